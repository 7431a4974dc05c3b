// Forward attention with fp8 (OCP e4m3fn) Q, K and V on gfx950.
//
// The skill guide's Workflow 3 (FlashAttention-3's FP8 forward): inputs cast
// to float8_e4m3fn, forward only.  Both contractions run on
// v_mfma_f32_32x32x64_f8f6f4 (fp8 in, fp32 accumulate):
//
//   S^T = K_j Q^T      A = K rows from LDS (32 bytes of d per lane), B = Q
//                      held in registers; scores scaled by
//                      scale * q_descale * k_descale.
//   online softmax     running max m in log2 units, weights
//                      P = 2^(S c - m) formed against m as it stands and
//                      only re-formed after raising m when some weight
//                      might exceed 448 (e4m3fn's largest value); fp32 row
//                      sums of the unrounded weights.
//   O^T += V_j^T P^T   P rounded to e4m3fn with v_cvt_pk_fp8_f32 straight
//                      from the S^T accumulator into the B operand; V^T
//                      read from the untransposed V tile with
//                      ds_read_b64_tr_b8.
//
// Two schedules of the key loop (Fp8Cfg), as in the 16-bit forward.
// Interleaved, for small grids: step j issues the PV MFMAs of tile j-1 and
// the QK MFMAs of tile j+1 among the exponentials of tile j, so one wave
// keeps its matrix core fed from its own instruction stream.  Phased, for
// grids that fill the chip: the weights of tile j, then PV(j) and S(j+1),
// with more waves per SIMD filling each other's phases.
//
// O = O^T * v_descale / l in bf16, LSE fp32.  One workgroup of 4 waves owns
// 128 queries (32 per wave, a query per lane); key tiles of 64 stream
// HBM -> LDS through a ring of 3 or 4 slots.  Causal masks, sliding windows and
// fewer K/V heads work as in the 16-bit forward.
//
// Operand layouts (measured on gfx950): the A and B operands of the fp8 MFMA
// use the same k order per lane half, so any consistent assignment of keys
// (or d) to the 32 byte slots of a lane works.  ds_read_b64_tr_b8 gives, in
// each group of 16 lanes, lane l as element j the byte l % 8 of the 8-byte
// word addressed by lane 2j + l / 8 of the group.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kW8 = 4;         // waves per workgroup
constexpr int kT8 = 64 * kW8;  // threads
constexpr int kBN8 = 64;       // keys per tile: one 64-deep k step of P V
constexpr int kQW8 = 32;       // queries per wave
constexpr int kBM8 = kW8 * kQW8;

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// LDS tile [64 rows][D bytes]: 16-byte chunk c of row r lives at chunk
// c ^ swz8(r).  Two read patterns must be free of bank conflicts (64 banks
// of 4 bytes; a ds_read_b128 serves 16 lanes per cycle, a 64-bit read 32):
//   K operand (ds_read_b128): 16 consecutive rows, one chunk;
//   V^T operand (ds_read_b64_tr_b8): a half-wave reads the 8 rows
//     {0..3, 8..11} (or {4..7, 12..15}) + 16 u of two adjacent chunks.
// At d = 128 two rows share a 256-byte bank line; with e = (r >> 1) & 7 the
// swizzle g(e) = 2 (e & 1) + (e & 4) + ((e >> 1) & 1) is a permutation of
// 0..7 (K reads: the 8 rows of one parity land on 8 distinct chunks) whose
// bits 1-2 take all four values on e in {0, 1, 4, 5} and on {2, 3, 6, 7}
// (transposing reads: the 2 x 8 chunks of a half-wave are distinct).  The
// plain e, used before, put chunk pairs of rows 0 and 2 on one bank group.
// At d = 64 four rows share a bank line and (r >> 2) & 3 satisfies both.
template <int D>
__device__ __forceinline__ int swz8(int r) {
  if constexpr (D == 128) {
    const int e = (r >> 1) & 7;
    return ((e & 1) << 1) | (e & 4) | ((e >> 1) & 1);
  } else {
    return (r >> 2) & 3;
  }
}
template <int D>
__device__ __forceinline__ int off8(int r, int byte) {
  return r * D + ((((byte >> 4) ^ swz8<D>(r)) << 4) | (byte & 15));
}

// 64 rows of a [N][D]-byte tensor into the swizzled tile; lane i of a wave
// instruction fills LDS bytes 16*i .. 16*i+15 of its block (1 KiB).
template <int D>
struct Tile8Copy {
  static constexpr int CH = D / 16;
  static constexpr int RPI = 64 / CH;
  static constexpr int NI = kBN8 / RPI / kW8;
  static_assert(NI >= 1 && NI * RPI * kW8 == kBN8, "tile split");
  static __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, uint32_t row_bytes, uint32_t tile_off,
                                               uint8_t* lds, int lane, int wave) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = (wave * NI + i) * RPI + lane / CH;
      const int c = (lane % CH) ^ swz8<D>(r);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(lds + (wave * NI + i) * RPI * D),
                                               16, (uint32_t)r * row_bytes + (uint32_t)(c * 16), tile_off, 0, 0);
    }
  }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc8(const uint8_t* base, int n, int64_t stride, int d) {
  const uint32_t bytes = rsrc_bytes((int64_t)(n - 1) * stride + d);
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, __builtin_bit_cast(int, bytes), 0x00020000);
}

__device__ __forceinline__ u32x4 lds16(const uint8_t* base, int off) { return *(const u32x4*)(base + off); }
__device__ __forceinline__ i32x2 lds_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(p));
}

// Per-lane LDS byte offsets within one tile slot.  K operand: row col
// (+32 per key block, which keeps the swizzle), bytes 64 ks + 32 half + 16 hl.
// V^T operand (transposing reads): the lane's row for read u = 0 (+16 rows
// per u, again swizzle-invariant), columns 32 db + 16 (g % 2) + 8 (lane % 2).
template <int D>
struct Tile8Addr {
  int k[D / 64][2];
  int v[D / 32];
  __device__ __forceinline__ void init(int lane) {
    const int col = lane & 31, half = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks)
#pragma unroll
      for (int hl = 0; hl < 2; ++hl) k[ks][hl] = off8<D>(col, 64 * ks + 32 * half + 16 * hl);
    const int g = lane >> 4, pl = lane & 15, je = pl >> 1;
    const int row = 8 * (je >> 2) + 4 * (g >> 1) + (je & 3);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) v[db] = off8<D>(row, 32 * db + 16 * (g & 1) + 8 * (pl & 1));
  }
};

// The A operands of S^T = K Q^T for one K tile: [key block][k step].
template <int D>
__device__ __forceinline__ void load_k8(const uint8_t* __restrict__ Kt, const Tile8Addr<D>& ta,
                                        i32x8 (&ka)[2][D / 64]) {
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks) {
      const u32x4 lo = lds16(Kt, ta.k[ks][0] + 32 * mb * D);
      const u32x4 hi = lds16(Kt, ta.k[ks][1] + 32 * mb * D);
      ka[mb][ks] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2],
                         (int)hi[3]};
    }
}

// S^T (64 keys x 32 queries, two 32-key blocks) from loaded K operands.
template <int D>
__device__ __forceinline__ void scores8(const i32x8 (&ka)[2][D / 64], const i32x8 (&qf)[D / 64], f32x16 (&s)[2]) {
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    s[mb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks) s[mb] = mfma_fp8(ka[mb][ks], qf[ks], s[mb]);
  }
}

// The A operands of O^T += V^T P^T for one V tile, per 32-wide d block:
// slot 8u + e of a lane holds key 32(u/2) + 16(u%2) + 8(e/4) + 4 half + e%4.
template <int D>
__device__ __forceinline__ void load_v8(const uint8_t* __restrict__ Vt, const Tile8Addr<D>& ta,
                                        i32x8 (&va)[D / 32]) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const i32x2 t = lds_tr8(Vt + ta.v[db] + 16 * u * D);
      va[db][2 * u] = t[0];
      va[db][2 * u + 1] = t[1];
    }
}

constexpr float kP8Max = 448.0f;  // largest finite e4m3fn

__device__ __forceinline__ void wait_lds_reads() { __builtin_amdgcn_s_waitcnt(0xC07F); }  // lgkmcnt(0)

// -inf for the scores of tile j that query qi does not admit (only tiles
// crossing the key tail or an edge of this wave's band).
template <bool BAND>
__device__ __forceinline__ void mask8(f32x16 (&s)[2], int j0, int Nk, int wl, int wr, int qw0, int qi, int half) {
  if ((j0 + kBN8 > Nk) ||
      (BAND && ((wr >= 0 && j0 + kBN8 - 1 > qw0 + wr) || (wl >= 0 && j0 < qw0 + kQW8 - 1 - wl)))) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + 32 * mb + acc_row(half, r);
        if (key >= Nk || (BAND && ((wr >= 0 && key > qi + wr) || (wl >= 0 && key < qi - wl))))
          s[mb][r] = -__builtin_inff();
      }
  }
}

// One step of the software-pipelined loop, for tile j:
//
//   O^T += V_{j-1}^T P_{j-1}^T   (P and the V operands carried in registers
//                                 from the previous step)
//   P_j = 2^(S_j c - m)          (VALU)
//   S_{j+1} = K_{j+1} Q^T        (into the registers of S_j once read)
//
// The eight MFMAs are spread through the ~100 VALU instructions of the
// weights, so a wave keeps its matrix core busy while it issues its own
// exponentials; the other wave on the SIMD fills the gaps.  Slot t mod 4
// of the ring holds tile jt0 + t; the step fills the slot of tile j+3
// (that of tile j-1, whose V operands are already in registers).
//
// The weights are formed against the running maximum m as it stands.  Only
// if some lane's sum of its 16 weights of a row exceeds 448 (a weight
// might not fit e4m3fn), or m is unset (m = -1e30 makes every admitted
// weight +inf), does the wave take the slow path: S_j again from K_j
// (still in its slot), row maximum, raise m, rescale O^T (which by then
// holds V_{j-1} P_{j-1}) and l, weights again.  So m never lags the row
// maximum by more than log2(448) and the fast path needs no maximum.
template <int D, bool BAND, bool FIRST>
__device__ __forceinline__ void fwd8_step(int j, int n_kt, f32x16 (&s)[2], i32x8& pf, i32x8 (&va)[D / 32],
                                          const uint8_t* __restrict__ Kj, const uint8_t* __restrict__ Kn,
                                          const uint8_t* __restrict__ Vj, uint8_t* __restrict__ Kdst,
                                          uint8_t* __restrict__ Vdst, __amdgpu_buffer_rsrc_t krs,
                                          __amdgpu_buffer_rsrc_t vrs, uint32_t krow, uint32_t vrow,
                                          const i32x8 (&qf)[D / 64], f32x16 (&acc)[D / 32], float& m, float& l,
                                          int Nk, int wl, int wr, int qw0, float c, int lane, int wave,
                                          const Tile8Addr<D>& ta) {
  using TC = Tile8Copy<D>;
  constexpr int DB = D / 32;
  const int j0 = j * kBN8;
  const int half = lane >> 5;
  const int qi = qw0 + (lane & 31);

  if (j + 3 < n_kt) {
    TC::issue(krs, krow, (uint32_t)(j + 3) * kBN8 * krow, Kdst, lane, wave);
    TC::issue(vrs, vrow, (uint32_t)(j + 3) * kBN8 * vrow, Vdst, lane, wave);
  }
  mask8<BAND>(s, j0, Nk, wl, wr, qw0, qi, half);

  // K(j+1) operands (reading K(j+1) when j+1 = n_kt reads a stale slot
  // whose scores are never used; it keeps the MFMAs in one block with the
  // exponentials)
  i32x8 ka[2][D / 64];
  load_k8<D>(Kn, ta, ka);
  __builtin_amdgcn_sched_barrier(0);

  // The eight MFMAs, each followed by a share of the weights' VALU work, in
  // chunks the scheduler may not reorder:
  //   PV(j-1) per d block (operands ready), with the V(j) reads that
  //   replace its operands and the weights of key block 0;
  //   S(j+1) block 0 (s[0] is consumed), with the exponent arguments of all
  //   of key block 1 and half its exponentials;
  //   S(j+1) block 1 (s[1] is consumed), with the rest.
  constexpr int KS = D / 64;
  float p[2][16];
  float x1[16];
  float ls0 = 0.f, ls1 = 0.f;
  const float mneg = -m;
  auto w0 = [&](int r) {
    p[0][r] = exp2_fast(__builtin_fmaf(s[0][r], c, mneg));
    ls0 += p[0][r];
  };
  if constexpr (FIRST) {
#pragma unroll
    for (int r = 0; r < 16; ++r) w0(r);
  } else {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      acc[db] = mfma_fp8(va[db], pf, acc[db]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const i32x2 t = lds_tr8(Vj + ta.v[db] + 16 * u * D);
        va[db][2 * u] = t[0];
        va[db][2 * u + 1] = t[1];
      }
#pragma unroll
      for (int r = db * (16 / DB); r < (db + 1) * (16 / DB); ++r) w0(r);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    s[0] = ks == 0 ? mfma_fp8(ka[0][0], qf[0], f32x16{}) : mfma_fp8(ka[0][ks], qf[ks], s[0]);
#pragma unroll
    for (int r = ks * (16 / KS); r < (ks + 1) * (16 / KS); ++r) x1[r] = __builtin_fmaf(s[1][r], c, mneg);
#pragma unroll
    for (int r = ks * (8 / KS); r < (ks + 1) * (8 / KS); ++r) {
      p[1][r] = exp2_fast(x1[r]);
      ls1 += p[1][r];
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    s[1] = ks == 0 ? mfma_fp8(ka[1][0], qf[0], f32x16{}) : mfma_fp8(ka[1][ks], qf[ks], s[1]);
#pragma unroll
    for (int r = 8 + ks * (8 / KS); r < 8 + (ks + 1) * (8 / KS); ++r) {
      p[1][r] = exp2_fast(x1[r]);
      ls1 += p[1][r];
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (FIRST) {  // the V(j) operands, for the epilogue or the next step
    load_v8<D>(Vj, ta, va);
  }
  float ls = ls0 + ls1;
  if (__any(!(ls <= kP8Max))) {  // rare (also catches +inf and NaN sums)
    asm volatile("" ::: "memory");
    f32x16 so[2];
    {
      i32x8 kj[2][D / 64];
      load_k8<D>(Kj, ta, kj);
      scores8<D>(kj, qf, so);
    }
    mask8<BAND>(so, j0, Nk, wl, wr, qw0, qi, half);
    float mx = so[0][0];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, so[mb][r]);
    const float mnew = fmaxf(m, max_pair32(mx) * c);
    const float alpha = exp2_fast(m - mnew);
    m = mnew;
    l *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] *= alpha;
    const float mneg2 = -m;
    ls = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[mb][r] = exp2_fast(__builtin_fmaf(so[mb][r], c, mneg2));
        ls += p[mb][r];
      }
  }
  l += ls;

  // P_j rounded into the B operand: byte 16 mb + r holds the key of
  // accumulator register r of block mb, matching load_v8's slots (both
  // halves of each word are written, so the old contents pass through
  // unused instead of a zeroed register)
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; r += 4) {
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[mb][r], p[mb][r + 1], pf[4 * mb + r / 4], false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(p[mb][r + 2], p[mb][r + 3], w, true);
      pf[4 * mb + r / 4] = w;
    }
  // the V reads must have left LDS before the barrier, after which tile
  // j+4 may land in the slot
  wait_lds_reads();

  // tile j+2 must have landed (its K is read next step); tile j+3 may fly on
  if (j + 3 < n_kt) {
    wait_vmcnt<2 * TC::NI>();
  } else {
    wait_loads();
  }
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// Two schedules of the key loop, as in the 16-bit forward: interleaved
// (fwd8_step; two waves per SIMD at d = 128, where a wave needs ~234
// registers, three at d = 64) for grids too small to give every CU two
// workgroups, and phased (fwd8_step_phased: the weights of tile j, then
// PV(j) and S(j+1); ~150 registers at d = 128, so three waves share a SIMD
// with a 3-slot ring, four at d = 64) for the others.
template <int D, bool PHASED>
struct Fp8Cfg {
  static constexpr int WAVES_PER_SIMD = PHASED ? (D == 64 ? 4 : 3) : (D == 64 ? 3 : 2);
  static constexpr int NBUF = PHASED && D == 128 ? 3 : 4;
};
// Workgroups from which the phased schedule is used.  Measured crossover:
// at d = 128 the interleaved schedule is 8% faster at 512 workgroups and
// the phased one 5% faster at 768; at d = 64 the interleaved one is 8-9%
// faster up to 1024.
template <int D>
constexpr int64_t kPhasedMinBlocks8 = D == 64 ? 1536 : 768;

// One step of the phased schedule for tile j: the weights of S(j) (the
// rare rescale finds S(j) still in registers), P(j) rounded into the B
// operand, then PV(j) and S(j+1) with their LDS operands read a few MFMAs
// ahead.  Step j requests tile j + NBUF - 1 into the slot of tile j-1.
template <int D, bool BAND>
__device__ __forceinline__ void fwd8_step_phased(int j, int n_kt, f32x16 (&s)[2], const uint8_t* __restrict__ Vj,
                                                 const uint8_t* __restrict__ Kn, uint8_t* __restrict__ Kdst,
                                                 uint8_t* __restrict__ Vdst, __amdgpu_buffer_rsrc_t krs,
                                                 __amdgpu_buffer_rsrc_t vrs, uint32_t krow, uint32_t vrow,
                                                 const i32x8 (&qf)[D / 64], f32x16 (&acc)[D / 32], float& m, float& l,
                                                 int Nk, int wl, int wr, int qw0, float c, int lane, int wave,
                                                 const Tile8Addr<D>& ta) {
  using TC = Tile8Copy<D>;
  constexpr int DB = D / 32;
  constexpr int KS = D / 64;
  constexpr int PD = Fp8Cfg<D, true>::NBUF - 1;
  const int j0 = j * kBN8;
  const int half = lane >> 5;
  const int qi = qw0 + (lane & 31);
  if (j + PD < n_kt) {
    TC::issue(krs, krow, (uint32_t)(j + PD) * kBN8 * krow, Kdst, lane, wave);
    TC::issue(vrs, vrow, (uint32_t)(j + PD) * kBN8 * vrow, Vdst, lane, wave);
  }
  mask8<BAND>(s, j0, Nk, wl, wr, qw0, qi, half);
  // P(j) rounded into the B operand as it is formed: byte 16 mb + r holds
  // the key of accumulator register r of block mb, matching load_v8's slots
  i32x8 pf;
  float ls = 0.f;
  auto weights8 = [&](float mneg) {
    ls = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        float w4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w4[e] = exp2_fast(__builtin_fmaf(s[mb][r + e], c, mneg));
          ls += w4[e];
        }
        // both halves of the word are written: the first conversion's
        // "old" operand is w4[0]'s own register (dead after it), not a
        // zero that would cost a move
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(w4[0], w4[1], __builtin_bit_cast(int, w4[0]), false);
        pf[4 * mb + r / 4] = __builtin_amdgcn_cvt_pk_fp8_f32(w4[2], w4[3], w, true);
      }
  };
  weights8(-m);
  if (__any(!(ls <= kP8Max))) {  // rare (also catches +inf and NaN sums)
    asm volatile("" ::: "memory");
    float mx = s[0][0];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][r]);
    const float mnew = fmaxf(m, max_pair32(mx) * c);
    const float alpha = exp2_fast(m - mnew);
    m = mnew;
    l *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] *= alpha;
    weights8(-m);
  }
  l += ls;
  __builtin_amdgcn_sched_barrier(0);
  // PV(j), then S(j+1) (after the last tile: a stale slot, never used)
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    i32x8 va;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const i32x2 t = lds_tr8(Vj + ta.v[db] + 16 * u * D);
      va[2 * u] = t[0];
      va[2 * u + 1] = t[1];
    }
    acc[db] = mfma_fp8(va, pf, acc[db]);
  }
  {
    i32x8 ka[2][KS];
    load_k8<D>(Kn, ta, ka);
    scores8<D>(ka, qf, s);
  }
  sched_reads_ahead<DB + 2 * KS, 4 * DB + 4 * KS>();
  // tile j+2 (read next step) must have landed; later ones may fly on
  if (j + PD < n_kt) {
    wait_vmcnt<(PD - 2) * 2 * TC::NI>();
  } else {
    wait_loads();
  }
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

template <int D, bool BAND, bool PHASED>
__global__ __launch_bounds__(kT8) __attribute__((amdgpu_waves_per_eu(Fp8Cfg<D, PHASED>::WAVES_PER_SIMD, Fp8Cfg<D, PHASED>::WAVES_PER_SIMD))) void fwd_fp8_kernel(Fp8Params p) {
  constexpr int KS = D / 64;
  constexpr int DB = D / 32;
  constexpr int TILE = kBN8 * D;
  constexpr int NBUF = Fp8Cfg<D, PHASED>::NBUF;
  using TC = Tile8Copy<D>;

  struct Smem {  // one LDS object (see the 16-bit forward)
    uint8_t k[NBUF][TILE];
    uint8_t v[NBUF][TILE];
  };
  __shared__ __attribute__((aligned(1024))) Smem sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int BH = p.B * p.H;
  const int n_qt = (p.Nq + kBM8 - 1) / kBM8;
  const int t = blockIdx.x;
  const int qt = n_qt - 1 - t / BH;  // heaviest query tiles first
  const int bh = t - (t / BH) * BH;
  const int b = bh / p.H, h = bh - b * p.H;
  const int hk = h / p.G;
  const int q0 = qt * kBM8;
  const int qw0 = q0 + wave * kQW8;
  const int qi = qw0 + col;

  const uint8_t* qp = p.q + b * p.sq.b + h * p.sq.h;
  const uint8_t* kp = p.k + b * p.sk.b + hk * p.sk.h;
  const uint8_t* vp = p.v + b * p.sv.b + hk * p.sv.h;

  int kend = p.Nk, jt0 = 0;
  if (BAND) {
    const int qlast = min(q0 + kBM8, p.Nq) - 1;
    if (p.wr >= 0) kend = min(p.Nk, qlast + p.wr + 1);
    if (p.wl >= 0) jt0 = max(0, q0 - p.wl) / kBN8;
  }
  const int n_kt = (kend + kBN8 - 1) / kBN8;

  const __amdgpu_buffer_rsrc_t krs = head_rsrc8(kp, p.Nk, p.sk.s, D);
  const __amdgpu_buffer_rsrc_t vrs = head_rsrc8(vp, p.Nk, p.sv.s, D);
  const uint32_t krow = (uint32_t)p.sk.s, vrow = (uint32_t)p.sv.s;

  // Q^T as the B operand: lane holds Q[qi][64 ks + 32 half .. +31]
  i32x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 lo = u32x4{0, 0, 0, 0}, hi = u32x4{0, 0, 0, 0};
    if (qi < p.Nq) {
      lo = *(const u32x4*)(qp + qi * p.sq.s + 64 * ks + 32 * half);
      hi = *(const u32x4*)(qp + qi * p.sq.s + 64 * ks + 32 * half + 16);
    }
    qf[ks] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
#pragma unroll
  for (int t0 = 0; t0 < NBUF - 1; ++t0) {
    const int jj = jt0 + t0;
    if (jj < n_kt) {
      TC::issue(krs, krow, (uint32_t)jj * kBN8 * krow, sm.k[t0], lane, wave);
      TC::issue(vrs, vrow, (uint32_t)jj * kBN8 * vrow, sm.v[t0], lane, wave);
    }
  }
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  float m = -1e30f, l = 0.f;
  const float c = p.c;
  Tile8Addr<D> ta;
  ta.init(lane);

  // tiles jt0 and jt0+1 landed (S(jt0) now, V(jt0) and K(jt0+1) in the first step)
  if (n_kt - jt0 >= NBUF - 1) {
    wait_vmcnt<(NBUF - 3) * 2 * TC::NI>();
  } else {
    wait_loads();
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qf[ks] ^= (int)p.qflip;
  lds_barrier();

  if constexpr (PHASED) {
    if (jt0 < n_kt) {
      f32x16 sa[2];
      {
        i32x8 ka[2][KS];
        load_k8<D>(sm.k[0], ta, ka);
        scores8<D>(ka, qf, sa);
      }
      auto wrap = [](int x) { return x >= NBUF ? x - NBUF : x; };
      int j = jt0;
      // Whole turns of the ring with every slot a constant, so the LDS
      // addresses are immediate offsets (8 fewer VALU instructions per
      // tile; 3% measured at 16K d = 128), then the rest one by one.
      for (; j + NBUF <= n_kt; j += NBUF) {
#pragma unroll
        for (int r = 0; r < NBUF; ++r)
          fwd8_step_phased<D, BAND>(j + r, n_kt, sa, sm.v[r], sm.k[(r + 1) % NBUF], sm.k[(r + NBUF - 1) % NBUF],
                                    sm.v[(r + NBUF - 1) % NBUF], krs, vrs, krow, vrow, qf, acc, m, l, p.Nk, p.wl, p.wr,
                                    qw0, c, lane, wave, ta);
      }
      int sl = (j - jt0) % NBUF;  // slot of tile j
      for (; j < n_kt; ++j) {
        const int sp = wrap(sl + NBUF - 1);  // slot of tile j-1
        fwd8_step_phased<D, BAND>(j, n_kt, sa, sm.v[sl], sm.k[wrap(sl + 1)], sm.k[sp], sm.v[sp], krs, vrs, krow, vrow,
                                  qf, acc, m, l, p.Nk, p.wl, p.wr, qw0, c, lane, wave, ta);
        sl = wrap(sl + 1);
      }
    }
  } else if (jt0 < n_kt) {
    // Tile jt0 + t lives in slot t mod 4.
    f32x16 sa[2];
    i32x8 pf = i32x8{};
    i32x8 va[DB];
    {
      i32x8 ka[2][KS];
      load_k8<D>(sm.k[0], ta, ka);
      scores8<D>(ka, qf, sa);
    }
    fwd8_step<D, BAND, true>(jt0, n_kt, sa, pf, va, sm.k[0], sm.k[1], sm.v[0], sm.k[3], sm.v[3], krs, vrs, krow,
                             vrow, qf, acc, m, l, p.Nk, p.wl, p.wr, qw0, c, lane, wave, ta);
    for (int j = jt0 + 1; j < n_kt; ++j) {
      const int sl = (j - jt0) & 3;
      fwd8_step<D, BAND, false>(j, n_kt, sa, pf, va, sm.k[sl], sm.k[(sl + 1) & 3], sm.v[sl], sm.k[(sl + 3) & 3],
                                sm.v[(sl + 3) & 3], krs, vrs, krow, vrow, qf, acc, m, l, p.Nk, p.wl, p.wr, qw0, c,
                                lane, wave, ta);
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = mfma_fp8(va[db], pf, acc[db]);
  }

  // ---- epilogue: O = O^T * v_descale / l in bf16, LSE
  const float lt = sum_pair32(l);
  if (qi < p.Nq) {
    uint16_t* op = p.o + b * p.so.b + h * p.so.h + qi * p.so.s;
    const float f = lt > 0.f ? p.vscale / lt : 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + 8 * g4 + 4 * half;
        const f32x16& a = acc[db];
        *(u32x2*)(op + d0) = u32x2{pack2<DT_BF16>(a[4 * g4 + 0] * f, a[4 * g4 + 1] * f),
                                   pack2<DT_BF16>(a[4 * g4 + 2] * f, a[4 * g4 + 3] * f)};
      }
    if (half == 0) p.lse[(int64_t)bh * p.Nq + qi] = lt > 0.f ? (m + log2_fast(lt)) * kLn2 : -__builtin_inff();
  }
}

template <int D, bool BAND>
hipError_t launch8(const Fp8Params& p, hipStream_t stream) {
  const int n_qt = (p.Nq + kBM8 - 1) / kBM8;
  const int64_t blocks = (int64_t)n_qt * p.B * p.H;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (blocks >= kPhasedMinBlocks8<D>) {
    hipLaunchKernelGGL((fwd_fp8_kernel<D, BAND, true>), dim3((unsigned)blocks), dim3(kT8), 0, stream, p);
  } else {
    hipLaunchKernelGGL((fwd_fp8_kernel<D, BAND, false>), dim3((unsigned)blocks), dim3(kT8), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8Params& p, int d, bool banded, hipStream_t stream) {
  if (d == 64) return banded ? launch8<64, true>(p, stream) : launch8<64, false>(p, stream);
  return banded ? launch8<128, true>(p, stream) : launch8<128, false>(p, stream);
}

}  // namespace fa
