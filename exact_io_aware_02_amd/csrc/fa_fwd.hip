// Forward attention kernel for gfx950.
//
// One workgroup of 4 waves owns BM = 128 query rows of one (batch, head);
// each wave owns 32 of them and their softmax state, so the row max and row
// sum never leave the wave (FlashAttention-2's point of less communication
// between warps, refbase Q&A on FA2's improvements).  K/V tiles of BN = 32
// keys stream from HBM straight into LDS (buffer_load ... lds, no staging
// registers) through a ring of 4 slots (3 in the phased schedule at
// d = 128, see FwdCfg).  Per tile and wave:
//
//   S^T = K_j Q^T          32x32x16 MFMAs; A = K rows from LDS, B = Q held
//                          in registers for the whole loop.  Each lane
//                          then holds 16 keys x 1 query of every 32x32
//                          block, so the row max and sum are in-lane plus
//                          one exchange with lane i^32.
//   online softmax         P = 2^(S*c - m) with c = |scale| log2 e against
//                          the running max m as it stands; l += sum P.
//                          Only when some lane's sum of its 16 weights of a
//                          row exceeds 2^15 (or m is unset) is m raised to
//                          the row max and O^T, l rescaled by 2^(m - m');
//                          a stale m changes no result (O = O^T / l uses
//                          the same m in both) and needs no per-element
//                          maximum.
//   O^T += V_j^T P^T       A = V^T via ds_read_b64_tr_b16 from the
//                          untransposed V tile; B = P^T repacked in place
//                          from the S^T accumulator (no LDS round trip).
//
// Two schedules of the key loop (FwdCfg).  Interleaved, for small grids:
// step j issues the PV MFMAs of tile j-1 and the S MFMAs of tile j+1 among
// the exponentials of tile j, in chunks the scheduler keeps in order, so
// one wave's matrix core and VALU work at the same time (the overlap FA3
// gets from asynchrony on Hopper, glossary article's FA-3 section); the V
// operands and P of tile j-1 stay in registers across the step boundary.
// Phased, for grids that fill the chip: the exponentials of tile j, then
// PV(j) and S(j+1); with fewer registers three waves (d = 128) or four
// (d = 64) share a SIMD and fill each other's phases.
//
// Epilogue: O = O^T / l, LSE = (m + log2 l) * ln 2 (O = 0, LSE = -inf for
// a row that admits no key).  Masks: query i admits keys i - wl .. i + wr
// (a negative bound is absent; causal is wr = 0; the skill guide's
// Workflow 2 step 3 sliding window is (wl, wr)).  Key tiles outside every
// query's band of the workgroup are never loaded; tiles that cross an edge
// of a wave's band, or the key tail, are masked elementwise.  With fewer
// K/V heads (the same step's multi-query attention) query head h reads
// K/V head h / G.
//
// This is the blocking / online-softmax / single merged write-back
// pipeline of the glossary article's "FlashAttention の仕組み" figure
// (steps 1-4) and its "Online Softmax" section, with tile sizes and data
// movement chosen for CDNA4 (64-wide waves, 160 KB LDS, 32x32x16 MFMA).
#include <algorithm>
#include <atomic>
#include <vector>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBN = 32;            // keys per pipeline tile
// Each wave owns 32 queries (one 32-query MFMA column block): 64 per wave
// halves the LDS bytes per MFMA but needs ~260 registers at d = 128 and
// ~220 at d = 64, and measured slower at both.
constexpr int kQW = 32;                // queries per wave
constexpr int kBM = kWaves * kQW;      // queries per workgroup

// Two schedules of the key loop (see fwd_step and fwd_step_phased):
//  * interleaved: a wave spreads the PV and S MFMAs of neighbouring tiles
//    through the exponentials of the current one, so it keeps its matrix
//    core fed by itself.  This needs the V operands, P and (at d = 128)
//    S(j+1) carried in registers (~210 at d = 128, two waves per SIMD;
//    ~140 at d = 64, three) and is used for grids too small to give every
//    CU two workgroups;
//  * phased: the exponentials, then the MFMAs, with the waves sharing a
//    SIMD filling each other's phases.  It needs ~160 registers at d = 128
//    (three waves per SIMD, with a 3-slot ring so three workgroups fit the
//    LDS) and ~105 at d = 64 (four).  On full grids it measured 7-12%
//    faster at d = 128 and 2-8% at d = 64; on small grids, where a SIMD
//    has one wave, 8% slower.
template <int D, bool PHASED>
struct FwdCfg {
  static constexpr int WAVES_PER_SIMD = PHASED ? (D == 64 ? 4 : 3) : (D == 64 ? 3 : 2);
  static constexpr int NBUF = PHASED && D == 128 ? 3 : 4;  // K/V ring slots
  // interleaved, d = 128: S(j+1) in registers of its own; otherwise it
  // overwrites S(j) after the weights
  static constexpr bool SEP_S = !PHASED && D == 128;
};
// Workgroups from which the phased schedule is used.  Measured crossover:
// at d = 128 the interleaved schedule is 6-8% faster up to 768 workgroups
// and the phased one faster from 1024; at d = 64 the interleaved one is
// 5-15% faster up to 1024 and the two are even at 1536.
template <int D>
constexpr int64_t kPhasedMinBlocks = D == 64 ? 1536 : 1024;

static_assert(kBN == 32, "K/V tiles are the 32-row tiles of fa_device.h");
template <int D, int NW = kWaves>  // NW: the waves of a key group, which share its tile copies
struct TileCopy {
  static constexpr int NI = TileLayout<D>::template copy_insts<NW>();  // instructions per wave per tile
  static __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, uint32_t row_bytes, uint32_t tile_byte_off,
                                               uint16_t* lds, int lane, int wave) {
    TileLayout<D>::template issue<NW>(rs, row_bytes, tile_byte_off, lds, lane, wave);
  }
};

template <int DT>
__device__ __forceinline__ float dot2_sum(uint32_t packed, float acc);
template <>
__device__ __forceinline__ float dot2_sum<DT_F16>(uint32_t packed, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, packed), __builtin_bit_cast(f16x2, 0x3c003c00u), acc, false);
}
template <>
__device__ __forceinline__ float dot2_sum<DT_BF16>(uint32_t packed, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), __builtin_bit_cast(bf16x2, 0x3f803f80u),
                                         acc, false);
}

template <int kNQB>
struct RowState {
  float m[kNQB];  // running max, log2 units (scaled by c)
  float l[kNQB];  // this lane's partial row sum (lane i^32 holds the rest)
};

// -inf for the scores of tile j (keys j0 ..) that a query does not admit
// (only tiles crossing the key tail or an edge of this wave's band).
template <bool BAND, int kNQB>
__device__ __forceinline__ void mask_tile(f32x16 (&s)[kNQB], int j0, int Nk, int wl, int wr, int qw0, int col,
                                          int half) {
  constexpr int QW = 32 * kNQB;
  if ((j0 + kBN > Nk) ||
      (BAND && ((wr >= 0 && j0 + kBN - 1 > qw0 + wr) || (wl >= 0 && j0 < qw0 + QW - 1 - wl)))) {
#pragma unroll
    for (int nb = 0; nb < kNQB; ++nb) {
      const int qi = qw0 + 32 * nb + col;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + acc_row(half, r);
        if (key >= Nk || (BAND && ((wr >= 0 && key > qi + wr) || (wl >= 0 && key < qi - wl))))
          s[nb][r] = -__builtin_inff();
      }
    }
  }
}

__device__ __forceinline__ void wait_lds_reads() { __builtin_amdgcn_s_waitcnt(0xC07F); }  // lgkmcnt(0)

// Weights of tile j: P = 2^(S c - m) against the running maximum as it
// stands, the normaliser's partial sums (of the undropped weights),
// dropout, and the packing into the MFMA B operand, one packed word (two
// keys of one query block) at a time: word w = 4 kk + e of block nb holds
// accumulator registers 8 kk + 2 e and +1.
template <int DT, bool DROP>
__device__ __forceinline__ uint32_t weight_word(const f32x16& s, int w, float c, float mneg, float (&ls)[2],
                                                const u32x4& rnd, uint32_t thr) {
  const int r = 2 * w;
  float p0 = exp2_fast(__builtin_fmaf(s[r], c, mneg));
  float p1 = exp2_fast(__builtin_fmaf(s[r + 1], c, mneg));
  if constexpr (DT == DT_BF16 || DROP) {  // bf16 rounding (2^-9) is too coarse for the normaliser
    ls[0] = r == 0 ? p0 : ls[0] + p0;
    ls[1] = r == 0 ? p1 : ls[1] + p1;
  }
  if constexpr (DROP) {  // register r holds key 8*(r/4) + 4*half + r%4 of the tile
    if (((rnd[r >> 2] >> (8 * (r & 3))) & 0xffu) < thr) p0 = 0.f;
    if (((rnd[(r + 1) >> 2] >> (8 * ((r + 1) & 3))) & 0xffu) < thr) p1 = 0.f;
  }
  const uint32_t pw = pack2<DT>(p0, p1);
  if constexpr (DT == DT_F16 && !DROP) {  // fp16-rounded P is accurate enough: sum pairs in one op
    if (r == 0) ls[0] = ls[1] = 0.f;
    ls[w & 1] = dot2_sum<DT>(pw, ls[w & 1]);
  }
  return pw;
}

template <int DT, bool DROP>
__device__ __forceinline__ void weights(const f32x16& s, float c, float m, float (&ls)[2], u32x4 (&pfo)[2],
                                        const u32x4& rnd, uint32_t thr) {
#pragma unroll
  for (int w = 0; w < 8; ++w) pfo[w >> 2][w & 3] = weight_word<DT, DROP>(s, w, c, -m, ls, rnd, thr);
}

constexpr float kLaneSumMax = 32768.0f;  // 2^15: each weight fits fp16 and bf16

// One step of the software-pipelined loop, for tile j:
//
//   O^T += V_{j-1}^T P_{j-1}^T   (P and the V operands carried in registers
//                                 from the previous step)
//   P_j = 2^(S_j c - m)          (VALU)
//   S_{j+1} = K_{j+1} Q^T        (into the registers of S_j once read)
//
// The MFMAs of both products are spread through the VALU work of the
// weights in chunks the scheduler may not reorder, so one wave keeps its
// matrix core fed from its own instruction stream (the overlap of
// FA3's asynchrony, glossary article's FA-3 section, by scheduling).  The
// LDS ring has four slots, tile jt0 + t in slot t mod 4; step j fills the
// slot of tile j+3, that of tile j-1 whose V operands are already in
// registers.  The __restrict__ tile pointers tell the compiler these reads
// never alias the in-flight copy; the vmcnt wait and barrier at the end
// order the ring.
//
// The weights are formed against the running maximum m as it stands.
// Only if a lane's sum of its 16 weights of a row exceeds 2^15, or m is
// unset (m = -1e30 makes every admitted weight +inf), does the wave take
// the slow path: S_j again from K_j (still in its slot), row maximum,
// raise m, rescale O^T (which by then holds V_{j-1} P_{j-1}) and l,
// weights again.  The result is the same for any m (O = O^T / l uses one
// m for both); m only keeps the weights in range.
template <int D, int DT, bool BAND, bool DROP, bool FIRST, int kNQB = 1>
__device__ __forceinline__ void fwd_step(int j, int n_kt, f32x16 (&s)[kNQB], f32x16 (&sn)[kNQB], u32x4 (&pf)[2][kNQB],
                                         u32x4 (&va)[2][D / 32], const uint16_t* __restrict__ Kj,
                                         const uint16_t* __restrict__ Kn, const uint16_t* __restrict__ Vj,
                                         uint16_t* __restrict__ Kdst, uint16_t* __restrict__ Vdst,
                                         __amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs, uint32_t krow,
                                         uint32_t vrow, uint32_t ktb, uint32_t vtb, const u32x4 (&qf)[kNQB][D / 16],
                                         f32x16 (&acc)[D / 32][kNQB], RowState<kNQB>& st, int Nk, int wl, int wr,
                                         int qw0, float c, int lane, int wave, const TileLayout<D>& ta,
                                         const DropoutParams& dp, uint32_t bh) {
  using TC = TileCopy<D>;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  const int j0 = j * kBN;
  const int col = lane & 31, half = lane >> 5;

  if constexpr (FwdCfg<D, false>::SEP_S) {
    // K(j) is no longer read (S(j) stays in registers), so K runs four
    // tiles ahead: K(j+4) into K(j)'s slot, V(j+3) into V(j-1)'s
    if (j + 4 < n_kt) TC::issue(krs, krow, (uint32_t)(j + 4) * ktb, Kdst, lane, wave);
    if (j + 3 < n_kt) TC::issue(vrs, vrow, (uint32_t)(j + 3) * vtb, Vdst, lane, wave);
  } else {
    if (j + 3 < n_kt) {
      TC::issue(krs, krow, (uint32_t)(j + 3) * ktb, Kdst, lane, wave);
      TC::issue(vrs, vrow, (uint32_t)(j + 3) * vtb, Vdst, lane, wave);
    }
  }
  mask_tile<BAND>(s, j0, Nk, wl, wr, qw0, col, half);

  // K(j+1) operands (reading K(j+1) when j+1 = n_kt reads a stale slot
  // whose scores are never used; it keeps the MFMAs in one block with the
  // exponentials)
  constexpr bool kSep = FwdCfg<D, false>::SEP_S;
  constexpr int kKLead = 2;  // with kSep, K(j+1) operands are read this many chunks ahead of use
  u32x4 ka[KS];
  if constexpr (!kSep || FIRST) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ka[ks] = lds_rowmajor<D>(Kn, ta, ks);
  }
  u32x4 rnd[kNQB];
#pragma unroll
  for (int nb = 0; nb < kNQB; ++nb) {
    rnd[nb] = u32x4{0, 0, 0, 0};
    if constexpr (DROP)  // this lane's 16 keys of tile j: one generator call
      rnd[nb] = philox4x32_10(2u * (uint32_t)j + (uint32_t)half, (uint32_t)(qw0 + 32 * nb + col), bh, dp.offset,
                              dp.seed_lo, dp.seed_hi);
  }
  __builtin_amdgcn_sched_barrier(0);

  // PV(j-1) chunks, each with the V(j) reads that replace its operands and
  // an equal share of the weights' packed words; then the S(j+1) MFMAs,
  // which overwrite S(j) once every word has read it.
  float ls[kNQB][2];
  u32x4 pn[kNQB][2];
  float mneg[kNQB];
#pragma unroll
  for (int nb = 0; nb < kNQB; ++nb) mneg[nb] = -st.m[nb];
  constexpr int NW = 8 * kNQB;  // packed words per lane
  // With room for it (d = 128: one wave per SIMD), S(j+1) goes to separate
  // registers, so its MFMAs can share the weights' VALU work too: chunks of
  // two MFMAs (PV first, then S) and one packed word each.
  if constexpr (kSep && !FIRST) {
    constexpr int NPVM = 2 * DB * kNQB, NSM = KS * kNQB, NCH = (NPVM + NSM) / 2;
    constexpr int CPK = kNQB / 2 > 0 ? kNQB / 2 : 1;  // S chunks per k step (two MFMAs per chunk)
    static_assert(NCH == NW, "one packed word per chunk");
    static_assert(kNQB <= 2, "S chunk layout");
#pragma unroll
    for (int g = 0; g < NCH; ++g) {
      {  // K(j+1) operand of k step ks, kKLead k steps ahead of its MFMAs
        const int ks = (g - NPVM / 2) / CPK * (kNQB == 1 ? 2 : 1) + kKLead;
        if ((g - NPVM / 2) % CPK == 0 && ks >= 0 && ks < KS) {
          ka[ks] = lds_rowmajor<D>(Kn, ta, ks);
          if (kNQB == 1 && ks + 1 < KS) ka[ks + 1] = lds_rowmajor<D>(Kn, ta, ks + 1);
        }
        if (g == NPVM / 2 - 1) {  // the first k steps
#pragma unroll
          for (int k0 = 0; k0 < kKLead && k0 < KS; ++k0) ka[k0] = lds_rowmajor<D>(Kn, ta, k0);
        }
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int x = 2 * g + h2;
        if (x < NPVM) {  // x = ((kk DB) + db) kNQB + nb
          const int nb = x % kNQB, kd = x / kNQB, kk = kd / DB, db = kd % DB;
          acc[db][nb] = mfma32<DT>(va[kk][db], pf[kk][nb], acc[db][nb]);
          if (nb == kNQB - 1) va[kk][db] = lds_transposed_a<D>(Vj, ta, kk, db);
        } else {  // y = ks kNQB + nb
          const int y = x - NPVM, nb = y % kNQB, ks = y / kNQB;
          sn[nb] = mfma32<DT>(ka[ks], qf[nb][ks], ks == 0 ? f32x16{} : sn[nb]);
        }
      }
      const int nb = g / 8, w = g % 8;
      pn[nb][w >> 2][w & 3] = weight_word<DT, DROP>(s[nb], w, c, mneg[nb], ls[nb], rnd[nb], dp.thr);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else if constexpr (!FIRST) {
    constexpr int NPV = 2 * DB;
    static_assert(NW % NPV == 0, "words per chunk");
#pragma unroll
    for (int g = 0; g < NPV; ++g) {
      const int kk = g / DB, db = g % DB;
#pragma unroll
      for (int nb = 0; nb < kNQB; ++nb) acc[db][nb] = mfma32<DT>(va[kk][db], pf[kk][nb], acc[db][nb]);
      va[kk][db] = lds_transposed_a<D>(Vj, ta, kk, db);
#pragma unroll
      for (int x = g * (NW / NPV); x < (g + 1) * (NW / NPV); ++x) {
        const int nb = x / 8, w = x % 8;
        pn[nb][w >> 2][w & 3] = weight_word<DT, DROP>(s[nb], w, c, mneg[nb], ls[nb], rnd[nb], dp.thr);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
#pragma unroll
    for (int nb = 0; nb < kNQB; ++nb) weights<DT, DROP>(s[nb], c, st.m[nb], ls[nb], pn[nb], rnd[nb], dp.thr);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int db = 0; db < DB; ++db) va[kk][db] = lds_transposed_a<D>(Vj, ta, kk, db);
  }
  if constexpr (kSep && FIRST) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int nb = 0; nb < kNQB; ++nb) sn[nb] = mfma32<DT>(ka[ks], qf[nb][ks], ks == 0 ? f32x16{} : sn[nb]);
  } else if constexpr (!kSep) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int nb = 0; nb < kNQB; ++nb) s[nb] = mfma32<DT>(ka[ks], qf[nb][ks], ks == 0 ? f32x16{} : s[nb]);
    }
  }
  bool raise = false;
#pragma unroll
  for (int nb = 0; nb < kNQB; ++nb) raise |= !(ls[nb][0] + ls[nb][1] <= kLaneSumMax);
  if (__any(raise)) {  // rare (also catches +inf and NaN sums)
    asm volatile("" ::: "memory");
    f32x16 so[kNQB];
    if constexpr (kSep) {  // S(j) is still in s
#pragma unroll
      for (int nb = 0; nb < kNQB; ++nb) so[nb] = s[nb];
    } else {  // S(j) was overwritten: again from K(j), still in its slot
#pragma unroll
      for (int nb = 0; nb < kNQB; ++nb) so[nb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 a = lds_rowmajor<D>(Kj, ta, ks);
#pragma unroll
        for (int nb = 0; nb < kNQB; ++nb) so[nb] = mfma32<DT>(a, qf[nb][ks], so[nb]);
      }
      mask_tile<BAND>(so, j0, Nk, wl, wr, qw0, col, half);
    }
#pragma unroll
    for (int nb = 0; nb < kNQB; ++nb) {
      float mx = so[nb][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, so[nb][r]);
      const float mnew = fmaxf(st.m[nb], max_pair32(mx) * c);
      const float alpha = exp2_fast(st.m[nb] - mnew);
      st.m[nb] = mnew;
      st.l[nb] *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db][nb] *= alpha;
      weights<DT, DROP>(so[nb], c, st.m[nb], ls[nb], pn[nb], rnd[nb], dp.thr);
    }
  }
#pragma unroll
  for (int nb = 0; nb < kNQB; ++nb) {
    st.l[nb] += ls[nb][0] + ls[nb][1];
    pf[0][nb] = pn[nb][0];
    pf[1][nb] = pn[nb][1];
  }

  // the V reads must have left LDS before the barrier, after which tile
  // j+4 may land in the slot
  wait_lds_reads();

  if constexpr (FwdCfg<D, false>::SEP_S) {
    // K(j+2) and V(j+1) (read next step) must have landed; the copies
    // issued after them (K(j+3), V(j+2), K(j+4), V(j+3)) may fly on
    if (j + 4 < n_kt) {
      wait_vmcnt<4 * TC::NI>();
    } else {
      wait_loads();
    }
  } else {
    // tile j+2 must have landed (its K is read next step); tile j+3 may fly on
    if (j + 3 < n_kt) {
      wait_vmcnt<2 * TC::NI>();
    } else {
      wait_loads();
    }
  }
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// One step of the phased schedule, for tile j: the weights of tile j
// against the running maximum (VALU; the rare rescale finds S(j) still in
// registers), then PV(j) and S(j+1) (MFMA, their LDS operands read a few
// MFMAs ahead), which overwrite S(j).  The waves sharing a SIMD fill each
// other's phases.  The ring holds NBUF tiles; step j requests tile
// j + NBUF - 1 into the slot of tile j-1, read in full by the last step.
template <int D, int DT, bool BAND, bool DROP, int kNQB, int NW = kWaves, int NB = FwdCfg<D, true>::NBUF>
__device__ __forceinline__ void fwd_step_phased(int j, int n_kt, f32x16 (&s)[kNQB], const uint16_t* __restrict__ Vj,
                                            const uint16_t* __restrict__ Kn, uint16_t* __restrict__ Kdst,
                                            uint16_t* __restrict__ Vdst, __amdgpu_buffer_rsrc_t krs,
                                            __amdgpu_buffer_rsrc_t vrs, uint32_t krow, uint32_t vrow, uint32_t ktb,
                                            uint32_t vtb, const u32x4 (&qf)[kNQB][D / 16], f32x16 (&acc)[D / 32][kNQB],
                                            RowState<kNQB>& st, int Nk, int wl, int wr, int qw0, float c, int lane,
                                            int wave, const TileLayout<D>& ta, const DropoutParams& dp, uint32_t bh) {
  using TC = TileCopy<D, NW>;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  const int j0 = j * kBN;
  const int col = lane & 31, half = lane >> 5;
  constexpr int PD = NB - 1;  // tile j+PD goes to the slot of tile j-1
  if (j + PD < n_kt) {
    TC::issue(krs, krow, (uint32_t)(j + PD) * ktb, Kdst, lane, wave);
    TC::issue(vrs, vrow, (uint32_t)(j + PD) * vtb, Vdst, lane, wave);
  }
  mask_tile<BAND>(s, j0, Nk, wl, wr, qw0, col, half);
  u32x4 rnd[kNQB];
#pragma unroll
  for (int nb = 0; nb < kNQB; ++nb) {
    rnd[nb] = u32x4{0, 0, 0, 0};
    if constexpr (DROP)
      rnd[nb] = philox4x32_10(2u * (uint32_t)j + (uint32_t)half, (uint32_t)(qw0 + 32 * nb + col), bh, dp.offset,
                              dp.seed_lo, dp.seed_hi);
  }
  float ls[kNQB][2];
  u32x4 pn[kNQB][2];
#pragma unroll
  for (int nb = 0; nb < kNQB; ++nb) weights<DT, DROP>(s[nb], c, st.m[nb], ls[nb], pn[nb], rnd[nb], dp.thr);
  bool raise = false;
#pragma unroll
  for (int nb = 0; nb < kNQB; ++nb) raise |= !(ls[nb][0] + ls[nb][1] <= kLaneSumMax);
  if (__any(raise)) {  // rare: S(j) is still in s
    asm volatile("" ::: "memory");
#pragma unroll
    for (int nb = 0; nb < kNQB; ++nb) {
      float mx = s[nb][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[nb][r]);
      const float mnew = fmaxf(st.m[nb], max_pair32(mx) * c);
      const float alpha = exp2_fast(st.m[nb] - mnew);
      st.m[nb] = mnew;
      st.l[nb] *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db][nb] *= alpha;
      weights<DT, DROP>(s[nb], c, st.m[nb], ls[nb], pn[nb], rnd[nb], dp.thr);
    }
  }
#pragma unroll
  for (int nb = 0; nb < kNQB; ++nb) st.l[nb] += ls[nb][0] + ls[nb][1];
  __builtin_amdgcn_sched_barrier(0);
  // At d = 64 (four waves per SIMD) a wave issuing its MFMAs goes first:
  // 1-3% measured; at d = 128 it made no difference.
  if constexpr (D == 64) __builtin_amdgcn_s_setprio(1);
  // PV(j), then S(j+1) (after the last tile: a stale slot, never used)
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const u32x4 a = lds_transposed_a<D>(Vj, ta, kk, db);
#pragma unroll
      for (int nb = 0; nb < kNQB; ++nb) acc[db][nb] = mfma32<DT>(a, pn[nb][kk], acc[db][nb]);
    }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const u32x4 a = lds_rowmajor<D>(Kn, ta, ks);
#pragma unroll
    for (int nb = 0; nb < kNQB; ++nb) s[nb] = mfma32<DT>(a, qf[nb][ks], ks == 0 ? f32x16{} : s[nb]);
  }
  sched_reads_ahead<(2 * DB + KS) * kNQB, 4 * DB + KS>();
  if constexpr (D == 64) __builtin_amdgcn_s_setprio(0);
  // tile j+2 (read next step) must have landed; later ones may fly on
  if (j + PD < n_kt) {
    wait_vmcnt<(PD - 2) * 2 * TC::NI>();
  } else {
    wait_loads();
  }
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// A step of the phased ring for a wave with no work on tile j: its share
// of the copy of tile j + NBUF - 1 (into the slot of tile j - 1), the wait
// for tile j + 1 and the barrier, as in fwd_step_phased.
template <int D, int NW = kWaves, int NB = FwdCfg<D, true>::NBUF>
__device__ __forceinline__ void fwd_idle_phased(int j, int n_kt, uint16_t* __restrict__ Kdst,
                                                uint16_t* __restrict__ Vdst, __amdgpu_buffer_rsrc_t krs,
                                                __amdgpu_buffer_rsrc_t vrs, uint32_t krow, uint32_t vrow, uint32_t ktb,
                                                uint32_t vtb, int lane, int wave) {
  using TC = TileCopy<D, NW>;
  constexpr int PD = NB - 1;
  if (j + PD < n_kt) {
    TC::issue(krs, krow, (uint32_t)(j + PD) * ktb, Kdst, lane, wave);
    TC::issue(vrs, vrow, (uint32_t)(j + PD) * vtb, Vdst, lane, wave);
    wait_vmcnt<(PD - 2) * 2 * TC::NI>();
  } else {
    wait_loads();
  }
  lds_barrier();
}

// Key tiles [lo, hi) of query block qb (kBM queries): those some query of
// the block admits (all of them without a band).
__host__ __device__ __forceinline__ void block_tiles(int qb, int Nq, int Nk, int wl, int wr, bool band, int& lo,
                                                     int& hi) {
  const int q0 = qb * kBM;
  int kend = Nk, j0 = 0;
  if (band) {
    const int qlast = min(q0 + kBM, Nq) - 1;
    if (wr >= 0) kend = min(Nk, qlast + wr + 1);
    if (wl >= 0) j0 = max(0, q0 - wl) / kBN;
  }
  lo = j0;
  hi = max(j0, (kend + kBN - 1) / kBN);
}

// Chunks of a query block of n key tiles (at least one, so that a block
// with no admitted key still writes O = 0, LSE = -inf).
__host__ __device__ __forceinline__ int block_chunks(int n, int chunk) { return n > 0 ? (n + chunk - 1) / chunk : 1; }

// Position of item `target` in the chunk order (query blocks n_qt-1 .. 0,
// each with block_chunks(...) chunks): with split_only, items are the
// split blocks (two or more chunks) instead of the chunks.  Returns the
// block (-1 if none), the item's index within it, the block's chunk count
// and the partial slots of the split blocks before it.  Each wave scans 64
// blocks per step, one per lane, with a prefix sum over the lanes; the
// results are the same in every lane and every wave.
struct ChunkPos {
  int qb, idx, sb, base;
};
template <bool BAND>
__device__ __forceinline__ ChunkPos locate_chunk(const FwdParams& p, int n_qt, int target, bool split_only) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  for (int g = 0; g < n_qt; g += 64) {
    const int qb = n_qt - 1 - (g + lane);
    int sb = 0;
    if (qb >= 0) {
      int lo, hi;
      block_tiles(qb, p.Nq, p.Nk, p.wl, p.wr, BAND, lo, hi);
      sb = block_chunks(hi - lo, p.chunk);
    }
    const int unit = split_only ? (sb > 1 ? 1 : 0) : sb;
    const int slots = sb > 1 ? sb : 0;
    int pu = unit, ps = slots;  // inclusive prefix sums over the lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int x = __shfl_up(pu, o), y = __shfl_up(ps, o);
      if (lane >= o) {
        pu += x;
        ps += y;
      }
    }
    const uint64_t hit = __ballot(pu > target);
    if (hit) {
      const int L = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
      ChunkPos r;
      r.qb = __builtin_amdgcn_readfirstlane(__shfl(qb, L));
      r.sb = __builtin_amdgcn_readfirstlane(__shfl(sb, L));
      r.idx = __builtin_amdgcn_readfirstlane(target - (__shfl(pu, L) - __shfl(unit, L)));
      r.base = __builtin_amdgcn_readfirstlane(base + __shfl(ps, L) - __shfl(slots, L));
      return r;
    }
    target -= __builtin_amdgcn_readfirstlane(__shfl(pu, 63));
    base += __builtin_amdgcn_readfirstlane(__shfl(ps, 63));
  }
  return ChunkPos{-1, 0, 0, 0};
}

// Intra-workgroup key split for grids that give a CU at most one
// workgroup (one wave per SIMD otherwise): KSPLIT = 3 groups of four waves own
// the same 128 queries, and group g takes the g-th of KSPLIT equal runs of
// the block's key tiles through a ring of its own.  Each group forms the
// partial state (O^T, m, l) of its keys; the groups > 0 hand theirs to
// group 0 through LDS, which merges them in group order by the online
// softmax rule (m = max m_g, O^T = sum 2^(m_g - m) O^T_g, l likewise) and
// writes O and LSE.  Every wave executes the same number of barriers:
// groups with fewer tiles add barrier-only steps.
template <int D>
constexpr int kKSplit = 3;
// The groups run the phased schedule at d = 128 (three waves per SIMD,
// 3-slot rings): 8% faster than two groups on the interleaved one at
// B1 H2 N16384.  At d = 64 four phased groups need <= 128 registers and
// spill; three interleaved ones measured faster.
template <int D>
constexpr bool kKSplitPhased = D == 128;

// Key-chunked forward (CHUNK, fa_fwd_splitk): workgroup t takes chunk
// t / BH of head t % BH, the chunks listed from the last query block to
// the first (the heaviest first under a causal band), each block's n key
// tiles cut into ceil(n / p.chunk) near-equal runs.  A block of one chunk writes O and
// LSE; the chunks of a split block write their partial state (O^T, m, l)
// to p.part, which fwd_merge_kernel combines.
// GW: waves per query block (and per key group), 32 queries each.  Four
// everywhere but the small-block split below, which runs six groups of two
// waves on 64-query blocks with three-slot rings (its LDS: six rings).
template <int D, bool PHASED, int GW>
constexpr int kFwdWavesPerSimd = GW < kWaves ? 3 : FwdCfg<D, PHASED>::WAVES_PER_SIMD;

template <int D, int DT, bool BAND, bool DROP, bool PHASED, int KSPLIT, bool CHUNK, int GW = kWaves>
__global__ __launch_bounds__(64 * GW * KSPLIT) __attribute__((amdgpu_waves_per_eu(
    kFwdWavesPerSimd<D, PHASED, GW>, kFwdWavesPerSimd<D, PHASED, GW>))) void fwd_kernel(FwdParams p) {
  static_assert(!CHUNK || KSPLIT == 1, "key chunks run whole workgroups");
  static_assert(GW == kWaves || (PHASED && !CHUNK), "two-wave groups run the phased step");
  constexpr int kNQB = 1;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int BMG = GW * kQW;  // queries per block
  constexpr int NBUF = GW < kWaves ? 3 : FwdCfg<D, PHASED>::NBUF;  // K/V ring (see fwd_step, fwd_step_phased)
  constexpr int TILE = kTileElems<D>;

  // One LDS object for the whole ring: the compiler gives every separate
  // __shared__ variable its own alias scope, and then makes each LDS read
  // wait for the in-flight copies into the same variable, which would
  // serialise the prefetch with the compute it is meant to hide under.
  struct Smem {
    uint16_t k[KSPLIT][NBUF][TILE];
    uint16_t v[KSPLIT][NBUF][TILE];
  };
  __shared__ __attribute__((aligned(1024))) Smem sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave_all / GW;          // key group (0 without a split)
  const int wave = wave_all - grp * GW;   // wave within the group: its 32 queries
  auto& Ks = sm.k[grp];
  auto& Vs = sm.v[grp];

  // Heaviest query tiles first: block t covers query tile (last - t / BH),
  // head t % BH.  Consecutive blocks land on different XCDs round-robin,
  // so a head's tiles share one XCD's L2 when B*H is a multiple of 8.
  const int BH = p.B * p.H;
  const int n_qt = (p.Nq + BMG - 1) / BMG;
  const int t = blockIdx.x;
  const int bh = t - (t / BH) * BH;
  int qt = n_qt - 1 - t / BH;
  int ck_lo = 0, ck_hi = 0, slot = -1;  // CHUNK: this chunk's key tiles and partial slot (-1: O directly)
  if constexpr (CHUNK) {  // chunk c of sb near-equal runs of its block's tiles
    const ChunkPos cp = locate_chunk<BAND>(p, n_qt, t / BH, false);
    int lo, hi;
    block_tiles(cp.qb, p.Nq, p.Nk, p.wl, p.wr, BAND, lo, hi);
    qt = cp.qb;
    ck_lo = lo + (int)((int64_t)cp.idx * (hi - lo) / cp.sb);
    ck_hi = lo + (int)((int64_t)(cp.idx + 1) * (hi - lo) / cp.sb);
    if (cp.sb > 1) slot = cp.base + cp.idx;
  }
  const int b = bh / p.H, h = bh - b * p.H;
  const int q0 = qt * BMG;
  const int qw0 = q0 + wave * kQW;

  const int hk = h / p.G;  // K/V head shared by p.G consecutive query heads
  const uint16_t* qp = p.q + b * p.sq.b + h * p.sq.h;
  const uint16_t* kp = p.k + b * p.sk.b + hk * p.sk.h;
  const uint16_t* vp = p.v + b * p.sv.b + hk * p.sv.h;

  // key tiles [jt0, n_kt): those some query of the block admits; with a
  // split, this group's run of them
  int kend = p.Nk, jt0 = 0;
  if (BAND) {
    const int qlast = min(q0 + BMG, p.Nq) - 1;
    if (p.wr >= 0) kend = min(p.Nk, qlast + p.wr + 1);
    if (p.wl >= 0) jt0 = max(0, q0 - p.wl) / kBN;
  }
  int n_kt = (kend + kBN - 1) / kBN;
  if constexpr (CHUNK) {
    jt0 = ck_lo;
    n_kt = ck_hi;
  }
  int per = 0;  // tiles of the longest run
  if constexpr (KSPLIT > 1) {
    const int all = max(0, n_kt - jt0);
    per = (all + KSPLIT - 1) / KSPLIT;
    const int ja = min(n_kt, jt0 + grp * per);
    n_kt = min(n_kt, ja + per);
    jt0 = ja;
  }

  const __amdgpu_buffer_rsrc_t krs = head_rsrc(kp, p.Nk, p.sk.s, D);
  const __amdgpu_buffer_rsrc_t vrs = head_rsrc(vp, p.Nk, p.sv.s, D);
  const uint32_t krow = (uint32_t)(p.sk.s * 2), vrow = (uint32_t)(p.sv.s * 2);
  const uint32_t ktb = kBN * krow, vtb = kBN * vrow;
  using TC = TileCopy<D, GW>;

  // Q^T as the B operand, resident in registers: lane holds
  // Q[qw0 + 32*nb + col][16*ks + 8*half .. +7].  Its loads go first so the
  // vmcnt wait below can leave tile 2 in flight.
  u32x4 qf[kNQB][KS];
#pragma unroll
  for (int nb = 0; nb < kNQB; ++nb) {
    const int qi = qw0 + 32 * nb + col;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 x = u32x4{0, 0, 0, 0};
      if (qi < p.Nq) x = *(const u32x4*)(qp + qi * p.sq.s + 16 * ks + 8 * half);
      qf[nb][ks] = x;
    }
  }
  // prologue: tiles jt0 .. jt0+NBUF-2 in flight (tile jt0 + t lives in
  // slot t mod NBUF), and K of tile jt0+3 where K runs four tiles ahead
  constexpr bool kSep = FwdCfg<D, PHASED>::SEP_S;
#pragma unroll
  for (int t0 = 0; t0 < NBUF - 1; ++t0) {
    const int jj = jt0 + t0;
    if (jj < n_kt) {
      TC::issue(krs, krow, (uint32_t)jj * ktb, Ks[t0], lane, wave);
      TC::issue(vrs, vrow, (uint32_t)jj * vtb, Vs[t0], lane, wave);
    }
  }
  if constexpr (kSep) {
    if (jt0 + 3 < n_kt) TC::issue(krs, krow, (uint32_t)(jt0 + 3) * ktb, Ks[3], lane, wave);
  }

  f32x16 acc[DB][kNQB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int nb = 0; nb < kNQB; ++nb) acc[db][nb] = f32x16{};
  RowState<kNQB> st;
#pragma unroll
  for (int nb = 0; nb < kNQB; ++nb) {
    st.m[nb] = -1e30f;
    st.l[nb] = 0.f;
  }
  const float c = p.c;

  TileLayout<D> ta;
  ta.init(lane);

  // tiles jt0 and jt0+1 landed (K(jt0) for S(jt0) now, V(jt0) and
  // K(jt0+1) in the first step); the later ones may fly on (with K four
  // ahead: V(jt0+1), K(jt0+2), V(jt0+2) and K(jt0+3))
  if (kSep && n_kt - jt0 > 3) {
    wait_vmcnt<4 * TC::NI>();
  } else if (!kSep && n_kt - jt0 >= NBUF - 1) {
    wait_vmcnt<(NBUF - 3) * 2 * TC::NI>();
  } else {
    wait_loads();
  }
#pragma unroll
  for (int nb = 0; nb < kNQB; ++nb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[nb][ks] ^= p.qflip;
  lds_barrier();

  if constexpr (PHASED) {
    if (jt0 < n_kt) {
      // This wave's own tiles [wlo, whi): those one of its queries admits.
      // The workgroup's band can reach further (its other waves' queries);
      // there the wave's weights would be exact zeros, so it only takes
      // its part in the ring (copies, wait, barrier) and skips the work.
      // The result is bit for bit the same (O never holds -0).
      int wlo = jt0, whi = n_kt;
      if constexpr (BAND) {
        if (p.wl >= 0) wlo = max(wlo, max(0, qw0 - p.wl) / kBN);
        if (p.wr >= 0) whi = min(whi, (qw0 + kQW - 1 + p.wr) / kBN + 1);
        whi = max(whi, wlo);
      }
      auto wrap = [](int x) { return x >= NBUF ? x - NBUF : x; };
      int sl = 0;  // slot of tile j
      int j = jt0;
      auto idle = [&]() {
        const int sp = wrap(sl + NBUF - 1);  // slot of tile j-1
        fwd_idle_phased<D, GW, NBUF>(j, n_kt, Ks[sp], Vs[sp], krs, vrs, krow, vrow, ktb, vtb, lane, wave);
        sl = wrap(sl + 1);
      };
      for (; j < wlo; ++j) idle();
      if (j < whi) {
        f32x16 sa[kNQB];
#pragma unroll
        for (int nb = 0; nb < kNQB; ++nb) sa[nb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const u32x4 a = lds_rowmajor<D>(Ks[sl], ta, ks);
#pragma unroll
          for (int nb = 0; nb < kNQB; ++nb) sa[nb] = mfma32<DT>(a, qf[nb][ks], sa[nb]);
        }
        auto one = [&]() {
          const int sp = wrap(sl + NBUF - 1);  // slot of tile j-1
          fwd_step_phased<D, DT, BAND, DROP, kNQB, GW, NBUF>(j, n_kt, sa, Vs[sl], Ks[wrap(sl + 1)], Ks[sp], Vs[sp], krs, vrs,
                                                   krow, vrow, ktb, vtb, qf, acc, st, p.Nk, p.wl, p.wr, qw0, c, lane,
                                                   wave, ta, p.drop, (uint32_t)bh);
          sl = wrap(sl + 1);
        };
        // Whole turns of the ring with every slot a constant (LDS addresses
        // as immediate offsets; 0.6-0.9% at 16K causal d = 128), from the
        // first step whose tile sits in slot 0.  With dropout the unrolled
        // turn spills registers at d = 128, so it steps one by one.
        if constexpr (!DROP) {
          for (; j < whi && sl != 0; ++j) one();
          for (; j + NBUF <= whi; j += NBUF) {
#pragma unroll
            for (int r = 0; r < NBUF; ++r)
              fwd_step_phased<D, DT, BAND, DROP, kNQB, GW, NBUF>(j + r, n_kt, sa, Vs[r], Ks[(r + 1) % NBUF],
                                                       Ks[(r + NBUF - 1) % NBUF], Vs[(r + NBUF - 1) % NBUF], krs, vrs,
                                                       krow, vrow, ktb, vtb, qf, acc, st, p.Nk, p.wl, p.wr, qw0, c, lane,
                                                       wave, ta, p.drop, (uint32_t)bh);
          }
        }
        for (; j < whi; ++j) one();
      }
      for (; j < n_kt; ++j) idle();
    }
  } else if (jt0 < n_kt) {
    // Tile jt0 + t lives in slot t mod 4.
    f32x16 sa[kNQB];
#pragma unroll
    for (int nb = 0; nb < kNQB; ++nb) sa[nb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 a = lds_rowmajor<D>(Ks[0], ta, ks);
#pragma unroll
      for (int nb = 0; nb < kNQB; ++nb) sa[nb] = mfma32<DT>(a, qf[nb][ks], sa[nb]);
    }
    if constexpr (kSep) {  // the first step copies K(jt0+4) into K(jt0)'s slot
      wait_lds_reads();
      lds_barrier();
    }
    u32x4 pf[2][kNQB];
    u32x4 va[2][DB];
    // with S(j+1) in registers of its own, sa and sb alternate
    f32x16 sb[kNQB];
    fwd_step<D, DT, BAND, DROP, true>(jt0, n_kt, sa, sb, pf, va, Ks[0], Ks[1], Vs[0], Ks[kSep ? 0 : 3], Vs[3], krs, vrs, krow,
                                      vrow, ktb, vtb, qf, acc, st, p.Nk, p.wl, p.wr, qw0, c, lane, wave, ta, p.drop,
                                      (uint32_t)bh);
    if constexpr (kSep) {
#pragma unroll
      for (int nb = 0; nb < kNQB; ++nb) sa[nb] = sb[nb];
    }
    int j = jt0 + 1;
    if constexpr (kSep) {
      if constexpr (!DROP) {
        // single steps (S(j+1) copied back) until tile j sits in slot 0,
        // then whole turns of the ring with constant slots (LDS addresses
        // as immediates), two swapped pairs per turn: -1 to -3% on grids of
        // 512 blocks
        for (; j < n_kt && ((j - jt0) & 3) != 0; ++j) {
          const int sl = (j - jt0) & 3;
          fwd_step<D, DT, BAND, DROP, false>(j, n_kt, sa, sb, pf, va, Ks[sl], Ks[(sl + 1) & 3], Vs[sl], Ks[sl],
                                             Vs[(sl + 3) & 3], krs, vrs, krow, vrow, ktb, vtb, qf, acc, st, p.Nk, p.wl,
                                             p.wr, qw0, c, lane, wave, ta, p.drop, (uint32_t)bh);
#pragma unroll
          for (int nb = 0; nb < kNQB; ++nb) sa[nb] = sb[nb];
        }
        for (; j + 3 < n_kt; j += 4) {
#pragma unroll
          for (int r = 0; r < 4; r += 2) {
            fwd_step<D, DT, BAND, DROP, false>(j + r, n_kt, sa, sb, pf, va, Ks[r], Ks[r + 1], Vs[r], Ks[r],
                                               Vs[(r + 3) & 3], krs, vrs, krow, vrow, ktb, vtb, qf, acc, st, p.Nk, p.wl,
                                               p.wr, qw0, c, lane, wave, ta, p.drop, (uint32_t)bh);
            fwd_step<D, DT, BAND, DROP, false>(j + r + 1, n_kt, sb, sa, pf, va, Ks[r + 1], Ks[(r + 2) & 3], Vs[r + 1],
                                               Ks[r + 1], Vs[r], krs, vrs, krow, vrow, ktb, vtb, qf, acc, st, p.Nk,
                                               p.wl, p.wr, qw0, c, lane, wave, ta, p.drop, (uint32_t)bh);
          }
        }
      }
      // two steps per iteration with the roles of sa and sb swapped, so
      // S(j+1) is not copied back every step
      for (; j + 1 < n_kt; j += 2) {
        const int sl = (j - jt0) & 3, sl2 = (sl + 1) & 3;
        fwd_step<D, DT, BAND, DROP, false>(j, n_kt, sa, sb, pf, va, Ks[sl], Ks[sl2], Vs[sl], Ks[sl], Vs[(sl + 3) & 3], krs,
                                           vrs, krow, vrow, ktb, vtb, qf, acc, st, p.Nk, p.wl, p.wr, qw0, c, lane, wave, ta,
                                           p.drop, (uint32_t)bh);
        fwd_step<D, DT, BAND, DROP, false>(j + 1, n_kt, sb, sa, pf, va, Ks[sl2], Ks[(sl2 + 1) & 3], Vs[sl2], Ks[sl2],
                                           Vs[sl], krs, vrs, krow, vrow, ktb, vtb, qf, acc, st, p.Nk, p.wl, p.wr, qw0, c,
                                           lane, wave, ta, p.drop, (uint32_t)bh);
      }
    }
    // d = 64: whole turns of the 4-slot ring with constant slots (LDS
    // addresses as immediates; 157 registers, three waves per SIMD still):
    // B2 H8 N2048 29.3 -> 27.2 us, B2 H8 N512 -5%, others within +-1% or
    // faster.
    if constexpr (!kSep && !DROP) {
      for (; j < n_kt && ((j - jt0) & 3) != 0; ++j) {
        const int sl = (j - jt0) & 3;
        fwd_step<D, DT, BAND, DROP, false>(j, n_kt, sa, sb, pf, va, Ks[sl], Ks[(sl + 1) & 3], Vs[sl], Ks[(sl + 3) & 3],
                                           Vs[(sl + 3) & 3], krs, vrs, krow, vrow, ktb, vtb, qf, acc, st, p.Nk, p.wl, p.wr,
                                           qw0, c, lane, wave, ta, p.drop, (uint32_t)bh);
      }
      for (; j + 4 <= n_kt; j += 4) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          fwd_step<D, DT, BAND, DROP, false>(j + r, n_kt, sa, sb, pf, va, Ks[r], Ks[(r + 1) & 3], Vs[r], Ks[(r + 3) & 3],
                                             Vs[(r + 3) & 3], krs, vrs, krow, vrow, ktb, vtb, qf, acc, st, p.Nk, p.wl, p.wr,
                                             qw0, c, lane, wave, ta, p.drop, (uint32_t)bh);
      }
    }
    for (; j < n_kt; ++j) {
      const int sl = (j - jt0) & 3;
      fwd_step<D, DT, BAND, DROP, false>(j, n_kt, sa, sb, pf, va, Ks[sl], Ks[(sl + 1) & 3], Vs[sl],
                                         Ks[kSep ? sl : (sl + 3) & 3], Vs[(sl + 3) & 3], krs, vrs, krow, vrow, ktb, vtb, qf, acc,
                                         st, p.Nk, p.wl, p.wr, qw0, c, lane, wave, ta, p.drop, (uint32_t)bh);
      if constexpr (kSep) {
#pragma unroll
        for (int nb = 0; nb < kNQB; ++nb) sa[nb] = sb[nb];
      }
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int nb = 0; nb < kNQB; ++nb) acc[db][nb] = mfma32<DT>(va[kk][db], pf[kk][nb], acc[db][nb]);
  }

  if constexpr (KSPLIT > 1) {
    // Barriers of a run of m tiles: one per step, plus the one after S of
    // the first tile when S(j+1) has registers of its own.  Pad the
    // shorter runs to the longest.
    auto barriers = [&](int m) { return m > 0 ? m + (kSep ? 1 : 0) : 0; };
    for (int i = barriers(max(0, n_kt - jt0)); i < barriers(per); ++i) lds_barrier();
    // every group is done with its ring: reuse it for the hand-over
    constexpr int NV = DB * 16 + 2;  // floats per lane: O^T, m, l
    static_assert((size_t)(KSPLIT - 1) * GW * NV * 64 * 4 <= sizeof(Smem), "hand-over fits the rings");
    float* xo = reinterpret_cast<float*>(&sm) + (size_t)((grp - 1) * GW + wave) * NV * 64 + lane;
    lds_barrier();
    if (grp > 0) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo[(db * 16 + r) * 64] = acc[db][0][r];
      xo[(DB * 16) * 64] = st.m[0];
      xo[(DB * 16 + 1) * 64] = st.l[0];
    }
    lds_barrier();
    if (grp > 0) return;
#pragma unroll
    for (int g = 1; g < KSPLIT; ++g) {
      const float* xi = reinterpret_cast<const float*>(&sm) + (size_t)((g - 1) * GW + wave) * NV * 64 + lane;
      const float mg = xi[(DB * 16) * 64], lg = xi[(DB * 16 + 1) * 64];
      const float mn = fmaxf(st.m[0], mg);
      const float a0 = exp2_fast(st.m[0] - mn), ag = exp2_fast(mg - mn);
      st.m[0] = mn;
      st.l[0] = st.l[0] * a0 + lg * ag;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][0][r] = acc[db][0][r] * a0 + xi[(db * 16 + r) * 64] * ag;
    }
  }

  if constexpr (CHUNK) {
    if (slot >= 0) {  // a chunk of a split block: its partial state
      float* pb = p.part + ((size_t)bh * p.P + slot) * (size_t)(kBM * (D + 2));
      const int row = wave * kQW + col;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x16& a = acc[db][0];
          *(f32x4*)(pb + row * D + db * 32 + 8 * g4 + 4 * half) =
              f32x4{a[4 * g4], a[4 * g4 + 1], a[4 * g4 + 2], a[4 * g4 + 3]};
        }
      const float lt = sum_pair32(st.l[0]);
      if (half == 0) {
        pb[kBM * D + row] = st.m[0];
        pb[kBM * D + kBM + row] = lt;
      }
      return;
    }
  }

  // ---- epilogue: O = O^T / l, LSE
  uint16_t* op = p.o + b * p.so.b + h * p.so.h;
#pragma unroll
  for (int nb = 0; nb < kNQB; ++nb) {
    const float lt = sum_pair32(st.l[nb]);
    const int qi = qw0 + 32 * nb + col;
    if (qi < p.Nq) {
      // a row that admits no key: O = 0, LSE = -inf
      const float inv = lt > 0.f ? (DROP ? p.drop.scale : 1.0f) / lt : 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = db * 32 + 8 * g4 + 4 * half;
          const f32x16& a = acc[db][nb];
          u32x2 w = u32x2{pack2<DT>(a[4 * g4 + 0] * inv, a[4 * g4 + 1] * inv),
                          pack2<DT>(a[4 * g4 + 2] * inv, a[4 * g4 + 3] * inv)};
          *(u32x2*)(op + qi * p.so.s + d0) = w;
        }
      if (half == 0) p.lse[(int64_t)bh * p.Nq + qi] = lt > 0.f ? (st.m[nb] + log2_fast(lt)) * kLn2 : -__builtin_inff();
    }
  }
}

// Merge of a split query block's chunks (fa_fwd_splitk): workgroup t takes
// rows [RPW (t % NRG), +RPW) of the ((t / NRG) / BH)-th split block of head
// (t / NRG) % BH, in the chunk kernel's order; a thread merges one 4-wide
// column group of one row.  Per row, in chunk order: M = max m_s,
// L = sum 2^(m_s - M) l_s, O = sum 2^(m_s - M) O^T_s / L (times the dropout
// scale), LSE = (M + log2 L) ln 2 (O = 0, LSE = -inf for a row that admits
// no key).
template <int D>
constexpr int kMergeRows = kThreads / (D / 4);  // rows per merge workgroup
constexpr int kMergeBatch = 8;                  // partial slots loaded together

template <int D, int DT, bool BAND, bool DROP>
__global__ __launch_bounds__(kThreads) void fwd_merge_kernel(FwdParams p) {
  constexpr int CH = D / 4;  // float4 column groups per row
  constexpr int RPW = kMergeRows<D>;
  constexpr int NRG = kBM / RPW;
  const int BH = p.B * p.H;
  const int n_qt = (p.Nq + kBM - 1) / kBM;
  const int t = blockIdx.x;
  const int rg = t % NRG, rest = t / NRG;
  const int bh = rest % BH;
  const ChunkPos cp = locate_chunk<BAND>(p, n_qt, rest / BH, true);
  const int qt = cp.qb, ns = cp.sb, base = cp.base;
  const int row = rg * RPW + (int)threadIdx.x / CH;
  const int qi = qt * kBM + row;
  if (qt < 0 || qi >= p.Nq) return;
  const int ch = threadIdx.x % CH;
  const int b = bh / p.H, h = bh - b * p.H;
  const size_t SLOT = (size_t)kBM * (D + 2);
  const float* pb = p.part + ((size_t)bh * p.P + base) * SLOT;
  const float* pm = pb + kBM * D + row;        // m of slot s at pm[s * SLOT]
  const float* pl = pb + kBM * D + kBM + row;  // l likewise
  const float* po = pb + row * D + 4 * ch;     // this thread's 4 columns
  // Slots in batches of kMergeBatch whose loads all go out before the
  // first use (one memory latency per batch instead of one per pass);
  // batches fold in by the online-softmax rule.  With one batch (the
  // usual case) this is max over the slots, then the sums in slot order.
  float M = -1e30f, L = 0.f;
  f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < ns; s0 += kMergeBatch) {
    // unconditional loads (past the last slot they repeat it, which
    // leaves the max unchanged), so that none waits for another
    float mv[kMergeBatch], lv[kMergeBatch];
    f32x4 ov[kMergeBatch];
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      const size_t si = (size_t)min(s0 + i, ns - 1) * SLOT;
      mv[i] = pm[si];
      lv[i] = pl[si];
      ov[i] = *(const f32x4*)(po + si);
    }
    float Mb = M;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) Mb = fmaxf(Mb, mv[i]);
    if (s0 > 0) {  // rescale what the earlier batches summed
      const float r = exp2_fast(M - Mb);
      L *= r;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] *= r;
    }
    M = Mb;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      if (s0 + i < ns) {
        const float a = exp2_fast(mv[i] - M);
        L += a * lv[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] += a * ov[i][e];
      }
    }
  }
  const float inv = L > 0.f ? (DROP ? p.drop.scale : 1.0f) / L : 0.f;
  uint16_t* op = p.o + b * p.so.b + h * p.so.h + qi * p.so.s + 4 * ch;
  *(u32x2*)op = u32x2{pack2<DT>(o[0] * inv, o[1] * inv), pack2<DT>(o[2] * inv, o[3] * inv)};
  if (ch == 0) p.lse[(int64_t)bh * p.Nq + qi] = L > 0.f ? (M + log2_fast(L)) * kLn2 : -__builtin_inff();
}

template <int D, int DT, bool BAND, bool DROP, bool PHASED, int KSPLIT, int GW>
hipError_t launch_t(const FwdParams& p, int64_t blocks, hipStream_t stream) {
  hipLaunchKernelGGL((fwd_kernel<D, DT, BAND, DROP, PHASED, KSPLIT, false, GW>), dim3((unsigned)blocks),
                     dim3(64 * GW * KSPLIT), 0, stream, p);
  return hipGetLastError();
}

template <int D, int DT, bool BAND, bool DROP>
hipError_t launch_chunked_t(const FwdParams& p, const FwdSplitPlan& plan, hipStream_t stream) {
  const int64_t BH = (int64_t)p.B * p.H;
  hipLaunchKernelGGL((fwd_kernel<D, DT, BAND, DROP, true, 1, true>), dim3((unsigned)(plan.n_chunks * BH)),
                     dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.n_split == 0) return e;
  hipLaunchKernelGGL((fwd_merge_kernel<D, DT, BAND, DROP>), dim3((unsigned)(plan.n_split * BH * (kBM / kMergeRows<D>))),
                     dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D, int DT>
hipError_t launch_chunked(const FwdParams& p, const FwdSplitPlan& plan, bool banded, hipStream_t stream) {
  if (p.drop.thr > 0)
    return banded ? launch_chunked_t<D, DT, true, true>(p, plan, stream)
                  : launch_chunked_t<D, DT, false, true>(p, plan, stream);
  return banded ? launch_chunked_t<D, DT, true, false>(p, plan, stream)
                : launch_chunked_t<D, DT, false, false>(p, plan, stream);
}

template <int D, int DT, bool PHASED, int KSPLIT, int GW = kWaves>
hipError_t launch_ds(const FwdParams& p, bool banded, int64_t blocks, hipStream_t stream) {
  if (p.drop.thr > 0)
    return banded ? launch_t<D, DT, true, true, PHASED, KSPLIT, GW>(p, blocks, stream)
                  : launch_t<D, DT, false, true, PHASED, KSPLIT, GW>(p, blocks, stream);
  return banded ? launch_t<D, DT, true, false, PHASED, KSPLIT, GW>(p, blocks, stream)
                : launch_t<D, DT, false, false, PHASED, KSPLIT, GW>(p, blocks, stream);
}

// Compute units of the current device (cached per device; 256 on MI355X).
int device_cus() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cus[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// The intra-workgroup key split pays when the heaviest query block has at
// least this many key tiles; below, the merge costs more than it saves.
constexpr int kKSplitMinTiles = 32;
// At d = 64, from this many key tiles on, the split runs on 64-query blocks
// with six groups of two waves (three-slot rings): each heavy block's keys
// in sixths on twice the blocks.  Measured on grids of 256 128-query
// blocks: B1 H2 N16384 131 -> 93 us, B1 H4 N8192 72 -> 56 us; with 64
// tiles (B2 H8 N2048) no change, with 32-36 (B2 H16 N1024, a 1000-key
// window at N4096) 15-17% slower, where the blocks' own latency dominates.
constexpr int kSmallBlockSplitMinTiles = 128;

template <int D, int DT>
hipError_t launch_dc(const FwdParams& p, bool banded, hipStream_t stream) {
  const int n_qt = (p.Nq + kBM - 1) / kBM;
  const int64_t blocks = (int64_t)n_qt * p.B * p.H;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (blocks >= kPhasedMinBlocks<D>) return launch_ds<D, DT, true, 1>(p, banded, blocks, stream);
  // at most one workgroup per CU: split each block's keys over more waves
  if (blocks <= device_cus()) {
    constexpr int enough = D == 64 ? kSmallBlockSplitMinTiles : kKSplitMinTiles;
    int most = 0;  // key tiles of the heaviest block (n_qt <= the CU count here)
    for (int qb = 0; qb < n_qt && most < enough; ++qb) {
      int lo, hi;
      block_tiles(qb, p.Nq, p.Nk, p.wl, p.wr, banded, lo, hi);
      most = max(most, hi - lo);
    }
    if constexpr (D == 64) {  // (six rings of 16 KiB slots would not fit the LDS at d = 128)
      if (most >= kSmallBlockSplitMinTiles) {
        const int64_t blocks64 = (int64_t)((p.Nq + 63) / 64) * p.B * p.H;
        return launch_ds<D, DT, true, 6, 2>(p, banded, blocks64, stream);
      }
    }
    if (most >= kKSplitMinTiles) return launch_ds<D, DT, kKSplitPhased<D>, kKSplit<D>>(p, banded, blocks, stream);
  }
  return launch_ds<D, DT, false, 1>(p, banded, blocks, stream);
}

// Chunk plan (fa_fwd_splitk).  Grids of at most kSplitMaxBlocks query
// blocks leave CUs idle behind the heaviest blocks of a causal band.  Each
// block's key tiles are cut into near-equal chunks of at most `chunk`
// tiles, with `chunk` the smallest length (but at least kMinChunkTiles)
// whose chunks all fit the chip at once: at most 3 (d = 128) or 4
// (d = 64) workgroups per CU, the waves per SIMD of the phased schedule
// the chunks run; a second round of workgroups would double the time.
// The partial results cost a merge kernel (~10 us for ~20 MB of them), so
// the plan is kept only when its longest chunk is at least
// kChunkMinSaving tiles shorter than the critical path without it (the
// intra-workgroup split's run where that applies), or kChunkMinSaving2
// when the grid already gives every CU a workgroup and a second one to
// some: there the unsplit blocks already share the CUs about evenly, and
// chunks paid only on long rows (B1 H4 N16384 d128: -5%; B1 H16 N4096 d128:
// +3% with 32).  Planned for the MI355X's 256 CUs (a fixed number, so the
// workspace size depends on the sizes alone).
constexpr int kChipCUs = 256;
constexpr int kSplitMaxBlocks = 2 * kChipCUs;
constexpr int kMinChunkTiles = 8;
constexpr int kChunkMinSaving = 32;
constexpr int kChunkMinSaving2 = 96;

}  // namespace

FwdSplitPlan fwd_split_plan(int B, int H, int Nq, int Nk, int d, int wl, int wr) {
  FwdSplitPlan pl{0, 0, 0, 0};
  if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0) return pl;
  const int n_qt = (Nq + kBM - 1) / kBM;
  const int64_t BH = (int64_t)B * H;
  if (n_qt * BH > kSplitMaxBlocks) return pl;
  const bool band = wl >= 0 || wr >= 0;
  int64_t W = 0;
  for (int qb = 0; qb < n_qt; ++qb) {
    int lo, hi;
    block_tiles(qb, Nq, Nk, wl, wr, band, lo, hi);
    W += hi - lo;
  }
  const int64_t slots = (int64_t)(d == 64 ? 4 : 3) * kChipCUs;  // resident workgroups
  const int64_t per_bh = std::max<int64_t>(1, slots / BH);
  int most = 0;
  std::vector<int> tiles(n_qt);
  for (int qb = 0; qb < n_qt; ++qb) {
    int lo, hi;
    block_tiles(qb, Nq, Nk, wl, wr, band, lo, hi);
    tiles[qb] = hi - lo;
    most = std::max(most, hi - lo);
  }
  auto count = [&](int chunk) {
    int64_t n = 0;
    for (int x : tiles) n += block_chunks(x, chunk);
    return n;
  };
  int chunk = (int)std::max<int64_t>(kMinChunkTiles, (W + per_bh - 1) / per_bh);
  while (chunk < most && count(chunk) > per_bh) chunk += std::max(1, chunk / 32);
  // the critical path without chunks: the heaviest block, in runs of the
  // intra-workgroup split where fa_fwd_ex would use it
  const int unsplit = n_qt * BH <= kChipCUs && most >= kKSplitMinTiles
                          ? (most + (d == 64 ? kKSplit<64> : kKSplit<128>) - 1) / (d == 64 ? kKSplit<64> : kKSplit<128>)
                          : most;
  if (chunk + (n_qt * BH <= kChipCUs ? kChunkMinSaving : kChunkMinSaving2) > unsplit) return pl;
  int n_chunks = 0, n_split = 0, P = 0;
  for (int x : tiles) {
    const int sb = block_chunks(x, chunk);
    n_chunks += sb;
    if (sb > 1) {
      ++n_split;
      P += sb;
    }
  }
  if (n_split == 0) return pl;
  pl.chunk = chunk;
  pl.n_chunks = n_chunks;
  pl.n_split = n_split;
  pl.P = P;
  return pl;
}

size_t fwd_splitk_workspace_bytes(int B, int H, int Nq, int Nk, int d, int wl, int wr) {
  const FwdSplitPlan pl = fwd_split_plan(B, H, Nq, Nk, d, wl, wr);
  if (pl.chunk == 0) return 0;
  const size_t n = (size_t)B * H * pl.P * kBM * (size_t)(d + 2) * sizeof(float);
  return (n + 255) & ~(size_t)255;
}

hipError_t launch_fwd_splitk(const FwdParams& p, const FwdSplitPlan& plan, int d, int dtype, bool banded,
                             hipStream_t stream) {
  if (d == 64)
    return dtype == DT_F16 ? launch_chunked<64, DT_F16>(p, plan, banded, stream)
                           : launch_chunked<64, DT_BF16>(p, plan, banded, stream);
  return dtype == DT_F16 ? launch_chunked<128, DT_F16>(p, plan, banded, stream)
                         : launch_chunked<128, DT_BF16>(p, plan, banded, stream);
}

hipError_t launch_fwd(const FwdParams& p, int d, int dtype, bool banded, hipStream_t stream) {
  if (d == 64) return dtype == DT_F16 ? launch_dc<64, DT_F16>(p, banded, stream) : launch_dc<64, DT_BF16>(p, banded, stream);
  return dtype == DT_F16 ? launch_dc<128, DT_F16>(p, banded, stream) : launch_dc<128, DT_BF16>(p, banded, stream);
}

}  // namespace fa
