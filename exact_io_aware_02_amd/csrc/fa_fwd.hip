// Forward attention kernel for gfx950.
//
// One workgroup of 4 waves owns BM query rows of one (batch, head); each
// wave owns 32 of them at d = 128 (64, as two 32-query MFMA column blocks,
// at d = 64) and their softmax state, so the row max and row sum never
// leave the wave (FlashAttention-2's point of less communication between
// warps, refbase Q&A on FA2's improvements).  K/V tiles of BN = 32 keys
// stream from HBM straight into LDS (buffer_load ... lds, no staging
// registers) through a 4-slot ring.  Per tile and wave:
//
//   S^T = K_j Q^T          32x32x16 MFMAs; A = K rows from LDS, B = Q held
//                          in registers for the whole loop.  Each lane
//                          then holds 16 keys x 1 query of every 32x32
//                          block, so the row max and sum are in-lane plus
//                          one exchange with lane i^32.
//   online softmax         m' = max(m, max_j S*c) with c = |scale| log2 e;
//                          P = 2^(S*c - m); l += sum P; O^T *= 2^(m - m').
//                          The running max is only raised (and O^T, l
//                          rescaled) when some row's tile max exceeds it by
//                          more than 2^8; otherwise P <= 2^8 is computed
//                          against the stale max, which changes no result
//                          (O = O^T / l uses the same m in both).
//   O^T += V_j^T P^T       A = V^T via ds_read_b64_tr_b16 from the
//                          untransposed V tile; B = P^T repacked in place
//                          from the S^T accumulator (no LDS round trip).
//
// The loop is software pipelined: the MFMAs for S of tile j+1 are issued
// among the exponentials of tile j, so the matrix core and the VALU of a
// SIMD work at the same time within one wave (the overlap FA3 gets from
// asynchrony on Hopper, glossary article's FA-3 section).
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
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBN = 32;            // keys per pipeline tile
// Queries per wave are 32 * NQB (NQB = 32-query MFMA column blocks): 64
// halves the LDS bytes per MFMA but needs ~260 registers at d = 128.
template <int D>
struct FwdTile {
  static constexpr int NQB = D == 64 ? 2 : 1;
  static constexpr int QW = 32 * NQB;       // queries per wave
  static constexpr int BM = kWaves * QW;    // queries per workgroup
  static constexpr int WAVES_PER_SIMD = 2;
};
constexpr float kRescaleSlack = 8.0f;  // log2 units

template <int D>
using TileCopy = TileCopyT<D, kBN, kWaves>;

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

// One step of the software-pipelined loop: tile j's softmax and O += P V,
// while the MFMAs form S for tile j+1 into `sn`.  A wave's issue stream
// alternates those independent MFMAs with the exponentials of tile j, so
// the matrix core and the VALU of one SIMD stay busy together even without
// the other wave's help.  The LDS ring has four slots (tile t in slot
// t mod 4): step j reads K(j+1) and V(j) and fills slot (j+3) mod 4.
// The __restrict__ tile pointers tell the compiler the reads never alias
// the in-flight copy, so it does not wait for that copy before reading;
// the vmcnt wait and barrier at the end order the ring.
template <int D, int DT, bool BAND, bool DROP, int kNQB = FwdTile<D>::NQB>
__device__ __forceinline__ void fwd_step(int j, int n_kt, f32x16 (&s)[kNQB], f32x16 (&sn)[kNQB],
                                         const uint16_t* __restrict__ Kn, const uint16_t* __restrict__ Vt,
                                         uint16_t* __restrict__ Kdst, uint16_t* __restrict__ Vdst,
                                         __amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs, uint32_t krow,
                                         uint32_t vrow, uint32_t ktb, uint32_t vtb, const u32x4 (&qf)[kNQB][D / 16],
                                         f32x16 (&acc)[D / 32][kNQB], RowState<kNQB>& st, int Nk, int wl, int wr, int qw0, float c,
                                         int lane, int wave, const TileAddr<D>& ta, const DropoutParams& dp,
                                         uint32_t bh) {
  using TC = TileCopy<D>;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  const int j0 = j * kBN;
  const int col = lane & 31, half = lane >> 5;

  if (j + 3 < n_kt) {
    TC::issue(krs, krow, (uint32_t)(j + 3) * ktb, Kdst, lane, wave);
    TC::issue(vrs, vrow, (uint32_t)(j + 3) * vtb, Vdst, lane, wave);
  }

  // ---- masks (only tiles crossing the key tail or an edge of this wave's band)
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
  // ---- row max; lazy rescale
  float mxc[kNQB];
  bool raise = false;
#pragma unroll
  for (int nb = 0; nb < kNQB; ++nb) {
    float mx = fmaxf(s[nb][0], s[nb][1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) mx = fmaxf(fmaxf(mx, s[nb][r]), s[nb][r + 1]);
    mx = max_pair32(mx);
    mxc[nb] = mx * c;
    raise |= mxc[nb] > st.m[nb] + kRescaleSlack;
  }
  if (__any(raise)) {
#pragma unroll
    for (int nb = 0; nb < kNQB; ++nb) {
      const float mnew = fmaxf(st.m[nb], mxc[nb]);
      const float alpha = exp2_fast(st.m[nb] - mnew);
      st.m[nb] = mnew;
      st.l[nb] *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db][nb] *= alpha;
    }
  }

  // ---- S(j+1) = K(j+1) Q^T, issued first so the MFMAs run under the exponentials
#pragma unroll
  for (int nb = 0; nb < kNQB; ++nb) sn[nb] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const u32x4 a = lds_b128(Kn, ta.rm[ks]);
#pragma unroll
    for (int nb = 0; nb < kNQB; ++nb) sn[nb] = mfma32<DT>(a, qf[nb][ks], sn[nb]);
  }

  // ---- P = 2^(S c - m) packed into the MFMA B operand (after dropout:
  // the normaliser sums the undropped weights, the kept ones are rescaled
  // once in the epilogue)
  u32x4 pf[2][kNQB];
  float ls[kNQB][2];
#pragma unroll
  for (int nb = 0; nb < kNQB; ++nb) {
    const float mneg = -st.m[nb];
    ls[nb][0] = ls[nb][1] = 0.f;
    u32x4 rnd = u32x4{0, 0, 0, 0};
    if constexpr (DROP)  // this lane's 16 keys of tile j: one generator call
      rnd = philox4x32_10(2u * (uint32_t)j + (uint32_t)half, (uint32_t)(qw0 + 32 * nb + col), bh, dp.offset,
                          dp.seed_lo, dp.seed_hi);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 8 * kk + 2 * e;
        float p0 = exp2_fast(__builtin_fmaf(s[nb][r], c, mneg));
        float p1 = exp2_fast(__builtin_fmaf(s[nb][r + 1], c, mneg));
        if constexpr (DT == DT_BF16 || DROP) {  // bf16 rounding (2^-9) is too coarse for the normaliser
          ls[nb][0] = (r == 0) ? p0 : ls[nb][0] + p0;
          ls[nb][1] = (r == 0) ? p1 : ls[nb][1] + p1;
        }
        if constexpr (DROP) {  // register r holds key 8*(r/4) + 4*half + r%4 of the tile
          if (((rnd[r >> 2] >> (8 * (r & 3))) & 0xffu) < dp.thr) p0 = 0.f;
          if (((rnd[(r + 1) >> 2] >> (8 * ((r + 1) & 3))) & 0xffu) < dp.thr) p1 = 0.f;
        }
        w[e] = pack2<DT>(p0, p1);
      }
      if constexpr (DT == DT_F16 && !DROP) {  // fp16-rounded P is accurate enough: sum pairs in one op
#pragma unroll
        for (int e = 0; e < 4; ++e) ls[nb][e & 1] = dot2_sum<DT>(w[e], ls[nb][e & 1]);
      }
      pf[kk][nb] = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
  // ---- O^T += V^T P^T
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const u32x4 a = lds_transposed_a<D>(Vt, ta, kk, db);
#pragma unroll
      for (int nb = 0; nb < kNQB; ++nb) acc[db][nb] = mfma32<DT>(a, pf[kk][nb], acc[db][nb]);
    }
#pragma unroll
  for (int nb = 0; nb < kNQB; ++nb) st.l[nb] += ls[nb][0] + ls[nb][1];

  // tile j+2 must have landed (K read next step, V the step after); j+3 may fly on
  if (j + 3 < n_kt) {
    wait_vmcnt<2 * TC::NI>();
  } else {
    wait_loads();
  }
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

template <int D, int DT, bool BAND, bool DROP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(FwdTile<D>::WAVES_PER_SIMD,
                                                                          FwdTile<D>::WAVES_PER_SIMD))) void fwd_kernel(FwdParams p) {
  constexpr int kNQB = FwdTile<D>::NQB;
  constexpr int kQW = FwdTile<D>::QW;
  constexpr int kBM = FwdTile<D>::BM;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int NBUF = 4;  // K/V ring (see fwd_step)
  constexpr int TILE = kBN * D;

  // One LDS object for the whole ring: the compiler gives every separate
  // __shared__ variable its own alias scope, and then makes each LDS read
  // wait for the in-flight copies into the same variable, which would
  // serialise the prefetch with the compute it is meant to hide under.
  struct Smem {
    uint16_t k[NBUF][TILE];
    uint16_t v[NBUF][TILE];
  };
  __shared__ __attribute__((aligned(1024))) Smem sm;
  auto& Ks = sm.k;
  auto& Vs = sm.v;

  const int tid = threadIdx.x;
  const int lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Heaviest query tiles first: block t covers query tile (last - t / BH),
  // head t % BH.  Consecutive blocks land on different XCDs round-robin,
  // so a head's tiles share one XCD's L2 when B*H is a multiple of 8.
  const int BH = p.B * p.H;
  const int n_qt = (p.Nq + kBM - 1) / kBM;
  const int t = blockIdx.x;
  const int qt = n_qt - 1 - t / BH;
  const int bh = t - (t / BH) * BH;
  const int b = bh / p.H, h = bh - b * p.H;
  const int q0 = qt * kBM;
  const int qw0 = q0 + wave * kQW;

  const int hk = h / p.G;  // K/V head shared by p.G consecutive query heads
  const uint16_t* qp = p.q + b * p.sq.b + h * p.sq.h;
  const uint16_t* kp = p.k + b * p.sk.b + hk * p.sk.h;
  const uint16_t* vp = p.v + b * p.sv.b + hk * p.sv.h;

  // key tiles [jt0, n_kt): those some query of the block admits
  int kend = p.Nk, jt0 = 0;
  if (BAND) {
    const int qlast = min(q0 + kBM, p.Nq) - 1;
    if (p.wr >= 0) kend = min(p.Nk, qlast + p.wr + 1);
    if (p.wl >= 0) jt0 = max(0, q0 - p.wl) / kBN;
  }
  const int n_kt = (kend + kBN - 1) / kBN;

  const __amdgpu_buffer_rsrc_t krs = head_rsrc(kp, p.Nk, p.sk.s, D);
  const __amdgpu_buffer_rsrc_t vrs = head_rsrc(vp, p.Nk, p.sv.s, D);
  const uint32_t krow = (uint32_t)(p.sk.s * 2), vrow = (uint32_t)(p.sv.s * 2);
  const uint32_t ktb = kBN * krow, vtb = kBN * vrow;
  using TC = TileCopy<D>;

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
  // prologue: tiles jt0 .. jt0+2 in flight (tile j lives in slot j mod 4)
#pragma unroll
  for (int t0 = 0; t0 < 3; ++t0) {
    const int jj = jt0 + t0;
    if (jj < n_kt) {
      TC::issue(krs, krow, (uint32_t)jj * ktb, Ks[jj & 3], lane, wave);
      TC::issue(vrs, vrow, (uint32_t)jj * vtb, Vs[jj & 3], lane, wave);
    }
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

  TileAddr<D> ta;
  ta.init(lane);

  if (n_kt - jt0 > 2) {
    wait_vmcnt<2 * TC::NI>();
  } else {
    wait_loads();
  }
#pragma unroll
  for (int nb = 0; nb < kNQB; ++nb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[nb][ks] ^= p.qflip;
  lds_barrier();

  // S(0)
  f32x16 sa[kNQB], sb[kNQB];
#pragma unroll
  for (int nb = 0; nb < kNQB; ++nb) sa[nb] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const u32x4 a = lds_b128(Ks[jt0 & 3], ta.rm[ks]);
#pragma unroll
    for (int nb = 0; nb < kNQB; ++nb) sa[nb] = mfma32<DT>(a, qf[nb][ks], sa[nb]);
  }

  // (Unrolling by two so that S alternates between the two register sets
  // without the copy costs ~60 more registers and spills at d = 64.)
  for (int j = jt0; j < n_kt; ++j) {
    const int sl = j & 3;
    fwd_step<D, DT, BAND, DROP>(j, n_kt, sa, sb, Ks[(sl + 1) & 3], Vs[sl], Ks[(sl + 3) & 3], Vs[(sl + 3) & 3], krs,
                                vrs, krow, vrow, ktb, vtb, qf, acc, st, p.Nk, p.wl, p.wr, qw0, c, lane, wave, ta,
                                p.drop, (uint32_t)bh);
#pragma unroll
    for (int nb = 0; nb < kNQB; ++nb) sa[nb] = sb[nb];
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

template <int D, int DT, bool BAND, bool DROP>
hipError_t launch_t(const FwdParams& p, hipStream_t stream) {
  constexpr int kBM = FwdTile<D>::BM;
  const int n_qt = (p.Nq + kBM - 1) / kBM;
  const int64_t blocks = (int64_t)n_qt * p.B * p.H;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_kernel<D, DT, BAND, DROP>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D, int DT>
hipError_t launch_dc(const FwdParams& p, bool banded, hipStream_t stream) {
  if (p.drop.thr > 0) return banded ? launch_t<D, DT, true, true>(p, stream) : launch_t<D, DT, false, true>(p, stream);
  return banded ? launch_t<D, DT, true, false>(p, stream) : launch_t<D, DT, false, false>(p, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, int d, int dtype, bool banded, hipStream_t stream) {
  if (d == 64) return dtype == DT_F16 ? launch_dc<64, DT_F16>(p, banded, stream) : launch_dc<64, DT_BF16>(p, banded, stream);
  return dtype == DT_F16 ? launch_dc<128, DT_F16>(p, banded, stream) : launch_dc<128, DT_BF16>(p, banded, stream);
}

}  // namespace fa
