// Forward attention kernel for gfx950.
//
// One workgroup of 4 waves owns BM = 256 query rows of one (batch, head);
// each wave owns 64 of them (two 32-query MFMA column blocks) and their
// softmax state, so the row max and row sum never leave the wave
// (FlashAttention-2's point of less communication between warps, refbase
// Q&A on FA2's improvements).  K/V tiles of BN = 64 keys stream from HBM
// straight into LDS (global_load_lds_dwordx4, no staging registers),
// double buffered.  Per tile and wave:
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
// The loop is software pipelined: S for tile j+1 is computed by MFMA while
// the VALU exponentiates tile j, so the matrix cores and the vector/
// transcendental units work at the same time (the overlap FA3 gets from
// asynchrony on Hopper, glossary article's FA-3 section, done here within
// one wave).
//
// Epilogue: O = O^T / l, LSE = (m + log2 l) * ln 2.  Causal: tiles wholly
// after a workgroup's last query are never loaded; tiles that cross a
// wave's diagonal or the key tail are masked elementwise.
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
  static constexpr bool UNROLL_RING = false;  // true: constant slot addresses (but spills at d=128)
  static constexpr int QK_LOOKAHEAD = 4;     // K operand reads issued ahead of their MFMAs
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

// S^T (32 keys x 64 queries) of one tile: A = K rows from LDS, B = Q^T.
// The issue order is pinned (LA operand reads ahead, then the MFMAs of one
// k-step per read) so at most LA + 1 K operands are live: the scheduler
// would otherwise hoist all of them.
template <int D, int DT, int kNQB, int LA = FwdTile<D>::QK_LOOKAHEAD>
__device__ __forceinline__ void qk(f32x16 (&s)[kNQB], const uint16_t* Kt, const u32x4 (&qf)[kNQB][D / 16],
                                   const TileAddr<D>& ta) {
  constexpr int KS = D / 16;
#pragma unroll
  for (int nb = 0; nb < kNQB; ++nb) s[nb] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const u32x4 a = lds_b128(Kt, ta.rm[ks]);
#pragma unroll
    for (int nb = 0; nb < kNQB; ++nb) s[nb] = mfma32<DT>(a, qf[nb][ks], s[nb]);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);  // DS read x LA
#pragma unroll
  for (int i = 0; i < KS - LA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, kNQB, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // DS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, LA * kNQB, 0);
}

template <int kNQB>
struct RowState {
  float m[kNQB];  // running max, log2 units (scaled by c)
  float l[kNQB];  // this lane's partial row sum (lane i^32 holds the rest)
};

// One K/V tile of the forward loop.  The __restrict__ tile pointers tell
// the compiler the LDS reads of tile j never alias the asynchronous copy
// into tile j+2's slot, so it does not wait for that copy before reading;
// the explicit vmcnt wait + barrier at the end orders the ring.
template <int D, int DT, bool CAUSAL, int kNQB = FwdTile<D>::NQB>
__device__ __forceinline__ void fwd_iter(int j, int n_kt, const uint16_t* __restrict__ Kt,
                                         const uint16_t* __restrict__ Vt, uint16_t* __restrict__ Kdst,
                                         uint16_t* __restrict__ Vdst, __amdgpu_buffer_rsrc_t krs,
                                         __amdgpu_buffer_rsrc_t vrs, uint32_t krow, uint32_t vrow, uint32_t ktb,
                                         uint32_t vtb, const u32x4 (&qf)[kNQB][D / 16], f32x16 (&acc)[D / 32][kNQB],
                                         RowState<kNQB>& st, int Nk, int qw0, float c, int lane, int wave,
                                         const TileAddr<D>& ta) {
  using TC = TileCopy<D>;
  constexpr int DB = D / 32;
  const int j0 = j * kBN;
  const int ln = lane;
  const int col = ln & 31, half = ln >> 5;

  if (j + 2 < n_kt) {
    TC::issue(krs, krow, (uint32_t)(j + 2) * ktb, Kdst, ln, wave);
    TC::issue(vrs, vrow, (uint32_t)(j + 2) * vtb, Vdst, ln, wave);
  }

  // ---- S^T = K Q^T
  f32x16 s[kNQB];
  qk<D, DT, kNQB>(s, Kt, qf, ta);

  // ---- masks (only tiles crossing the key tail or this wave's diagonal)
  if ((j0 + kBN > Nk) || (CAUSAL && j0 + kBN - 1 > qw0)) {
#pragma unroll
    for (int nb = 0; nb < kNQB; ++nb) {
      const int qi = qw0 + 32 * nb + col;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + acc_row(half, r);
        if (key >= Nk || (CAUSAL && key > qi)) s[nb][r] = -__builtin_inff();
      }
    }
  }
  // ---- row max; lazy rescale
  float mxc[kNQB];
  bool raise = false;
#pragma unroll
  for (int nb = 0; nb < kNQB; ++nb) {
    float mx = s[nb][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[nb][r]);
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
  // ---- P = 2^(S c - m) packed into the MFMA B operand; row sums from the packed values
  u32x4 pf[2][kNQB];
#pragma unroll
  for (int nb = 0; nb < kNQB; ++nb) {
    const float mneg = -st.m[nb];
    float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 8 * kk + 2 * e;
        const float p0 = exp2_fast(__builtin_fmaf(s[nb][r], c, mneg));
        const float p1 = exp2_fast(__builtin_fmaf(s[nb][r + 1], c, mneg));
        w[e] = pack2<DT>(p0, p1);
        if constexpr (DT == DT_BF16) {  // bf16 rounding (2^-9) is too coarse for the normaliser
          ls0 = (r == 0) ? p0 : ls0 + p0;
          ls1 = (r == 0) ? p1 : ls1 + p1;
        }
      }
      if constexpr (DT == DT_F16) {  // fp16-rounded P is accurate enough: sum pairs in one op
        ls0 = dot2_sum<DT>(w[0], ls0);
        ls1 = dot2_sum<DT>(w[1], ls1);
        ls0 = dot2_sum<DT>(w[2], ls0);
        ls1 = dot2_sum<DT>(w[3], ls1);
      }
      pf[kk][nb] = u32x4{w[0], w[1], w[2], w[3]};
    }
    st.l[nb] += ls0 + ls1;
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

  // tile j+1 (issued one step earlier) must have landed; tile j+2 may fly on
  if (j + 2 < n_kt) {
    wait_vmcnt<2 * TC::NI>();
  } else {
    wait_loads();
  }
  lds_barrier();
}

template <int D, int DT, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(FwdTile<D>::WAVES_PER_SIMD,
                                                                          FwdTile<D>::WAVES_PER_SIMD))) void fwd_kernel(FwdParams p) {
  constexpr int kNQB = FwdTile<D>::NQB;
  constexpr int kQW = FwdTile<D>::QW;
  constexpr int kBM = FwdTile<D>::BM;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int NBUF = 3;  // K/V ring: tile j+2 loads while tile j is computed
  constexpr int TILE = kBN * D;

  __shared__ __attribute__((aligned(1024))) uint16_t Ks[NBUF][TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t Vs[NBUF][TILE];

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

  const uint16_t* qp = p.q + b * p.sq.b + h * p.sq.h;
  const uint16_t* kp = p.k + b * p.sk.b + h * p.sk.h;
  const uint16_t* vp = p.v + b * p.sv.b + h * p.sv.h;

  int kend = p.Nk;
  if (CAUSAL) kend = min(p.Nk, min(q0 + kBM, p.Nq));
  const int n_kt = (kend + kBN - 1) / kBN;

  const __amdgpu_buffer_rsrc_t krs = head_rsrc(kp, p.Nk, p.sk.s, D);
  const __amdgpu_buffer_rsrc_t vrs = head_rsrc(vp, p.Nk, p.sv.s, D);
  const uint32_t krow = (uint32_t)(p.sk.s * 2), vrow = (uint32_t)(p.sv.s * 2);
  const uint32_t ktb = kBN * krow, vtb = kBN * vrow;
  using TC = TileCopy<D>;

  // prologue: tiles 0 and 1 in flight before Q is touched
  TC::issue(krs, krow, 0, Ks[0], lane, wave);
  TC::issue(vrs, vrow, 0, Vs[0], lane, wave);
  if (n_kt > 1) {
    TC::issue(krs, krow, ktb, Ks[1], lane, wave);
    TC::issue(vrs, vrow, vtb, Vs[1], lane, wave);
  }

  // Q^T as the B operand, resident in registers: lane holds
  // Q[qw0 + 32*nb + col][16*ks + 8*half .. +7].
  u32x4 qf[kNQB][KS];
#pragma unroll
  for (int nb = 0; nb < kNQB; ++nb) {
    const int qi = qw0 + 32 * nb + col;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 x = u32x4{0, 0, 0, 0};
      if (qi < p.Nq) x = *(const u32x4*)(qp + qi * p.sq.s + 16 * ks + 8 * half);
      qf[nb][ks] = x ^ p.qflip;
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

  wait_loads();
  lds_barrier();

  static_assert(NBUF == 3, "the loops below assume a 3-slot ring");
  if constexpr (FwdTile<D>::UNROLL_RING) {
    // unrolled by the ring depth: every slot address is a compile-time
    // constant, folded into the LDS instructions' offsets
    for (int j = 0; j < n_kt; j += 3) {
      fwd_iter<D, DT, CAUSAL>(j, n_kt, Ks[0], Vs[0], Ks[2], Vs[2], krs, vrs, krow, vrow, ktb, vtb, qf, acc, st, p.Nk,
                              qw0, c, lane, wave, ta);
      if (j + 1 >= n_kt) break;
      fwd_iter<D, DT, CAUSAL>(j + 1, n_kt, Ks[1], Vs[1], Ks[0], Vs[0], krs, vrs, krow, vrow, ktb, vtb, qf, acc, st,
                              p.Nk, qw0, c, lane, wave, ta);
      if (j + 2 >= n_kt) break;
      fwd_iter<D, DT, CAUSAL>(j + 2, n_kt, Ks[2], Vs[2], Ks[1], Vs[1], krs, vrs, krow, vrow, ktb, vtb, qf, acc, st,
                              p.Nk, qw0, c, lane, wave, ta);
    }
  } else {
    int buf = 0;
    for (int j = 0; j < n_kt; ++j) {
      // prefetch tile j+2 into the slot tile j-1 used (free since the last barrier)
      int nbuf = buf + 2;
      nbuf = nbuf >= NBUF ? nbuf - NBUF : nbuf;
      fwd_iter<D, DT, CAUSAL>(j, n_kt, Ks[buf], Vs[buf], Ks[nbuf], Vs[nbuf], krs, vrs, krow, vrow, ktb, vtb, qf, acc,
                              st, p.Nk, qw0, c, lane, wave, ta);
      buf = buf + 1 >= NBUF ? 0 : buf + 1;
    }
  }

  // ---- epilogue: O = O^T / l, LSE
  uint16_t* op = p.o + b * p.so.b + h * p.so.h;
#pragma unroll
  for (int nb = 0; nb < kNQB; ++nb) {
    const float lt = sum_pair32(st.l[nb]);
    const int qi = qw0 + 32 * nb + col;
    if (qi < p.Nq) {
      const float inv = 1.0f / lt;
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
      if (half == 0) p.lse[(int64_t)bh * p.Nq + qi] = (st.m[nb] + log2_fast(lt)) * kLn2;
    }
  }
}

template <int D, int DT, bool CAUSAL>
hipError_t launch_t(const FwdParams& p, hipStream_t stream) {
  constexpr int kBM = FwdTile<D>::BM;
  const int n_qt = (p.Nq + kBM - 1) / kBM;
  const int64_t blocks = (int64_t)n_qt * p.B * p.H;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_kernel<D, DT, CAUSAL>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D, int DT>
hipError_t launch_dc(const FwdParams& p, bool causal, hipStream_t stream) {
  return causal ? launch_t<D, DT, true>(p, stream) : launch_t<D, DT, false>(p, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, int d, int dtype, bool causal, hipStream_t stream) {
  if (d == 64) return dtype == DT_F16 ? launch_dc<64, DT_F16>(p, causal, stream) : launch_dc<64, DT_BF16>(p, causal, stream);
  return dtype == DT_F16 ? launch_dc<128, DT_F16>(p, causal, stream) : launch_dc<128, DT_BF16>(p, causal, stream);
}

}  // namespace fa
