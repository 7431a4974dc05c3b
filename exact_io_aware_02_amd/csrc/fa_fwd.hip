// Forward attention kernel for gfx950.
//
// One workgroup of 4 waves owns BM = 4 * 32 * NQB query rows of one
// (batch, head); each wave owns 32 * NQB of them and their softmax state,
// so the row max / row sum never leave the wave (FlashAttention-2's
// point of less communication between warps, refbase Q&A on FA2's
// improvements).  K/V tiles of BN = 64 keys stream HBM -> registers ->
// LDS, double buffered: the loads of tile j+1 are in flight while tile j is
// computed.  Per tile and wave:
//
//   S^T = K_j Q^T          32x32x16 MFMAs; A = K rows from LDS, B = Q held
//                          in registers for the whole loop.  Each lane then
//                          holds 16 keys x 1 query of every 32x32 block, so
//                          the row max and sum are in-lane, plus one
//                          exchange with lane i^32.
//   online softmax         m' = max(m, max_j S*c); alpha = 2^(m - m');
//                          P = 2^(S*c - m'); l = alpha*l + sum P;
//                          O^T *= alpha   (c = |scale| * log2 e)
//   O^T += V_j^T P^T       A = V^T via ds_read_b64_tr_b16 from the
//                          untransposed V tile, B = P^T repacked in place
//                          from the S^T accumulator (no LDS round trip).
//
// Epilogue: O = O^T / l, LSE = (m + log2 l) * ln 2.  Causal: tiles wholly
// after a workgroup's last query are never loaded; tiles wholly after a
// wave's last query are skipped by that wave; only tiles that cross the
// diagonal or the key tail are masked elementwise.
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
constexpr int kBN = 64;

template <int D, int DT, bool CAUSAL, int NQB>
__global__ __launch_bounds__(kThreads) void fwd_kernel(FwdParams p) {
  constexpr int QW = 32 * NQB;        // queries per wave
  constexpr int BM = kWaves * QW;     // queries per workgroup
  constexpr int KS = D / 16;          // k-steps of S^T = K Q^T
  constexpr int DB = D / 32;          // 32-row blocks of O^T
  constexpr int RB = kBN / 32;        // 32-key blocks per tile
  constexpr int CH = D / 8;           // 16-byte chunks per row
  constexpr int RPP = kThreads / CH;  // rows per load pass
  constexpr int PASSES = kBN / RPP;

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kBN * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][kBN * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, col = lane & 31, half = lane >> 5;

  // Heaviest query tiles first: block t covers query tile (last - t / BH),
  // head t % BH.  Consecutive blocks land on different XCDs round-robin,
  // so a head's tiles share one XCD's L2 when B*H is a multiple of 8.
  const int BH = p.B * p.H;
  const int n_qt = (p.Nq + BM - 1) / BM;
  const int t = blockIdx.x;
  const int qt = n_qt - 1 - t / BH;
  const int bh = t - (t / BH) * BH;
  const int b = bh / p.H, h = bh - b * p.H;
  const int q0 = qt * BM;
  const int qw0 = q0 + wave * QW;

  const uint16_t* qp = p.q + b * p.sq.b + h * p.sq.h;
  const uint16_t* kp = p.k + b * p.sk.b + h * p.sk.h;
  const uint16_t* vp = p.v + b * p.sv.b + h * p.sv.h;

  // Q^T as the B operand, resident in registers: lane holds
  // Q[qw0 + 32*nb + col][16*ks + 8*half .. +7].
  u32x4 qf[NQB][KS];
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
    const int qi = qw0 + 32 * nb + col;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 x = u32x4{0, 0, 0, 0};
      if (qi < p.Nq) x = *(const u32x4*)(qp + qi * p.sq.s + 16 * ks + 8 * half);
      qf[nb][ks] = x ^ p.qflip;
    }
  }

  int kend = p.Nk;
  if (CAUSAL) kend = min(p.Nk, min(q0 + BM, p.Nq));
  const int n_kt = (kend + kBN - 1) / kBN;

  u32x4 kreg[PASSES], vreg[PASSES];
  const int lrow = tid / CH, lch = tid % CH;
  auto load_tile = [&](int j) {
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
      const int key = j * kBN + lrow + i * RPP;
      u32x4 kx = u32x4{0, 0, 0, 0}, vx = u32x4{0, 0, 0, 0};
      if (key < p.Nk) {
        kx = *(const u32x4*)(kp + key * p.sk.s + lch * 8);
        vx = *(const u32x4*)(vp + key * p.sv.s + lch * 8);
      }
      kreg[i] = kx;
      vreg[i] = vx;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
      const int r = lrow + i * RPP;
      const int off = r * D + ((lch ^ swz<D>(r)) << 3);
      *(u32x4*)(&Ks[buf][off]) = kreg[i];
      *(u32x4*)(&Vs[buf][off]) = vreg[i];
    }
  };

  f32x16 acc[DB][NQB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int nb = 0; nb < NQB; ++nb) acc[db][nb] = f32x16{};
  float m[NQB], l[NQB];
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
    m[nb] = -1e30f;
    l[nb] = 0.f;
  }
  const float c = p.c;
  const bool wave_has_rows = qw0 < p.Nq;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < n_kt; ++j) {
    const int buf = j & 1;
    const int j0 = j * kBN;
    if (j + 1 < n_kt) load_tile(j + 1);

    const bool active = wave_has_rows && !(CAUSAL && j0 > qw0 + QW - 1);
    if (active) {
      const uint16_t* Kt = Ks[buf];
      const uint16_t* Vt = Vs[buf];
      // ---- S^T = K Q^T
      f32x16 s[RB][NQB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int nb = 0; nb < NQB; ++nb) s[rb][nb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const u32x4 a = load_rowmajor_op<D>(Kt, rb * 32 + col, ks, half);
#pragma unroll
          for (int nb = 0; nb < NQB; ++nb) s[rb][nb] = mfma32<DT>(a, qf[nb][ks], s[rb][nb]);
        }
      }
      // ---- masks (only tiles crossing the key tail or the diagonal)
      const bool need_mask = (j0 + kBN > p.Nk) || (CAUSAL && j0 + kBN - 1 > qw0);
      if (need_mask) {
#pragma unroll
        for (int nb = 0; nb < NQB; ++nb) {
          const int qi = qw0 + 32 * nb + col;
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = j0 + rb * 32 + acc_row(half, r);
              if (key >= p.Nk || (CAUSAL && key > qi)) s[rb][nb][r] = -__builtin_inff();
            }
        }
      }
      // ---- online softmax
#pragma unroll
      for (int nb = 0; nb < NQB; ++nb) {
        float mx = s[0][nb][0];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[rb][nb][r]);
        mx = fmaxf(mx, xor32(mx));
        const float mnew = fmaxf(m[nb], mx * c);
        const float alpha = exp2_fast(m[nb] - mnew);
        m[nb] = mnew;
        float rs = 0.f;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float pv = exp2_fast(__builtin_fmaf(s[rb][nb][r], c, -mnew));
            s[rb][nb][r] = pv;
            rs += pv;
          }
        l[nb] = l[nb] * alpha + rs;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db][nb] *= alpha;
      }
      // ---- O^T += V^T P^T
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          u32x4 pf[NQB];
#pragma unroll
          for (int nb = 0; nb < NQB; ++nb) pf[nb] = pack_acc8<DT>(s[rb][nb], kk);
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const u32x4 a = load_transposed_a<D>(Vt, lane, rb * 32 + kk * 16, db);
#pragma unroll
            for (int nb = 0; nb < NQB; ++nb) acc[db][nb] = mfma32<DT>(a, pf[nb], acc[db][nb]);
          }
        }
      }
    }

    if (j + 1 < n_kt) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, LSE
  uint16_t* op = p.o + b * p.so.b + h * p.so.h;
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
    const float lt = l[nb] + xor32(l[nb]);
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
      if (half == 0) p.lse[(int64_t)bh * p.Nq + qi] = (m[nb] + log2_fast(lt)) * kLn2;
    }
  }
}

template <int D, int DT, bool CAUSAL, int NQB>
hipError_t launch_t(const FwdParams& p, hipStream_t stream) {
  constexpr int BM = kWaves * 32 * NQB;
  const int n_qt = (p.Nq + BM - 1) / BM;
  const int64_t blocks = (int64_t)n_qt * p.B * p.H;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_kernel<D, DT, CAUSAL, NQB>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D, int DT>
hipError_t launch_dc(const FwdParams& p, bool causal, hipStream_t stream) {
  return causal ? launch_t<D, DT, true, 1>(p, stream) : launch_t<D, DT, false, 1>(p, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, int d, int dtype, bool causal, hipStream_t stream) {
  if (d == 64) return dtype == DT_F16 ? launch_dc<64, DT_F16>(p, causal, stream) : launch_dc<64, DT_BF16>(p, causal, stream);
  return dtype == DT_F16 ? launch_dc<128, DT_F16>(p, causal, stream) : launch_dc<128, DT_BF16>(p, causal, stream);
}

}  // namespace fa
