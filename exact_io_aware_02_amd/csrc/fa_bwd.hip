// Backward attention kernels for gfx950 (recompute, no stored P).
//
// The forward keeps only O and the per-row log-sum-exp; the backward
// rebuilds P = exp(scale * q.k - lse) tile by tile instead of reading an
// N x N matrix (skill guide quick start: tiling and recomputation; refbase
// entry, "Capability").  With D_i = dO_i . O_i (= sum_j P_ij dP_ij):
//
//   dV = P^T dO        dP = dO V^T        dS = P * (dP - D)
//   dK = scale dS^T Q  dQ = scale dS K
//
// Three kernels, deterministic (no atomics):
//   dsum_kernel  D_i = dO_i . O_i                       (HBM bound, tiny)
//   dkdv_kernel  one workgroup per 128 keys; loops over 64-query tiles;
//                K and V stay in registers, Q / dO / lse / D tiles stream
//                through LDS double buffered.  S = Q K^T and dP = dO V^T
//                come out with a key per lane, which is exactly the B
//                operand layout for dV^T += dO^T P and dK^T += Q^T dS; the
//                transposed A operands (dO^T, Q^T) are read from the
//                untransposed LDS tiles with ds_read_b64_tr_b16.
//   dq_kernel    one workgroup per 128 queries; loops over 64-key tiles
//                like the forward; S^T and dP^T have a query per lane;
//                dQ^T += K^T dS^T with K^T read transposed from LDS.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <int DT>
__device__ __forceinline__ float lo_f32(uint32_t w);
template <int DT>
__device__ __forceinline__ float hi_f32(uint32_t w);
template <>
__device__ __forceinline__ float lo_f32<DT_F16>(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2, w)[0];
}
template <>
__device__ __forceinline__ float hi_f32<DT_F16>(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2, w)[1];
}
template <>
__device__ __forceinline__ float lo_f32<DT_BF16>(uint32_t w) {
  return __builtin_bit_cast(float, w << 16);
}
template <>
__device__ __forceinline__ float hi_f32<DT_BF16>(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xffff0000u);
}

// ------------------------------------------------------------ D = rowsum(dO * O)
template <int D, int DT>
__global__ __launch_bounds__(kThreads) void dsum_kernel(BwdParams p, int blocks_per_bh) {
  constexpr int CH = D / 8;
  constexpr int RPB = kThreads / CH;
  const int bh = blockIdx.x / blocks_per_bh;
  const int rblk = blockIdx.x - bh * blocks_per_bh;
  const int b = bh / p.H, h = bh - b * p.H;
  const int row = rblk * RPB + threadIdx.x / CH;
  const int ch = threadIdx.x % CH;
  float acc = 0.f;
  if (row < p.Nq) {
    const u32x4 x = *(const u32x4*)(p.dout + b * p.sdo.b + h * p.sdo.h + row * p.sdo.s + ch * 8);
    const u32x4 y = *(const u32x4*)(p.o + b * p.so.b + h * p.so.h + row * p.so.s + ch * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc += lo_f32<DT>(x[i]) * lo_f32<DT>(y[i]) + hi_f32<DT>(x[i]) * hi_f32<DT>(y[i]);
  }
#pragma unroll
  for (int off = CH / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (ch == 0 && row < p.Nq) p.dsum[(int64_t)bh * p.Nq + row] = acc;
}

// Write a [d x 32] fp32 accumulator block column (one row of the output per
// lane) as 4-element groups: out row `row`, columns 32*db + acc_row(half, r).
template <int DT, int DB>
__device__ __forceinline__ void store_rows(uint16_t* rowp, const f32x16 (&acc)[DB], float mul, int half) {
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = db * 32 + 8 * g4 + 4 * half;
      const f32x16& a = acc[db];
      u32x2 w = u32x2{pack2<DT>(a[4 * g4 + 0] * mul, a[4 * g4 + 1] * mul),
                      pack2<DT>(a[4 * g4 + 2] * mul, a[4 * g4 + 3] * mul)};
      *(u32x2*)(rowp + d0) = w;
    }
}

// ------------------------------------------------------------ dK, dV
template <int D, int DT, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void dkdv_kernel(BwdParams p) {
  constexpr int KW = 32;                // keys per wave
  constexpr int BNK = kWaves * KW;      // keys per workgroup
  constexpr int BMQ = 64;               // queries per streamed tile
  constexpr int QB = BMQ / 32;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int CH = D / 8;
  constexpr int RPP = kThreads / CH;
  constexpr int PASSES = BMQ / RPP;

  __shared__ __attribute__((aligned(16))) uint16_t Qs[2][BMQ * D];
  __shared__ __attribute__((aligned(16))) uint16_t Os[2][BMQ * D];  // dO tile
  __shared__ __attribute__((aligned(16))) float Ls[2][BMQ];         // lse * log2(e), +inf past Nq
  __shared__ __attribute__((aligned(16))) float Dsm[2][BMQ];        // D_i

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, col = lane & 31, half = lane >> 5;
  const int BH = p.B * p.H;
  const int t = blockIdx.x;
  const int kt = t / BH;  // ascending key tiles: the causal-heaviest first
  const int bh = t - kt * BH;
  const int b = bh / p.H, h = bh - b * p.H;
  const int k0 = kt * BNK;
  const int kw0 = k0 + wave * KW;
  const int key = kw0 + col;

  const uint16_t* qp = p.q + b * p.sq.b + h * p.sq.h;
  const uint16_t* dop = p.dout + b * p.sdo.b + h * p.sdo.h;
  const float* lsep = p.lse + (int64_t)bh * p.Nq;
  const float* dsp = p.dsum + (int64_t)bh * p.Nq;

  // K and V of this wave's keys as B operands (K^T, V^T): lane holds
  // row `key`, columns 16*ks + 8*half .. +7.
  u32x4 kf[KS], vf[KS];
  {
    const uint16_t* kp = p.k + b * p.sk.b + h * p.sk.h;
    const uint16_t* vp = p.v + b * p.sv.b + h * p.sv.h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 x = u32x4{0, 0, 0, 0}, y = u32x4{0, 0, 0, 0};
      if (key < p.Nk) {
        x = *(const u32x4*)(kp + key * p.sk.s + 16 * ks + 8 * half);
        y = *(const u32x4*)(vp + key * p.sv.s + 16 * ks + 8 * half);
      }
      kf[ks] = x;
      vf[ks] = y;
    }
  }

  const int qt0 = CAUSAL ? (k0 / BMQ) : 0;
  const int n_qt = (p.Nq + BMQ - 1) / BMQ;

  u32x4 qreg[PASSES], oreg[PASSES];
  float lreg = 0.f, dreg = 0.f;
  const int lrow = tid / CH, lch = tid % CH;
  auto load_tile = [&](int it) {
    const int i0 = it * BMQ;
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
      const int q = i0 + lrow + i * RPP;
      u32x4 x = u32x4{0, 0, 0, 0}, y = u32x4{0, 0, 0, 0};
      if (q < p.Nq) {
        x = *(const u32x4*)(qp + q * p.sq.s + lch * 8);
        y = *(const u32x4*)(dop + q * p.sdo.s + lch * 8);
      }
      qreg[i] = x;
      oreg[i] = y;
    }
    if (tid < BMQ) {
      const int q = i0 + tid;
      lreg = q < p.Nq ? lsep[q] * kLog2e : __builtin_inff();
      dreg = q < p.Nq ? dsp[q] : 0.f;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
      const int r = lrow + i * RPP;
      const int off = r * D + ((lch ^ swz<D>(r)) << 3);
      *(u32x4*)(&Qs[buf][off]) = qreg[i];
      *(u32x4*)(&Os[buf][off]) = oreg[i];
    }
    if (tid < BMQ) {
      Ls[buf][tid] = lreg;
      Dsm[buf][tid] = dreg;
    }
  };

  f32x16 adk[DB], adv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    adk[db] = f32x16{};
    adv[db] = f32x16{};
  }
  const float c = p.c;

  if (qt0 < n_qt) {
    load_tile(qt0);
    store_tile(0);
  }
  __syncthreads();

  for (int it = qt0; it < n_qt; ++it) {
    const int buf = (it - qt0) & 1;
    const int i0 = it * BMQ;
    if (it + 1 < n_qt) load_tile(it + 1);

    const bool active = kw0 < p.Nk && !(CAUSAL && i0 + BMQ - 1 < kw0);
    if (active) {
      const uint16_t* Qt = Qs[buf];
      const uint16_t* Ot = Os[buf];
      f32x16 s[QB], dp[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        s[qb] = f32x16{};
        dp[qb] = f32x16{};
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const u32x4 aq = load_rowmajor_op<D>(Qt, qb * 32 + col, ks, half);
          const u32x4 ao = load_rowmajor_op<D>(Ot, qb * 32 + col, ks, half);
          s[qb] = mfma32<DT>(aq, kf[ks], s[qb]);
          dp[qb] = mfma32<DT>(ao, vf[ks], dp[qb]);
        }
      // P and dS; rows are queries i0 + 32*qb + acc_row(half, r).
      const bool need_mask = CAUSAL && (i0 < kw0 + KW - 1);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int rq = qb * 32 + 8 * g4 + 4 * half;
          const float4 lv = *(const float4*)(&Ls[buf][rq]);
          const float4 dv = *(const float4*)(&Dsm[buf][rq]);
          const float lz[4] = {lv.x, lv.y, lv.z, lv.w};
          const float dz[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g4 + e;
            float pv = exp2_fast(__builtin_fmaf(s[qb][r], c, -lz[e]));
            if (need_mask && key > i0 + rq + e) pv = 0.f;
            s[qb][r] = pv;
            dp[qb][r] = pv * (dp[qb][r] - dz[e]);
          }
        }
      // dV^T += dO^T P ; dK^T += Q^T dS   (k runs over this tile's queries)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const u32x4 bp = pack_acc8<DT>(s[qb], kk);
          const u32x4 bd = pack_acc8<DT>(dp[qb], kk);
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const u32x4 ao = load_transposed_a<D>(Ot, lane, qb * 32 + kk * 16, db);
            adv[db] = mfma32<DT>(ao, bp, adv[db]);
            const u32x4 aq = load_transposed_a<D>(Qt, lane, qb * 32 + kk * 16, db);
            adk[db] = mfma32<DT>(aq, bd, adk[db]);
          }
        }
    }

    if (it + 1 < n_qt) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (key < p.Nk) {
    store_rows<DT, DB>(p.dk + b * p.sdk.b + h * p.sdk.h + key * p.sdk.s, adk, p.scale, half);
    store_rows<DT, DB>(p.dv + b * p.sdv.b + h * p.sdv.h + key * p.sdv.s, adv, 1.0f, half);
  }
}

// ------------------------------------------------------------ dQ
template <int D, int DT, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void dq_kernel(BwdParams p) {
  constexpr int QW = 32;
  constexpr int BM = kWaves * QW;
  constexpr int BN = 64;
  constexpr int RB = BN / 32;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int CH = D / 8;
  constexpr int RPP = kThreads / CH;
  constexpr int PASSES = BN / RPP;

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][BN * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, col = lane & 31, half = lane >> 5;
  const int BH = p.B * p.H;
  const int n_qt = (p.Nq + BM - 1) / BM;
  const int t = blockIdx.x;
  const int qt = n_qt - 1 - t / BH;
  const int bh = t - (t / BH) * BH;
  const int b = bh / p.H, h = bh - b * p.H;
  const int q0 = qt * BM;
  const int qw0 = q0 + wave * QW;
  const int qi = qw0 + col;

  const uint16_t* kp = p.k + b * p.sk.b + h * p.sk.h;
  const uint16_t* vp = p.v + b * p.sv.b + h * p.sv.h;

  u32x4 qf[KS], of[KS];
  {
    const uint16_t* qp = p.q + b * p.sq.b + h * p.sq.h;
    const uint16_t* dop = p.dout + b * p.sdo.b + h * p.sdo.h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 x = u32x4{0, 0, 0, 0}, y = u32x4{0, 0, 0, 0};
      if (qi < p.Nq) {
        x = *(const u32x4*)(qp + qi * p.sq.s + 16 * ks + 8 * half);
        y = *(const u32x4*)(dop + qi * p.sdo.s + 16 * ks + 8 * half);
      }
      qf[ks] = x;
      of[ks] = y;
    }
  }
  const float lse2 = qi < p.Nq ? p.lse[(int64_t)bh * p.Nq + qi] * kLog2e : __builtin_inff();
  const float dsv = qi < p.Nq ? p.dsum[(int64_t)bh * p.Nq + qi] : 0.f;

  int kend = p.Nk;
  if (CAUSAL) kend = min(p.Nk, min(q0 + BM, p.Nq));
  const int n_kt = (kend + BN - 1) / BN;

  u32x4 kreg[PASSES], vreg[PASSES];
  const int lrow = tid / CH, lch = tid % CH;
  auto load_tile = [&](int j) {
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
      const int kk = j * BN + lrow + i * RPP;
      u32x4 x = u32x4{0, 0, 0, 0}, y = u32x4{0, 0, 0, 0};
      if (kk < p.Nk) {
        x = *(const u32x4*)(kp + kk * p.sk.s + lch * 8);
        y = *(const u32x4*)(vp + kk * p.sv.s + lch * 8);
      }
      kreg[i] = x;
      vreg[i] = y;
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

  f32x16 adq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) adq[db] = f32x16{};
  const float c = p.c;

  if (n_kt > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int j = 0; j < n_kt; ++j) {
    const int buf = j & 1;
    const int j0 = j * BN;
    if (j + 1 < n_kt) load_tile(j + 1);
    const bool active = qw0 < p.Nq && !(CAUSAL && j0 > qw0 + QW - 1);
    if (active) {
      const uint16_t* Kt = Ks[buf];
      const uint16_t* Vt = Vs[buf];
      f32x16 s[RB], dp[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        s[rb] = f32x16{};
        dp[rb] = f32x16{};
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const u32x4 ak = load_rowmajor_op<D>(Kt, rb * 32 + col, ks, half);
          const u32x4 av = load_rowmajor_op<D>(Vt, rb * 32 + col, ks, half);
          s[rb] = mfma32<DT>(ak, qf[ks], s[rb]);
          dp[rb] = mfma32<DT>(av, of[ks], dp[rb]);
        }
      const bool need_mask = (j0 + BN > p.Nk) || (CAUSAL && j0 + BN - 1 > qw0);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pv = exp2_fast(__builtin_fmaf(s[rb][r], c, -lse2));
          if (need_mask) {
            const int kk = j0 + rb * 32 + acc_row(half, r);
            if (kk >= p.Nk || (CAUSAL && kk > qi)) pv = 0.f;
          }
          dp[rb][r] = pv * (dp[rb][r] - dsv);
        }
      // dQ^T += K^T dS^T  (k runs over this tile's keys)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const u32x4 bd = pack_acc8<DT>(dp[rb], kk);
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const u32x4 ak = load_transposed_a<D>(Kt, lane, rb * 32 + kk * 16, db);
            adq[db] = mfma32<DT>(ak, bd, adq[db]);
          }
        }
    }
    if (j + 1 < n_kt) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (qi < p.Nq) store_rows<DT, DB>(p.dq + b * p.sdq.b + h * p.sdq.h + qi * p.sdq.s, adq, p.scale, half);
}

template <int D, int DT, bool CAUSAL>
hipError_t launch_t(const BwdParams& p, int stages, hipStream_t stream) {
  const int64_t BH = (int64_t)p.B * p.H;
  constexpr int RPB = kThreads / (D / 8);
  const int64_t dsum_bpb = (p.Nq + RPB - 1) / RPB;
  const int64_t g0 = dsum_bpb * BH;
  const int64_t g1 = (int64_t)((p.Nk + 127) / 128) * BH;
  const int64_t g2 = (int64_t)((p.Nq + 127) / 128) * BH;
  if (g0 > 0x7fffffff || g1 > 0x7fffffff || g2 > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipError_t e = hipSuccess;
  if ((stages & 1) && g0 > 0) {  // Nq may be 0 (then dK = dV = 0 and there is no dQ)
    hipLaunchKernelGGL((dsum_kernel<D, DT>), dim3((unsigned)g0), dim3(kThreads), 0, stream, p, (int)dsum_bpb);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((stages & 2) && g1 > 0) {
    hipLaunchKernelGGL((dkdv_kernel<D, DT, CAUSAL>), dim3((unsigned)g1), dim3(kThreads), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((stages & 4) && g2 > 0) {
    hipLaunchKernelGGL((dq_kernel<D, DT, CAUSAL>), dim3((unsigned)g2), dim3(kThreads), 0, stream, p);
    e = hipGetLastError();
  }
  return e;
}

template <int D, int DT>
hipError_t launch_dc(const BwdParams& p, bool causal, int stages, hipStream_t stream) {
  return causal ? launch_t<D, DT, true>(p, stages, stream) : launch_t<D, DT, false>(p, stages, stream);
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p, int d, int dtype, bool causal, int stages, hipStream_t stream) {
  if (d == 64)
    return dtype == DT_F16 ? launch_dc<64, DT_F16>(p, causal, stages, stream)
                           : launch_dc<64, DT_BF16>(p, causal, stages, stream);
  return dtype == DT_F16 ? launch_dc<128, DT_F16>(p, causal, stages, stream)
                         : launch_dc<128, DT_BF16>(p, causal, stages, stream);
}

}  // namespace fa
