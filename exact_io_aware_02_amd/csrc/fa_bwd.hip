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
//   prep_kernel  D_i = dO_i . O_i and lse_i * log2(e) per query row, into
//                the workspace (HBM bound, tiny).
//   dkdv_kernel  a workgroup owns 128 keys (32 per wave) with K and V held
//                in registers; 32-query tiles of Q, dO and the two row
//                statistics stream HBM -> LDS through a 3-slot ring.
//                S = Q K^T and dP = dO V^T come out with a key per lane,
//                which is the B-operand layout of dV^T += dO^T P and
//                dK^T += Q^T dS; the transposed A operands (dO^T, Q^T) are
//                read from the same untransposed LDS tiles with
//                ds_read_b64_tr_b16.
//   dq_kernel    a workgroup owns 128 queries (32 per wave) with Q and dO
//                in registers; 32-key tiles of K and V stream through a
//                3-slot ring like the forward.  S^T and dP^T have a query
//                per lane (its lse and D are lane-local); dQ^T += K^T dS^T
//                reads K^T transposed from the K tile.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kT = 32;        // rows per streamed tile (queries in dkdv, keys in dq)
constexpr int kNBuf = 3;      // ring slots: tile t+2 loads while tile t is computed
constexpr int kStatPad = 64;  // per-(b,h) stride of the workspace statistics, rounded up to this

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

__host__ __device__ __forceinline__ int stat_stride(int Nq) { return (Nq + kStatPad - 1) / kStatPad * kStatPad; }

// ------------------------------------------------------------ D and lse*log2(e)
template <int D, int DT>
__global__ __launch_bounds__(kThreads) void prep_kernel(BwdParams p, int blocks_per_bh) {
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
  // rows in [Nq, stat_stride) get zeros: the kernels then treat them as
  // queries with zero Q/dO rows, which contribute nothing
  if (ch == 0 && row < stat_stride(p.Nq)) {
    const int64_t o = (int64_t)bh * stat_stride(p.Nq) + row;
    p.dsum[o] = acc;
    p.lse2[o] = row < p.Nq ? p.lse[(int64_t)bh * p.Nq + row] * kLog2e : 0.f;
  }
}

// Write a [d x 32] fp32 accumulator block column (one output row per lane)
// as 4-element groups: columns 32*db + acc_row(half, r) of row `rowp`.
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

// 32x32 accumulator = init + rows of a row-major LDS tile (32 rows) times B
// held in registers, contracting over d.
template <int D, int DT>
__device__ __forceinline__ f32x16 rows_times_regs(const uint16_t* tile, const u32x4 (&bf)[D / 16],
                                                  const TileAddr<D>& ta, f32x16 s = f32x16{}) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) s = mfma32<DT>(lds_b128(tile, ta.rm[ks]), bf[ks], s);
  return s;
}

// acc[db] += tile^T (d x 32 tile rows, read transposed) x B (32 tile rows x
// 32, packed from a 32x32 accumulator in its register k order).
template <int D, int DT>
__device__ __forceinline__ void tile_t_times(f32x16 (&acc)[D / 32], const uint16_t* tile, const u32x4 (&bp)[2],
                                             const TileAddr<D>& ta) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] = mfma32<DT>(lds_transposed_a<D>(tile, ta, kk, db), bp[kk], acc[db]);
}

// ------------------------------------------------------------ dK, dV
template <int D, int DT, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void dkdv_kernel(BwdParams p) {
  constexpr int KW = 32;            // keys per wave
  constexpr int BNK = kWaves * KW;  // keys per workgroup
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  using TC = TileCopyT<D, kT, kWaves>;
  constexpr int NLOADS = 2 * TC::NI + 2;  // per wave per tile: Q, dO, 8 lse2 and 8 D values

  // One LDS object (separate __shared__ variables get separate alias
  // scopes, and the compiler then waits for every in-flight copy into a
  // variable before reading any part of it).
  struct Smem {
    uint16_t q[kNBuf][kT * D];
    uint16_t o[kNBuf][kT * D];  // dO
    float l[kNBuf][kT];         // lse * log2(e)
    float d[kNBuf][kT];         // D
  };
  __shared__ __attribute__((aligned(1024))) Smem sm;
  auto& Qs = sm.q;
  auto& Os = sm.o;
  auto& Ls = sm.l;
  auto& Dsm = sm.d;

  const int tid = threadIdx.x;
  const int lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const __amdgpu_buffer_rsrc_t qrs = head_rsrc(qp, p.Nq, p.sq.s, D);
  const __amdgpu_buffer_rsrc_t ors = head_rsrc(dop, p.Nq, p.sdo.s, D);
  const int sst = stat_stride(p.Nq);
  const __amdgpu_buffer_rsrc_t lrs = f32_rsrc(p.lse2 + (int64_t)bh * sst, sst);
  const __amdgpu_buffer_rsrc_t drs = f32_rsrc(p.dsum + (int64_t)bh * sst, sst);
  const uint32_t qrow = (uint32_t)(p.sq.s * 2), orow = (uint32_t)(p.sdo.s * 2);

  const int qt0 = CAUSAL ? (k0 / kT) : 0;
  const int n_qt = (p.Nq + kT - 1) / kT;

  auto issue = [&](int it, int slot) {
    TC::issue(qrs, qrow, (uint32_t)it * kT * qrow, Qs[slot], lane, wave);
    TC::issue(ors, orow, (uint32_t)it * kT * orow, Os[slot], lane, wave);
    vec_to_lds<8>(lrs, (uint32_t)(it * kT + 8 * wave) * 4, Ls[slot] + 8 * wave, lane);
    vec_to_lds<8>(drs, (uint32_t)(it * kT + 8 * wave) * 4, Dsm[slot] + 8 * wave, lane);
  };
  if (qt0 < n_qt) issue(qt0, 0);
  if (qt0 + 1 < n_qt) issue(qt0 + 1, 1);

  // K^T and V^T of this wave's keys as B operands: lane holds row `key`,
  // columns 16*ks + 8*half .. +7 (zeros past Nk).
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
  f32x16 adk[DB], adv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    adk[db] = f32x16{};
    adv[db] = f32x16{};
  }
  const float c = p.c;

  TileAddr<D> ta;
  ta.init(lane);

  wait_loads();
  lds_barrier();

  int slot = 0;
  for (int it = qt0; it < n_qt; ++it) {
    const int i0 = it * kT;
    int nslot = slot + 2;
    nslot = nslot >= kNBuf ? nslot - kNBuf : nslot;
    if (it + 2 < n_qt) issue(it + 2, nslot);

    // Queries past Nq read as zero rows with zero statistics, so they add
    // nothing to dK or dV; keys past Nk are never written.
    const bool active = kw0 < p.Nk && !(CAUSAL && i0 + kT - 1 < kw0);
    // The tile pointers are __restrict__ parameters of the inlined body so
    // that its LDS reads carry alias scopes; the compiler then leaves the
    // in-flight copy into another slot alone (the wait + barrier below
    // order the ring).
    auto body = [&](const uint16_t* __restrict__ Qt, const uint16_t* __restrict__ Ot, const float* __restrict__ Lt,
                    const float* __restrict__ Dt) {
      // S = Q K^T and dP = dO V^T: rows are queries i0 + acc_row(half, r); column = this lane's key
      f32x16 s = rows_times_regs<D, DT>(Qt, kf, ta);
      // dP - D in one pass: the dP accumulator starts at -D of its row
      f32x16 dinit;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const float4 dv = *(const float4*)(&Dt[8 * g4 + 4 * half]);
        dinit[4 * g4 + 0] = -dv.x;
        dinit[4 * g4 + 1] = -dv.y;
        dinit[4 * g4 + 2] = -dv.z;
        dinit[4 * g4 + 3] = -dv.w;
      }
      f32x16 dp = rows_times_regs<D, DT>(Ot, vf, ta, dinit);
      const bool need_mask = CAUSAL && (i0 < kw0 + KW - 1);
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int rq = 8 * g4 + 4 * half;
        const float4 lv = *(const float4*)(&Lt[rq]);
        const float lz[4] = {lv.x, lv.y, lv.z, lv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g4 + e;
          float pv = exp2_fast(__builtin_fmaf(s[r], c, -lz[e]));
          if (need_mask && key > i0 + rq + e) pv = 0.f;
          s[r] = pv;
          dp[r] = pv * dp[r];
        }
      }
      const u32x4 bp[2] = {pack_acc8<DT>(s, 0), pack_acc8<DT>(s, 1)};
      const u32x4 bd[2] = {pack_acc8<DT>(dp, 0), pack_acc8<DT>(dp, 1)};
      tile_t_times<D, DT>(adv, Ot, bp, ta);  // dV^T += dO^T P
      tile_t_times<D, DT>(adk, Qt, bd, ta);  // dK^T += Q^T dS
    };
    if (active) body(Qs[slot], Os[slot], Ls[slot], Dsm[slot]);

    if (it + 2 < n_qt) {
      wait_vmcnt<NLOADS>();
    } else {
      wait_loads();
    }
    lds_barrier();
    slot = slot + 1 >= kNBuf ? 0 : slot + 1;
  }

  if (key < p.Nk) {
    store_rows<DT, DB>(p.dk + b * p.sdk.b + h * p.sdk.h + key * p.sdk.s, adk, p.scale, half);
    store_rows<DT, DB>(p.dv + b * p.sdv.b + h * p.sdv.h + key * p.sdv.s, adv, 1.0f, half);
  }
}

// ------------------------------------------------------------ dQ
template <int D, int DT, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void dq_kernel(BwdParams p) {
  constexpr int QW = 32;
  constexpr int BM = kWaves * QW;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  using TC = TileCopyT<D, kT, kWaves>;

  struct Smem {  // one LDS object, as in dkdv_kernel
    uint16_t k[kNBuf][kT * D];
    uint16_t v[kNBuf][kT * D];
  };
  __shared__ __attribute__((aligned(1024))) Smem sm;
  auto& Ks = sm.k;
  auto& Vs = sm.v;

  const int tid = threadIdx.x;
  const int lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const __amdgpu_buffer_rsrc_t krs = head_rsrc(kp, p.Nk, p.sk.s, D);
  const __amdgpu_buffer_rsrc_t vrs = head_rsrc(vp, p.Nk, p.sv.s, D);
  const uint32_t krow = (uint32_t)(p.sk.s * 2), vrow = (uint32_t)(p.sv.s * 2);

  int kend = p.Nk;
  if (CAUSAL) kend = min(p.Nk, min(q0 + BM, p.Nq));
  const int n_kt = (kend + kT - 1) / kT;

  auto issue = [&](int j, int slot) {
    TC::issue(krs, krow, (uint32_t)j * kT * krow, Ks[slot], lane, wave);
    TC::issue(vrs, vrow, (uint32_t)j * kT * vrow, Vs[slot], lane, wave);
  };
  if (n_kt > 0) issue(0, 0);
  if (n_kt > 1) issue(1, 1);

  // Q^T and dO^T of this wave's queries as B operands (zeros past Nq).
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
  const int sst = stat_stride(p.Nq);
  const float lse2 = qi < p.Nq ? p.lse2[(int64_t)bh * sst + qi] : __builtin_inff();
  const float dsv = qi < p.Nq ? p.dsum[(int64_t)bh * sst + qi] : 0.f;
  f32x16 dinit;  // every dP^T accumulator starts at -D of this lane's query
#pragma unroll
  for (int r = 0; r < 16; ++r) dinit[r] = -dsv;

  f32x16 adq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) adq[db] = f32x16{};
  const float c = p.c;

  TileAddr<D> ta;
  ta.init(lane);

  wait_loads();
  lds_barrier();

  int slot = 0;
  for (int j = 0; j < n_kt; ++j) {
    const int j0 = j * kT;
    int nslot = slot + 2;
    nslot = nslot >= kNBuf ? nslot - kNBuf : nslot;
    if (j + 2 < n_kt) issue(j + 2, nslot);

    const bool active = qw0 < p.Nq && !(CAUSAL && j0 > qw0 + QW - 1);
    auto body = [&](const uint16_t* __restrict__ Kt, const uint16_t* __restrict__ Vt) {  // as in dkdv_kernel
      // S^T = K Q^T and dP^T = V dO^T: rows are keys j0 + acc_row(half, r); column = this lane's query
      f32x16 s = rows_times_regs<D, DT>(Kt, qf, ta);
      f32x16 dp = rows_times_regs<D, DT>(Vt, of, ta, dinit);  // dP^T - D
      const bool need_mask = (j0 + kT > p.Nk) || (CAUSAL && j0 + kT - 1 > qw0);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pv = exp2_fast(__builtin_fmaf(s[r], c, -lse2));
        if (need_mask) {
          const int kk = j0 + acc_row(half, r);
          if (kk >= p.Nk || (CAUSAL && kk > qi)) pv = 0.f;
        }
        dp[r] = pv * dp[r];
      }
      const u32x4 bd[2] = {pack_acc8<DT>(dp, 0), pack_acc8<DT>(dp, 1)};
      tile_t_times<D, DT>(adq, Kt, bd, ta);  // dQ^T += K^T dS^T
    };
    if (active) body(Ks[slot], Vs[slot]);

    if (j + 2 < n_kt) {
      wait_vmcnt<2 * TC::NI>();
    } else {
      wait_loads();
    }
    lds_barrier();
    slot = slot + 1 >= kNBuf ? 0 : slot + 1;
  }

  if (qi < p.Nq) store_rows<DT, DB>(p.dq + b * p.sdq.b + h * p.sdq.h + qi * p.sdq.s, adq, p.scale, half);
}

template <int D, int DT, bool CAUSAL>
hipError_t launch_t(const BwdParams& p, int stages, hipStream_t stream) {
  const int64_t BH = (int64_t)p.B * p.H;
  constexpr int RPB = kThreads / (D / 8);
  const int64_t prep_bpb = (stat_stride(p.Nq) + RPB - 1) / RPB;
  const int64_t g0 = prep_bpb * BH;
  const int64_t g1 = (int64_t)((p.Nk + 127) / 128) * BH;
  const int64_t g2 = (int64_t)((p.Nq + 127) / 128) * BH;
  if (g0 > 0x7fffffff || g1 > 0x7fffffff || g2 > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipError_t e = hipSuccess;
  if ((stages & 1) && g0 > 0) {  // Nq may be 0 (then dK = dV = 0 and there is no dQ)
    hipLaunchKernelGGL((prep_kernel<D, DT>), dim3((unsigned)g0), dim3(kThreads), 0, stream, p, (int)prep_bpb);
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

size_t bwd_workspace_bytes(int B, int H, int Nq) {
  // D and lse*log2(e): two fp32 arrays of stat_stride(Nq) values per (b, h)
  const size_t n = (size_t)B * (size_t)H * (size_t)stat_stride(Nq) * sizeof(float) * 2;
  return (n + 255) & ~(size_t)255;
}

float* bwd_lse2_region(void* workspace, int B, int H, int Nq) {
  return static_cast<float*>(workspace) + (size_t)B * (size_t)H * (size_t)stat_stride(Nq);
}

hipError_t launch_bwd(const BwdParams& p, int d, int dtype, bool causal, int stages, hipStream_t stream) {
  if (d == 64)
    return dtype == DT_F16 ? launch_dc<64, DT_F16>(p, causal, stages, stream)
                           : launch_dc<64, DT_BF16>(p, causal, stages, stream);
  return dtype == DT_F16 ? launch_dc<128, DT_F16>(p, causal, stages, stream)
                         : launch_dc<128, DT_BF16>(p, causal, stages, stream);
}

}  // namespace fa
