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
//   prep_kernel  -D_i = -dO_i . O_i and lse_i * log2(e) per query row, into
//                the workspace (HBM bound, tiny).
//   dkdv_kernel  a workgroup of NPAIR pairs of waves owns 32 * KB * NPAIR
//                keys (at d = 128 four pairs of 64 keys, or six of 32 with
//                dropout or a sliding window; at d = 64 four of 32); the
//                two waves of a pair share its keys and split the work by
//                role (A: K in registers, S, P, dV; B: V in registers, dP,
//                dS, dK, with P handed over through LDS), skewed so that
//                one role's MFMAs run under the other's VALU work.
//                32-query tiles of Q, dO and the two row statistics stream
//                HBM -> LDS through a 4-slot ring.  S = Q K^T and dP = dO V^T
//                come out with a key per lane, which is the B-operand
//                layout of dV^T += dO^T P and dK^T += Q^T dS; the
//                transposed A operands (dO^T, Q^T) are read from the same
//                untransposed LDS tiles with ds_read_b64_tr_b16.
//   dq_kernel    a workgroup owns 128 queries (32 per wave) with Q and dO
//                in registers; 32-key tiles of K and V stream through a
//                4-slot ring.  S^T and dP^T have a query
//                per lane (its lse and D are lane-local); dQ^T += K^T dS^T
//                reads K^T transposed from the K tile.  Each step forms
//                dS of tile j on the VALU, then issues dQ(j) and the S and
//                dP MFMAs of tile j+1 as one interleaved run.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kT = 32;        // rows per streamed tile (queries in dkdv, keys in dq)
constexpr int kStatPad = 64;  // per-(b,h) stride of the workspace statistics, rounded up to this
constexpr int kChipCUs = 256;  // MI355X (workspace sizes are planned for it, so they depend on the sizes alone)

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
    p.dsum[o] = -acc;  // stored negated: it seeds the dP accumulators
    // a row that admitted no key has lse = -inf; +inf here makes its
    // recomputed P = 2^(s c - lse2) zero
    const float l = row < p.Nq ? p.lse[(int64_t)bh * p.Nq + row] : 0.f;
    p.lse2[o] = l == -__builtin_inff() ? __builtin_inff() : l * kLog2e;
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
                                                  const TileLayout<D>& ta, f32x16 s = f32x16{}) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) s = mfma32<DT>(lds_rowmajor<D>(tile, ta, ks), bf[ks], s);
  return s;
}

// acc[db] += tile^T (d x 32 tile rows, read transposed) x B (32 tile rows x
// 32, packed from a 32x32 accumulator in its register k order).
template <int D, int DT>
__device__ __forceinline__ void tile_t_times(f32x16 (&acc)[D / 32], const uint16_t* tile, const u32x4 (&bp)[2],
                                             const TileLayout<D>& ta) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] = mfma32<DT>(lds_transposed_a<D>(tile, ta, kk, db), bp[kk], acc[db]);
}

// The same two products for KB 32-key blocks at once: each LDS operand read
// feeds one MFMA per block (s[kb] starts at init).
template <int D, int DT, int KB>
__device__ __forceinline__ void rows_times_regs_kb(f32x16 (&s)[KB], const uint16_t* tile,
                                                   const u32x4 (&bf)[KB][D / 16], const TileLayout<D>& ta,
                                                   const f32x16& init) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const u32x4 a = lds_rowmajor<D>(tile, ta, ks);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) s[kb] = mfma32<DT>(a, bf[kb][ks], ks == 0 ? init : s[kb]);
  }
}
template <int D, int DT, int KB>
__device__ __forceinline__ void tile_t_times_kb(f32x16 (&acc)[KB][D / 32], const uint16_t* tile,
                                                const u32x4 (&bp)[KB][2], const TileLayout<D>& ta) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const u32x4 a = lds_transposed_a<D>(tile, ta, kk, db);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) acc[kb][db] = mfma32<DT>(a, bp[kb][kk], acc[kb][db]);
    }
}

// Issue order of a run of MFMAs fed by LDS operand reads: NO1 operands of
// R1 read instructions each, then NO2 operands of R2 each, every operand
// feeding KB consecutive MFMAs.  After each MFMA the reads of the operand
// LEAD operands ahead have gone out (the first LEAD operands' reads go
// first), so a read runs about LEAD * KB MFMAs ahead of its use while only
// LEAD operands are in flight.  PRE more reads (an accumulator's initial
// values) go out first.
template <int NO1, int R1, int NO2, int R2>
constexpr int reads_through(int o) {  // read instructions of operands 0 .. o
  return o < NO1 ? R1 * (o + 1) : R1 * NO1 + R2 * (o - NO1 + 1);
}
template <int KB, int NO1, int R1, int NO2, int R2, int LEAD, int I, int ISSUED>
__device__ __forceinline__ void sched_ops_step() {
  constexpr int NM = KB * (NO1 + NO2);
  if constexpr (I < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    constexpr int o = I / KB + LEAD < NO1 + NO2 - 1 ? I / KB + LEAD : NO1 + NO2 - 1;
    constexpr int T = reads_through<NO1, R1, NO2, R2>(o);
    if constexpr (T > ISSUED) __builtin_amdgcn_sched_group_barrier(0x100, T - ISSUED, 0);
    sched_ops_step<KB, NO1, R1, NO2, R2, LEAD, I + 1, (T > ISSUED ? T : ISSUED)>();
  }
}
template <int KB, int NO1, int R1, int NO2, int R2, int LEAD, int PRE = 0>
__device__ __forceinline__ void sched_ops() {
  constexpr int first = reads_through<NO1, R1, NO2, R2>(LEAD - 1);
  __builtin_amdgcn_sched_group_barrier(0x100, PRE + first, 0);
  sched_ops_step<KB, NO1, R1, NO2, R2, LEAD, 0, first>();
}

// Wait until the ring tile just after the one being consumed has landed:
// `later` tiles were requested after it (at most MAXT, each L loads per
// wave), and vmcnt counts in request order, so leaving min(later, MAXT) * L
// loads outstanding is enough.
template <int MAXT, int L>
__device__ __forceinline__ void wait_ring(int later) {
  static_assert(MAXT * L < 64, "vmcnt range");
  if (later >= MAXT) {
    wait_vmcnt<MAXT * L>();
    return;
  }
  switch (later) {
#define FA_WAIT_CASE(n) \
  case n:               \
    if constexpr (n < MAXT) wait_vmcnt<n * L>(); \
    break;
    FA_WAIT_CASE(1) FA_WAIT_CASE(2) FA_WAIT_CASE(3) FA_WAIT_CASE(4) FA_WAIT_CASE(5) FA_WAIT_CASE(6)
#undef FA_WAIT_CASE
    default:
      wait_loads();
  }
}

// dK/dV workgroups hold NPAIR pairs of waves, each wave KB blocks of 32
// keys.  With KB = 1 at d = 128 a wave needs ~160 registers: six pairs
// (twelve waves, three per SIMD) in one workgroup per CU measured 6% faster
// than four pairs (two per SIMD).  With KB = 2 a pair owns 64 keys: every
// LDS operand read feeds two MFMAs (one per key block), a barrier covers
// twice the MFMA work per wave, and a wave needs ~255 registers, so four
// pairs share a CU (two waves per SIMD; waves w and w + 4 share one, so
// each SIMD holds one wave of each role).  At d = 128 that measured 6-7%
// faster than six single-block pairs on 16K causal rows and 15% faster on
// non-causal ones; with dropout (the keep-byte transpose is per 32 keys)
// the single-block kernel runs.  At d = 64 a wave needs at most 128: two
// workgroups of four single-block pairs share a CU (four waves per SIMD,
// 20% faster than two).  A dQ wave at d = 64 needs at most 168 registers
// (three per SIMD: 10% faster than two).
template <int D, int KB = 1>
constexpr int kDkvPairs = KB == 2 ? 4 : D == 64 ? 4 : 6;
template <int D, int KB = 1>
constexpr int kDkvWavesPerSimd = KB == 2 ? 2 : D == 64 ? 4 : 3;
// key blocks per wave of the dK/dV kernel without a left band edge (a
// sliding window runs the single-block kernel, see launch_t)
template <int D, bool DROP>
constexpr int kDkvKB = (D == 128 && !DROP) ? 2 : 1;
// keys per dK/dV workgroup of that kernel
template <int D, bool DROP>
constexpr int kDkvKeys = 32 * kDkvKB<D, DROP> * kDkvPairs<D, kDkvKB<D, DROP>>;
// causal bands run the two-block kernel from this many of its key blocks
constexpr int64_t kDkvTwoMinBlocks = 65;
template <int D>
constexpr int kDqWavesPerSimd = D == 64 ? 3 : 2;

// ------------------------------------------------------------ dK, dV
// NPAIR pairs of waves (four at d = 64; at d = 128 four pairs of KB = 2
// key blocks, six of one with dropout or a window).  The two waves of a
// pair own the same 32 * KB keys and split the four contractions of a
// query tile by role:
//   role A (waves 0 .. NPAIR-1): K rows in registers; S = Q K^T,
//                       P = 2^(S c - lse2), dV^T += dO^T P; P goes to its
//                       partner through LDS.
//   role B (waves NPAIR .. 2 NPAIR-1): V rows in registers;
//                       dP - D = dO V^T - D, dS = P (dP - D), dK^T += Q^T dS.
// Each wave holds one operand set and one 32 x d accumulator instead of
// two, and the loop is skewed so that within one phase the MFMAs of one
// role run while the other role works on the VALU:
//   phase 1: A  P(t) from S(t), hand P(t) over      B  dP(t); dK += .. dS(t-1)
//   barrier
//   phase 2: A  dV += .. P(t); S(t+1)               B  dS(t) = P(t) (dP(t) - D)
// Query tiles (Q, dO and the two row statistics) stream HBM -> LDS through
// a 4-slot ring; tile t+3 is requested in phase 2 of step t.
template <int D, int DT, bool BAND, bool DROP, int KB>
__global__ __launch_bounds__((128 * kDkvPairs<D, KB>)) __attribute__((amdgpu_waves_per_eu(kDkvWavesPerSimd<D, KB>, kDkvWavesPerSimd<D, KB>))) void dkdv_kernel(BwdParams p) {
  static_assert(KB == 1 || !DROP, "dropout runs one key block per wave");
  constexpr int KW = 32 * KB;       // keys per pair
  constexpr int NPAIR = kDkvPairs<D, KB>;  // pairs per workgroup
  constexpr int NCOPY = 4;             // waves of a role that copy its tiles
  constexpr int BNK = NPAIR * KW;   // keys per workgroup
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int NB = 4;             // ring slots (a power of two)
  constexpr int PD = NB - 1;        // prefetch distance: tile t+PD is requested in step t
  static_assert(kT == 32, "Q/dO tiles are the 32-row tiles of fa_device.h");
  // a Q or dO tile is copied by the four waves of one role
  constexpr int NLOADS = TileLayout<D>::template copy_insts<NCOPY>() + 1;  // per wave per tile: its share of Q (A) or dO (B), 8 statistics

  // One LDS object (separate __shared__ variables get separate alias
  // scopes, and the compiler then waits for every in-flight copy into a
  // variable before reading any part of it).
  struct Smem {
    uint16_t q[NB][kTileElems<D>];
    uint16_t o[NB][kTileElems<D>];  // dO
    float l[NB][kT];         // lse * log2(e)
    float d[NB][kT];         // -D
    f32x4 x[2][NPAIR][KB][4][64];  // fp32 P hand-over, double buffered: [step & 1][pair][key block][register group][lane]
    // dropout keep bytes of a pair's 32 keys x 32 queries, [step & 1][pair][key][query]
    uint8_t mk[DROP ? 2 : 1][NPAIR][KW * kT];
  };
  __shared__ __attribute__((aligned(1024))) Smem sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool role_a = wave < NPAIR;
  const int pair = role_a ? wave : wave - NPAIR;
  const int Hkv = p.H / p.G;
  const int BH = p.B * Hkv;
  // workgroups per key tile: one per (batch, K/V head, run sp of the steps)
  const int t = blockIdx.x;
  const int kt = t / (BH * p.S);  // ascending key tiles: the causal-heaviest first
  const int rem = t - kt * BH * p.S;
  const int bhk = rem / p.S;
  const int sp = rem - bhk * p.S;
  const int b = bhk / Hkv, hk = bhk - b * Hkv;
  const int k0 = kt * BNK;
  const int kw0 = k0 + pair * KW;
  const int key = kw0 + col;  // the lane's key of key block 0 (block kb: key + 32 kb)

  const int sst = stat_stride(p.Nq);
  const int64_t tstride = role_a ? p.sq.s : p.sdo.s;
  const uint32_t trow = (uint32_t)(tstride * 2);

  // Query tiles [qlo, qhi) of each of the G query heads of K/V head hk:
  // those with a query whose band admits a key of this workgroup.  The
  // steps run over u = g * nq + (it - qlo) for head hk * G + g.
  const int n_qt = (p.Nq + kT - 1) / kT;
  int qlo = 0, qhi = n_qt;
  if (BAND) {
    if (p.wr >= 0) qlo = max(0, k0 - p.wr) / kT;
    if (p.wl >= 0) qhi = min(n_qt, (k0 + BNK - 1 + p.wl) / kT + 1);
  }
  const int nq = max(0, qhi - qlo);
  // this workgroup's run [u0, u0 + U) of the S near-equal runs of the G * nq
  // steps (the query heads' tile sequences back to back)
  const int Utot = p.G * nq;
  const int u0 = (int)((int64_t)sp * Utot / p.S);
  const int U = (int)((int64_t)(sp + 1) * Utot / p.S) - u0;
  const int h0 = hk * p.G + (nq > 0 ? u0 / nq : 0);
  const int it0 = qlo + (nq > 0 ? u0 % nq : 0);

  // requests go out in step order; (iss_h, iss_it) is the next one's tile
  int iss_h = h0, iss_it = it0;
  auto issue = [&](int slot) {
    // role A streams Q and lse2, role B dO and -D
    const uint16_t* tp = role_a ? p.q + b * p.sq.b + iss_h * p.sq.h : p.dout + b * p.sdo.b + iss_h * p.sdo.h;
    const __amdgpu_buffer_rsrc_t trs = head_rsrc(tp, p.Nq, tstride, D);
    const __amdgpu_buffer_rsrc_t srs =
        f32_rsrc((role_a ? p.lse2 : p.dsum) + ((int64_t)b * p.H + iss_h) * sst, sst);
    if (pair < NCOPY) {  // four waves of the role, a quarter of the tile and 8 statistics each
      TileLayout<D>::template issue<NCOPY>(trs, trow, (uint32_t)iss_it * kT * trow, role_a ? sm.q[slot] : sm.o[slot],
                                           lane, pair);
      vec_to_lds<8>(srs, (uint32_t)(iss_it * kT + 8 * pair) * 4, (role_a ? sm.l[slot] : sm.d[slot]) + 8 * pair, lane);
    }
    if (++iss_it == qhi) {
      iss_it = qlo;
      ++iss_h;
    }
  };

  // The two roles run separate copies of the loop (one barrier per step in
  // each, so they stay in step): a shared loop would merge the roles'
  // registers through copies at every join.
  auto run = [&](auto role_tag) {
    constexpr bool A = decltype(role_tag)::value;
    // K rows (A) or V rows (B) of the pair's keys as B operands: lane holds
    // row `key`, columns 16*ks + 8*half .. +7 (zeros past Nk).
    u32x4 kv[KB][KS];
    {
      const uint16_t* rp = A ? p.k + b * p.sk.b + hk * p.sk.h : p.v + b * p.sv.b + hk * p.sv.h;
      const int64_t rs = A ? p.sk.s : p.sv.s;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          u32x4 x = u32x4{0, 0, 0, 0};
          if (key + 32 * kb < p.Nk) x = *(const u32x4*)(rp + (key + 32 * kb) * rs + 16 * ks + 8 * half);
          kv[kb][ks] = x;
        }
    }
    for (int i = 0; i < PD; ++i)
      if (i < U) issue(i);
    // The slot before the first tile's (not loaded before tile qt0 + PD)
    // is read by B's first dK update with dS = 0: make it finite zeros.
    if constexpr (!A) {
      u32x4* z = (u32x4*)sm.q[NB - 1];
#pragma unroll
      for (int i = pair * 64 + lane; i < TileLayout<D>::BYTES / 16; i += 64 * NPAIR) z[i] = u32x4{0, 0, 0, 0};
    }

    f32x16 acc[KB][DB];  // dV^T (A) or dK^T (B) of each key block
    f32x16 sd[KB];       // A: S of the next tile; B: dP - D of the current one
    u32x4 pk[KB][2];     // A: P; B: dS of the previous tile
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[kb][db] = f32x16{};
      sd[kb] = f32x16{};
      pk[kb][0] = pk[kb][1] = u32x4{0, 0, 0, 0};
    }
    const float c = p.c;

    TileLayout<D> ta;
    ta.init(lane);

    // Tile pointers are __restrict__ parameters of inlined lambdas so that
    // their LDS reads carry alias scopes; the compiler then leaves the
    // in-flight copies into other slots alone (the vmcnt waits and barriers
    // order the ring).  The tile of step u lives in slot u mod NB.
    wait_ring<PD - 2, NLOADS>(U - 2);  // the tiles of steps 0 and 1 landed
    lds_barrier();

    // One step.  (Unrolling by the ring depth would turn the slot bases
    // into immediates, but makes this compiler spill role A's registers.)
    int it = it0;            // query tile of the current step
    int hcur = h0;           // its query head
    auto step = [&](int u) {
      const int SL = u & (NB - 1);
      const int XB = SL & 1;
      const int i0 = it * kT;

      // ---------------- phase 1
      if constexpr (A) {
        auto phase = [&](const float* __restrict__ Lt, f32x4* __restrict__ X, uint8_t* Mk) {
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const float4 lv = *(const float4*)(&Lt[8 * g4 + 4 * half]);
            const float lz[4] = {lv.x, lv.y, lv.z, lv.w};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                sd[kb][4 * g4 + e] = exp2_fast(__builtin_fmaf(sd[kb][4 * g4 + e], c, -lz[e]));
          }
          // tiles that cross an edge of the pair's band
          if (BAND && ((p.wr >= 0 && i0 < kw0 + KW - 1 - p.wr) || (p.wl >= 0 && i0 + kT - 1 > kw0 + p.wl))) {
            // (the empty asm keeps this a branch: if-converted, the compares
            // would run on every tile)
            asm volatile("");
            // query of register r is i0 + 4*half + ro(r), ro(r) = 8*(r/4) + r%4;
            // key > query + wr  <=>  kd - wr > ro;  key < query - wl  <=>  kd + wl < ro
            // key - query offset of the lane's registers; with two key
            // blocks the lane id is re-read here instead of kept live
            // through the loop (registers)
            int kd0 = key - 4 * half;
            if constexpr (KB > 1) {
              uint32_t lo, ln;
              asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %1, -1, %0" : "=&v"(lo), "=v"(ln));
              kd0 = kw0 + (int)(ln & 31u) - 4 * (int)((ln >> 5) & 1u);
            }
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
              const int kd = kd0 + 32 * kb - i0;
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int ro = ((r >> 2) << 3) + (r & 3);
                if ((p.wr >= 0 && kd - p.wr > ro) || (p.wl >= 0 && kd + p.wl < ro)) sd[kb][r] = 0.f;
              }
            }
          }
          // P in fp32 to the partner (exact dS, no unpacking there)
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4)
              X[64 * (4 * kb + g4) + lane] =
                  f32x4{sd[kb][4 * g4], sd[kb][4 * g4 + 1], sd[kb][4 * g4 + 2], sd[kb][4 * g4 + 3]};
          if constexpr (DROP) {
            // The forward's draw for query i0 + col and the 16 keys of the
            // pair with key bit 2 = half (one call per lane), turned to a
            // key-major byte matrix in LDS; then this lane (key col) reads
            // the bytes of its 16 queries back, four per word.
            const u32x4 rnd = philox4x32_10(2u * (uint32_t)(kw0 >> 5) + (uint32_t)half, (uint32_t)(i0 + col),
                                            (uint32_t)(b * p.H + hcur), p.drop.offset, p.drop.seed_lo,
                                            p.drop.seed_hi);
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
              for (int bb = 0; bb < 4; ++bb) Mk[(8 * a + 4 * half + bb) * kT + col] = (uint8_t)(rnd[a] >> (8 * bb));
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const uint32_t kw = *(const uint32_t*)&Mk[col * kT + 8 * g4 + 4 * half];
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (((kw >> (8 * e)) & 0xffu) < p.drop.thr) sd[0][4 * g4 + e] = 0.f;
            }
          }
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            pk[kb][0] = pack_acc8<DT>(sd[kb], 0);  // P (kept P with dropout) for dV
            pk[kb][1] = pack_acc8<DT>(sd[kb], 1);
          }
        };
        phase(sm.l[SL], &sm.x[XB][pair][0][0][0], &sm.mk[DROP ? XB : 0][pair][0]);
      } else {
        auto phase = [&](const uint16_t* __restrict__ Ot, const float* __restrict__ Dt,
                         const uint16_t* __restrict__ Qprev) {
          // at d = 64 (four waves per SIMD) a wave issuing MFMAs goes first
          // (1-2.5% measured); at d = 128 it was 1% slower
          if constexpr (D == 64) __builtin_amdgcn_s_setprio(1);
          // dP - D in one pass: the accumulator starts at -D of its row
          // (with dropout at 0: -D is added after the mask)
          f32x16 dinit = f32x16{};
          if constexpr (!DROP) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const float4 dv = *(const float4*)(&Dt[8 * g4 + 4 * half]);
              dinit[4 * g4 + 0] = dv.x;
              dinit[4 * g4 + 1] = dv.y;
              dinit[4 * g4 + 2] = dv.z;
              dinit[4 * g4 + 3] = dv.w;
            }
          }
          if constexpr (KB == 1) {
            rows_times_regs_kb<D, DT, KB>(sd, Ot, kv, ta, dinit);
            // dK^T += Q^T dS of the previous tile, after dP: dS of this tile
            // (the next phase) waits only for dP, so its MFMAs go first
            tile_t_times_kb<D, DT, KB>(acc, Qprev, pk, ta);
            // issue order: operand reads kReadLead MFMAs ahead of their use
            sched_reads_ahead<2 * DB + KS, (4 * DB + 4 + KS)>();
          } else {
            // with two key blocks dK goes first: dS of the previous tile
            // then dies before dP is born (registers)
            tile_t_times_kb<D, DT, KB>(acc, Qprev, pk, ta);
            rows_times_regs_kb<D, DT, KB>(sd, Ot, kv, ta, dinit);
            sched_ops<KB, 2 * DB, 2, KS, 1, 2, 4>();
          }
          if constexpr (D == 64) __builtin_amdgcn_s_setprio(0);
        };
        // on the first step dS = 0 and the previous slot holds zeros
        phase(sm.o[SL], sm.d[SL], sm.q[(SL + NB - 1) & (NB - 1)]);
      }

      // step u+1's tile must have landed (A reads its Q rows next); the
      // later requested ones fly on
      wait_ring<PD - 2, NLOADS>(U - 1 - (u + 1));
      lds_barrier();
      // step u+PD's slot held step u-1's tile, whose last reader (B's dK)
      // finished before the barrier
      if (u + PD < U) issue((SL + PD) & (NB - 1));

      // ---------------- phase 2
      if constexpr (A) {
        auto phase = [&](const uint16_t* __restrict__ Ot, const uint16_t* __restrict__ Qn) {
          if constexpr (D == 64) __builtin_amdgcn_s_setprio(1);
          tile_t_times_kb<D, DT, KB>(acc, Ot, pk, ta);  // dV^T += dO^T P
          // S of the next tile (after the last tile this reads a stale slot
          // and the result is never used)
          rows_times_regs_kb<D, DT, KB>(sd, Qn, kv, ta, f32x16{});
          if constexpr (KB == 1)
            sched_reads_ahead<2 * DB + KS, 4 * DB + KS>();
          else
            sched_ops<KB, 2 * DB, 2, KS, 1, 2>();
          if constexpr (D == 64) __builtin_amdgcn_s_setprio(0);
        };
        phase(sm.o[SL], sm.q[(SL + 1) & (NB - 1)]);
      } else {
        auto phase = [&](const f32x4* __restrict__ X, const uint8_t* __restrict__ Mk, const float* __restrict__ Dt) {
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const f32x4 pv = X[64 * (4 * kb + g4) + lane];
              if constexpr (DROP) {  // dS = P (keep * scale * dP - D)
                const uint32_t kw = *(const uint32_t*)&Mk[col * kT + 8 * g4 + 4 * half];
                const float4 nd = *(const float4*)(&Dt[8 * g4 + 4 * half]);
                const float ndv[4] = {nd.x, nd.y, nd.z, nd.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const float m = ((kw >> (8 * e)) & 0xffu) >= p.drop.thr ? p.drop.scale : 0.f;
                  sd[kb][4 * g4 + e] = pv[e] * __builtin_fmaf(m, sd[kb][4 * g4 + e], ndv[e]);
                }
              } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) sd[kb][4 * g4 + e] *= pv[e];
              }
            }
            pk[kb][0] = pack_acc8<DT>(sd[kb], 0);
            pk[kb][1] = pack_acc8<DT>(sd[kb], 1);
          }
        };
        phase(&sm.x[XB][pair][0][0][0], &sm.mk[DROP ? XB : 0][pair][0], sm.d[SL]);
      }
      if (++it == qhi) {
        it = qlo;
        ++hcur;
      }
    };
    // A step with no work for this pair: its part in the ring's copies,
    // wait and barrier.
    auto idle = [&](int u) {
      const int SL = u & (NB - 1);
      wait_ring<PD - 2, NLOADS>(U - 1 - (u + 1));
      lds_barrier();
      if (u + PD < U) issue((SL + PD) & (NB - 1));
      if (++it == qhi) {
        it = qlo;
        ++hcur;
      }
    };
    // With equal heads the steps are one run of query tiles, and this
    // pair's own steps [ulo, uhi) are those whose queries admit one of its
    // keys; outside them (tiles the workgroup's band reaches for its other
    // pairs) its P and dS would be exact zeros, so it idles there (the
    // result is bit for bit the same).
    int ulo = 0, uhi = U;
    if (BAND && p.G == 1) {
      int plo = qlo, phi = qhi;
      if (p.wr >= 0) plo = max(plo, max(0, kw0 - p.wr) / kT);
      if (p.wl >= 0) phi = min(phi, (kw0 + KW - 1 + p.wl) / kT + 1);
      ulo = min(U, max(0, plo - it0));
      uhi = max(ulo, min(U, phi - it0));
    }
    int u = 0;
    for (; u < ulo; ++u) idle(u);
    if (u < uhi) {
      if constexpr (A) {  // S of the first own step's tile
        auto s_tile = [&](const uint16_t* __restrict__ Qt) { rows_times_regs_kb<D, DT, KB>(sd, Qt, kv, ta, f32x16{}); };
        s_tile(sm.q[u & (NB - 1)]);
      }
      for (; u < uhi; ++u) step(u);
      // the previous-tile product of the last own step: B's dK (its slot is
      // refilled only after the next step's barrier)
      if constexpr (!A) {
        auto last = [&](const uint16_t* __restrict__ Qt) { tile_t_times_kb<D, DT, KB>(acc, Qt, pk, ta); };
        last(sm.q[(uhi - 1) & (NB - 1)]);
      }
    }
    for (; u < U; ++u) idle(u);

#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int kk = key + 32 * kb;
      if (kk < p.Nk) {
        if (p.S > 1) {  // fp32 partial row of dK (B) or dV (A), scaled by the reduction
          float* rowp = p.part + ((((size_t)(A ? 1 : 0) * p.S + sp) * BH + bhk) * (size_t)p.Nk + kk) * D;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4)
              *(f32x4*)(rowp + db * 32 + 8 * g4 + 4 * half) = f32x4{acc[kb][db][4 * g4], acc[kb][db][4 * g4 + 1],
                                                                    acc[kb][db][4 * g4 + 2], acc[kb][db][4 * g4 + 3]};
        } else if constexpr (A) {
          store_rows<DT, DB>(p.dv + b * p.sdv.b + hk * p.sdv.h + kk * p.sdv.s, acc[kb], DROP ? p.drop.scale : 1.0f,
                             half);
        } else {
          store_rows<DT, DB>(p.dk + b * p.sdk.b + hk * p.sdk.h + kk * p.sdk.s, acc[kb], p.scale, half);
        }
      }
    }
  };
  if (role_a) {
    run(std::true_type{});
  } else {
    run(std::false_type{});
  }
}

// dK, dV = the scaled sums of the S partials, 8 values of one row per
// thread, in a fixed order (deterministic).
template <int D, int DT>
__global__ __launch_bounds__(kThreads) void dkdv_reduce_kernel(BwdParams p, int rows) {
  constexpr int CH = D / 8;  // 8-value chunks per row
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= 2 * (int64_t)rows * CH) return;
  const int which = (int)(i / ((int64_t)rows * CH));  // 0: dK, 1: dV
  const int64_t rc = i - (int64_t)which * rows * CH;
  const int row = (int)(rc / CH), ch = (int)(rc - (int64_t)row * CH);
  const int bhk = row / p.Nk, key = row - bhk * p.Nk;
  const int Hkv = p.H / p.G;
  const int b = bhk / Hkv, hk = bhk - b * Hkv;
  float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < p.S; ++s) {
    const float* src = p.part + (((size_t)which * p.S + s) * rows + row) * (size_t)D + 8 * ch;
    const f32x4 x0 = *(const f32x4*)src, x1 = *(const f32x4*)(src + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[e] += x0[e];
      a[4 + e] += x1[e];
    }
  }
  const float mul = which == 0 ? p.scale : (p.drop.thr > 0 ? p.drop.scale : 1.0f);
  uint16_t* dst = which == 0 ? p.dk + b * p.sdk.b + hk * p.sdk.h + key * p.sdk.s
                             : p.dv + b * p.sdv.b + hk * p.sdv.h + key * p.sdv.s;
  *(u32x4*)(dst + 8 * ch) = u32x4{pack2<DT>(a[0] * mul, a[1] * mul), pack2<DT>(a[2] * mul, a[3] * mul),
                                  pack2<DT>(a[4] * mul, a[5] * mul), pack2<DT>(a[6] * mul, a[7] * mul)};
}

// ------------------------------------------------------------ dQ
// dQ: a workgroup owns 128 queries (32 per wave) with Q and dO in
// registers; 32-key tiles of K and V stream through a 4-slot ring (tile
// t + 3 requested while tile t is used).  Software pipeline, step j:
//
//   VALU   P(j) = 2^(S(j) c - lse), masks, dS(j) = P (dP(j) - D), packed;
//   MFMA   dQ^T += K(j)^T dS(j)^T, S(j+1)^T = K(j+1) Q^T and
//          dP(j+1)^T = V(j+1) dO^T - D, interleaved and written over the
//          S(j), dP(j) registers just consumed, with their LDS operands
//          read a few MFMAs ahead.
//
// Each wave alternates a VALU phase and an MFMA phase; the two waves on a
// SIMD (two workgroups) fill each other's phases.
//
// Grids of at most one workgroup per CU whose heaviest query block has
// kDqSplitMinTiles key tiles or more run KSPLIT = kDqWavesPerSimd groups of
// four waves per workgroup (KSPLIT waves per SIMD): group g takes the g-th
// of KSPLIT near-equal runs of the block's key tiles through a ring of its
// own, and the groups' dQ^T partial sums are added in group order through
// LDS.  Every wave executes the same number of barriers (groups with fewer
// tiles add barrier-only steps).
template <int D, int DT, bool BAND, bool DROP, int KSPLIT>
__global__ __launch_bounds__(kThreads * KSPLIT) __attribute__((amdgpu_waves_per_eu(kDqWavesPerSimd<D>, kDqWavesPerSimd<D>))) void dq_kernel(BwdParams p) {
  constexpr int QW = 32;
  constexpr int BM = kWaves * QW;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int NB = 4;  // ring slots
  static_assert(kT == 32, "K/V tiles are the 32-row tiles of fa_device.h");
  static_assert(KSPLIT == 1 || KSPLIT == kDqWavesPerSimd<D>, "one wave of each group per SIMD");
  constexpr int NI = TileLayout<D>::template copy_insts<kWaves>();  // copy instructions per wave per tile

  struct Smem {  // one LDS object, as in dkdv_kernel
    uint16_t k[KSPLIT][NB][kTileElems<D>];
    uint16_t v[KSPLIT][NB][kTileElems<D>];
  };
  __shared__ __attribute__((aligned(1024))) Smem sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave_all / kWaves;        // key group (0 without a split)
  const int wave = wave_all - grp * kWaves;  // wave within the group: its 32 queries
  auto& Ks = sm.k[grp];
  auto& Vs = sm.v[grp];
  const int BH = p.B * p.H;
  const int n_qt = (p.Nq + BM - 1) / BM;
  const int t = blockIdx.x;
  const int qt = n_qt - 1 - t / BH;
  const int bh = t - (t / BH) * BH;
  const int b = bh / p.H, h = bh - b * p.H;
  const int q0 = qt * BM;
  const int qw0 = q0 + wave * QW;
  const int qi = qw0 + col;

  const int hk = h / p.G;  // K/V head shared by p.G consecutive query heads
  const uint16_t* kp = p.k + b * p.sk.b + hk * p.sk.h;
  const uint16_t* vp = p.v + b * p.sv.b + hk * p.sv.h;
  const __amdgpu_buffer_rsrc_t krs = head_rsrc(kp, p.Nk, p.sk.s, D);
  const __amdgpu_buffer_rsrc_t vrs = head_rsrc(vp, p.Nk, p.sv.s, D);
  const uint32_t krow = (uint32_t)(p.sk.s * 2), vrow = (uint32_t)(p.sv.s * 2);

  // key tiles [jt0, n_kt): those some query of the block admits; with a
  // split, this group's run of them
  int kend = p.Nk, jt0 = 0;
  if (BAND) {
    const int qlast = min(q0 + BM, p.Nq) - 1;
    if (p.wr >= 0) kend = min(p.Nk, qlast + p.wr + 1);
    if (p.wl >= 0) jt0 = max(0, q0 - p.wl) / kT;
  }
  int n_kt = (kend + kT - 1) / kT;
  int per = 0;  // tiles of the longest run
  if constexpr (KSPLIT > 1) {
    const int all = max(0, n_kt - jt0);
    per = (all + KSPLIT - 1) / KSPLIT;
    const int ja = min(n_kt, jt0 + grp * per);
    n_kt = min(n_kt, ja + per);
    jt0 = ja;
  }

  // tile jt0 + t lives in slot t mod 4
  auto issue = [&](int j, int slot) {
    TileLayout<D>::template issue<kWaves>(krs, krow, (uint32_t)j * kT * krow, Ks[slot], lane, wave);
    TileLayout<D>::template issue<kWaves>(vrs, vrow, (uint32_t)j * kT * vrow, Vs[slot], lane, wave);
  };
#pragma unroll
  for (int t0 = 0; t0 < 3; ++t0)
    if (jt0 + t0 < n_kt) issue(jt0 + t0, t0);

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
  const float ndsv = qi < p.Nq ? p.dsum[(int64_t)bh * sst + qi] : 0.f;  // -D
  f32x16 dinit;  // every dP^T accumulator starts at -D of this lane's query
#pragma unroll
  for (int r = 0; r < 16; ++r) dinit[r] = DROP ? 0.f : ndsv;  // with dropout -D is added after the mask

  f32x16 adq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) adq[db] = f32x16{};
  const float c = p.c;

  TileLayout<D> ta;
  ta.init(lane);

  // tiles jt0 and jt0+1 landed (S(jt0) now, tile jt0+1 in the first step)
  if (n_kt - jt0 > 2) {
    wait_vmcnt<2 * NI>();
  } else {
    wait_loads();
  }
  lds_barrier();

  // This wave's own key tiles [wlo, whi): those one of its queries admits.
  // Outside them (tiles the workgroup's band reaches for its other waves)
  // the wave's dS would be exact zeros: it only takes its part in the
  // ring's copies, waits and barriers (the result is bit for bit the same).
  int wlo = jt0, whi = n_kt;
  if constexpr (BAND) {
    if (p.wl >= 0) wlo = max(wlo, max(0, qw0 - p.wl) / kT);
    if (p.wr >= 0) whi = min(whi, (qw0 + QW - 1 + p.wr) / kT + 1);
    whi = max(whi, wlo);
  }
  auto idle = [&](int jj) {
    const int sl = (jj - jt0) & 3;
    if (jj + 3 < n_kt) {
      issue(jj + 3, (sl + 3) & 3);
      wait_vmcnt<2 * NI>();
    } else {
      wait_loads();
    }
    lds_barrier();
  };
  int j = jt0;
  for (; j < wlo; ++j) idle(j);

  // S(j)^T and dP(j)^T - D of the first own tile: rows are keys
  // j0 + acc_row(half, r), column this lane's query
  f32x16 s, dp;
  if (j < whi) {
    s = rows_times_regs<D, DT>(Ks[(j - jt0) & 3], qf, ta);
    dp = rows_times_regs<D, DT>(Vs[(j - jt0) & 3], of, ta, dinit);
  }
  auto step = [&](int j, int sl) {  // sl = (j - jt0) mod 4, the slot of tile j
    const int j0 = j * kT;
    if (j + 3 < n_kt) issue(j + 3, (sl + 3) & 3);

    // ---- VALU phase: dS(j)
    u32x4 rnd = u32x4{0, 0, 0, 0};
    if constexpr (DROP)  // the forward's draw for this query and the lane's 16 keys of tile j
      rnd = philox4x32_10(2u * (uint32_t)j + (uint32_t)half, (uint32_t)qi, (uint32_t)bh, p.drop.offset,
                          p.drop.seed_lo, p.drop.seed_hi);
    const bool need_mask = (j0 + kT > p.Nk) || (BAND && ((p.wr >= 0 && j0 + kT - 1 > qw0 + p.wr) ||
                                                          (p.wl >= 0 && j0 < qw0 + QW - 1 - p.wl)));
    float pv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) pv[r] = exp2_fast(__builtin_fmaf(s[r], c, -lse2));
    if (need_mask) {
      // one branch per tile (the empty asm keeps it a branch: per element,
      // the compiler would branch sixteen times on every tile)
      asm volatile("");
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = j0 + acc_row(half, r);
        if (kk >= p.Nk || (BAND && ((p.wr >= 0 && kk > qi + p.wr) || (p.wl >= 0 && kk < qi - p.wl)))) pv[r] = 0.f;
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if constexpr (DROP) {  // dS = P (keep * scale * dP - D)
        const float m = ((rnd[r >> 2] >> (8 * (r & 3))) & 0xffu) >= p.drop.thr ? p.drop.scale : 0.f;
        dp[r] = pv[r] * __builtin_fmaf(m, dp[r], ndsv);
      } else {
        dp[r] = pv[r] * dp[r];
      }
    }
    const u32x4 bd[2] = {pack_acc8<DT>(dp, 0), pack_acc8<DT>(dp, 1)};
    __builtin_amdgcn_sched_barrier(0);

    // ---- MFMA phase: dQ(j), S(j+1), dP(j+1) (reading tile j+1's stale
    // slot when j+1 = n_kt; those scores are never used)
    {
      const uint16_t* __restrict__ Kt = Ks[sl];
      const uint16_t* __restrict__ Kn = Ks[(sl + 1) & 3];
      const uint16_t* __restrict__ Vn = Vs[(sl + 1) & 3];
#pragma unroll
      for (int i = 0; i < KS; ++i) {
        if (i < 2 * DB) {
          const int kk = i / DB, db = i % DB;
          adq[db] = mfma32<DT>(lds_transposed_a<D>(Kt, ta, kk, db), bd[kk], adq[db]);
        }
        s = mfma32<DT>(lds_rowmajor<D>(Kn, ta, i), qf[i], i == 0 ? f32x16{} : s);
        dp = mfma32<DT>(lds_rowmajor<D>(Vn, ta, i), of[i], i == 0 ? dinit : dp);
      }
      sched_reads_ahead<2 * DB + 2 * KS, 4 * DB + 2 * KS>();
    }

    // tile j+2 (read next step) must have landed; tile j+3 may fly on
    if (j + 3 < n_kt) {
      wait_vmcnt<2 * NI>();
    } else {
      wait_loads();
    }
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // At d = 64 whole turns of the ring run with constant slots (LDS
  // addresses as immediates): -4 to -5% at 16K and B4 H32 N4096; at d = 128
  // (two waves per SIMD, 240 registers) it measured within +-0.8%.
  if constexpr (D == 64 && !DROP) {
    for (; j < whi && ((j - jt0) & 3) != 0; ++j) step(j, (j - jt0) & 3);
    for (; j + 4 <= whi; j += 4) {
#pragma unroll
      for (int r = 0; r < 4; ++r) step(j + r, r);
    }
  }
  for (; j < whi; ++j) step(j, (j - jt0) & 3);
  for (; j < n_kt; ++j) idle(j);

  if constexpr (KSPLIT > 1) {
    // one barrier per step: pad the shorter runs to the longest
    for (int i = max(0, n_kt - jt0); i < per; ++i) lds_barrier();
    // every group is done with its ring: reuse it for the partial sums
    constexpr int NV = DB * 16;
    static_assert((size_t)(KSPLIT - 1) * kWaves * NV * 64 * 4 <= sizeof(Smem), "partials fit the rings");
    float* xo = reinterpret_cast<float*>(&sm) + (size_t)((grp - 1) * kWaves + wave) * NV * 64 + lane;
    lds_barrier();
    if (grp > 0) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo[(db * 16 + r) * 64] = adq[db][r];
    }
    lds_barrier();
    if (grp > 0) return;
#pragma unroll
    for (int g = 1; g < KSPLIT; ++g) {
      const float* xi = reinterpret_cast<const float*>(&sm) + (size_t)((g - 1) * kWaves + wave) * NV * 64 + lane;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) adq[db][r] += xi[(db * 16 + r) * 64];
    }
  }

  if (qi < p.Nq) store_rows<DT, DB>(p.dq + b * p.sdq.b + h * p.sdq.h + qi * p.sdq.s, adq, p.scale, half);
}

// dK/dV and dQ are independent once the row statistics exist.  When the
// dK/dV grid is at most two waves of the chip, each kernel leaves most CUs
// idle, so dQ runs beside dK/dV on a side stream: an event recorded on the
// caller's stream after the statistics forks it (dK/dV is issued first),
// and one recorded on the side stream joins it back, so every result is
// ordered on the caller's stream as before.  One
// side stream and two events per device, created on first use outside
// graph capture and kept until the process ends; the lock pairs each fork
// and join with their own event records when host threads call at once.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  int cus = 0;
  bool ready = false;
};
constexpr int kMaxSideDevices = 64;
std::mutex g_side_mu;
SideStream g_side[kMaxSideDevices];

// The side stream of the current device, creating it if needed; nullptr if
// there is none (then everything runs on the caller's stream).  Call with
// g_side_mu held.
SideStream* side_stream(hipStream_t caller) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxSideDevices) return nullptr;
  SideStream& ss = g_side[dev];
  if (ss.ready) return &ss;
  // creating streams and events is not allowed while a graph is captured
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(caller, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return nullptr;
  if (hipDeviceGetAttribute(&ss.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ss.cus <= 0)
    return nullptr;
  if (!ss.s && hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) != hipSuccess) {
    ss.s = nullptr;
    return nullptr;
  }
  if (!ss.fork && hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess) {
    ss.fork = nullptr;
    return nullptr;
  }
  if (!ss.join && hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess) {
    ss.join = nullptr;
    return nullptr;
  }
  ss.ready = true;
  return &ss;
}

// The dQ kernel's key split pays when the heaviest query block has at least
// this many key tiles (as in the forward).
constexpr int kDqSplitMinTiles = 32;

// Launch the dQ kernel on `st`: with the key split when the grid gives a
// CU at most one workgroup and some block has enough key tiles.
template <int D, int DT, bool BAND, bool DROP>
hipError_t launch_dq(const BwdParams& p, int64_t g2, int cus, hipStream_t st) {
  bool split = false;
  if (g2 <= cus) {
    const int n_qt = (p.Nq + 127) / 128;
    for (int qb = 0; qb < n_qt && !split; ++qb) {
      int kend = p.Nk, j0 = 0;
      if (BAND) {
        const int qlast = std::min(qb * 128 + 128, p.Nq) - 1;
        if (p.wr >= 0) kend = std::min(p.Nk, qlast + p.wr + 1);
        if (p.wl >= 0) j0 = std::max(0, qb * 128 - p.wl) / kT;
      }
      split = (kend + kT - 1) / kT - j0 >= kDqSplitMinTiles;
    }
  }
  if (split) {
    constexpr int KSP = kDqWavesPerSimd<D>;
    hipLaunchKernelGGL((dq_kernel<D, DT, BAND, DROP, KSP>), dim3((unsigned)g2), dim3(kThreads * KSP), 0, st, p);
  } else {
    hipLaunchKernelGGL((dq_kernel<D, DT, BAND, DROP, 1>), dim3((unsigned)g2), dim3(kThreads), 0, st, p);
  }
  return hipGetLastError();
}

int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return kChipCUs;
  return n;
}

template <int D, int DT, bool BAND, bool DROP>
hipError_t launch_t(const BwdParams& p, int stages, bool side_ok, hipStream_t stream) {
  const int64_t BH = (int64_t)p.B * p.H;
  const int64_t BHkv = (int64_t)p.B * (p.H / p.G);
  constexpr int RPB = kThreads / (D / 8);
  const int64_t prep_bpb = (stat_stride(p.Nq) + RPB - 1) / RPB;
  const int64_t g0 = prep_bpb * BH;
  // Two key blocks per wave at d = 128 without dropout, unless the band
  // has a left edge (a window: there the single-block kernel measured 1-7%
  // faster, B1 H16 N16384 with windows (64, 64) to (4096, 0)), or a causal
  // band leaves the grid at most kDkvTwoMinBlocks - 1 two-block key blocks
  // (the heaviest block's run is then the critical path, and the smaller
  // blocks shorten it: B1 H1 N16384 0.388 -> 0.351 ms, B1 H2 N8192 0.223 ->
  // 0.197, B1 H4 N4096 0.136 -> 0.119; at 128 blocks the two were within
  // +-4% either way).
  const int64_t blocks2 = (int64_t)((p.Nk + kDkvKeys<D, false> - 1) / kDkvKeys<D, false>) * BHkv;
  const bool two = kDkvKB<D, DROP> == 2 && p.wl < 0 && (!BAND || blocks2 >= kDkvTwoMinBlocks);
  const int BNK = two ? kDkvKeys<D, DROP> : 32 * kDkvPairs<D, 1>;  // keys per dK/dV workgroup
  const int64_t g1 = (int64_t)((p.Nk + BNK - 1) / BNK) * BHkv * p.S;
  const int64_t rrows = BHkv * (int64_t)p.Nk;  // rows of dK (and of dV)
  const int64_t gr = (2 * rrows * (D / 8) + kThreads - 1) / kThreads;
  const int64_t g2 = (int64_t)((p.Nq + 127) / 128) * BH;
  if (g0 > 0x7fffffff || g1 > 0x7fffffff || g2 > 0x7fffffff || rrows > 0x7fffffff || gr > 0x7fffffff)
    return hipErrorInvalidConfiguration;
  hipError_t e = hipSuccess;
  if ((stages & 1) && g0 > 0) {  // Nq may be 0 (then dK = dV = 0 and there is no dQ)
    hipLaunchKernelGGL((prep_kernel<D, DT>), dim3((unsigned)g0), dim3(kThreads), 0, stream, p, (int)prep_bpb);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const bool both = side_ok && (stages & 2) && g1 > 0 && (stages & 4) && g2 > 0;
  std::unique_lock<std::mutex> lk(g_side_mu, std::defer_lock);
  SideStream* side = nullptr;
  if (both) {
    lk.lock();
    side = side_stream(stream);
    // dK/dV workgroups resident per CU: one at d = 128, two at d = 64 (the
    // grid before any split of its key blocks' steps)
    if (side && g1 / p.S > (int64_t)2 * side->cus * (D == 64 ? 2 : 1)) side = nullptr;
    // A captured call's fork makes the side stream part of that capture
    // until the capture ends.  Later calls of the same capture may go on
    // using it; another call (eager, or captured elsewhere) must not
    // enqueue onto it, so it runs dQ on its own stream.
    if (side) {
      hipStreamCaptureStatus cs = hipStreamCaptureStatusNone, cc = hipStreamCaptureStatusNone;
      unsigned long long is = 0, ic = 0;
      if (hipStreamGetCaptureInfo(side->s, &cs, &is) != hipSuccess) {
        side = nullptr;
      } else if (cs != hipStreamCaptureStatusNone) {
        if (hipStreamGetCaptureInfo(stream, &cc, &ic) != hipSuccess || cc != hipStreamCaptureStatusActive ||
            cs != hipStreamCaptureStatusActive || ic != is)
          side = nullptr;
      }
    }
    if (!side) lk.unlock();
  }
  // The fork follows the statistics; dK/dV is issued before dQ so that its
  // workgroups (the heaviest key blocks, the critical path) take the CUs
  // first, and dQ's fill the CUs that the light key blocks free.
  if (side && (e = hipEventRecord(side->fork, stream)) != hipSuccess) return e;
  if ((stages & 2) && g1 > 0) {
    if constexpr (kDkvKB<D, DROP> == 2) {
      if (two)
        hipLaunchKernelGGL((dkdv_kernel<D, DT, BAND, DROP, 2>), dim3((unsigned)g1), dim3(128 * kDkvPairs<D, 2>), 0,
                           stream, p);
      else
        hipLaunchKernelGGL((dkdv_kernel<D, DT, BAND, DROP, 1>), dim3((unsigned)g1), dim3(128 * kDkvPairs<D, 1>), 0,
                           stream, p);
    } else {
      hipLaunchKernelGGL((dkdv_kernel<D, DT, BAND, DROP, 1>), dim3((unsigned)g1), dim3(128 * kDkvPairs<D, 1>), 0,
                         stream, p);
    }
    e = hipGetLastError();
    if (e == hipSuccess && p.S > 1) {
      hipLaunchKernelGGL((dkdv_reduce_kernel<D, DT>), dim3((unsigned)gr), dim3(kThreads), 0, stream, p, (int)rrows);
      e = hipGetLastError();
    }
  }
  if (side) {
    // the fork was recorded, so the side stream is joined back even if a
    // launch fails
    hipError_t ej = hipStreamWaitEvent(side->s, side->fork, 0);
    if (ej == hipSuccess && e == hipSuccess) ej = launch_dq<D, DT, BAND, DROP>(p, g2, side->cus, side->s);
    hipError_t er = hipEventRecord(side->join, side->s);
    if (er == hipSuccess) er = hipStreamWaitEvent(stream, side->join, 0);
    return e != hipSuccess ? e : ej != hipSuccess ? ej : er;
  }
  if (e != hipSuccess) return e;
  if ((stages & 4) && g2 > 0) e = launch_dq<D, DT, BAND, DROP>(p, g2, device_cus(), stream);
  return e;
}

template <int D, int DT>
hipError_t launch_dc(const BwdParams& p, bool banded, int stages, bool side_ok, hipStream_t stream) {
  if (p.drop.thr > 0)
    return banded ? launch_t<D, DT, true, true>(p, stages, side_ok, stream)
                  : launch_t<D, DT, false, true>(p, stages, side_ok, stream);
  return banded ? launch_t<D, DT, true, false>(p, stages, side_ok, stream)
                : launch_t<D, DT, false, false>(p, stages, side_ok, stream);
}

// ------------------------------------------------------------ scratch
// The workspace of the allocation-free backward: a file-scope device array,
// one copy per GPU, kept until the process ends.  Host code never uses its
// name as an address (on the host it is only a stand-in for the symbol):
// the device address comes from hipGetSymbolAddress, once per device, with
// that device current.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];
static_assert(kNoAllocScratchBytes % 256 == 0, "scratch size");

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxSideDevices];

}  // namespace

size_t bwd_workspace_bytes(int B, int H, int Nq) {
  // -D and lse*log2(e): two fp32 arrays of stat_stride(Nq) values per (b, h)
  const size_t n = (size_t)B * (size_t)H * (size_t)stat_stride(Nq) * sizeof(float) * 2;
  return (n + 255) & ~(size_t)255;
}

float* bwd_lse2_region(void* workspace, int B, int H, int Nq) {
  return static_cast<float*>(workspace) + (size_t)B * (size_t)H * (size_t)stat_stride(Nq);
}

// dK/dV runs per key block with fewer K/V heads (G > 1): enough
// workgroups to balance a causal band over the chip, at least 1024 (four
// per CU), S the smallest divisor of G that gets there (else G), so each
// run is whole query heads.  With equal heads (G = 1) a key block's query
// tiles are cut into S = 2 runs when the grid has fewer dK/dV workgroups
// than the chip holds at once (one per CU at d = 128, two at d = 64) and
// Nk >= kEqSplitMinKeys: the heaviest causal block (all query tiles) is
// then the critical path, and dK/dV is issued before dQ, so the runs take
// CUs that would idle.  Measured: B1 H2 N16384 d128 0.61 -> 0.55 ms, B1 H1
// N16384 0.53 -> 0.36 ms, B1 H2 N8192 0.43 -> 0.32 ms, B1 H2 N16384 d64
// 0.51 -> 0.42 ms, B1 H16 N2048 d64 -5%, B2 H8 N2048 d64 +-1%.  Four runs
// at B2 H8 N2048 d64 cost 30% (67 MB of partial sums against a short
// critical path).
constexpr int kEqSplitMinKeys = 2048;
int bwd_kv_splits(int B, int H, int H_kv, int Nk, int d) {
  if (H_kv <= 0 || H % H_kv != 0) return 1;
  const int G = H / H_kv;
  // (the key blocks of the kernel without dropout; the same S serves both)
  const int bnk = d == 64 ? kDkvKeys<64, false> : kDkvKeys<128, false>;
  const int64_t base = (int64_t)((Nk + bnk - 1) / bnk) * B * H_kv;
  if (G == 1) return base < (int64_t)kChipCUs * (d == 64 ? 2 : 1) && Nk >= kEqSplitMinKeys ? 2 : 1;
  for (int S = 1; S < G; ++S)
    if (G % S == 0 && base * S >= 1024) return S;
  return G;
}

size_t bwd_split_workspace_bytes(int B, int H, int H_kv, int Nq, int Nk, int d) {
  const size_t stats = bwd_workspace_bytes(B, H, Nq);
  const int S = bwd_kv_splits(B, H, H_kv, Nk, d);
  if (S <= 1) return stats;
  return stats + 2 * (size_t)S * (size_t)B * (size_t)H_kv * (size_t)Nk * (size_t)d * sizeof(float);
}

hipError_t launch_bwd(const BwdParams& p, int d, int dtype, bool banded, int stages, hipStream_t stream,
                      bool side_ok) {
  if (d == 64)
    return dtype == DT_F16 ? launch_dc<64, DT_F16>(p, banded, stages, side_ok, stream)
                           : launch_dc<64, DT_BF16>(p, banded, stages, side_ok, stream);
  return dtype == DT_F16 ? launch_dc<128, DT_F16>(p, banded, stages, side_ok, stream)
                         : launch_dc<128, DT_BF16>(p, banded, stages, side_ok, stream);
}

hipError_t bwd_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxSideDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!a) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = a;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace fa
