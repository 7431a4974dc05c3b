// Kernel parameter blocks and host-side launchers (internal to libfa.so).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct DropoutParams {
  uint32_t thr;    // keep iff the element's random byte >= thr (0: no dropout)
  float scale;     // 256 / (256 - thr), applied to the kept weights
  uint32_t seed_lo, seed_hi, offset;
};

// Element strides {batch, head, seq}; the d dimension is contiguous.
struct Strides {
  int64_t b, h, s;
};

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  Strides sq, sk, sv, so;
  int B, H, Nq, Nk;
  int G;           // query heads per K/V head (K/V head of query head h is h / G)
  int wl, wr;      // admitted keys of query i: [i - wl, i + wr]; a negative bound is absent
  DropoutParams drop;
  float c;         // |scale| * log2(e), clamped away from 0
  uint32_t qflip;  // 0x80008000 when scale < 0 (Q is negated on load), else 0
  // Key-chunked forward (fa_fwd_splitk): chunk = key tiles per chunk (0:
  // not chunked), P = partial slots per (b, h), part = their fp32 storage
  // ([B*H][P][128 rows][d] partial O^T rows, then [128] m, then [128] l).
  int chunk;
  int P;
  float* part;
};

// The key-chunk plan of fa_fwd_splitk for these sizes: chunk = 0 when the
// grid fills the chip or no query block would be split.
struct FwdSplitPlan {
  int chunk;     // key tiles (32 keys) per chunk
  int n_chunks;  // workgroups per (b, h)
  int n_split;   // query blocks split into two or more chunks, per (b, h)
  int P;         // partial slots per (b, h)
};
FwdSplitPlan fwd_split_plan(int B, int H, int Nq, int Nk, int d, int wl, int wr);
size_t fwd_splitk_workspace_bytes(int B, int H, int Nq, int Nk, int d, int wl, int wr);
hipError_t launch_fwd_splitk(const FwdParams& p, const FwdSplitPlan& plan, int d, int dtype, bool banded,
                             hipStream_t stream);

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const float* lse;
  const uint16_t* dout;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* dsum;  // workspace: -D_i = -(dO_i . O_i), fp32, rows padded per (b, h)
  float* lse2;  // workspace: lse_i * log2(e), same layout
  Strides sq, sk, sv, so, sdo, sdq, sdk, sdv;
  int B, H, Nq, Nk;
  int G;        // query heads per K/V head (as FwdParams)
  int wl, wr;   // admitted-key band (as FwdParams)
  DropoutParams drop;
  float scale;  // the softmax scale as given
  float c;      // scale * log2(e) (signed)
  // dK/dV of a key block split over S workgroups: the block's steps (its
  // G query heads' query tiles, back to back) cut into S near-equal runs;
  // each workgroup writes fp32 partial sums to `part` ([2][S][B*H_kv][Nk][d]:
  // dK^T then dV^T, unscaled) and a reduction kernel adds them in run
  // order; S = 1 accumulates every step in registers (part unused).
  int S;
  float* part;
};

// fp8 (OCP e4m3fn) forward: q, k, v are bytes, o is bf16.
struct Fp8Params {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  uint16_t* o;
  float* lse;
  Strides sq, sk, sv, so;  // elements (bytes for q, k, v)
  int B, H, Nq, Nk;
  int G;           // query heads per K/V head
  int wl, wr;      // admitted-key band (as FwdParams)
  float c;         // |scale * q_descale * k_descale| * log2(e), clamped away from 0
  uint32_t qflip;  // 0x80808080 when that product is negative (Q negated on load), else 0
  float vscale;    // v_descale
};
hipError_t launch_fwd_fp8(const Fp8Params& p, int d, bool banded, hipStream_t stream);

// Return hipSuccess or the launch error.  d in {64,128}, dtype 0 = fp16,
// 1 = bf16; the caller has validated every argument.  `banded`: some bound
// of the admitted-key band is present (causal is the band wr = 0).
hipError_t launch_fwd(const FwdParams& p, int d, int dtype, bool banded, hipStream_t stream);
// Backward workspace: the two per-row statistics (-D and lse * log2 e),
// each B*H rows of Nq rounded up to 64 fp32 values (H = query heads).
size_t bwd_workspace_bytes(int B, int H, int Nq);
float* bwd_lse2_region(void* workspace, int B, int H, int Nq);
// Split of each K/V head's query heads for the dK/dV stage (1 = none) and
// the workspace bytes that split needs in total (statistics included).
int bwd_kv_splits(int B, int H, int H_kv, int Nk, int d);
size_t bwd_split_workspace_bytes(int B, int H, int H_kv, int Nq, int Nk, int d);
// stages: OR of 1 (row statistics), 2 (dK, dV), 4 (dQ), run in that order.
// side_ok = false keeps every stage on `stream` (no side stream for dQ).
hipError_t launch_bwd(const BwdParams& p, int d, int dtype, bool banded, int stages, hipStream_t stream,
                      bool side_ok = true);
// Bytes of the file-scope scratch array that serves as the workspace of
// the allocation-free backward, and its address on the current device
// (looked up once per device with hipGetSymbolAddress).
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;  // FA_BWD_NOALLOC_SCRATCH_BYTES of fa.h
hipError_t bwd_scratch(void** ptr);

}  // namespace fa
