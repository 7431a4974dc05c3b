// C ABI of libfa.so: argument validation, device check and dispatch.
// Every check runs before the first HIP call, so an invalid call enqueues
// nothing and touches no device.  Declarations and the contract are in
// include/fa.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/fa.h"
#include "fa_kernels.h"

static_assert(fa::kNoAllocScratchBytes == FA_BWD_NOALLOC_SCRATCH_BYTES, "scratch size of fa.h and the kernels");

namespace {

thread_local char g_msg[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return status;
}

constexpr int kMaxDevices = 64;
// 0 = not checked yet, 1 = gfx950, 2 = other architecture.
std::atomic<int> g_arch_state[kMaxDevices];

int check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(FA_ERR_DEVICE, "no HIP device available (%s)", hipGetErrorString(e));
  }
  if (dev >= kMaxDevices) return fail(FA_ERR_DEVICE, "device ordinal %d out of range", dev);
  int st = g_arch_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(FA_ERR_DEVICE, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
    }
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch_state[dev].store(st, std::memory_order_release);
    if (st == 2) return fail(FA_ERR_UNSUPPORTED, "device %d is %s; these kernels are built for gfx950", dev, prop.gcnArchName);
  }
  if (st == 2) return fail(FA_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
  return FA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Largest element offset touched within one (b, h) slice, and the whole-tensor
// extent, for overflow checks and aliasing.
struct Extent {
  int64_t lo_bytes, hi_bytes;  // [lo, hi) byte range relative to the base pointer
};

// elem: bytes per element (2, or 1 for fp8); strides must keep every row
// 16-byte aligned.
int check_tensor(const char* name, const void* ptr, const int64_t st[3], int B, int H, int N, int d, Extent* ext,
                 int elem = 2) {
  ext->lo_bytes = 0;
  ext->hi_bytes = 0;
  if (N == 0) return FA_OK;  // empty tensor: never dereferenced
  if (!ptr) return fail(FA_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(ptr)) return fail(FA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  const int unit = 16 / elem;
  for (int i = 0; i < 3; ++i) {
    if (st[i] < 0) return fail(FA_ERR_INVALID_ARG, "%s stride[%d] = %lld is negative", name, i, (long long)st[i]);
    if (st[i] % unit != 0)
      return fail(FA_ERR_INVALID_ARG, "%s stride[%d] = %lld is not a multiple of %d elements", name, i,
                  (long long)st[i], unit);
  }
  if (N > 1 && st[2] < d) return fail(FA_ERR_INVALID_ARG, "%s seq stride %lld < d = %d (rows overlap)", name, (long long)st[2], d);
  // within one (b, h) slice the kernels use 32-bit-safe offsets, and a
  // buffer resource's byte count (an unsigned 32-bit field) spans the slice
  constexpr int64_t kMaxSliceElems = 0x7fffffffLL;
  static_assert(kMaxSliceElems * 2 <= 0xffffffffLL, "a 16-bit head slice must fit a 32-bit byte count");
  const int64_t slice_max = (int64_t)(N - 1) * st[2] + d;
  if (slice_max > kMaxSliceElems) return fail(FA_ERR_INVALID_ARG, "%s: per-head extent exceeds 2^31 elements", name);
  const int64_t last = (int64_t)(B - 1) * st[0] + (int64_t)(H - 1) * st[1] + (int64_t)(N - 1) * st[2] + d;
  if (last > (INT64_MAX / 4)) return fail(FA_ERR_INVALID_ARG, "%s: extent overflows", name);
  ext->lo_bytes = 0;
  ext->hi_bytes = last * elem;
  return FA_OK;
}

// An output's distinct (b, h, row, column) elements must sit at distinct
// addresses, or the workgroups that write them race.  Taking the dimensions
// of size > 1 in increasing stride order (the contiguous d first), each
// stride must clear the span of the dimensions inside it.  Every dense or
// row-padded layout (BHSD, BSHD) passes; a zero stride or two dimensions
// sharing a stride do not.  Runs after check_tensor, so the spans fit int64.
int check_output_layout(const char* name, const int64_t st[3], int B, int H, int N, int d) {
  if (N == 0) return FA_OK;
  int64_t dims[3][2] = {{st[0], B}, {st[1], H}, {st[2], N}};
  for (int i = 1; i < 3; ++i)  // insertion sort by stride
    for (int j = i; j > 0 && dims[j][0] < dims[j - 1][0]; --j)
      for (int f = 0; f < 2; ++f) {
        const int64_t t = dims[j][f];
        dims[j][f] = dims[j - 1][f];
        dims[j - 1][f] = t;
      }
  int64_t span = d;
  for (int i = 0; i < 3; ++i) {
    if (dims[i][1] <= 1) continue;
    if (dims[i][0] < span)
      return fail(FA_ERR_INVALID_ARG, "%s: strides {%lld, %lld, %lld} put distinct elements at one address", name,
                  (long long)st[0], (long long)st[1], (long long)st[2]);
    span += (dims[i][1] - 1) * dims[i][0];
  }
  return FA_OK;
}

// Rows in all (b, h) slices together; far below this every byte count the
// library forms (tensor extents, LSE, workspaces) fits in 64 bits.
constexpr int64_t kMaxTotalRows = (int64_t)1 << 48;

bool rows_fit(int B, int H, int Nq, int Nk) {
  const int64_t bh = (int64_t)B * H;  // both < 2^31: no overflow
  if (bh > 0x7fffffffLL) return false;
  return bh * (Nq > Nk ? Nq : Nk) <= kMaxTotalRows;
}

bool overlaps(const void* a, const Extent& ea, const void* b, const Extent& eb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  const uintptr_t a1 = a0 + (uintptr_t)ea.hi_bytes, b1 = b0 + (uintptr_t)eb.hi_bytes;
  return a0 < b1 && b0 < a1;
}

int check_common(int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype) {
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0)
    return fail(FA_ERR_INVALID_ARG, "negative size (B=%d H=%d Nq=%d Nk=%d)", B, H, Nq, Nk);
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dim d=%d unsupported (64 or 128)", d);
  if (dtype != FA_FP16 && dtype != FA_BF16)
    return fail(FA_ERR_UNSUPPORTED, "dtype %d unsupported (FA_FP16=0 or FA_BF16=1; fp32 is not supported)", dtype);
  if (!std::isfinite(scale)) return fail(FA_ERR_INVALID_ARG, "scale is not finite");
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1 (got %d)", causal);
  if (Nq > 0 && B > 0 && H > 0 && Nk < 1) return fail(FA_ERR_INVALID_ARG, "Nk must be >= 1 when there are queries");
  if ((int64_t)B * H > 0x7fffffffLL) return fail(FA_ERR_INVALID_ARG, "B*H overflows");
  if (!rows_fit(B, H, Nq, Nk)) return fail(FA_ERR_INVALID_ARG, "B*H*max(Nq, Nk) exceeds 2^48 rows");
  return FA_OK;
}

int check_heads(int B, int H, int H_kv) {
  if (B == 0 || H == 0) return FA_OK;
  if (H_kv < 1) return fail(FA_ERR_INVALID_ARG, "H_kv = %d must be >= 1", H_kv);
  if (H % H_kv != 0) return fail(FA_ERR_INVALID_ARG, "H_kv = %d does not divide H = %d", H_kv, H);
  return FA_OK;
}

// Admitted keys of query i: [i - wl, i + wr], a negative bound meaning none.
// Causal is wr = 0 (and tighter than any right window).  A bound that
// excludes nothing (wl >= Nq: i - wl < 0; wr >= Nk: i + wr >= Nk) is
// dropped, which also keeps the kernels' index sums far from overflow.
struct Band {
  int wl, wr;
  bool present() const { return wl >= 0 || wr >= 0; }
};
Band make_band(int causal, int window_left, int window_right, int Nq, int Nk) {
  Band b;
  b.wl = (window_left < 0 || window_left >= Nq) ? -1 : window_left;
  b.wr = causal ? 0 : ((window_right < 0 || window_right >= Nk) ? -1 : window_right);
  return b;
}

// Dropout probability p in [0, 1) -> keep iff random byte >= thr, with
// thr = min(255, rint(256 p)) and kept weights scaled by 256 / (256 - thr).
int make_dropout(float p, uint64_t seed, uint32_t offset, fa::DropoutParams* out) {
  if (!(p >= 0.0f && p < 1.0f)) return fail(FA_ERR_INVALID_ARG, "dropout_p = %g is not in [0, 1)", (double)p);
  const double t = std::nearbyint((double)p * 256.0);
  out->thr = t > 255.0 ? 255u : (uint32_t)t;
  out->scale = (float)(256.0 / (256.0 - (double)out->thr));
  out->seed_lo = (uint32_t)seed;
  out->seed_hi = (uint32_t)(seed >> 32);
  out->offset = offset;
  return FA_OK;
}

float softmax_c(float scale) {
  // |scale| * log2(e); a tiny floor keeps c > 0 so masked (-inf) scores stay
  // -inf after scaling.  For |scale| below it the weights are uniform to
  // well under fp32 rounding either way.
  float c = std::fabs(scale) * 1.4426950408889634f;
  return c < 1e-30f ? 1e-30f : c;
}

void contiguous_strides(int H, int N, int d, int64_t st[3]) {
  st[2] = d;
  st[1] = (int64_t)N * d;
  st[0] = (int64_t)H * N * d;
}

}  // namespace

extern "C" {

int fa_abi_version(void) { return 6; }

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_DEVICE: return "FA_ERR_DEVICE";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH";
    default: return "FA_UNKNOWN_STATUS";
  }
}

const char* fa_last_error_message(void) { return g_msg; }

}  // extern "C"

namespace {

// The forward behind fa_fwd_ex and fa_fwd_splitk.  `splitk`: the key-chunked
// launch with the caller's workspace when the sizes have a chunk plan.
int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv, int Nq,
             int Nk, int d, float scale, int causal, int window_left, int window_right, float dropout_p,
             uint64_t seed, uint32_t offset, int dtype,
             const int64_t q_strides[3], const int64_t k_strides[3], const int64_t v_strides[3],
             const int64_t o_strides[3], void* workspace, size_t workspace_bytes, bool splitk, void* stream) {
  g_msg[0] = '\0';
  int st = check_common(B, H, Nq, Nk, d, scale, causal, dtype);
  if (st) return st;
  if ((st = check_heads(B, H, H_kv))) return st;
  fa::DropoutParams drop;
  if ((st = make_dropout(dropout_p, seed, offset, &drop))) return st;
  if (!q_strides || !k_strides || !v_strides || !o_strides) return fail(FA_ERR_INVALID_ARG, "a strides array is NULL");
  if (B == 0 || H == 0 || Nq == 0) return FA_OK;
  Extent eq, ek, ev, eo;
  if ((st = check_tensor("q", q, q_strides, B, H, Nq, d, &eq))) return st;
  if ((st = check_tensor("k", k, k_strides, B, H_kv, Nk, d, &ek))) return st;
  if ((st = check_tensor("v", v, v_strides, B, H_kv, Nk, d, &ev))) return st;
  if ((st = check_tensor("o", o, o_strides, B, H, Nq, d, &eo))) return st;
  if ((st = check_output_layout("o", o_strides, B, H, Nq, d))) return st;
  if (!lse) return fail(FA_ERR_INVALID_ARG, "lse is NULL");
  if (reinterpret_cast<uintptr_t>(lse) & 3u) return fail(FA_ERR_INVALID_ARG, "lse is not 4-byte aligned");
  Extent el{0, (int64_t)B * H * Nq * 4};
  if (overlaps(o, eo, q, eq) || overlaps(o, eo, k, ek) || overlaps(o, eo, v, ev))
    return fail(FA_ERR_INVALID_ARG, "o overlaps an input");
  if (overlaps(lse, el, q, eq) || overlaps(lse, el, k, ek) || overlaps(lse, el, v, ev) || overlaps(lse, el, o, eo))
    return fail(FA_ERR_INVALID_ARG, "lse overlaps another tensor");
  const Band band = make_band(causal, window_left, window_right, Nq, Nk);
  fa::FwdSplitPlan plan{0, 0, 0, 0};
  if (splitk) {
    plan = fa::fwd_split_plan(B, H, Nq, Nk, d, band.wl, band.wr);
    const size_t need = fa::fwd_splitk_workspace_bytes(B, H, Nq, Nk, d, band.wl, band.wr);
    if (need > 0) {
      if (!workspace) return fail(FA_ERR_INVALID_ARG, "workspace is NULL");
      if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return fail(FA_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
      if (workspace_bytes < need)
        return fail(FA_ERR_INVALID_ARG, "workspace_bytes = %zu < required %zu", workspace_bytes, need);
      const Extent ew{0, (int64_t)need};
      if (overlaps(workspace, ew, q, eq) || overlaps(workspace, ew, k, ek) || overlaps(workspace, ew, v, ev) ||
          overlaps(workspace, ew, o, eo) || overlaps(workspace, ew, lse, el))
        return fail(FA_ERR_INVALID_ARG, "workspace overlaps a tensor");
    }
  }
  if ((st = check_device())) return st;

  fa::FwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.sq = {q_strides[0], q_strides[1], q_strides[2]};
  p.sk = {k_strides[0], k_strides[1], k_strides[2]};
  p.sv = {v_strides[0], v_strides[1], v_strides[2]};
  p.so = {o_strides[0], o_strides[1], o_strides[2]};
  p.B = B;
  p.H = H;
  p.Nq = Nq;
  p.Nk = Nk;
  p.G = H / H_kv;
  p.wl = band.wl;
  p.wr = band.wr;
  p.drop = drop;
  p.c = softmax_c(scale);
  p.qflip = std::signbit(scale) ? 0x80008000u : 0u;
  p.chunk = plan.chunk;
  p.P = plan.P;
  p.part = static_cast<float*>(workspace);
  hipError_t e = plan.chunk > 0
                     ? fa::launch_fwd_splitk(p, plan, d, dtype, band.present(), static_cast<hipStream_t>(stream))
                     : fa::launch_fwd(p, d, dtype, band.present(), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_LAUNCH, "forward launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv, int Nq,
              int Nk, int d, float scale, int causal, int window_left, int window_right, float dropout_p,
              uint64_t seed, uint32_t offset, int dtype,
              const int64_t q_strides[3], const int64_t k_strides[3], const int64_t v_strides[3],
              const int64_t o_strides[3], void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, scale, causal, window_left, window_right, dropout_p, seed,
                  offset, dtype, q_strides, k_strides, v_strides, o_strides, nullptr, 0, false, stream);
}

size_t fa_fwd_splitk_workspace_bytes(int B, int H, int Nq, int Nk, int d, int causal, int window_left,
                                     int window_right) {
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0 || (d != 64 && d != 128) || (causal != 0 && causal != 1)) return 0;
  if (!rows_fit(B, H, Nq, Nk)) return 0;
  const Band band = make_band(causal, window_left, window_right, Nq, Nk);
  return fa::fwd_splitk_workspace_bytes(B, H, Nq, Nk, d, band.wl, band.wr);
}

int fa_fwd_splitk(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv, int Nq,
                  int Nk, int d, float scale, int causal, int window_left, int window_right, float dropout_p,
                  uint64_t seed, uint32_t offset, int dtype,
                  const int64_t q_strides[3], const int64_t k_strides[3], const int64_t v_strides[3],
                  const int64_t o_strides[3], void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, scale, causal, window_left, window_right, dropout_p, seed,
                  offset, dtype, q_strides, k_strides, v_strides, o_strides, workspace, workspace_bytes, true, stream);
}

int fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                   int d, float scale, int causal, int dtype, const int64_t q_strides[3],
                   const int64_t k_strides[3], const int64_t v_strides[3], const int64_t o_strides[3],
                   void* stream) {
  return fa_fwd_ex(q, k, v, o, lse, B, H, H, Nq, Nk, d, scale, causal, -1, -1, 0.0f, 0, 0, dtype, q_strides, k_strides,
                   v_strides, o_strides, stream);
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk, int d,
           float scale, int causal, int dtype, void* stream) {
  int64_t sq[3], sk[3];
  contiguous_strides(H, Nq, d, sq);
  contiguous_strides(H, Nk, d, sk);
  return fa_fwd_strided(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, dtype, sq, sk, sk, sq, stream);
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv, int Nq,
               int Nk, int d, float scale, int causal, int window_left, int window_right, float q_descale,
               float k_descale, float v_descale, const int64_t q_strides[3], const int64_t k_strides[3],
               const int64_t v_strides[3], const int64_t o_strides[3], void* stream) {
  g_msg[0] = '\0';
  int st = check_common(B, H, Nq, Nk, d, scale, causal, FA_BF16);
  if (st) return st;
  if ((st = check_heads(B, H, H_kv))) return st;
  if (!std::isfinite(q_descale) || !std::isfinite(k_descale) || !std::isfinite(v_descale))
    return fail(FA_ERR_INVALID_ARG, "a descale factor is not finite");
  const double cs = (double)scale * (double)q_descale * (double)k_descale;
  if (!std::isfinite(cs) || std::fabs(cs) > 3.0e38)
    return fail(FA_ERR_INVALID_ARG, "scale * q_descale * k_descale overflows fp32");
  if (!q_strides || !k_strides || !v_strides || !o_strides) return fail(FA_ERR_INVALID_ARG, "a strides array is NULL");
  if (B == 0 || H == 0 || Nq == 0) return FA_OK;
  Extent eq, ek, ev, eo;
  if ((st = check_tensor("q", q, q_strides, B, H, Nq, d, &eq, 1))) return st;
  if ((st = check_tensor("k", k, k_strides, B, H_kv, Nk, d, &ek, 1))) return st;
  if ((st = check_tensor("v", v, v_strides, B, H_kv, Nk, d, &ev, 1))) return st;
  if ((st = check_tensor("o", o, o_strides, B, H, Nq, d, &eo))) return st;
  if ((st = check_output_layout("o", o_strides, B, H, Nq, d))) return st;
  if (!lse) return fail(FA_ERR_INVALID_ARG, "lse is NULL");
  if (reinterpret_cast<uintptr_t>(lse) & 3u) return fail(FA_ERR_INVALID_ARG, "lse is not 4-byte aligned");
  Extent el{0, (int64_t)B * H * Nq * 4};
  if (overlaps(o, eo, q, eq) || overlaps(o, eo, k, ek) || overlaps(o, eo, v, ev))
    return fail(FA_ERR_INVALID_ARG, "o overlaps an input");
  if (overlaps(lse, el, q, eq) || overlaps(lse, el, k, ek) || overlaps(lse, el, v, ev) || overlaps(lse, el, o, eo))
    return fail(FA_ERR_INVALID_ARG, "lse overlaps another tensor");
  if ((st = check_device())) return st;

  fa::Fp8Params p;
  p.q = static_cast<const uint8_t*>(q);
  p.k = static_cast<const uint8_t*>(k);
  p.v = static_cast<const uint8_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.sq = {q_strides[0], q_strides[1], q_strides[2]};
  p.sk = {k_strides[0], k_strides[1], k_strides[2]};
  p.sv = {v_strides[0], v_strides[1], v_strides[2]};
  p.so = {o_strides[0], o_strides[1], o_strides[2]};
  p.B = B;
  p.H = H;
  p.Nq = Nq;
  p.Nk = Nk;
  p.G = H / H_kv;
  const Band band = make_band(causal, window_left, window_right, Nq, Nk);
  p.wl = band.wl;
  p.wr = band.wr;
  p.c = softmax_c((float)cs);
  p.qflip = std::signbit((float)cs) ? 0x80808080u : 0u;
  p.vscale = v_descale;
  hipError_t e = fa::launch_fwd_fp8(p, d, band.present(), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_LAUNCH, "fp8 forward launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

size_t fa_bwd_ex_workspace_bytes(int B, int H, int H_kv, int Nq, int Nk, int d, int dtype) {
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0 || (d != 64 && d != 128) || (dtype != FA_FP16 && dtype != FA_BF16)) return 0;
  if (H > 0 && (H_kv < 1 || H % H_kv != 0)) return 0;
  if (!rows_fit(B, H, Nq, Nk)) return 0;
  return fa::bwd_split_workspace_bytes(B, H, H > 0 ? H_kv : 1, Nq, Nk, d);
}

size_t fa_bwd_workspace_bytes(int B, int H, int Nq, int Nk, int d, int dtype) {
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0 || (d != 64 && d != 128) || (dtype != FA_FP16 && dtype != FA_BF16)) return 0;
  if (!rows_fit(B, H, Nq, Nk)) return 0;
  return fa::bwd_workspace_bytes(B, H, Nq);
}

}  // extern "C"

namespace {

// The backward behind fa_bwd_ex and fa_bwd_noalloc.  With `noalloc` the
// workspace is the library's file-scope scratch array (workspace and
// workspace_bytes are ignored), every stage stays on `stream`, and sizes
// whose workspace exceeds the array are rejected.
int bwd_impl(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
             void* dq, void* dk, void* dv, int B, int H, int H_kv, int Nq, int Nk, int d, float scale, int causal,
             int window_left, int window_right, float dropout_p, uint64_t seed, uint32_t offset, int dtype,
             const int64_t q_strides[3], const int64_t k_strides[3],
             const int64_t v_strides[3], const int64_t o_strides[3], const int64_t do_strides[3],
             const int64_t dq_strides[3], const int64_t dk_strides[3], const int64_t dv_strides[3],
             void* workspace, size_t workspace_bytes, int stages, void* stream, bool noalloc) {
  g_msg[0] = '\0';
  int st = check_common(B, H, Nq, Nk, d, scale, causal, dtype);
  if (st) return st;
  if ((st = check_heads(B, H, H_kv))) return st;
  fa::DropoutParams drop;
  if ((st = make_dropout(dropout_p, seed, offset, &drop))) return st;
  if (stages <= 0 || (stages & ~FA_BWD_ALL)) return fail(FA_ERR_INVALID_ARG, "stages = %d is not a nonzero OR of FA_BWD_*", stages);
  if (!q_strides || !k_strides || !v_strides || !o_strides || !do_strides || !dq_strides || !dk_strides || !dv_strides)
    return fail(FA_ERR_INVALID_ARG, "a strides array is NULL");
  if (B == 0 || H == 0) return FA_OK;
  if (Nq == 0 && Nk == 0) return FA_OK;  // with Nq = 0 and Nk > 0, dK = dV = 0 are written
  Extent eq, ek, ev, eo, edo, edq, edk, edv;
  if ((st = check_tensor("q", q, q_strides, B, H, Nq, d, &eq))) return st;
  if ((st = check_tensor("k", k, k_strides, B, H_kv, Nk, d, &ek))) return st;
  if ((st = check_tensor("v", v, v_strides, B, H_kv, Nk, d, &ev))) return st;
  if ((st = check_tensor("o", o, o_strides, B, H, Nq, d, &eo))) return st;
  if ((st = check_tensor("dout", dout, do_strides, B, H, Nq, d, &edo))) return st;
  if ((st = check_tensor("dq", dq, dq_strides, B, H, Nq, d, &edq))) return st;
  if ((st = check_tensor("dk", dk, dk_strides, B, H_kv, Nk, d, &edk))) return st;
  if ((st = check_tensor("dv", dv, dv_strides, B, H_kv, Nk, d, &edv))) return st;
  if ((st = check_output_layout("dq", dq_strides, B, H, Nq, d))) return st;
  if ((st = check_output_layout("dk", dk_strides, B, H_kv, Nk, d))) return st;
  if ((st = check_output_layout("dv", dv_strides, B, H_kv, Nk, d))) return st;
  if (Nq > 0 && !lse) return fail(FA_ERR_INVALID_ARG, "lse is NULL");
  if (reinterpret_cast<uintptr_t>(lse) & 3u) return fail(FA_ERR_INVALID_ARG, "lse is not 4-byte aligned");
  const size_t need = fa_bwd_workspace_bytes(B, H, Nq, Nk, d, dtype);
  if (noalloc) {
    if (need > fa::kNoAllocScratchBytes)
      return fail(FA_ERR_INVALID_ARG,
                  "these sizes need %zu bytes of workspace, more than the %zu of the allocation-free scratch "
                  "(B * H * round_up(Nq, 64) must be at most %zu)",
                  need, fa::kNoAllocScratchBytes, fa::kNoAllocScratchBytes / 8);
    workspace = nullptr;
    workspace_bytes = 0;
  } else {
    if (need > 0 && !workspace) return fail(FA_ERR_INVALID_ARG, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
      return fail(FA_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
    if (workspace_bytes < need)
      return fail(FA_ERR_INVALID_ARG, "workspace_bytes = %zu < required %zu", workspace_bytes, need);
  }
  // fewer K/V heads: split each K/V head's query heads over more dK/dV
  // workgroups when the workspace holds their partial sums
  const int splits = fa::bwd_kv_splits(B, H, H_kv, Nk, d);
  const size_t need_split = fa::bwd_split_workspace_bytes(B, H, H_kv, Nq, Nk, d);
  const bool split = splits > 1 && (stages & FA_BWD_DKDV) && workspace_bytes >= need_split;
  const size_t used = split ? need_split : need;
  const void* ins[6] = {q, k, v, o, dout, lse};
  const Extent eins[6] = {eq, ek, ev, eo, edo, Extent{0, (int64_t)B * H * Nq * 4}};
  void* outs[4] = {dq, dk, dv, workspace};
  const Extent eouts[4] = {edq, edk, edv, Extent{0, noalloc ? 0 : (int64_t)used}};
  const char* onames[4] = {"dq", "dk", "dv", "workspace"};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], eouts[i], ins[j], eins[j])) return fail(FA_ERR_INVALID_ARG, "%s overlaps an input", onames[i]);
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], eouts[i], outs[j], eouts[j]))
        return fail(FA_ERR_INVALID_ARG, "%s overlaps %s", onames[i], onames[j]);
  }
  if ((st = check_device())) return st;
  if (noalloc) {
    hipError_t es = fa::bwd_scratch(&workspace);
    if (es != hipSuccess || !workspace) {
      (void)hipGetLastError();
      return fail(FA_ERR_DEVICE, "scratch lookup (hipGetSymbolAddress) failed: %s", hipGetErrorString(es));
    }
  }

  fa::BwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<const uint16_t*>(o);
  p.lse = lse;
  p.dout = static_cast<const uint16_t*>(dout);
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  p.dsum = static_cast<float*>(workspace);
  p.lse2 = fa::bwd_lse2_region(workspace, B, H, Nq);
  p.sq = {q_strides[0], q_strides[1], q_strides[2]};
  p.sk = {k_strides[0], k_strides[1], k_strides[2]};
  p.sv = {v_strides[0], v_strides[1], v_strides[2]};
  p.so = {o_strides[0], o_strides[1], o_strides[2]};
  p.sdo = {do_strides[0], do_strides[1], do_strides[2]};
  p.sdq = {dq_strides[0], dq_strides[1], dq_strides[2]};
  p.sdk = {dk_strides[0], dk_strides[1], dk_strides[2]};
  p.sdv = {dv_strides[0], dv_strides[1], dv_strides[2]};
  p.B = B;
  p.H = H;
  p.Nq = Nq;
  p.Nk = Nk;
  p.G = H / H_kv;
  const Band band = make_band(causal, window_left, window_right, Nq, Nk);
  p.wl = band.wl;
  p.wr = band.wr;
  p.drop = drop;
  p.scale = scale;
  p.c = scale * 1.4426950408889634f;
  p.S = split ? splits : 1;
  p.part = split ? reinterpret_cast<float*>(static_cast<char*>(workspace) + need) : nullptr;
  hipError_t e = fa::launch_bwd(p, d, dtype, band.present(), stages, static_cast<hipStream_t>(stream), !noalloc);
  if (e != hipSuccess) return fail(FA_ERR_LAUNCH, "backward launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
              void* dq, void* dk, void* dv, int B, int H, int H_kv, int Nq, int Nk, int d, float scale, int causal,
              int window_left, int window_right, float dropout_p, uint64_t seed, uint32_t offset, int dtype,
              const int64_t q_strides[3], const int64_t k_strides[3],
              const int64_t v_strides[3], const int64_t o_strides[3], const int64_t do_strides[3],
              const int64_t dq_strides[3], const int64_t dk_strides[3], const int64_t dv_strides[3],
              void* workspace, size_t workspace_bytes, int stages, void* stream) {
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, B, H, H_kv, Nq, Nk, d, scale, causal, window_left, window_right,
                  dropout_p, seed, offset, dtype, q_strides, k_strides, v_strides, o_strides, do_strides, dq_strides,
                  dk_strides, dv_strides, workspace, workspace_bytes, stages, stream, false);
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                   void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk, int d, float scale, int causal,
                   int dtype, void* stream) {
  int64_t sq[3], sk[3];
  contiguous_strides(H, Nq, d, sq);
  contiguous_strides(H, Nk, d, sk);
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, B, H, H, Nq, Nk, d, scale, causal, -1, -1, 0.0f, 0, 0, dtype,
                  sq, sk, sk, sq, sq, sq, sk, sk, nullptr, 0, FA_BWD_ALL, stream, true);
}

int fa_bwd_stages(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                  void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk, int d, float scale, int causal,
                  int dtype, const int64_t q_strides[3], const int64_t k_strides[3], const int64_t v_strides[3],
                  const int64_t o_strides[3], const int64_t do_strides[3], const int64_t dq_strides[3],
                  const int64_t dk_strides[3], const int64_t dv_strides[3], void* workspace,
                  size_t workspace_bytes, int stages, void* stream) {
  return fa_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, B, H, H, Nq, Nk, d, scale, causal, -1, -1, 0.0f, 0, 0, dtype,
                   q_strides,
                   k_strides, v_strides, o_strides, do_strides, dq_strides, dk_strides, dv_strides, workspace,
                   workspace_bytes, stages, stream);
}

int fa_bwd_strided(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                   void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk, int d, float scale, int causal,
                   int dtype, const int64_t q_strides[3], const int64_t k_strides[3], const int64_t v_strides[3],
                   const int64_t o_strides[3], const int64_t do_strides[3], const int64_t dq_strides[3],
                   const int64_t dk_strides[3], const int64_t dv_strides[3], void* workspace,
                   size_t workspace_bytes, void* stream) {
  return fa_bwd_stages(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nk, d, scale, causal, dtype, q_strides, k_strides,
                       v_strides, o_strides, do_strides, dq_strides, dk_strides, dv_strides, workspace,
                       workspace_bytes, FA_BWD_ALL, stream);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
           void* dk, void* dv, int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
           void* workspace, size_t workspace_bytes, void* stream) {
  int64_t sq[3], sk[3];
  contiguous_strides(H, Nq, d, sq);
  contiguous_strides(H, Nk, d, sk);
  return fa_bwd_strided(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nk, d, scale, causal, dtype, sq, sk, sk, sq, sq,
                        sq, sk, sk, workspace, workspace_bytes, stream);
}

}  // extern "C"
