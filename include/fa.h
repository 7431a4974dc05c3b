/*
 * fa.h - exact scaled dot-product attention on AMD Instinct MI355X (gfx950).
 *
 * What is computed (per batch b and head h):
 *
 *     S   = scale * Q K^T                      (Nq x Nk, never stored)
 *     P   = softmax_rows(S)                    (causal: entries j > i are -inf)
 *     O   = P V                                (Nq x d)
 *     LSE = log sum_j exp(S_ij)                (natural log, per query row)
 *
 * This is the "standard attention" the "Flash Attention" skill guide replaces
 * in Workflow 1, step 2 (softmax of q k^T / sqrt(d_k), times v), computed the
 * way the glossary article's "FlashAttention の仕組み" section and its four-step
 * figure describe: Q/K/V split into blocks that live in on-chip memory, an
 * online softmax whose running maximum and normaliser are updated as each
 * key block arrives, and one merged write of the result, so the Nq x Nk score
 * matrix is never written to HBM.  The backward recomputes P from the saved
 * LSE instead of storing it (skill guide quick start: tiling and
 * recomputation; refbase entry, "Capability").
 *
 * Causal masking is top-left aligned: query i attends to keys j <= i (the
 * reading of the pages' causal=True / is_causal=True that matches PyTorch
 * when Nq != Nk).  A causal row therefore always sees key 0.
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The
 *    library never allocates, frees or retains them, and never synchronises.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued asynchronously on it; a kernel fault shows at the
 *    caller's next synchronisation, as usual in HIP.  The current HIP device
 *    (hipSetDevice) must be the one that owns `stream` and the pointers:
 *    kernels and fa_bwd's side stream go to the current device.
 *  - Element type of Q, K, V, O, dO, dQ, dK, dV is `dtype` (FA_FP16 or
 *    FA_BF16; fp32 is not supported, as the skill guide's "精度が落ちる"
 *    issue and the glossary article's FP32 anti-pattern state), except in
 *    fa_fwd_fp8 (e4m3fn Q, K, V; bf16 O).  LSE and the backward workspace
 *    are fp32.
 *  - Head dimension d must be 64 or 128.
 *  - Default layout ("BHSD", the SDPA layout of the skill guide's quick
 *    start): Q/O are [B][H][Nq][d], K/V are [B][H][Nk][d], contiguous.
 *    The *_strided variants take, per tensor, three element strides
 *    {batch, head, seq}; the d dimension must be contiguous (stride 1).
 *    This covers the flash_attn layout [B][N][H][d] ("BSHD", skill guide
 *    Workflow 2 step 2) with strides {N*H*d, d, H*d}.
 *  - LSE is always a contiguous fp32 array [B][H][Nq].
 *  - `scale` is any finite float (1/sqrt(d) is the pages' default).
 *  - B, H or Nq equal to 0: nothing to do, FA_OK.  Nk must be >= 1 when
 *    Nq >= 1 (a softmax over no keys is undefined).
 *  - Each base pointer must be 16-byte aligned and each stride a multiple of
 *    8 elements (16 for fa_fwd_fp8's byte tensors); element offsets within
 *    one (b, h) slice must fit in 31 bits (offsets across batches and heads
 *    are 64-bit).  O must not alias Q, K or V; dQ/dK/dV must not alias any input.
 *    An output's strides must give its distinct elements distinct addresses:
 *    with its dimensions of size > 1 in increasing stride order, each stride
 *    at least the span of the dimensions inside it (dense and row-padded
 *    BHSD/BSHD pass; a zero stride is for inputs only).
 *  - B * H * max(Nq, Nk) must not exceed 2^48 rows (the workspace-size
 *    queries return 0 beyond it).
 *  - Return value: FA_OK (0) or an fa_status code.  Arguments are checked
 *    before any HIP call; on error nothing is enqueued.  A thread-local
 *    human-readable detail is available from fa_last_error_message().
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1, /* null pointer, bad size/stride/alignment, aliasing, small workspace */
  FA_ERR_UNSUPPORTED = 2, /* d not in {64,128}, dtype not fp16/bf16, device is not gfx950 */
  FA_ERR_DEVICE = 3,      /* no HIP device, or a device query failed */
  FA_ERR_LAUNCH = 4       /* the kernel launch itself reported an error */
} fa_status;

typedef enum { FA_FP16 = 0, FA_BF16 = 1 } fa_dtype;

/* Forward, BHSD contiguous.
 *   q   [B][H][Nq][d]   in
 *   k,v [B][H][Nk][d]   in
 *   o   [B][H][Nq][d]   out, O = softmax(scale Q K^T) V in dtype (RNE)
 *   lse [B][H][Nq] fp32 out, natural-log sum of exp(scale q.k) per row
 *   causal: 0 or 1. */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
           void* stream);

/* Forward with explicit element strides {batch, head, seq} for q, k, v, o.
 * Same kernels as fa_fwd. */
int fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
                   const int64_t q_strides[3], const int64_t k_strides[3],
                   const int64_t v_strides[3], const int64_t o_strides[3],
                   void* stream);

/* Forward with fewer K/V heads, a sliding window and/or dropout (the skill
 * guide's Workflow 2: step 3's multi-query attention with K/V shared across
 * heads and sliding-window attention with window_size = (left, right), and
 * step 2's dropout_p argument of flash_attn_func).
 *   H_kv: heads of k and v, dividing H; query head h uses K/V head
 *     h / (H / H_kv), so consecutive query heads share one (H_kv = H is
 *     plain multi-head attention, H_kv = 1 multi-query attention).
 *   window_left, window_right: query i admits keys i - window_left ..
 *     i + window_right, bounds inclusive; a negative value leaves that
 *     side unbounded ((-1, -1): no window).  causal = 1 additionally limits
 *     keys to j <= i.  Positions are top-left aligned as for causal.
 *   A query row that admits no key (possible with a window when Nq > Nk)
 *   gets O = 0 and LSE = -inf.
 *   dropout_p in [0, 1): each attention weight (after the softmax) is
 *     dropped with probability thr/256, thr = min(255, rint(256 dropout_p)),
 *     and kept ones are scaled by 256/(256 - thr); LSE is that of the
 *     undropped scores.  Element (b, h, i, j) (h a query head) is kept iff
 *     byte (j & 3) of word ((j >> 3) & 3) of Philox4x32-10 (Salmon et al.,
 *     SC'11) at counter {2*(j >> 5) + ((j >> 2) & 1), i, b*H + h, offset}
 *     with key {seed mod 2^32, seed >> 32} is >= thr.  The same (seed,
 *     offset) in fa_bwd_ex reproduces the mask.  This counter layout is part
 *     of the ABI: it does not follow how a kernel assigns keys to lanes, and
 *     it changes only with fa_abi_version().  dropout_p = 0: no dropout.
 *   k, v: [B][H_kv][Nk][d] through their strides; everything else as in
 *   fa_fwd_strided. */
int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int H_kv, int Nq, int Nk, int d, float scale, int causal,
              int window_left, int window_right, float dropout_p, uint64_t seed, uint32_t offset, int dtype,
              const int64_t q_strides[3], const int64_t k_strides[3],
              const int64_t v_strides[3], const int64_t o_strides[3],
              void* stream);

/* Bytes of workspace fa_fwd_splitk needs for these sizes; 0 when it
 * needs none (the grid of 128-query blocks fills the chip, or no block's
 * keys would be split).  causal, window_left, window_right as in fa_fwd_ex. */
size_t fa_fwd_splitk_workspace_bytes(int B, int H, int Nq, int Nk, int d, int causal, int window_left,
                                     int window_right);

/* fa_fwd_ex for grids too small to fill the chip, with the key range of
 * each heavy query block split over several workgroups (the glossary
 * article's online-softmax merge of partial results across blocks; FA2
 * entry, "並列化改良": parallelism over the sequence as well as over batch
 * and heads).  Same arguments, results within fp32 rounding of fa_fwd_ex,
 * deterministic: the partial results (O, row max, row sum) of a block's
 * chunks are merged in chunk order by a second kernel on `stream`.
 *   workspace: caller-owned device memory of at least
 *   fa_fwd_splitk_workspace_bytes(...) bytes, 256-byte aligned, not
 *   overlapping any tensor; contents on entry ignored, on return
 *   unspecified.  When that size is 0, workspace may be NULL and the call
 *   runs exactly fa_fwd_ex's kernels. */
int fa_fwd_splitk(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int H_kv, int Nq, int Nk, int d, float scale, int causal,
                  int window_left, int window_right, float dropout_p, uint64_t seed, uint32_t offset, int dtype,
                  const int64_t q_strides[3], const int64_t k_strides[3],
                  const int64_t v_strides[3], const int64_t o_strides[3],
                  void* workspace, size_t workspace_bytes, void* stream);

/* Forward with fp8 inputs (the skill guide's Workflow 3, step 3:
 * FlashAttention-3's FP8 path, forward only, q, k and v cast to
 * float8_e4m3fn).
 *   q, k, v: OCP FP8 E4M3 "fn" bytes (1 sign, 4 exponent bits with bias 7,
 *     3 mantissa bits; no infinities, 0x7f/0xff are NaN, largest finite
 *     448), the layout of fa_fwd_ex with strides in elements = bytes;
 *     k, v have H_kv heads.
 *   q_descale, k_descale, v_descale: per-tensor factors the stored values
 *     are multiplied by, so the attention computed is that of
 *     q_descale*q, k_descale*k, v_descale*v (1.0 for a plain cast).
 *   o: bf16 [B][H][Nq][d] through o_strides, O = softmax(scale QK^T) V of
 *     the descaled inputs; lse: fp32 [B][H][Nq] natural log as fa_fwd_ex.
 *   H_kv, causal, window_left, window_right: as fa_fwd_ex; no dropout.
 * Arithmetic: Q K^T on the fp8 matrix cores with fp32 accumulation; the
 * softmax in fp32; the weights p_j = exp(s_j - m) (each <= 448, the
 * running maximum m lagging the row maximum by at most log2(448) in log2
 * units) rounded to e4m3fn (nearest even) for the P V product, the
 * normaliser l summed from the unrounded weights in fp32.  Rounding the weights dominates the
 * error: per element of O, |error| <= 2^-4 sum_j w_j |v_j| +
 * 2^-10 sum_j |v_j| / L, plus bf16 rounding, where w_j are the exact
 * softmax weights and L = sum_j exp(s_j - max s) >= 1 (each weight is off
 * by at most 2^-4 of itself, or 2^-10 below e4m3fn's normal range).  LSE is
 * as accurate as fa_fwd_ex's.
 * Inputs must hold no NaN bytes (0x7f, 0xff); the result for
 * them is unspecified.
 * Strides must be multiples of 16 elements; pointers 16-byte aligned.
 * scale * q_descale * k_descale must be finite in fp32.  There is no
 * backward for fp8. */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int H_kv, int Nq, int Nk, int d, float scale, int causal,
               int window_left, int window_right, float q_descale, float k_descale, float v_descale,
               const int64_t q_strides[3], const int64_t k_strides[3],
               const int64_t v_strides[3], const int64_t o_strides[3],
               void* stream);

/* Bytes of device workspace fa_bwd needs for these sizes (0 if the sizes are
 * invalid).  Holds two fp32 row statistics per (b, h): -D_i = -sum_d dO_i O_i
 * and lse_i * log2(e), each with its rows padded to a multiple of 64
 * (2 * B * H * round_up(Nq, 64) floats). */
size_t fa_bwd_workspace_bytes(int B, int H, int Nq, int Nk, int d, int dtype);

/* Backward of L = sum(O * dO): gradients of Q, K, V, BHSD contiguous.
 *   q,k,v,o,lse  the forward's inputs and outputs (lse exactly as fa_fwd wrote it)
 *   dout [B][H][Nq][d]  upstream gradient dO
 *   dq [B][H][Nq][d], dk/dv [B][H][Nk][d]  out, in dtype
 *   workspace: caller-owned device memory of at least
 *   fa_bwd_workspace_bytes(...) bytes, 256-byte aligned; contents on entry
 *   are ignored and on return unspecified.  A workspace of at least
 *   fa_bwd_ex_workspace_bytes(B, H, H, ...) bytes also lets the dK/dV stage
 *   split its key blocks when the grid leaves CUs idle (see there).  P is
 *   recomputed as exp(scale q.k - lse); dS = P * (dP - D) with dP = dO V^T.
 * Streams: all work is ordered on `stream`.  When the dK/dV grid is at most
 * two waves of the chip, the dQ kernel runs on a side stream that the
 * library forks from `stream` (after the row statistics, dK/dV issued
 * first) and joins back to it with events (one non-blocking stream and two
 * events per device, created by the first such call made outside graph
 * capture and kept until the process exits; calls from several host
 * threads take a short internal lock).  The fork and join are capturable:
 * every call of one capture may fork onto the side stream, and a call made
 * while a different capture holds it runs dQ on `stream` instead. */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv,
           int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
           void* workspace, size_t workspace_bytes, void* stream);

/* Backward with explicit {batch, head, seq} element strides for every
 * d-major tensor (q, k, v, o, dout, dq, dk, dv).  lse and workspace as in
 * fa_bwd. */
int fa_bwd_strided(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv,
                   int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
                   const int64_t q_strides[3], const int64_t k_strides[3],
                   const int64_t v_strides[3], const int64_t o_strides[3],
                   const int64_t do_strides[3], const int64_t dq_strides[3],
                   const int64_t dk_strides[3], const int64_t dv_strides[3],
                   void* workspace, size_t workspace_bytes, void* stream);

/* Stages of the backward, for callers that schedule them themselves.
 * fa_bwd_strided runs FA_BWD_ALL.  FA_BWD_PREP writes -D_i = -dO_i . O_i
 * and lse_i * log2(e) into the workspace; FA_BWD_DKDV (dK, dV) and FA_BWD_DQ (dQ) read it and are
 * independent of each other, so after PREP has completed they may run on
 * two streams at once.  Stages in one call run in the order PREP, DKDV, DQ
 * on `stream`, except that a call with both DKDV and DQ may run DQ on the
 * side stream described at fa_bwd.  Same arguments and checks as fa_bwd_strided; `stages` is a
 * nonzero OR of the flags below. */
enum { FA_BWD_PREP = 1, FA_BWD_DKDV = 2, FA_BWD_DQ = 4, FA_BWD_ALL = 7 };
int fa_bwd_stages(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  const void* dout, void* dq, void* dk, void* dv,
                  int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
                  const int64_t q_strides[3], const int64_t k_strides[3],
                  const int64_t v_strides[3], const int64_t o_strides[3],
                  const int64_t do_strides[3], const int64_t dq_strides[3],
                  const int64_t dk_strides[3], const int64_t dv_strides[3],
                  void* workspace, size_t workspace_bytes, int stages, void* stream);

/* Backward of fa_fwd_ex: the stages of fa_bwd_stages with fewer K/V heads,
 * a sliding window and/or dropout; H_kv, window_left, window_right, causal,
 * dropout_p, seed and offset as in the fa_fwd_ex call that produced o and
 * lse.  dk, dv are [B][H_kv][Nk][d] through their strides; a K/V
 * head's gradients sum the contributions of all query heads that use it.
 * The workspace is sized by fa_bwd_workspace_bytes(B, H, Nq, ...) with H
 * the number of query heads, or preferably by fa_bwd_ex_workspace_bytes:
 * a workspace that large lets the dK/dV stage split each key block's
 * query tiles (over its query heads) over more workgroups (their fp32
 * partial sums are added in a fixed order by a second kernel, so results
 * stay deterministic; they can differ from the unsplit order in the last
 * bits of fp32 rounding).  lse must be what fa_fwd_ex wrote (-inf for a
 * row that admits no key; such a row gets dq = 0). */
int fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const float* lse,
              const void* dout, void* dq, void* dk, void* dv,
              int B, int H, int H_kv, int Nq, int Nk, int d, float scale, int causal,
              int window_left, int window_right, float dropout_p, uint64_t seed, uint32_t offset, int dtype,
              const int64_t q_strides[3], const int64_t k_strides[3],
              const int64_t v_strides[3], const int64_t o_strides[3],
              const int64_t do_strides[3], const int64_t dq_strides[3],
              const int64_t dk_strides[3], const int64_t dv_strides[3],
              void* workspace, size_t workspace_bytes, int stages, void* stream);

/* Workspace bytes for the backward (fa_bwd_ex, or with H_kv = H any fa_bwd
 * entry point taking a workspace) that enables the split dK/dV stage: at
 * least fa_bwd_workspace_bytes(B, H, Nq, Nk, d, dtype); 0 if the sizes are
 * invalid.  The extra part holds 2 * S * B * H_kv * Nk * d fp32 partial
 * sums: each key block's steps (its query heads' query tiles) are cut into
 * S runs on as many workgroups, added in run order by a second kernel
 * (deterministic; results can differ from the unsplit order in the last
 * bits of fp32 rounding).  S > 1 with fewer K/V heads (whole query heads
 * per run, until there are 1024 workgroups); with H_kv = H, S = 2 when the
 * dK/dV grid (one workgroup per 256 keys at d = 128, 128 at d = 64, per
 * (b, head)) has fewer workgroups than the MI355X holds at once (256 at
 * d = 128, 512 at d = 64) and Nk >= 2048; otherwise S = 1 (no extra part). */
size_t fa_bwd_ex_workspace_bytes(int B, int H, int H_kv, int Nq, int Nk, int d, int dtype);

/* fa_bwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, kernels and results as fa_bwd on contiguous BHSD
 * tensors, with the workspace taken from a device array of
 * FA_BWD_NOALLOC_SCRATCH_BYTES that the library holds at file scope (one
 * per GPU, kept until the process ends; its address is looked up once per
 * device, on the first call made with that device current).  It calls no
 * allocating routine.
 *   Sizes whose workspace (fa_bwd_workspace_bytes) exceeds the array, i.e.
 *   B * H * round_up(Nq, 64) > FA_BWD_NOALLOC_SCRATCH_BYTES / 8, are
 *   rejected with FA_ERR_INVALID_ARG.  All stages run on `stream` (no side
 *   stream).  Every call on one GPU shares that GPU's array: calls that
 *   can overlap on one GPU (other streams, other threads, graphs replayed
 *   concurrently) race and must be ordered by the caller.  Nothing in the
 *   array needs to start at zero: each call writes every value it reads. */
#define FA_BWD_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv,
                   int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype, void* stream);

/* Static name of a status code ("FA_OK", ...); "FA_UNKNOWN_STATUS" otherwise. */
const char* fa_status_string(int status);

/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* fa_last_error_message(void);

/* Library ABI version, currently 6 (3 added fa_fwd_fp8, 4
 * fa_bwd_ex_workspace_bytes, 5 fa_bwd_noalloc, 6 fa_fwd_splitk). */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
