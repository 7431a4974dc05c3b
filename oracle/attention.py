"""Plain fp64 reference of exact scaled dot-product attention (CPU, numpy).

TEST INFRASTRUCTURE ONLY: the product path never imports this module.

What is computed, and where the pages define it:

* Forward.  "Flash Attention" skill guide, Workflow 1, step 2 ("Before
  (standard attention)"): the weights are the row softmax of
  ``q @ k^T / sqrt(d_k)`` and the output is those weights times ``v``.  The
  same guide's step 3 and step 4 snippets divide by 8.0 for head dim 64, and
  Workflow 2 step 2 passes ``softmax_scale=None`` for the automatic
  ``1/sqrt(d)``.  The scale is therefore an explicit argument here.
* Causal masking.  The ``causal=True`` / ``is_causal=True`` calls in the same
  guide (quick start, Workflow 2) and in the glossary article's SDPA pattern
  B.  Reading taken (pages silent on Nq != Nk): top-left alignment, query i
  sees keys j <= i, as PyTorch's ``is_causal``.
* Exactness.  The glossary article ("FlashAttention とは", and misconception 1)
  states the tiled method returns the same result as standard attention up
  to rounding; so this oracle is the definition itself, with the N x N score
  and probability matrices materialised, never the tiled algorithm.
* Log-sum-exp.  The pages give recomputation in the backward (skill guide
  quick start; the refbase Q&A entry on tiling and recomputation) but no
  formula.  Reading: ``lse_i = log sum_j exp(s_ij)`` with ``s = scale*q.k``,
  natural log, the quantity that lets P be recomputed as ``exp(s - lse)``.
* Backward.  The pages only say that training (forward + backward) is
  supported (glossary comparison table; misconception 2; FA2 FAQ Q2).  The
  gradients here are the textbook chain rule through softmax:
  ``dV = P^T dO``, ``dP = dO V^T``,
  ``dS = P * (dP - rowsum(P * dP))``, ``dQ = scale * dS K``,
  ``dK = scale * dS^T Q``.  Deliberately the ``rowsum(P*dP)`` form, not the
  ``rowsum(dO*O)`` identity a fast kernel uses, so parity tests that identity.

* Fewer K/V heads (multi-query / grouped-query attention).  The skill
  guide's Workflow 2, step 3 ("multi-query attention"): ``k`` and ``v`` may
  carry fewer heads than ``q`` and the call handles it.  Reading taken (the
  pages give no index map): ``H_kv`` divides ``H`` and query head ``h`` uses
  K/V head ``h // (H // H_kv)``, so consecutive query heads share one K/V
  head.  In the backward a K/V head's gradient is the sum over its query
  heads.
* Sliding window.  The same step ("sliding window attention"): a
  ``window_size=(left, right)`` pair, ``(-1, -1)`` meaning no window
  (Workflow 2, step 2), shown with ``causal=True``.  Reading taken: query i
  sees key j iff ``j >= i - left`` (when left >= 0) and ``j <= i + right``
  (when right >= 0), bounds inclusive, any negative value meaning that side
  is unbounded, and causal additionally requires ``j <= i``; indices are
  top-left aligned as for causal.  A row that sees no key at all has
  output 0 and log-sum-exp -inf (and contributes no gradient).

* Dropout.  The skill guide's Workflow 2, step 2 passes ``dropout_p=0.1``
  to ``flash_attn_func`` but defines no random numbers.  Reading taken:
  dropout acts on the attention weights after the softmax, as in
  FlashAttention: ``O = (P * keep * s_keep) V`` with the log-sum-exp of the
  undropped scores, ``s_keep`` restoring the expectation.  Both sides draw
  from one counter-based generator, Philox4x32-10 (Salmon, Moraes, Dror and
  Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11), implemented
  here from that definition: element (b, h, i, j) (h a query head) uses the
  counter ``(2*(j >> 5) + ((j >> 2) & 1), i, b*H + h, offset)`` and the key
  ``(seed mod 2^32, seed >> 32)``; its byte is byte ``j & 3`` of output word
  ``(j >> 3) & 3``; the element is kept iff byte >= thr with
  ``thr = min(255, rint(256 p))`` (p quantised to 1/256), and
  ``s_keep = 256 / (256 - thr)``.  (The counter layout lets one generator
  call serve the 16 keys of a 32-key tile that one GPU lane owns.)

Layout of every array: ``[batch, heads, seq, dim]`` (``[B, H, N, d]``), float64.
"""
import numpy as np

__all__ = [
    "attention_fwd64",
    "attention_rows_fwd64",
    "attention_bwd64",
    "attention_rows_dq64",
    "philox4x32_10",
    "dropout_threshold",
    "dropout_keep",
]

_M0, _M1, _W0, _W1 = 0xD2511F53, 0xCD9E8D57, 0x9E3779B9, 0xBB67AE85


def philox4x32_10(ctr, key):
    """Philox4x32-10 on arrays: ``ctr`` uint32 [..., 4], ``key`` uint32
    [..., 2] (broadcast).  Ten rounds; each multiplies words 0 and 2 by the
    two round constants into 64-bit products, and the new words are
    (hi(M1*x2) ^ x1 ^ k0, lo(M1*x2), hi(M0*x0) ^ x3 ^ k1, lo(M0*x0)); the key
    is bumped by the two Weyl constants before every round but the first."""
    c = np.asarray(ctr, dtype=np.uint64)
    k = np.asarray(key, dtype=np.uint64)
    x0, x1, x2, x3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0, k1 = k[..., 0], k[..., 1]
    m32 = np.uint64(0xFFFFFFFF)
    for r in range(10):
        if r > 0:
            k0 = (k0 + np.uint64(_W0)) & m32
            k1 = (k1 + np.uint64(_W1)) & m32
        p0 = np.uint64(_M0) * x0
        p1 = np.uint64(_M1) * x2
        x0, x1, x2, x3 = (p1 >> np.uint64(32)) ^ x1 ^ k0, p1 & m32, (p0 >> np.uint64(32)) ^ x3 ^ k1, p0 & m32
    return np.stack([x0, x1, x2, x3], axis=-1).astype(np.uint32)


def dropout_threshold(p):
    """(thr, s_keep) for dropout probability p in [0, 1) (see the module
    docstring); p is taken as the float32 the kernels receive."""
    p = float(np.float32(p))
    if not 0.0 <= p < 1.0:
        raise ValueError("dropout probability must be in [0, 1)")
    thr = min(255, int(np.rint(p * 256.0)))
    return thr, 256.0 / (256 - thr)


def dropout_keep(b, h, H, rows, nk, p, seed, offset):
    """Boolean keep mask [len(rows), nk] of query rows ``rows`` of (b, h)."""
    thr, _ = dropout_threshold(p)
    i = np.asarray(rows, dtype=np.uint64)[:, None]
    j = np.arange(nk, dtype=np.uint64)[None, :]
    ctr = np.stack(np.broadcast_arrays((j >> np.uint64(5)) * np.uint64(2) + ((j >> np.uint64(2)) & np.uint64(1)),
                                       i, np.uint64(b * H + h), np.uint64(offset)), axis=-1)
    seed = int(seed)
    w = philox4x32_10(ctr, (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))
    word = np.take_along_axis(w, ((j >> np.uint64(3)) & np.uint64(3)).astype(np.int64)[..., None]
                              .repeat(len(rows), axis=0), axis=-1)[..., 0]
    byte = (word >> ((j & np.uint64(3)) * np.uint64(8)).astype(np.uint32)) & np.uint32(0xFF)
    return byte >= thr


def _as64(x):
    a = np.asarray(x, dtype=np.float64)
    if a.ndim != 4:
        raise ValueError("expected a [B, H, N, d] array, got shape %r" % (a.shape,))
    return a


def _allowed(rows, nk, causal, window):
    """Boolean [len(rows), nk]: may query ``rows[r]`` attend key j (see the
    module docstring for the reading of causal and the window)."""
    left, right = int(window[0]), int(window[1])
    keys = np.arange(nk)[None, :]
    i = np.asarray(rows)[:, None]
    ok = np.ones((len(rows), nk), dtype=bool)
    if causal:
        ok &= keys <= i
    if left >= 0:
        ok &= keys >= i - left
    if right >= 0:
        ok &= keys <= i + right
    return ok


def _scores(q2, k2, scale, causal, rows, window=(-1, -1)):
    """s_ij = scale * q_i . k_j for the query rows ``rows`` (global indices);
    entries the mask forbids are -inf."""
    s = scale * (q2 @ k2.T)
    return np.where(_allowed(rows, k2.shape[0], causal, window), s, -np.inf)


def _softmax_rows(s):
    """Row softmax written out: p = exp(s - m) / sum exp(s - m) with
    m = row max (subtracting m changes nothing mathematically).  Also returns
    lse = m + log(sum exp(s - m)) = log sum exp(s).  A row of only -inf
    (no allowed key) gets p = 0 and lse = -inf."""
    m = np.max(s, axis=1, keepdims=True)
    empty = ~np.isfinite(m[:, 0])
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m)
    z = np.sum(e, axis=1, keepdims=True)
    p = e / np.where(z > 0, z, 1.0)
    with np.errstate(divide="ignore"):
        lse = (m + np.log(z))[:, 0]
    lse[empty] = -np.inf
    return p, lse


def _dropped(x, b, h, H, rows, dropout):
    """x * keep * s_keep for the rows of (b, h), or x without dropout."""
    if dropout is None:
        return x
    p, seed, offset = dropout
    _, s_keep = dropout_threshold(p)
    return np.where(dropout_keep(b, h, H, rows, x.shape[1], p, seed, offset), x * s_keep, 0.0)


def _kv_group(H, Hkv):
    if Hkv < 1 or H % Hkv:
        raise ValueError("K/V heads (%d) must divide query heads (%d)" % (Hkv, H))
    return H // Hkv


def _check(q, k, v):
    B, H, Nq, d = q.shape
    if k.shape[0] != B or v.shape != k.shape or k.shape[3] != d:
        raise ValueError("shape mismatch q%r k%r v%r" % (q.shape, k.shape, v.shape))
    return B, H, Nq, d, _kv_group(H, k.shape[1])


def attention_fwd64(q, k, v, scale, causal, window=(-1, -1), dropout=None):
    """O = softmax(scale * Q K^T [mask]) V and its log-sum-exp.

    q: [B, H, Nq, d]; k, v: [B, H_kv, Nk, d] with H_kv dividing H (any float
    dtype, widened to fp64).  Returns (o [B, H, Nq, d], lse [B, H, Nq]) in
    float64.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, Nq, d, G = _check(q, k, v)
    scale = float(scale)
    o = np.empty((B, H, Nq, d), dtype=np.float64)
    lse = np.empty((B, H, Nq), dtype=np.float64)
    rows = np.arange(Nq)
    for b in range(B):
        for h in range(H):
            s = _scores(q[b, h], k[b, h // G], scale, causal, rows, window)
            p, lse[b, h] = _softmax_rows(s)
            o[b, h] = _dropped(p, b, h, H, rows, dropout) @ v[b, h // G]
    return o, lse


def attention_rows_fwd64(q, k, v, scale, causal, rows, window=(-1, -1), dropout=None):
    """The forward restricted to selected query rows (each against all keys).

    rows: int array [B, H, R] of query indices.  Returns
    (o [B, H, R, d], lse [B, H, R]).  Row i of the result is exactly row
    rows[b,h,i] of ``attention_fwd64`` (softmax rows are independent).
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    rows = np.asarray(rows, dtype=np.int64)
    B, H, Nq, d, G = _check(q, k, v)
    if rows.ndim != 3 or rows.shape[:2] != (B, H):
        raise ValueError("rows must be [B, H, R]")
    R = rows.shape[2]
    o = np.empty((B, H, R, d), dtype=np.float64)
    lse = np.empty((B, H, R), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            r = rows[b, h]
            s = _scores(q[b, h][r], k[b, h // G], float(scale), causal, r, window)
            p, lse[b, h] = _softmax_rows(s)
            o[b, h] = _dropped(p, b, h, H, r, dropout) @ v[b, h // G]
    return o, lse


def attention_bwd64(q, k, v, do, scale, causal, window=(-1, -1), dropout=None):
    """Gradients of L = sum(O * dO) with respect to Q, K and V.

    Recomputes P from Q and K (its own P: nothing produced by a fast kernel
    is used), then applies the chain rule listed in the module docstring;
    a K/V head accumulates the gradients of every query head that uses it.
    With dropout the weights W = P * keep * s_keep replace P in O = W V, so
    dV = W^T dO and dS = P * (keep * s_keep * dP - rowsum(W * dP)).
    Returns (dq, dk, dv) with the shapes of q, k, v, in float64.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    B, H, Nq, d, G = _check(q, k, v)
    if do.shape != q.shape:
        raise ValueError("dO must have the shape of Q")
    scale = float(scale)
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    rows = np.arange(Nq)
    for b in range(B):
        for h in range(H):
            qq, kk, vv, g = q[b, h], k[b, h // G], v[b, h // G], do[b, h]
            p, _ = _softmax_rows(_scores(qq, kk, scale, causal, rows, window))
            wgt = _dropped(p, b, h, H, rows, dropout)
            dv[b, h // G] += wgt.T @ g
            dp = g @ vv.T
            ds = p * (_dropped(dp, b, h, H, rows, dropout) - np.sum(wgt * dp, axis=1, keepdims=True))
            dq[b, h] = scale * (ds @ kk)
            dk[b, h // G] += scale * (ds.T @ qq)
    return dq, dk, dv


def attention_rows_dq64(q, k, v, do, scale, causal, rows, window=(-1, -1), dropout=None):
    """dQ of ``attention_bwd64`` restricted to selected query rows.

    A query row's gradient depends only on its own softmax row (the same
    chain rule, row by row: dS_i = P_i * (dP_i - rowsum(W_i * dP_i)),
    dQ_i = scale * dS_i K), so it is computed here for the rows
    ``rows`` [B, H, R] alone, each against all keys.  Returns
    dq [B, H, R, d] in float64.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    rows = np.asarray(rows, dtype=np.int64)
    B, H, Nq, d, G = _check(q, k, v)
    if do.shape != q.shape:
        raise ValueError("dO must have the shape of Q")
    if rows.ndim != 3 or rows.shape[:2] != (B, H):
        raise ValueError("rows must be [B, H, R]")
    scale = float(scale)
    dq = np.empty((B, H, rows.shape[2], d), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            r = rows[b, h]
            kk, vv, g = k[b, h // G], v[b, h // G], do[b, h][r]
            p, _ = _softmax_rows(_scores(q[b, h][r], kk, scale, causal, r, window))
            wgt = _dropped(p, b, h, H, r, dropout)
            dp = g @ vv.T
            ds = p * (_dropped(dp, b, h, H, r, dropout) - np.sum(wgt * dp, axis=1, keepdims=True))
            dq[b, h] = scale * (ds @ kk)
    return dq
