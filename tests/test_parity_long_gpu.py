"""GPU parity at the largest sizes the tests reach: long rows, and a grid of
more than 65535 workgroups in every kernel.

- One head of 131072 queries and keys at d=128 bf16, causal, inputs x0.5
  (8x the benchmark's rows; 4096 key tiles in the heaviest query block).
  Forward through both routes for heavy blocks (``fa_fwd_splitk``'s chunks
  across workgroups, ``fa_fwd_ex``'s key split inside a workgroup), the
  backward with the statistics-only workspace and with the one that lets
  dK/dV split.
- 65536 rows at d=64 fp16 BSHD, 4 query heads on 1 K/V head, causal with a
  window of 4095 keys to the left, dropout 0.1 with a 64-bit seed.
- B9 H128 N8192 d64 bf16 causal: 73728 forward query blocks and dK/dV key
  blocks, 294912 statistics blocks (inputs: heads cut from one seeded pool of
  rows at seeded offsets, ``make_qkv_pooled``); four heads checked.

O, LSE and dQ are checked against the fp64 oracle on sampled query rows
(rows 0 and N-1 always); dK and dV through identities that hold at any size
(``grad_identities``): sum_j k_j dK_j^T = sum_i dQ_i q_i^T, sum_j v_j dV_j^T
= sum_i O_i dO_i^T and sum_j dK_j = 0, relative to the size of each side,
within about four times the deviation that rounding exact gradients to the
output type gives (2.4e-3 for bf16, a test of the oracle pins; 8x less for
fp16).
"""
import math
import sys

import numpy as np
import pytest
import torch

import exact_io_aware_02_amd as fa
from attn_inputs import make_qkv, make_qkv_pooled, sample_rows, to_bhsd64
from grad_identities import identity_errors
from oracle import attention_rows_dq64, attention_rows_fwd64, dropout_threshold

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL_O = {"fp16": 2e-3, "bf16": 1.6e-2}
TOL_LSE = 1e-3
TOL_GRAD = 2e-2
TOL_IDENT = {"fp16": 2e-3, "bf16": 1e-2}
ROWS = 128


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def fwd(route, q, k, v, scale, causal, window, layout, dropout):
    B, H, Nq, d = (q.shape[0], q.shape[1], q.shape[2], q.shape[3]) if layout == "bhsd" else \
        (q.shape[0], q.shape[2], q.shape[1], q.shape[3])
    Nk = k.shape[2] if layout == "bhsd" else k.shape[1]
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=DEV)
    if route == "splitk":
        nf = fa.fa_fwd_splitk_workspace_bytes(B, H, Nq, Nk, d, causal, window)
        ws = torch.empty(nf, dtype=torch.uint8, device=DEV) if nf else None
        fa.fa_fwd_splitk(q, k, v, o, lse, scale, causal, ws, window, layout, None, dropout)
    elif route == "ex":
        fa.fa_fwd_ex(q, k, v, o, lse, scale, causal, window, layout, None, dropout)
    else:
        fa.fa_fwd(q, k, v, o, lse, scale, causal)
    return o, lse


def bwd(route, q, k, v, o, lse, do, scale, causal, window, layout, dropout, code):
    B, H, Nq, d = (q.shape[0], q.shape[1], q.shape[2], q.shape[3]) if layout == "bhsd" else \
        (q.shape[0], q.shape[2], q.shape[1], q.shape[3])
    Hkv, Nk = (k.shape[1], k.shape[2]) if layout == "bhsd" else (k.shape[2], k.shape[1])
    g = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    if route == "split":
        nbytes = fa.fa_bwd_ex_workspace_bytes(B, H, Hkv, Nq, Nk, d, code)
    else:
        nbytes = fa.fa_bwd_workspace_bytes(B, H, Nq, Nk, d, code)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    if route == "plain":
        fa.fa_bwd(q, k, v, o, lse, do, *g, scale, causal, ws)
    else:
        fa.fa_bwd_ex(q, k, v, o, lse, do, *g, scale, causal, ws, window, fa.FA_BWD_ALL, layout, None, dropout)
    return g


def pick(a, rows):
    B, H = rows.shape[:2]
    return np.stack([np.stack([a[b, h][rows[b, h]] for h in range(H)]) for b in range(B)])


def check_rows(name, dt, q64, k64, v64, do64, o, lse, dq, scale, causal, rows, window, dropout):
    """O, LSE and dQ of the sampled rows against the oracle (64-bit arrays
    in [B, H, N, d]; o, lse, dq the kernels' results, likewise)."""
    ro, rl = attention_rows_fwd64(q64, k64, v64, scale, causal, rows, window=window, dropout=dropout)
    rq = attention_rows_dq64(q64, k64, v64, do64, scale, causal, rows, window=window, dropout=dropout)
    keep = dropout_threshold(dropout[0])[1] if dropout else 1.0
    assert np.isfinite(o).all() and np.isfinite(dq).all()
    live = np.isfinite(rl)
    np.testing.assert_array_equal(np.isneginf(pick(lse, rows)), ~live)
    err_o = np.abs(pick(o, rows) - ro).max()
    err_l = np.abs(pick(lse, rows)[live] - rl[live]).max()
    rel_q = np.linalg.norm(pick(dq, rows) - rq) / np.linalg.norm(rq)
    say("  %s: %d rows/head: O max-abs %.3e (tol %.2e), LSE %.3e, dQ rel-F %.3e"
        % (name, rows.shape[2], err_o, TOL_O[dt] * keep, err_l, rel_q))
    assert err_o <= TOL_O[dt] * keep and err_l <= TOL_LSE and rel_q <= TOL_GRAD


def check_identities(name, dt, q64, k64, v64, do64, o, dq, dk, dv):
    err = identity_errors(q64, k64, v64, do64, o, dq, dk, dv)
    say("  %s: K^T dK vs dQ^T Q %.2e, V^T dV vs O^T dO %.2e, |sum dK| %.2e" % (name, err["dk"], err["dv"],
                                                                            err["dk_sum"]))
    assert np.isfinite(dk).all() and np.isfinite(dv).all()
    assert max(err.values()) <= TOL_IDENT[dt]


def test_long_rows_131072_d128():
    N, d, dt = 131072, 128, "bf16"
    say("case long rows: B1 H1 N%d d%d %s causal" % (N, d, dt))
    inp = make_qkv(1, 1, N, N, d, dt, seed=811, in_scale=0.5, with_do=True)
    q, k, v, do = (inp[x].to(DEV) for x in ("q", "k", "v", "do"))
    s = 1.0 / math.sqrt(d)
    rows = sample_rows(1, 1, N, ROWS, 812)
    q64, k64, v64, do64 = (to_bhsd64(inp[x]) for x in ("q", "k", "v", "do"))
    outs = {}
    for route in ("splitk", "ex"):
        o, lse = fwd(route, q, k, v, s, True, (-1, -1), "bhsd", None)
        torch.cuda.synchronize()
        outs[route] = (o, lse)
        o64, l64 = to_bhsd64(o.cpu()), lse.cpu().numpy().astype(np.float64)
        ro, rl = attention_rows_fwd64(q64, k64, v64, s, True, rows)
        err_o, err_l = np.abs(pick(o64, rows) - ro).max(), np.abs(pick(l64, rows) - rl).max()
        say("  forward %s: O max-abs %.3e, LSE %.3e" % (route, err_o, err_l))
        assert np.isfinite(o64).all() and err_o <= TOL_O[dt] and err_l <= TOL_LSE
    o, lse = outs["splitk"]
    o64 = to_bhsd64(o.cpu())
    for route in ("plain", "split"):
        dq, dk, dv = bwd(route, q, k, v, o, lse, do, s, True, (-1, -1), "bhsd", None, fa.FA_BF16)
        torch.cuda.synchronize()
        dq64, dk64, dv64 = (to_bhsd64(x.cpu()) for x in (dq, dk, dv))
        check_rows("backward " + route, dt, q64, k64, v64, do64, o64, lse.cpu().numpy().astype(np.float64), dq64,
                   s, True, rows, (-1, -1), None)
        check_identities("backward " + route, dt, q64, k64, v64, do64, o64, dq64, dk64, dv64)


def test_long_rows_65536_gqa_window_dropout_bshd():
    N, d, dt, H, Hkv = 65536, 64, "fp16", 4, 1
    window, dropout = (4095, -1), (0.1, (3 << 32) + 17, 5)
    say("case long rows: B1 H%d on %d N%d d%d %s bshd causal window %s dropout %s" % (H, Hkv, N, d, dt, window,
                                                                                   dropout))
    inp = make_qkv(1, H, N, N, d, dt, "bshd", seed=821, with_do=True, Hkv=Hkv)
    q, k, v, do = (inp[x].to(DEV) for x in ("q", "k", "v", "do"))
    s = 1.0 / math.sqrt(d)
    o, lse = fwd("splitk", q, k, v, s, True, window, "bshd", dropout)
    dq, dk, dv = bwd("split", q, k, v, o, lse, do, s, True, window, "bshd", dropout, fa.FA_FP16)
    torch.cuda.synchronize()
    rows = sample_rows(1, H, N, ROWS, 822)
    q64, k64, v64, do64 = (to_bhsd64(inp[x], "bshd") for x in ("q", "k", "v", "do"))
    o64, dq64, dk64, dv64 = (to_bhsd64(x.cpu(), "bshd") for x in (o, dq, dk, dv))
    check_rows("window + dropout", dt, q64, k64, v64, do64, o64, lse.cpu().numpy().astype(np.float64), dq64, s,
               True, rows, window, dropout)
    check_identities("window + dropout", dt, q64, k64, v64, do64, o64, dq64, dk64, dv64)


def test_grid_beyond_65535_workgroups():
    B, H, N, d, dt = 9, 128, 8192, 64, "bf16"
    say("case large grid: B%d H%d N%d d%d %s causal (%d query blocks)" % (B, H, N, d, dt, B * H * N // 128))
    inp = make_qkv_pooled(B, H, N, d, dt, seed=831, with_do=True)
    q, k, v, do = (inp[x].to(DEV) for x in ("q", "k", "v", "do"))
    s = 1.0 / math.sqrt(d)
    o, lse = fwd("plain", q, k, v, s, True, (-1, -1), "bhsd", None)
    dq, dk, dv = bwd("plain", q, k, v, o, lse, do, s, True, (-1, -1), "bhsd", None, fa.FA_BF16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(832)
    heads = [(0, 0), (B - 1, H - 1)] + [(int(rng.integers(0, B)), int(rng.integers(0, H))) for _ in range(2)]
    for b, h in heads:
        sl = lambda t: t[b:b + 1, h:h + 1]  # noqa: E731
        q64, k64, v64, do64 = (to_bhsd64(sl(inp[x])) for x in ("q", "k", "v", "do"))
        o64, dq64, dk64, dv64 = (to_bhsd64(sl(x).cpu()) for x in (o, dq, dk, dv))
        l64 = sl(lse).cpu().numpy().astype(np.float64)
        rows = sample_rows(1, 1, N, 64, 833 + b * H + h)
        check_rows("head (%d, %d)" % (b, h), dt, q64, k64, v64, do64, o64, l64, dq64, s, True, rows, (-1, -1),
                   None)
        check_identities("head (%d, %d)" % (b, h), dt, q64, k64, v64, do64, o64, dq64, dk64, dv64)
