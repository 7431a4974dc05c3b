"""GPU parity of fewer K/V heads and sliding windows (fa_fwd_ex, fa_bwd_ex)
against the fp64 oracle, with the tolerances of tests/test_parity_gpu.py.

Cases cover: grouped and multi-query heads, both layouts, ragged lengths
(several tiles plus a tail), windows on one or both sides with and without
causal, rows that admit no key (O = 0, lse = -inf, dq = 0), and windows
wide enough to be no window at all.
"""
import sys

import numpy as np
import pytest
import torch

import exact_io_aware_02_amd as fa
from attn_inputs import make_qkv, to_bhsd64
from oracle import attention_bwd64, attention_fwd64

pytestmark = pytest.mark.gpu

TOL_O = {"fp16": 2e-3, "bf16": 1.6e-2}
TOL_LSE = 1e-3
TOL_GRAD = 2e-2
DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


CASES = [
    # name, B, H, Hkv, Nq, Nk, d, dtype, layout, causal, window
    ("gqa4to2_causal", 1, 8, 2, 256, 256, 64, "fp16", "bhsd", True, None),
    ("gqa4to2", 2, 4, 2, 190, 190, 64, "fp16", "bhsd", False, None),
    ("mqa_ragged_bshd", 1, 4, 1, 200, 300, 128, "bf16", "bshd", False, None),
    ("mqa_causal_d128", 1, 4, 1, 333, 333, 128, "bf16", "bhsd", True, None),
    ("win64_64", 1, 2, 2, 512, 512, 64, "fp16", "bhsd", False, (64, 64)),
    ("win100_causal_d128", 1, 2, 2, 700, 700, 128, "bf16", "bhsd", True, (100, -1)),
    ("win_right_only", 1, 2, 2, 300, 260, 64, "fp16", "bshd", False, (-1, 37)),
    ("win0_0_diagonal", 1, 2, 2, 130, 130, 64, "fp16", "bhsd", False, (0, 0)),
    ("win_empty_rows", 1, 2, 2, 300, 100, 64, "fp16", "bhsd", False, (10, 10)),
    ("gqa_win", 1, 6, 3, 257, 257, 128, "fp16", "bhsd", False, (33, 17)),
    ("gqa_win_causal_bf16", 2, 4, 2, 400, 400, 64, "bf16", "bshd", True, (130, 5)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fwd_bwd_matches_oracle(case):
    name, B, H, Hkv, Nq, Nk, d, dt, layout, causal, window = case
    say("case %s" % name)
    inp = make_qkv(B, H, Nq, Nk, d, dt, layout, seed=77, with_do=True, Hkv=Hkv)
    q, k, v, do = (inp[x].to(DEV) for x in ("q", "k", "v", "do"))
    scale = 1.0 / np.sqrt(d)
    o, lse = fa.attention_fwd(q, k, v, causal=causal, scale=scale, layout=layout, window=window)
    dq, dk, dv = fa.attention_bwd(q, k, v, o, lse, do, causal=causal, scale=scale, layout=layout, window=window)
    torch.cuda.synchronize()
    w = window if window is not None else (-1, -1)
    args = [to_bhsd64(inp[x], layout) for x in ("q", "k", "v")]
    o_ref, lse_ref = attention_fwd64(*args, scale, causal, window=w)
    got_o = to_bhsd64(o.cpu(), layout)
    got_l = lse.cpu().numpy().astype(np.float64)
    live = np.isfinite(lse_ref)
    assert np.isfinite(got_o).all()
    err_o = np.abs(got_o - o_ref).max()
    say("  O max-abs err %.3e (tol %.1e)" % (err_o, TOL_O[dt]))
    assert err_o <= TOL_O[dt]
    np.testing.assert_array_equal(np.isneginf(got_l), ~live)  # empty rows exactly -inf, others finite
    err_l = np.abs(got_l[live] - lse_ref[live]).max()
    say("  LSE max-abs err %.3e (empty rows %d)" % (err_l, int((~live).sum())))
    assert err_l <= TOL_LSE
    if (~live).any():
        assert np.all(got_o[~np.broadcast_to(live[..., None], got_o.shape)] == 0.0)
    g_ref = attention_bwd64(*args, to_bhsd64(inp["do"], layout), scale, causal, window=w)
    for nm, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), g_ref):
        got = to_bhsd64(g.cpu(), layout)
        assert np.isfinite(got).all(), nm
        if np.linalg.norm(r) < 1e-6:  # e.g. the (0, 0) window: one key per row, so dS = 0
            say("  %s: reference is zero, max|gpu| = %.2e" % (nm, np.abs(got).max()))
            assert np.abs(got).max() < 1e-3, nm
            continue
        rel = np.linalg.norm(got - r) / np.linalg.norm(r)
        say("  %s rel-F err %.3e" % (nm, rel))
        assert rel <= TOL_GRAD, nm
    if (~live).any():
        got_dq = to_bhsd64(dq.cpu(), layout)
        assert np.all(got_dq[~np.broadcast_to(live[..., None], got_dq.shape)] == 0.0)


def test_wide_window_is_bitwise_no_window():
    """A window that excludes nothing runs the unbanded kernels: same bits."""
    inp = make_qkv(1, 4, 300, 300, 64, "fp16", seed=5, with_do=True, Hkv=2)
    q, k, v = (inp[x].to(DEV) for x in ("q", "k", "v"))
    o0, l0 = fa.attention_fwd(q, k, v)
    o1, l1 = fa.attention_fwd(q, k, v, window=(300, 5000))
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_gqa_equals_repeated_heads():
    """Fewer K/V heads give the same bits as multi-head attention on K/V
    heads repeated G times (the kernels only change which head they read);
    the K/V gradients are the group sums of the repeated heads' gradients."""
    H, Hkv = 6, 2
    inp = make_qkv(1, H, 257, 257, 128, "bf16", seed=9, with_do=True, Hkv=Hkv)
    q, k, v, do = (inp[x].to(DEV) for x in ("q", "k", "v", "do"))
    kr, vr = (t.repeat_interleave(H // Hkv, dim=1).contiguous() for t in (k, v))
    o1, l1 = fa.attention_fwd(q, k, v, causal=True)
    o2, l2 = fa.attention_fwd(q, kr, vr, causal=True)
    dq1, dk1, dv1 = fa.attention_bwd(q, k, v, o1, l1, do, causal=True)
    dq2, dk2, dv2 = fa.attention_bwd(q, kr, vr, o2, l2, do, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(dq1, dq2)
    for g1, g2 in ((dk1, dk2), (dv1, dv2)):
        ref = g2.float().view(1, Hkv, H // Hkv, 257, 128).sum(2)
        err = (g1.float() - ref).abs().max().item() / ref.abs().max().item()
        say("  grouped K/V gradient vs summed repeated heads: %.3e" % err)
        assert err < 1e-2


def _bwd_ex(q, k, v, o, lse, do, causal, nbytes, window=None, dropout=None):
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    fa.fa_bwd_ex(q, k, v, o, lse, do, dq, dk, dv, 1.0 / np.sqrt(q.shape[-1]), causal, ws, window,
                 dropout=dropout)
    return dq, dk, dv


@pytest.mark.parametrize("H,Hkv,N,d,dt,causal,window,dropout", [
    (8, 2, 300, 128, "bf16", True, None, None),
    (4, 1, 257, 64, "fp16", False, None, None),
    (6, 3, 400, 64, "bf16", True, (100, -1), None),
    (8, 2, 256, 128, "bf16", True, None, (0.1, 7, 3)),
])
def test_split_kv_gradients_match_unsplit(H, Hkv, N, d, dt, causal, window, dropout):
    """The split dK/dV stage (partials reduced by a second kernel) against
    the single-pass one: dQ bit-identical, dK/dV equal up to fp32 summation
    order, and both within the oracle's tolerance."""
    say("case split_kv H%d Hkv%d N%d d%d %s causal=%d window=%r dropout=%r" % (H, Hkv, N, d, dt, causal, window,
                                                                                 dropout))
    inp = make_qkv(1, H, N, N, d, dt, seed=31, with_do=True, Hkv=Hkv)
    q, k, v, do = (inp[x].to(DEV) for x in ("q", "k", "v", "do"))
    s = 1.0 / np.sqrt(d)
    o, lse = fa.attention_fwd(q, k, v, causal=causal, scale=s, window=window, dropout=dropout)
    small = fa.fa_bwd_workspace_bytes(1, H, N, N, d, fa.FA_BF16 if dt == "bf16" else fa.FA_FP16)
    big = fa.fa_bwd_ex_workspace_bytes(1, H, Hkv, N, N, d, fa.FA_BF16 if dt == "bf16" else fa.FA_FP16)
    assert big > small
    g0 = _bwd_ex(q, k, v, o, lse, do, causal, small, window, dropout)
    g1 = _bwd_ex(q, k, v, o, lse, do, causal, big, window, dropout)
    torch.cuda.synchronize()
    assert torch.equal(g0[0], g1[0])
    for nm, a, b in zip(("dk", "dv"), g0[1:], g1[1:]):
        err = (a.float() - b.float()).abs().max().item() / max(b.float().abs().max().item(), 1e-30)
        say("  %s split vs unsplit: max rel %.2e" % (nm, err))
        assert err < 1e-2
    w = window if window is not None else (-1, -1)
    args = [to_bhsd64(inp[x]) for x in ("q", "k", "v")]
    g_ref = attention_bwd64(*args, to_bhsd64(inp["do"]), s, causal, window=w, dropout=dropout)
    for nm, g, r in zip(("dq", "dk", "dv"), g1, g_ref):
        rel = np.linalg.norm(to_bhsd64(g.cpu()) - r) / np.linalg.norm(r)
        say("  %s rel-F err (split) %.3e" % (nm, rel))
        assert rel <= TOL_GRAD, nm


def test_split_kv_16k_gqa_identities():
    """The benchmark's fewer-K/V-heads backward (16 query heads on 2 K/V
    heads, 16K causal d=128 bf16, split dK/dV): per K/V head the key sums
    sum_j dK_j = 0 and sum_j dV_j = sum over its query heads and rows of dO
    hold, and the split result matches the single-pass one."""
    say("case split_kv_16k")
    B, H, Hkv, N, d = 1, 16, 2, 16384, 128
    inp = make_qkv(B, H, N, N, d, "bf16", seed=3, in_scale=0.5, with_do=True, Hkv=Hkv)
    q, k, v, do = (inp[x].to(DEV) for x in ("q", "k", "v", "do"))
    o, lse = fa.attention_fwd(q, k, v, causal=True)
    small = fa.fa_bwd_workspace_bytes(B, H, N, N, d, fa.FA_BF16)
    big = fa.fa_bwd_ex_workspace_bytes(B, H, Hkv, N, N, d, fa.FA_BF16)
    g0 = _bwd_ex(q, k, v, o, lse, do, True, small)
    g1 = _bwd_ex(q, k, v, o, lse, do, True, big)
    torch.cuda.synchronize()
    assert torch.equal(g0[0], g1[0])
    for nm, a, b in zip(("dk", "dv"), g0[1:], g1[1:]):
        err = (a.float() - b.float()).abs().max().item() / b.float().abs().max().item()
        say("  %s split vs unsplit: max rel %.2e" % (nm, err))
        assert err < 1e-2
    dk, dv = g1[1].double(), g1[2].double()
    G = H // Hkv
    sum_do = do.double().view(B, Hkv, G, N, d).sum(dim=(2, 3))
    err_v = ((dv.sum(dim=2) - sum_do).abs().max() / sum_do.abs().max()).item()
    err_k = (dk.sum(dim=2).abs().max() / dk.abs().sum(dim=2).max()).item()
    say("  sum_j dV_j vs sum dO: %.2e; |sum_j dK_j| / sum_j |dK_j|: %.2e" % (err_v, err_k))
    assert err_v < 2e-2 and err_k < 2e-2
