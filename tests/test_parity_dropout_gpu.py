"""GPU parity of dropout (fa_fwd_ex / fa_bwd_ex with dropout_p > 0) against
the fp64 oracle drawing the same Philox4x32-10 mask.

Tolerances are those of tests/test_parity_gpu.py, the output one scaled by
the keep factor 256/(256 - thr) (the kept weights are that much larger).
"""
import sys

import numpy as np
import pytest
import torch

import exact_io_aware_02_amd as fa
from attn_inputs import make_qkv, to_bhsd64
from oracle import attention_bwd64, attention_fwd64, dropout_threshold

pytestmark = pytest.mark.gpu

TOL_O = {"fp16": 2e-3, "bf16": 1.6e-2}
TOL_LSE = 1e-3
TOL_GRAD = 2e-2
DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


CASES = [
    # name, B, H, Hkv, Nq, Nk, d, dtype, layout, causal, window, (p, seed, offset)
    ("p01_d64", 1, 2, 2, 256, 256, 64, "fp16", "bhsd", False, None, (0.1, 1234, 0)),
    ("p03_causal_d128_ragged", 1, 2, 2, 300, 300, 128, "bf16", "bhsd", True, None, (0.3, 99, 7)),
    ("p02_gqa_window_bshd", 2, 4, 2, 200, 230, 64, "fp16", "bshd", False, (40, 10), (0.2, (5 << 33) + 17, 3)),
    ("p05_d64_causal", 1, 3, 3, 190, 190, 64, "bf16", "bhsd", True, None, (0.5, 7, 123456)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_dropout_matches_oracle(case):
    name, B, H, Hkv, Nq, Nk, d, dt, layout, causal, window, dr = case
    say("case %s" % name)
    inp = make_qkv(B, H, Nq, Nk, d, dt, layout, seed=31, with_do=True, Hkv=Hkv)
    q, k, v, do = (inp[x].to(DEV) for x in ("q", "k", "v", "do"))
    scale = 1.0 / np.sqrt(d)
    o, lse = fa.attention_fwd(q, k, v, causal=causal, scale=scale, layout=layout, window=window, dropout=dr)
    dq, dk, dv = fa.attention_bwd(q, k, v, o, lse, do, causal=causal, scale=scale, layout=layout, window=window,
                                  dropout=dr)
    torch.cuda.synchronize()
    w = window if window is not None else (-1, -1)
    args = [to_bhsd64(inp[x], layout) for x in ("q", "k", "v")]
    o_ref, lse_ref = attention_fwd64(*args, scale, causal, window=w, dropout=dr)
    _, s_keep = dropout_threshold(dr[0])
    got_o = to_bhsd64(o.cpu(), layout)
    assert np.isfinite(got_o).all()
    err_o = np.abs(got_o - o_ref).max()
    say("  O max-abs err %.3e (tol %.1e)" % (err_o, TOL_O[dt] * s_keep))
    assert err_o <= TOL_O[dt] * s_keep
    err_l = np.abs(lse.cpu().numpy().astype(np.float64) - lse_ref).max()
    say("  LSE max-abs err %.3e" % err_l)
    assert err_l <= TOL_LSE
    g_ref = attention_bwd64(*args, to_bhsd64(inp["do"], layout), scale, causal, window=w, dropout=dr)
    for nm, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), g_ref):
        got = to_bhsd64(g.cpu(), layout)
        assert np.isfinite(got).all(), nm
        rel = np.linalg.norm(got - r) / np.linalg.norm(r)
        say("  %s rel-F err %.3e" % (nm, rel))
        assert rel <= TOL_GRAD, nm


def test_dropout_zero_is_bitwise_plain():
    inp = make_qkv(1, 2, 200, 200, 128, "bf16", seed=3, with_do=True)
    q, k, v, do = (inp[x].to(DEV) for x in ("q", "k", "v", "do"))
    o0, l0 = fa.attention_fwd(q, k, v, causal=True)
    o1, l1 = fa.attention_fwd(q, k, v, causal=True, dropout=(0.0, 5, 5))
    g0 = fa.attention_bwd(q, k, v, o0, l0, do, causal=True)
    g1 = fa.attention_bwd(q, k, v, o1, l1, do, causal=True, dropout=(0.0, 5, 5))
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    for a, b in zip(g0, g1):
        assert torch.equal(a, b)


def test_dropout_mask_changes_with_seed_and_offset():
    """Different (seed, offset) give different outputs; the same give the same bits."""
    inp = make_qkv(1, 2, 128, 128, 64, "fp16", seed=4)
    q, k, v = (inp[x].to(DEV) for x in ("q", "k", "v"))
    oa, _ = fa.attention_fwd(q, k, v, dropout=(0.25, 1, 0))
    ob, _ = fa.attention_fwd(q, k, v, dropout=(0.25, 1, 0))
    oc, _ = fa.attention_fwd(q, k, v, dropout=(0.25, 2, 0))
    od, _ = fa.attention_fwd(q, k, v, dropout=(0.25, 1, 1))
    torch.cuda.synchronize()
    assert torch.equal(oa, ob)
    assert not torch.equal(oa, oc) and not torch.equal(oa, od)
