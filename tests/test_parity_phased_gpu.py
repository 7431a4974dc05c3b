"""GPU parity of the forward's phased schedule, used from 1024 (d = 128) or
1536 (d = 64) workgroups of 128 queries upward (the other GPU tests mostly launch smaller grids, which
run the interleaved schedule).

Each case is a small problem repeated along the batch until the grid
reaches that many workgroups.  The first copy is checked against the fp64 oracle
(tolerances of the other parity tests).  Without dropout every copy must
then equal the first bit for bit.  With dropout the copies draw different
masks, since the generator's counter holds the batch index.
"""
import math
import sys

import numpy as np
import pytest
import torch

import exact_io_aware_02_amd as fa
from attn_inputs import make_qkv, to_bhsd64
from oracle import attention_fwd64, dropout_threshold

pytestmark = pytest.mark.gpu

TOL_O = {"fp16": 2e-3, "bf16": 1.6e-2}
TOL_LSE = 1e-3
DEV = "cuda:0"
PHASED_MIN_BLOCKS = {64: 1536, 128: 1024}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


CASES = [
    # name, B, H, Hkv, Nq, Nk, d, dtype, layout, causal, window, dropout
    ("d128_bf16_causal", 1, 2, 2, 300, 300, 128, "bf16", "bhsd", True, None, None),
    ("d128_fp16_noncausal_ragged", 1, 2, 2, 200, 333, 128, "fp16", "bhsd", False, None, None),
    ("d64_fp16_causal_bshd", 2, 2, 2, 257, 257, 64, "fp16", "bshd", True, None, None),
    ("d64_bf16_rect", 1, 3, 3, 130, 17, 64, "bf16", "bhsd", False, None, None),
    ("gqa4to1_causal_d128", 1, 4, 1, 333, 333, 128, "bf16", "bhsd", True, None, None),
    ("window_causal_d128", 1, 2, 2, 700, 700, 128, "bf16", "bhsd", True, (100, -1), None),
    ("window_empty_rows_d64", 1, 2, 2, 300, 100, 64, "fp16", "bhsd", False, (10, 10), None),
    ("gqa_window_bshd_d64", 2, 4, 2, 400, 400, 64, "bf16", "bshd", True, (130, 5), None),
    ("dropout_causal_d128", 1, 2, 2, 300, 300, 128, "bf16", "bhsd", True, None, (0.3, 99, 7)),
    ("dropout_gqa_window_d64", 2, 4, 2, 200, 230, 64, "fp16", "bshd", False, (40, 10), (0.2, 17, 3)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_phased_forward_matches_oracle(case):
    name, B, H, Hkv, Nq, Nk, d, dt, layout, causal, window, dr = case
    blocks = math.ceil(Nq / 128) * B * H
    R = math.ceil(PHASED_MIN_BLOCKS[d] / blocks)
    say("case %s: %d copies, %d workgroups" % (name, R, R * blocks))
    inp = make_qkv(B, H, Nq, Nk, d, dt, layout, seed=61, Hkv=Hkv)
    q, k, v = (inp[x].repeat(R, 1, 1, 1).to(DEV) for x in ("q", "k", "v"))
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.attention_fwd(q, k, v, causal=causal, scale=scale, layout=layout, window=window, dropout=dr)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    w = window if window is not None else (-1, -1)
    args = [to_bhsd64(inp[x], layout) for x in ("q", "k", "v")]
    o_ref, lse_ref = attention_fwd64(*args, scale, causal, window=w, dropout=dr)
    keep = dropout_threshold(dr[0])[1] if dr else 1.0
    got_o = to_bhsd64(o[:B], layout)
    got_l = lse[:B].numpy().astype(np.float64)
    live = np.isfinite(lse_ref)
    assert np.isfinite(got_o).all()
    err_o = np.abs(got_o - o_ref).max()
    say("  O max-abs err %.3e (tol %.1e)" % (err_o, TOL_O[dt] * keep))
    assert err_o <= TOL_O[dt] * keep
    np.testing.assert_array_equal(np.isneginf(got_l), ~live)
    err_l = np.abs(got_l[live] - lse_ref[live]).max()
    say("  LSE max-abs err %.3e" % err_l)
    assert err_l <= TOL_LSE
    if dr is None:
        for r in range(1, R):
            assert torch.equal(o[r * B:(r + 1) * B].view(torch.int16), o[:B].view(torch.int16)), r
            assert torch.equal(lse[r * B:(r + 1) * B], lse[:B]), r
