"""GPU parity of the backward's splits.

* dQ: a grid of at most one workgroup per CU whose heaviest query block has
  32 or more key tiles runs three (d = 64) or two (d = 128) groups of four
  waves per workgroup, each on its own run of the key tiles, their partial
  sums added through LDS (every case below).
* dK/dV with the workspace of fa_bwd_ex_workspace_bytes: each key block's
  steps (its query heads' query tiles) cut into runs on several
  workgroups, their fp32 partial sums added in run order by a second
  kernel.  With fewer K/V heads the runs are whole query heads (the GQA
  cases); with equal heads a grid of fewer dK/dV workgroups than the chip
  holds (256 at d = 128, 512 at d = 64) with Nk >= 2048 cuts each key
  block's query tiles into two runs (the eq_split cases, whose runs can
  start and end inside the causal band).

Every case checks dQ, dK, dV against the fp64 oracle (relative Frobenius
error <= 2e-2), that a second run is bitwise identical, and, where the
larger workspace splits dK/dV, that the unsplit stage agrees within the
same tolerance.
"""
import math
import sys

import numpy as np
import pytest
import torch

import exact_io_aware_02_amd as fa
from attn_inputs import make_qkv, to_bhsd64
from oracle import attention_bwd64

pytestmark = pytest.mark.gpu

TOL_GRAD = 2e-2
DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


CASES = [
    # name, B, H, Hkv, Nq, Nk, d, dtype, layout, causal, window, dropout
    ("d128_causal", 1, 2, 2, 1100, 1100, 128, "bf16", "bhsd", True, None, None),
    ("d64_causal_bshd", 2, 3, 3, 1500, 1500, 64, "fp16", "bshd", True, None, None),
    ("d128_rect", 1, 2, 2, 300, 1300, 128, "fp16", "bhsd", False, None, None),
    ("d64_window", 1, 2, 2, 1200, 1200, 64, "bf16", "bhsd", True, (900, -1), None),
    ("d128_window_empty_rows", 1, 2, 2, 1500, 1100, 128, "bf16", "bhsd", False, (1000, 200), None),
    ("d64_dropout", 1, 2, 2, 1100, 1100, 64, "fp16", "bhsd", True, None, (0.25, (3 << 32) + 7, 2)),
    ("d64_gqa", 1, 4, 2, 1100, 1100, 64, "bf16", "bhsd", True, None, None),
    ("d128_gqa_window_dropout", 1, 8, 2, 1300, 1300, 128, "fp16", "bhsd", True, (700, -1), (0.1, 77, 1)),
    ("d128_eq_split_causal", 1, 2, 2, 2500, 2500, 128, "bf16", "bhsd", True, None, None),
    ("d64_eq_split_bshd_ragged", 1, 2, 2, 2100, 2100, 64, "fp16", "bshd", True, None, None),
    ("d128_eq_split_window_rect", 1, 1, 1, 3000, 2200, 128, "bf16", "bhsd", False, (800, 100), None),
    ("d64_eq_split_dropout", 2, 1, 1, 2048, 2048, 64, "bf16", "bhsd", True, None, (0.2, (9 << 32) + 1, 4)),
]

CUS = 256  # MI355X


def splits_expected(B, H, Hkv, Nk, d):
    """Whether fa_bwd_ex_workspace_bytes asks for partial sums: fewer K/V
    heads, or equal heads whose dK/dV grid (32 keys per wave pair, 4 pairs
    at d = 64, 6 at d = 128) has fewer workgroups than the chip holds (one
    per CU at d = 128, two at d = 64), with Nk >= 2048."""
    blocks = -(-Nk // (32 * (4 if d == 64 else 6))) * B * Hkv
    return Hkv != H or (Nk >= 2048 and blocks < CUS * (2 if d == 64 else 1))


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_split_backward(case):
    name, B, H, Hkv, Nq, Nk, d, dt, layout, causal, window, dr = case
    code = fa.FA_FP16 if dt == "fp16" else fa.FA_BF16
    big = fa.fa_bwd_ex_workspace_bytes(B, H, Hkv, Nq, Nk, d, code)
    small = fa.fa_bwd_workspace_bytes(B, H, Nq, Nk, d, code)
    say("case bwd split %s: workspace %d (unsplit %d)" % (name, big, small))
    assert (big > small) == splits_expected(B, H, Hkv, Nk, d)
    inp = make_qkv(B, H, Nq, Nk, d, dt, layout, seed=83, with_do=True, Hkv=Hkv)
    q, k, v, do = (inp[x].to(DEV) for x in ("q", "k", "v", "do"))
    s = 1.0 / math.sqrt(d)
    w = window if window is not None else (-1, -1)
    o, lse = fa.attention_fwd(q, k, v, causal=causal, scale=s, layout=layout, window=window, dropout=dr)
    grads = lambda: [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]  # noqa: E731
    outs = []
    # a zeroed workspace, one of all-ones bytes (NaN partial sums, counters
    # at 2^32 - 1: the library must zero its counters and read only this
    # call's sums), and the statistics-only size (no split)
    for nbytes, fill in ((big, 0), (big, 0xFF), (small, 0)):
        ws = torch.full((nbytes,), fill, dtype=torch.uint8, device=DEV)
        g = grads()
        fa.fa_bwd_ex(q, k, v, o, lse, do, *g, s, causal, ws, w, fa.FA_BWD_ALL, layout, None, dr)
        outs.append(g)
    # the stages as three calls on an all-ones workspace (dK/dV without the
    # statistics stage zeroes the counters itself), then the whole backward
    # again on that workspace with another dO: equal to a fresh call with it
    ws = torch.full((big,), 0xFF, dtype=torch.uint8, device=DEV)
    g = grads()
    for stage in (fa.FA_BWD_PREP, fa.FA_BWD_DKDV, fa.FA_BWD_DQ):
        fa.fa_bwd_ex(q, k, v, o, lse, do, *g, s, causal, ws, w, stage, layout, None, dr)
    do2 = torch.flip(do, dims=(0,)).contiguous() * 0.5
    g2, g2_fresh = grads(), grads()
    fa.fa_bwd_ex(q, k, v, o, lse, do2, *g2, s, causal, ws, w, fa.FA_BWD_ALL, layout, None, dr)
    fa.fa_bwd_ex(q, k, v, o, lse, do2, *g2_fresh, s, causal, torch.zeros(big, dtype=torch.uint8, device=DEV), w,
                 fa.FA_BWD_ALL, layout, None, dr)
    torch.cuda.synchronize()
    for a, b, c in zip(outs[0], outs[1], g):
        assert torch.equal(a, b), "run to run (all-ones workspace)"
        assert torch.equal(a, c), "stages as separate calls"
    for a, b in zip(g2, g2_fresh):
        assert torch.equal(a, b), "a second call on the same workspace"
    args = [to_bhsd64(inp[x], layout) for x in ("q", "k", "v", "do")]
    refs = attention_bwd64(*args, s, causal, window=w, dropout=dr)
    for tag, g in (("split", outs[0]), ("unsplit dK/dV", outs[2])):
        for nm, x, r in zip(("dq", "dk", "dv"), g, refs):
            got = to_bhsd64(x.cpu(), layout)
            assert np.isfinite(got).all(), (tag, nm)
            rel = np.linalg.norm(got - r) / max(np.linalg.norm(r), 1e-30)
            say("  %s %s rel-F err %.3e" % (tag, nm, rel))
            assert rel <= TOL_GRAD, (tag, nm)
