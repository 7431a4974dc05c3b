"""fa_bwd_noalloc (the backward for callers that cannot allocate) against
fa_bwd through the C ABI.

Both run the same kernels in the same order, so their gradients must agree
bit for bit.  Two calls in a row, the second smaller, so the second runs on
the scratch the first left behind; then a call at the scratch's size limit,
one just past it (rejected before anything is enqueued), and one more
small call.
"""
import math
import sys

import pytest
import torch

import exact_io_aware_02_amd as fa
from attn_inputs import make_qkv

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _case(B, H, N, d, dt, causal, seed):
    say("case noalloc B%d H%d N%d d%d %s causal=%s" % (B, H, N, d, dt, causal))
    inp = make_qkv(B, H, N, N, d, dt, "bhsd", seed=seed, with_do=True)
    q, k, v, do = (inp[x].to(DEV) for x in ("q", "k", "v", "do"))
    s = 1.0 / math.sqrt(d)
    o, lse = fa.attention_fwd(q, k, v, causal=causal, scale=s)
    # fa_bwd with the workspace of fa_bwd_workspace_bytes, the size the
    # scratch array stands in for
    code = fa.FA_FP16 if dt == "fp16" else fa.FA_BF16
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, N, d, code), dtype=torch.uint8, device=DEV)
    ref = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    fa.fa_bwd(q, k, v, o, lse, do, *ref, s, causal, ws)
    got = [torch.full_like(q, 7.0), torch.full_like(k, 7.0), torch.full_like(v, 7.0)]
    fa.fa_bwd_noalloc(q, k, v, o, lse, do, *got, s, causal)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a, b), name
    return q, k, v, o, lse, do


def test_noalloc_matches_fa_bwd_twice_then_smaller():
    _case(2, 8, 1024, 64, "fp16", True, 61)
    _case(1, 2, 300, 128, "bf16", False, 62)


def test_noalloc_limit_and_rejection():
    rows_max = fa.FA_BWD_NOALLOC_SCRATCH_BYTES // 8  # B * H * round_up(Nq, 64)
    H = rows_max // 16384
    _case(1, H, 16384, 64, "fp16", True, 63)  # exactly the limit
    # one 64-row block more than the scratch holds: rejected on the host
    q = torch.zeros(1, H, 16384 + 1, 64, dtype=torch.float16, device=DEV)
    lse = torch.zeros(1, H, 16384 + 1, dtype=torch.float32, device=DEV)
    with pytest.raises(fa.FaError) as e:
        fa.fa_bwd_noalloc(q, q, q, q, lse, q, torch.empty_like(q), torch.empty_like(q), torch.empty_like(q), 0.125,
                          True)
    assert e.value.status == fa.FA_ERR_INVALID_ARG and "scratch" in str(e.value)
    del q, lse
    _case(1, 3, 200, 64, "bf16", True, 64)  # a valid call after the rejected one
