"""Replays of one captured HIP graph that holds the split and fp8 paths equal
their eager results bit for bit, replay after replay.

The shape, B1 H2 N4096 d128 causal, leaves most CUs idle (64 forward query
blocks, 44 dK/dV key blocks), so every call takes its split form: the key
chunks and merge of ``fa_fwd_splitk``, the intra-workgroup key split of
``fa_fwd_ex`` (here with dropout), the dK/dV partials and their reduction
in ``fa_bwd_ex`` with dQ forked onto the side stream, and the fp8 forward
(the test asserts that the forward's chunk plan and the backward's
workspace plan split this shape).
All four go into one graph.  Before each replay the program fills every
output with a different value and runs the same calls eagerly on buffers
of its own; after it, every output must equal the first eager run.  The
workspaces are reused by every replay, so partial sums or flags left from
an earlier replay would show.
"""
import math
import sys

import torch

import pytest

import exact_io_aware_02_amd as fa
from attn_inputs import make_qkv

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


class Calls:
    """Outputs and workspaces of the four calls; ``run`` issues them on the
    current stream."""

    def __init__(self, q, k, v, do, q8, k8, v8, s, drop):
        B, H, N, d = q.shape
        self.inp = (q, k, v, do, q8, k8, v8, s, drop)
        self.o1, self.o2 = torch.empty_like(q), torch.empty_like(q)
        self.o3 = torch.empty(q.shape, dtype=torch.bfloat16, device=DEV)
        self.l1, self.l2, self.l3 = (torch.empty((B, H, N), dtype=torch.float32, device=DEV) for _ in range(3))
        self.g = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
        nf = fa.fa_fwd_splitk_workspace_bytes(B, H, N, N, d, True)
        assert nf > 0  # the plan splits this shape
        self.fws = torch.empty(nf, dtype=torch.uint8, device=DEV)
        nb = fa.fa_bwd_ex_workspace_bytes(B, H, H, N, N, d, fa.FA_BF16)
        assert nb > fa.fa_bwd_workspace_bytes(B, H, N, N, d, fa.FA_BF16)  # room for the dK/dV partials
        self.bws = torch.empty(nb, dtype=torch.uint8, device=DEV)

    def outputs(self):
        return [self.o1, self.l1, self.o2, self.l2, self.o3, self.l3] + self.g

    def run(self):
        q, k, v, do, q8, k8, v8, s, drop = self.inp
        fa.fa_fwd_splitk(q, k, v, self.o1, self.l1, s, True, self.fws)
        fa.fa_fwd_ex(q, k, v, self.o2, self.l2, s, True, dropout=drop)
        fa.fa_bwd_ex(q, k, v, self.o1, self.l1, do, *self.g, s, True, self.bws)
        fa.fa_fwd_fp8(q8, k8, v8, self.o3, self.l3, s, True)


def test_split_paths_in_one_graph():
    B, H, N, d = 1, 2, 4096, 128
    say("case graph replay of the split paths: B%d H%d N%d d%d causal" % (B, H, N, d))
    inp = make_qkv(B, H, N, N, d, "bf16", seed=61, in_scale=0.5, with_do=True)
    q, k, v, do = (inp[x].to(DEV) for x in ("q", "k", "v", "do"))
    q8, k8, v8 = (inp[x].to(torch.float8_e4m3fn).to(DEV) for x in ("q", "k", "v"))
    s = 1.0 / math.sqrt(d)
    drop = (0.1, (9 << 32) + 3, 11)

    ref = Calls(q, k, v, do, q8, k8, v8, s, drop)
    ref.run()
    torch.cuda.synchronize()
    want = [t.clone() for t in ref.outputs()]
    assert all(torch.isfinite(t.float()).all() for t in want)

    cap = Calls(q, k, v, do, q8, k8, v8, s, drop)
    cap.run()  # first use of every path (and of the side stream) outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap.run()
    other = Calls(q, k, v, do, q8, k8, v8, s, drop)
    for r in range(4):
        for t in cap.outputs():
            t.fill_(float(r + 2))
        other.run()  # the program's own eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(cap.outputs(), want)):
            assert torch.equal(a, b), "replay %d output %d" % (r, i)
        for i, (a, b) in enumerate(zip(other.outputs(), want)):
            assert torch.equal(a, b), "eager run %d output %d" % (r, i)
    say("  4 replays and 4 eager runs bitwise equal to the first eager run")
