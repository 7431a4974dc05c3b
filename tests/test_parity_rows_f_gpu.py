"""GPU parity of the benchmark's 16K rows, in the launches ``bench.py`` times.

The 16K causal d=128 bf16 inputs (B1 H16 N16384, inputs x0.5) with, as in
the benchmark's ``rows_f`` and its main step: the plain causal case, 16
query heads on the first 2 K/V heads, a causal window (256, 256), and
dropout p = 0.1.  Forward through ``fa_fwd_splitk`` with its workspace, the
backward through ``fa_bwd_ex`` with the workspace that lets dK/dV split.
Checked against the fp64 oracle on 128 seeded query rows per head (rows 0
and N-1 always): O and LSE, and dQ of those rows (``attention_rows_dq64``;
a query row's gradient needs only its own softmax row).  dK and dV, whose
rows need every query, are checked through identities that hold at any
size: sum_j dK_j = 0 per K/V head (the rows of dS sum to zero, with
dropout too), without dropout sum_j dV_j = the sum of dO over the
query heads and rows that use the K/V head (the rows of P sum to one),
and in every case sum_j k_j dK_j^T = sum_i dQ_i q_i^T and sum_j v_j dV_j^T
= sum_i O_i dO_i^T over those query heads (``grad_identities``).
"""
import math
import sys

import numpy as np
import pytest
import torch

import exact_io_aware_02_amd as fa
from attn_inputs import WORKLOADS, sample_rows, to_bhsd64, workload_inputs
from grad_identities import identity_errors
from oracle import attention_rows_dq64, attention_rows_fwd64, dropout_threshold

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL_O = 1.6e-2   # bf16
TOL_LSE = 1e-3
TOL_GRAD = 2e-2  # relative Frobenius, here over the sampled rows' dQ
TOL_IDENT = 1e-2  # the d x d gradient identities: ~4x what bf16 rounding of exact outputs gives
ROWS = 128

CASES = [
    # name, K/V heads, window, dropout
    ("causal", 16, (-1, -1), None),
    ("gqa_16_on_2", 2, (-1, -1), None),
    ("window_256_256", 16, (256, 256), None),
    ("dropout_0.1", 16, (-1, -1), (0.1, 2024, 0)),
]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def inputs16k():
    w = WORKLOADS["fwd_causal_b1h16_n16384_d128_bf16_bhsd"]
    inp = workload_inputs(w)
    rng = np.random.default_rng(w.seed + 3000)
    do = torch.from_numpy(rng.standard_normal(inp["q"].shape, dtype=np.float32)).to(torch.bfloat16)
    rows = sample_rows(w.B, w.H, w.N, ROWS, w.seed + 4000)
    return w, inp, do, rows


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bench_rows_at_16k(inputs16k, case):
    name, hkv, window, dropout = case
    w, inp, do_cpu, rows = inputs16k
    B, H, N, d = w.B, w.H, w.N, w.d
    s = 1.0 / math.sqrt(d)
    say("case 16K %s" % name)
    q = inp["q"].to(DEV)
    k = inp["k"][:, :hkv].contiguous().to(DEV)
    v = inp["v"][:, :hkv].contiguous().to(DEV)
    do = do_cpu.to(DEV)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    nf = fa.fa_fwd_splitk_workspace_bytes(B, H, N, N, d, True, window)
    fws = torch.empty(nf, dtype=torch.uint8, device=DEV) if nf else None
    fa.fa_fwd_splitk(q, k, v, o, lse, s, True, fws, window, "bhsd", None, dropout)
    g = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    ws = torch.empty(fa.fa_bwd_ex_workspace_bytes(B, H, hkv, N, N, d, fa.FA_BF16), dtype=torch.uint8, device=DEV)
    fa.fa_bwd_ex(q, k, v, o, lse, do, *g, s, True, ws, window, fa.FA_BWD_ALL, "bhsd", None, dropout)
    torch.cuda.synchronize()

    qc, kc, vc = (to_bhsd64(x) for x in (inp["q"], inp["k"][:, :hkv], inp["v"][:, :hkv]))
    doc = to_bhsd64(do_cpu)
    ro, rl = attention_rows_fwd64(qc, kc, vc, s, True, rows, window=window, dropout=dropout)
    rq = attention_rows_dq64(qc, kc, vc, doc, s, True, rows, window=window, dropout=dropout)
    pick = lambda a: np.stack([np.stack([a[b, h][rows[b, h]] for h in range(H)]) for b in range(B)])  # noqa: E731
    og, lg, dqg = to_bhsd64(o.cpu()), lse.cpu().numpy().astype(np.float64), to_bhsd64(g[0].cpu())
    assert np.isfinite(og).all() and np.isfinite(lg).all() and np.isfinite(dqg).all()
    keep = dropout_threshold(dropout[0])[1] if dropout else 1.0
    err_o = np.abs(pick(og) - ro).max()
    err_l = np.abs(pick(lg) - rl).max()
    rel_q = np.linalg.norm(pick(dqg) - rq) / np.linalg.norm(rq)
    say("  %d rows/head: O max-abs %.3e (tol %.2e), LSE %.3e, dQ rel-F %.3e" % (ROWS, err_o, TOL_O * keep, err_l, rel_q))
    assert err_o <= TOL_O * keep and err_l <= TOL_LSE and rel_q <= TOL_GRAD

    gk, gv = to_bhsd64(g[1].cpu()), to_bhsd64(g[2].cpu())
    assert np.isfinite(gk).all() and np.isfinite(gv).all()
    rel_k = np.abs(gk.sum(axis=2)).max() / np.abs(gk).sum(axis=2).max()
    say("  |sum_j dK_j| / sum_j |dK_j| = %.2e" % rel_k)
    assert rel_k < TOL_GRAD
    if dropout is None:
        G = H // hkv
        sum_do = doc.reshape(B, hkv, G, N, d).sum(axis=(2, 3))
        rel_v = np.abs(gv.sum(axis=2) - sum_do).max() / np.abs(sum_do).max()
        say("  sum_j dV_j vs sum dO: rel %.2e" % rel_v)
        assert rel_v < TOL_GRAD
    err = identity_errors(qc, kc, vc, doc, og, dqg, gk, gv)
    say("  K^T dK vs dQ^T Q %.2e, V^T dV vs O^T dO %.2e" % (err["dk"], err["dv"]))
    assert err["dk"] <= TOL_IDENT and err["dv"] <= TOL_IDENT
