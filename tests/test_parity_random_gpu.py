"""GPU parity on seeded random combinations of every option, forward and
backward, against the fp64 oracle.

The structured tests change one or two options at a time; here each case
draws all of them at once from its own seed (printed before it runs):
batch and heads with a dividing number of K/V heads, ragged Nq and Nk
(every tenth case a long row of 4200 keys, which takes the split paths),
d, dtype, layout, causal, a window with random edges (rows that admit no
key included), dropout with 64-bit seeds (short rows only), the scale (times 0.5-2,
sometimes negative), the forward route (``fa_fwd_splitk``'s key chunks or
``fa_fwd_ex``) and the backward workspace (statistics only, or the size
that lets dK/dV split).  Tolerances as elsewhere: gradients 2e-2 relative
Frobenius, LSE 1e-3, O the absolute bound times the dropout scale plus
O's own rounding to the output type (reading 18: larger scales concentrate
the weights).
"""
import math
import sys

import numpy as np
import pytest
import torch

import exact_io_aware_02_amd as fa
from attn_inputs import make_qkv, to_bhsd64
from oracle import attention_bwd64, attention_fwd64, dropout_threshold

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL_O = {"fp16": 2e-3, "bf16": 1.6e-2}
UNIT = {"fp16": 2.0 ** -11, "bf16": 2.0 ** -8}
TOL_LSE = 1e-3
TOL_GRAD = 2e-2
N_CASES = 40


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def draw(i):
    rng = np.random.default_rng(5000 + i)
    long_row = i % 10 == 7
    d = int(rng.choice([64, 128]))
    if long_row:
        B, H, Nq = 1, int(rng.choice([1, 2])), 4200
        Nk = Nq
    else:
        B, H = int(rng.choice([1, 2])), int(rng.choice([1, 2, 3, 4, 6, 8]))
        Nq, Nk = (int(x) for x in rng.integers(1, 700, size=2))
        if rng.random() < 0.4:
            Nk = Nq
    Hkv = int(rng.choice([g for g in range(1, H + 1) if H % g == 0]))
    window = None
    if rng.random() < 0.4:
        window = tuple(int(rng.choice([-1, int(rng.integers(0, max(Nk, 2)))])) for _ in range(2))
    dropout = None
    if rng.random() < 0.25:
        dropout = (float(rng.choice([0.1, 0.25, 0.5])), int(rng.integers(0, 2 ** 63)), int(rng.integers(0, 2 ** 31)))
    if long_row:  # (the oracle's mask for 4200^2 weights costs tens of seconds; long rows with dropout are
        dropout = None  # covered by the split and 16K tests)
    scale = float(rng.uniform(0.5, 2.0)) / math.sqrt(d) * (-1.0 if rng.random() < 0.1 else 1.0)
    return dict(B=B, H=H, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d, dt=str(rng.choice(["fp16", "bf16"])),
                layout=str(rng.choice(["bhsd", "bhsd", "bshd"])), causal=bool(rng.random() < 0.5), window=window,
                dropout=dropout, scale=scale, splitk=bool(rng.random() < 0.5), big_ws=bool(rng.random() < 0.5),
                seed=int(rng.integers(0, 2 ** 31)))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    c = draw(i)
    say("case random %d: %s" % (i, c))
    B, H, Hkv, Nq, Nk, d, dt, layout = c["B"], c["H"], c["Hkv"], c["Nq"], c["Nk"], c["d"], c["dt"], c["layout"]
    causal, window, dropout, scale = c["causal"], c["window"], c["dropout"], c["scale"]
    inp = make_qkv(B, H, Nq, Nk, d, dt, layout, seed=c["seed"], with_do=True, Hkv=Hkv)
    q, k, v, do = (inp[x].to(DEV) for x in ("q", "k", "v", "do"))
    o, lse = fa.attention_fwd(q, k, v, causal=causal, scale=scale, layout=layout, window=window, dropout=dropout,
                              splitk=c["splitk"])
    code = fa.FA_FP16 if dt == "fp16" else fa.FA_BF16
    if c["big_ws"]:
        nbytes = fa.fa_bwd_ex_workspace_bytes(B, H, Hkv, Nq, Nk, d, code)
    else:
        nbytes = fa.fa_bwd_workspace_bytes(B, H, Nq, Nk, d, code)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=DEV)
    g = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    fa.fa_bwd_ex(q, k, v, o, lse, do, *g, scale, causal, ws, window if window else (-1, -1), fa.FA_BWD_ALL,
                 layout, None, dropout)
    torch.cuda.synchronize()

    w = window if window is not None else (-1, -1)
    args = [to_bhsd64(inp[x], layout) for x in ("q", "k", "v")]
    o_ref, lse_ref = attention_fwd64(*args, scale, causal, window=w, dropout=dropout)
    keep = dropout_threshold(dropout[0])[1] if dropout else 1.0
    got_o = to_bhsd64(o.cpu(), layout)
    got_l = lse.cpu().numpy().astype(np.float64)
    live = np.isfinite(lse_ref)
    assert np.isfinite(got_o).all()
    np.testing.assert_array_equal(np.isneginf(got_l), ~live)
    excess = np.abs(got_o - o_ref) - (TOL_O[dt] * keep + UNIT[dt] * np.abs(o_ref))
    err_l = np.abs(got_l[live] - lse_ref[live]).max() if live.any() else 0.0
    say("  O max-abs %.3e (worst excess over the bound %.2e), LSE %.3e, empty rows %d"
        % (np.abs(got_o - o_ref).max(), excess.max(), err_l, int((~live).sum())))
    assert excess.max() <= 0 and err_l <= TOL_LSE
    refs = attention_bwd64(*args, to_bhsd64(inp["do"], layout), scale, causal, window=w, dropout=dropout)
    for nm, x, r in zip(("dq", "dk", "dv"), g, refs):
        got = to_bhsd64(x.cpu(), layout)
        assert np.isfinite(got).all(), nm
        if np.linalg.norm(r) < 1e-6:  # e.g. one admitted key per row: dS = 0
            assert np.abs(got).max() < 1e-3, nm
            continue
        rel = np.linalg.norm(got - r) / np.linalg.norm(r)
        say("  %s rel-F %.3e" % (nm, rel))
        assert rel <= TOL_GRAD, nm
