"""GPU parity of the fp8 (e4m3fn) forward (fa_fwd_fp8) against the fp64 oracle.

The kernel rounds the attention weights to e4m3fn for the P V product, so O
is compared with the exact attention of the decoded inputs under the
tolerance that rounding implies (oracle ``fp8_rounding_model``):

* every element within the rigorous bound, and
* the mean of (error / model standard deviation)^2 at most 1.5 (the model
  is an upper bound in expectation; wrong keys, values or rounding push it
  far higher).

LSE uses the 16-bit path's tolerance (1e-3): the scores are exact fp8
products accumulated in fp32.  A second family of cases has integer scores
and scale ln 2, so every weight is a power of two that e4m3fn holds exactly;
there O must match the oracle to bf16 rounding (2^-8 relative).
"""
import math
import sys

import numpy as np
import pytest
import torch

import exact_io_aware_02_amd as fa
from attn_inputs import fp8_bytes, make_qkv, sample_rows, to_bhsd64
from oracle import attention_fp8_fwd64, attention_fp8_rows_fwd64, fp8_rounding_model

pytestmark = pytest.mark.gpu

TOL_LSE = 1e-3
TOL_Z2 = 1.5
DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def check(name, got_o, got_l, o_ref, lse_ref, bound, sigma):
    live = np.isfinite(lse_ref)
    assert np.isfinite(got_o).all()
    np.testing.assert_array_equal(np.isneginf(got_l), ~live)
    err = got_o - o_ref
    ratio = np.abs(err) / np.where(bound > 0, bound, 1e-30)
    livem = np.broadcast_to(live[..., None], err.shape)
    # sigma = 0 where nothing can round (one admitted key whose value is 0)
    flat = livem & (sigma == 0)
    assert np.all(err[flat] == 0.0)
    sm = livem & (sigma > 0)
    z2 = np.mean((err[sm] / sigma[sm]) ** 2) if sm.any() else 0.0
    err_l = np.abs(got_l[live] - lse_ref[live]).max() if live.any() else 0.0
    say("  %s: O max-abs %.3e, max err/bound %.3f, mean z^2 %.3f; LSE max-abs %.3e"
        % (name, np.abs(err).max(), ratio.max(), z2, err_l))
    assert np.all(got_o[~livem] == 0.0)
    assert ratio.max() <= 1.0
    assert z2 <= TOL_Z2
    assert err_l <= TOL_LSE


CASES = [
    # name, B, H, Hkv, Nq, Nk, d, layout, causal, window, descale, scale
    ("d64", 1, 2, 2, 256, 256, 64, "bhsd", False, None, (1.0, 1.0, 1.0), None),
    ("d128_causal", 1, 4, 4, 333, 333, 128, "bhsd", True, None, (1.0, 1.0, 1.0), None),
    ("ragged_bshd", 2, 4, 4, 200, 300, 64, "bshd", False, None, (1.0, 1.0, 1.0), None),
    ("gqa_causal_d128", 1, 8, 2, 257, 257, 128, "bhsd", True, None, (1.0, 1.0, 1.0), None),
    ("mqa_window", 1, 4, 1, 400, 400, 64, "bhsd", False, (64, 32), (1.0, 1.0, 1.0), None),
    ("win_causal_d128_bshd", 1, 2, 2, 700, 700, 128, "bshd", True, (100, -1), (1.0, 1.0, 1.0), None),
    ("empty_rows_window", 1, 2, 2, 300, 100, 64, "bhsd", False, (10, 10), (1.0, 1.0, 1.0), None),
    ("descales_negative_product", 1, 2, 2, 190, 190, 128, "bhsd", False, None, (0.5, -2.0, 3.0), None),
    ("large_scale_rescales", 1, 2, 2, 320, 320, 64, "bhsd", True, None, (1.0, 1.0, 1.0), 1.5),
    ("one_key", 1, 2, 2, 5, 1, 64, "bhsd", False, None, (1.0, 1.0, 1.0), None),
    ("one_tile", 1, 2, 1, 64, 64, 128, "bhsd", True, None, (1.0, 1.0, 0.5), None),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fp8_fwd_matches_oracle(case):
    name, B, H, Hkv, Nq, Nk, d, layout, causal, window, descale, scale = case
    say("case %s" % name)
    inp = make_qkv(B, H, Nq, Nk, d, "fp8", layout, seed=88, Hkv=Hkv)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    q, k, v = (inp[x].to(DEV) for x in ("q", "k", "v"))
    o, lse = fa.attention_fwd_fp8(q, k, v, causal=causal, scale=scale, layout=layout, window=window,
                                  descale=descale)
    torch.cuda.synchronize()
    w = window if window is not None else (-1, -1)
    q8, k8, v8 = (fp8_bytes(inp[x], layout) for x in ("q", "k", "v"))
    o_ref, lse_ref = attention_fp8_fwd64(q8, k8, v8, scale, causal, window=w, descale=descale)
    rows = np.tile(np.arange(Nq), (B, H, 1))
    bound, sigma = fp8_rounding_model(q8, k8, v8, scale, causal, rows, window=w, descale=descale)
    check(name, to_bhsd64(o.cpu(), layout), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref, bound, sigma)


def integer_score_inputs(B, H, Hkv, Nq, Nk, d, seed):
    """q rows with four entries of +-1, k entries in {-1, 0, 1}: every score
    q.k is an integer in [-4, 4]; v random e4m3fn."""
    rng = np.random.default_rng(seed)
    q = np.zeros((B, H, Nq, d), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            for i in range(Nq):
                pos = rng.choice(d, size=4, replace=False)
                q[b, h, i, pos] = rng.choice([-1.0, 1.0], size=4)
    k = rng.choice(np.array([-1.0, 0.0, 0.0, 1.0], dtype=np.float32), size=(B, Hkv, Nk, d))
    v = rng.standard_normal((B, Hkv, Nk, d), dtype=np.float32)
    return [torch.from_numpy(x).to(torch.float8_e4m3fn) for x in (q, k, v)]


@pytest.mark.parametrize("d,causal,Hkv", [(64, False, 2), (128, True, 2), (128, False, 1), (64, True, 4)])
def test_fp8_fwd_exact_weights(d, causal, Hkv):
    """scale * q_descale * k_descale = ln 2 makes each weight 2^(n - m) with
    integers n, m in [-4, 4]: exact in e4m3fn, so only fp32 accumulation and
    the bf16 output round."""
    B, H, Nq, Nk = 1, 4, 320, 333
    say("case exact_weights d=%d causal=%d Hkv=%d" % (d, causal, Hkv))
    q, k, v = integer_score_inputs(B, H, Hkv, Nq, Nk, d, seed=d + Hkv)
    descale = (0.5, 4.0, 1.0)
    scale = math.log(2.0) / (descale[0] * descale[1])
    o, lse = fa.attention_fwd_fp8(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale, descale=descale)
    torch.cuda.synchronize()
    q8, k8, v8 = (fp8_bytes(x) for x in (q, k, v))
    o_ref, lse_ref = attention_fp8_fwd64(q8, k8, v8, scale, causal, descale=descale)
    got = o.cpu().to(torch.float64).numpy()
    err = np.abs(got - o_ref)
    tol = 2.0 ** -8 * np.abs(o_ref) + 1e-4
    say("  O max err/tol %.3f, LSE max-abs %.3e" % ((err / tol).max(), np.abs(lse.cpu().numpy() - lse_ref).max()))
    assert np.all(err <= tol)
    assert np.abs(lse.cpu().numpy() - lse_ref).max() <= TOL_LSE


def test_fp8_fwd_16k_causal_sampled_rows():
    """The 16K-token causal d=128 shape (B=1, H=16, inputs 0.5 N(0,1) cast to
    e4m3fn) in the launch the benchmark times, checked on 256 seeded rows
    of every head (rows 0 and N-1 always)."""
    B, H, N, d = 1, 16, 16384, 128
    say("case fp8_16k_causal (sampled rows)")
    inp = make_qkv(B, H, N, N, d, "fp8", "bhsd", seed=3, in_scale=0.5)
    q, k, v = (inp[x].to(DEV) for x in ("q", "k", "v"))
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.attention_fwd_fp8(q, k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    rows = sample_rows(B, H, N, 256, seed=5)
    q8, k8, v8 = (fp8_bytes(inp[x]) for x in ("q", "k", "v"))
    o_ref, lse_ref = attention_fp8_rows_fwd64(q8, k8, v8, scale, True, rows)
    bound, sigma = fp8_rounding_model(q8, k8, v8, scale, True, rows)
    got_o = o.cpu().to(torch.float64).numpy()
    got_l = lse.cpu().numpy().astype(np.float64)
    go = np.stack([np.stack([got_o[0, h][rows[0, h]] for h in range(H)])])
    gl = np.stack([np.stack([got_l[0, h][rows[0, h]] for h in range(H)])])
    check("16k", go, gl, o_ref, lse_ref, bound, sigma)


LONG_CASES = [
    # name, H, Hkv, N, d, layout, causal, window, descale
    ("n131072_d128_causal", 1, 1, 131072, 128, "bhsd", True, None, (1.0, 1.0, 1.0)),
    ("n65536_d64_mqa_window_bshd_descales", 4, 1, 65536, 64, "bshd", False, (3000, 100), (0.5, 2.0, 1.5)),
]


@pytest.mark.parametrize("case", LONG_CASES, ids=[c[0] for c in LONG_CASES])
def test_fp8_fwd_long_rows(case):
    """Long rows (up to 2048 key tiles of 64 in the heaviest block), checked
    on 128 seeded rows per head under the rounding model (its fp32
    accumulation term grows with Nk)."""
    name, H, Hkv, N, d, layout, causal, window, descale = case
    say("case fp8 long rows %s" % name)
    inp = make_qkv(1, H, N, N, d, "fp8", layout, seed=91, in_scale=0.5, Hkv=Hkv)
    q, k, v = (inp[x].to(DEV) for x in ("q", "k", "v"))
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.attention_fwd_fp8(q, k, v, causal=causal, scale=scale, layout=layout, window=window,
                                  descale=descale)
    torch.cuda.synchronize()
    w = window if window is not None else (-1, -1)
    rows = sample_rows(1, H, N, 128, seed=92)
    q8, k8, v8 = (fp8_bytes(inp[x], layout) for x in ("q", "k", "v"))
    o_ref, lse_ref = attention_fp8_rows_fwd64(q8, k8, v8, scale, causal, rows, window=w, descale=descale)
    bound, sigma = fp8_rounding_model(q8, k8, v8, scale, causal, rows, window=w, descale=descale)
    got_o = to_bhsd64(o.cpu(), layout)
    got_l = lse.cpu().numpy().astype(np.float64)
    go = np.stack([np.stack([got_o[0, h][rows[0, h]] for h in range(H)])])
    gl = np.stack([np.stack([got_l[0, h][rows[0, h]] for h in range(H)])])
    check(name, go, gl, o_ref, lse_ref, bound, sigma)


def test_fp8_fwd_gqa_equals_repeated_heads():
    """Sharing a K/V head gives bit-for-bit the result of repeating it."""
    say("case fp8_gqa_vs_repeat")
    inp = make_qkv(1, 8, 300, 300, 128, "fp8", "bhsd", seed=9, Hkv=2)
    q, k, v = (inp[x].to(DEV) for x in ("q", "k", "v"))
    o1, l1 = fa.attention_fwd_fp8(q, k, v, causal=True)
    kr = k.view(torch.uint8).repeat_interleave(4, dim=1).view(torch.float8_e4m3fn)
    vr = v.view(torch.uint8).repeat_interleave(4, dim=1).view(torch.float8_e4m3fn)
    o2, l2 = fa.attention_fwd_fp8(q, kr, vr, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


PHASED_CASES = [
    # name, B, H, Hkv, Nq, Nk, d, layout, causal, window, descale
    ("d128_causal", 1, 2, 2, 333, 333, 128, "bhsd", True, None, (1.0, 1.0, 1.0)),
    ("d64_gqa_window_bshd", 2, 4, 2, 300, 300, 64, "bshd", True, (100, -1), (0.5, -2.0, 3.0)),
    ("d128_ragged_empty_rows", 1, 2, 1, 300, 100, 128, "bhsd", False, (10, 10), (1.0, 1.0, 1.0)),
]


@pytest.mark.parametrize("case", PHASED_CASES, ids=[c[0] for c in PHASED_CASES])
def test_fp8_fwd_phased_schedule(case):
    """From 768 (d = 128) or 1536 (d = 64) workgroups of 128 queries the
    fp8 forward runs its phased schedule: a small case repeated along the batch to that size, the first
    copy against the oracle and every copy bitwise equal to it."""
    name, B, H, Hkv, Nq, Nk, d, layout, causal, window, descale = case
    R = math.ceil({64: 1536, 128: 768}[d] / (math.ceil(Nq / 128) * B * H))
    say("case phased %s (%d copies)" % (name, R))
    inp = make_qkv(B, H, Nq, Nk, d, "fp8", layout, seed=71, Hkv=Hkv)
    rep = {x: inp[x].view(torch.uint8).repeat(R, 1, 1, 1).view(torch.float8_e4m3fn) for x in ("q", "k", "v")}
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.attention_fwd_fp8(*(rep[x].to(DEV) for x in ("q", "k", "v")), causal=causal, scale=scale,
                                  layout=layout, window=window, descale=descale)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    w = window if window is not None else (-1, -1)
    q8, k8, v8 = (fp8_bytes(inp[x], layout) for x in ("q", "k", "v"))
    o_ref, lse_ref = attention_fp8_fwd64(q8, k8, v8, scale, causal, window=w, descale=descale)
    rows = np.tile(np.arange(Nq), (B, H, 1))
    bound, sigma = fp8_rounding_model(q8, k8, v8, scale, causal, rows, window=w, descale=descale)
    check(name, to_bhsd64(o[:B], layout), lse[:B].numpy().astype(np.float64), o_ref, lse_ref, bound, sigma)
    for r in range(1, R):
        assert torch.equal(o[r * B:(r + 1) * B].view(torch.int16), o[:B].view(torch.int16)), r
        assert torch.equal(lse[r * B:(r + 1) * B], lse[:B]), r


@pytest.mark.parametrize("shape", ["interleaved", "phased"])
@pytest.mark.parametrize("d", [64, 128])
def test_fp8_rising_scores(d, shape):
    """Keys scaled by 1 + 3 j / N along the sequence (then rounded to
    e4m3fn, the bytes both sides get) and a scale of 2 / sqrt(d): under the
    causal mask a row's running maximum rises on almost every 64-key tile,
    so the lazy rescale's slow path runs in both schedules (the phased one
    from 768 / 1536 workgroups, reached by copies along the batch); against
    the oracle under the rounding model, copies bitwise equal."""
    B, H, N = 1, 2, 320
    blocks = math.ceil(N / 128) * B * H
    R = 1 if shape == "interleaved" else math.ceil({64: 1536, 128: 768}[d] / blocks)
    say("case fp8 rising scores d=%d %s (%d copies)" % (d, shape, R))
    inp = make_qkv(B, H, N, N, d, "fp8", "bhsd", seed=97)
    ramp = 1.0 + 3.0 * torch.arange(N, dtype=torch.float32) / N
    k = (inp["k"].float() * ramp[None, None, :, None]).to(torch.float8_e4m3fn)
    q, v = inp["q"], inp["v"]
    rep = [x.view(torch.uint8).repeat(R, 1, 1, 1).view(torch.float8_e4m3fn).to(DEV) for x in (q, k, v)]
    scale = 2.0 / math.sqrt(d)
    o, lse = fa.attention_fwd_fp8(*rep, causal=True, scale=scale)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    q8, k8, v8 = (fp8_bytes(x) for x in (q, k, v))
    o_ref, lse_ref = attention_fp8_fwd64(q8, k8, v8, scale, True)
    rows = np.tile(np.arange(N), (B, H, 1))
    bound, sigma = fp8_rounding_model(q8, k8, v8, scale, True, rows)
    check("rising d%d %s" % (d, shape), to_bhsd64(o[:B]), lse[:B].numpy().astype(np.float64), o_ref, lse_ref,
          bound, sigma)
    for r in range(1, R):
        assert torch.equal(o[r * B:(r + 1) * B].view(torch.int16), o[:B].view(torch.int16)), r
        assert torch.equal(lse[r * B:(r + 1) * B], lse[:B]), r


def draw_fp8(i):
    rng = np.random.default_rng(7000 + i)
    d = int(rng.choice([64, 128]))
    B, H = int(rng.choice([1, 2])), int(rng.choice([1, 2, 3, 4, 6]))
    Hkv = int(rng.choice([g for g in range(1, H + 1) if H % g == 0]))
    Nq, Nk = (int(x) for x in rng.integers(1, 600, size=2))
    window = None
    if rng.random() < 0.4:
        window = tuple(int(rng.choice([-1, int(rng.integers(0, max(Nk, 2)))])) for _ in range(2))
    descale = tuple(float(rng.choice([-1.0, 1.0, 1.0, 1.0]) * 2.0 ** rng.uniform(-2, 2)) for _ in range(3))
    scale = float(rng.uniform(0.5, 1.5)) / math.sqrt(d)
    return dict(B=B, H=H, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d, layout=str(rng.choice(["bhsd", "bhsd", "bshd"])),
                causal=bool(rng.random() < 0.5), window=window, descale=descale, scale=scale,
                seed=int(rng.integers(0, 2 ** 31)))


@pytest.mark.parametrize("i", range(20))
def test_fp8_random_case(i):
    """Seeded random combinations of the fp8 forward's options at once
    (heads and K/V heads, ragged Nq and Nk, d, layout, causal, random window
    edges, descale factors of either sign between 1/4 and 4, the scale),
    each printed before it runs; against the oracle under the rounding
    model, LSE within 1e-3."""
    c = draw_fp8(i)
    say("case fp8 random %d: %s" % (i, c))
    B, H, Hkv, Nq, Nk, d, layout = c["B"], c["H"], c["Hkv"], c["Nq"], c["Nk"], c["d"], c["layout"]
    inp = make_qkv(B, H, Nq, Nk, d, "fp8", layout, seed=c["seed"], Hkv=Hkv)
    q, k, v = (inp[x].to(DEV) for x in ("q", "k", "v"))
    o, lse = fa.attention_fwd_fp8(q, k, v, causal=c["causal"], scale=c["scale"], layout=layout,
                                  window=c["window"], descale=c["descale"])
    torch.cuda.synchronize()
    w = c["window"] if c["window"] is not None else (-1, -1)
    q8, k8, v8 = (fp8_bytes(inp[x], layout) for x in ("q", "k", "v"))
    o_ref, lse_ref = attention_fp8_fwd64(q8, k8, v8, c["scale"], c["causal"], window=w, descale=c["descale"])
    rows = np.tile(np.arange(Nq), (B, H, 1))
    bound, sigma = fp8_rounding_model(q8, k8, v8, c["scale"], c["causal"], rows, window=w, descale=c["descale"])
    check("random %d" % i, to_bhsd64(o.cpu(), layout), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref,
          bound, sigma)
