"""GPU parity of the forward's launch shapes, each on the same cases:

* small (the binding's default route for grids of at most one workgroup
  per CU: fa_fwd_splitk, which for these short blocks runs fa_fwd_ex's
  kernels);
* interleaved schedule (fa_fwd_ex): grids of more than one workgroup per
  CU up to the phased threshold;
* phased schedule: from 1024 (d = 128) or 1536 (d = 64) workgroups of 128
  queries upward;
* in test_chunked_forward, fa_fwd_splitk on shapes whose plan splits
  heavy query blocks' keys over several workgroups (the partial results
  merged by a second kernel);
* and, in test_intra_split_forward, the intra-workgroup key split of
  fa_fwd_ex for grids of at most one workgroup per CU whose heaviest block
  has 32 or more key tiles: three groups of four waves per workgroup (on
  the phased schedule at d = 128, the interleaved one at d = 64), each on
  its own run of the keys, merged through LDS; at d = 64 from 128 key
  tiles on, six groups of two waves on blocks of 64 queries (phased, with
  three-slot rings).

Each case is a small problem repeated along the batch until the grid
reaches the shape's size.  The first copy is checked against the fp64 oracle
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


SPLIT_MAX_BLOCKS = 256  # CUs of the MI355X


def copies(shape, blocks, d):
    """Copies of a case along the batch that put the grid in ``shape``."""
    if shape == "small":
        return max(1, SPLIT_MAX_BLOCKS // blocks)
    if shape == "interleaved":
        R = SPLIT_MAX_BLOCKS // blocks + 1
        assert R * blocks < PHASED_MIN_BLOCKS[d]
        return R
    return math.ceil(PHASED_MIN_BLOCKS[d] / blocks)


@pytest.mark.parametrize("shape", ["small", "interleaved", "phased"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_phased_forward_matches_oracle(case, shape):
    name, B, H, Hkv, Nq, Nk, d, dt, layout, causal, window, dr = case
    blocks = math.ceil(Nq / 128) * B * H
    R = copies(shape, blocks, d)
    say("case %s %s: %d copies, %d workgroups" % (name, shape, R, R * blocks))
    inp = make_qkv(B, H, Nq, Nk, d, dt, layout, seed=61, Hkv=Hkv)
    q, k, v = (inp[x].repeat(R, 1, 1, 1).to(DEV) for x in ("q", "k", "v"))
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.attention_fwd(q, k, v, causal=causal, scale=scale, layout=layout, window=window, dropout=dr,
                              splitk=shape == "small")
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


INTRA_CASES = [
    # name, B, H, Hkv, Nq, Nk, d, dtype, layout, causal, window, dropout
    ("d128_causal", 1, 2, 2, 1100, 1100, 128, "bf16", "bhsd", True, None, None),
    ("d64_causal_bshd", 2, 3, 3, 1500, 1500, 64, "fp16", "bshd", True, None, None),
    ("d128_noncausal_rect", 1, 2, 2, 300, 1300, 128, "fp16", "bhsd", False, None, None),
    ("d64_gqa_window", 1, 4, 2, 1200, 1200, 64, "bf16", "bhsd", True, (900, -1), None),
    ("d128_window_empty_rows", 1, 2, 2, 1500, 1100, 128, "bf16", "bhsd", False, (1000, 200), None),
    ("d64_dropout", 1, 2, 2, 1100, 1100, 64, "fp16", "bhsd", True, None, (0.25, (9 << 32) + 1, 4)),
    # d = 64, 128+ key tiles: six two-wave groups on 64-query blocks
    ("d64_long_causal", 1, 2, 2, 4500, 4500, 64, "bf16", "bhsd", True, None, None),
    ("d64_long_keys_rect", 1, 2, 2, 300, 5000, 64, "bf16", "bhsd", False, None, None),
    ("d64_long_gqa_window_bshd", 1, 4, 2, 4200, 4200, 64, "fp16", "bshd", True, (4100, -1), None),
    ("d64_long_dropout", 1, 1, 1, 4300, 4300, 64, "fp16", "bhsd", True, None, (0.15, (11 << 32) + 3, 6)),
]


@pytest.mark.parametrize("case", INTRA_CASES, ids=[c[0] for c in INTRA_CASES])
def test_intra_split_forward(case):
    """fa_fwd_ex on a grid of at most 256 workgroups whose heaviest block
    has 32+ key tiles (the intra-workgroup split; some groups of the light
    blocks get no tiles): against the oracle; the same inputs through
    fa_fwd_splitk agree to within the same tolerance."""
    name, B, H, Hkv, Nq, Nk, d, dt, layout, causal, window, dr = case
    say("case intra split %s" % name)
    inp = make_qkv(B, H, Nq, Nk, d, dt, layout, seed=67, Hkv=Hkv)
    q, k, v = (inp[x].to(DEV) for x in ("q", "k", "v"))
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.attention_fwd(q, k, v, causal=causal, scale=scale, layout=layout, window=window, dropout=dr,
                              splitk=False)
    o2, lse2 = fa.attention_fwd(q, k, v, causal=causal, scale=scale, layout=layout, window=window, dropout=dr)
    o3, lse3 = fa.attention_fwd(q, k, v, causal=causal, scale=scale, layout=layout, window=window, dropout=dr,
                                splitk=False)
    torch.cuda.synchronize()
    assert torch.equal(o, o3) and torch.equal(lse, lse3), "run to run"
    w = window if window is not None else (-1, -1)
    args = [to_bhsd64(inp[x], layout) for x in ("q", "k", "v")]
    o_ref, lse_ref = attention_fwd64(*args, scale, causal, window=w, dropout=dr)
    keep = dropout_threshold(dr[0])[1] if dr else 1.0
    live = np.isfinite(lse_ref)
    for tag, oo, ll in (("intra split", o, lse), ("chunked", o2, lse2)):
        got_o = to_bhsd64(oo.cpu(), layout)
        got_l = ll.cpu().numpy().astype(np.float64)
        err_o = np.abs(got_o - o_ref).max()
        np.testing.assert_array_equal(np.isneginf(got_l), ~live)
        err_l = np.abs(got_l[live] - lse_ref[live]).max()
        say("  %s: O max-abs err %.3e, LSE %.3e" % (tag, err_o, err_l))
        assert err_o <= TOL_O[dt] * keep and err_l <= TOL_LSE, tag


CHUNK_CASES = [
    # name, B, H, Hkv, Nq, Nk, d, dtype, layout, causal, window, dropout
    ("d64_causal_4k", 1, 1, 1, 4096, 4096, 64, "fp16", "bhsd", True, None, None),
    ("d128_causal_4k", 1, 2, 2, 4096, 4096, 128, "bf16", "bhsd", True, None, None),
    ("d128_long_keys", 1, 1, 1, 256, 8192, 128, "fp16", "bhsd", False, None, None),
    ("d64_gqa_window_bshd", 1, 2, 1, 8192, 8192, 64, "bf16", "bshd", False, (6000, 300), None),
    ("d128_dropout_causal", 1, 1, 1, 6000, 6000, 128, "bf16", "bhsd", True, None, (0.2, (5 << 32) + 9, 5)),
    ("d128_window_empty_rows", 1, 2, 2, 6000, 5000, 128, "fp16", "bhsd", False, (300, 5000), None),
]


@pytest.mark.parametrize("case", CHUNK_CASES, ids=[c[0] for c in CHUNK_CASES])
def test_chunked_forward(case):
    """fa_fwd_splitk where its plan chunks the keys: against the oracle,
    bitwise repeatable, and within tolerance of fa_fwd_ex."""
    name, B, H, Hkv, Nq, Nk, d, dt, layout, causal, window, dr = case
    w = window if window is not None else (-1, -1)
    nbytes = fa.fa_fwd_splitk_workspace_bytes(B, H, Nq, Nk, d, causal, w)
    say("case chunked %s: workspace %d bytes" % (name, nbytes))
    assert nbytes > 0
    inp = make_qkv(B, H, Nq, Nk, d, dt, layout, seed=73, Hkv=Hkv)
    q, k, v = (inp[x].to(DEV) for x in ("q", "k", "v"))
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.attention_fwd(q, k, v, causal=causal, scale=scale, layout=layout, window=window, dropout=dr)
    o2, lse2 = fa.attention_fwd(q, k, v, causal=causal, scale=scale, layout=layout, window=window, dropout=dr)
    o3, lse3 = fa.attention_fwd(q, k, v, causal=causal, scale=scale, layout=layout, window=window, dropout=dr,
                                splitk=False)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "run to run"
    args = [to_bhsd64(inp[x], layout) for x in ("q", "k", "v")]
    o_ref, lse_ref = attention_fwd64(*args, scale, causal, window=w, dropout=dr)
    keep = dropout_threshold(dr[0])[1] if dr else 1.0
    live = np.isfinite(lse_ref)
    for tag, oo, ll in (("chunked", o, lse), ("fa_fwd_ex", o3, lse3)):
        got_o = to_bhsd64(oo.cpu(), layout)
        got_l = ll.cpu().numpy().astype(np.float64)
        assert np.isfinite(got_o).all(), tag
        err_o = np.abs(got_o - o_ref).max()
        np.testing.assert_array_equal(np.isneginf(got_l), ~live)
        err_l = np.abs(got_l[live] - lse_ref[live]).max()
        say("  %s: O max-abs err %.3e, LSE %.3e" % (tag, err_o, err_l))
        assert err_o <= TOL_O[dt] * keep and err_l <= TOL_LSE, tag


RISE_CASES = [("d64_fp16", 64, "fp16"), ("d128_bf16", 128, "bf16")]
RISE_SHAPES = ["small", "interleaved", "phased", "intra", "intra_long", "chunked"]


@pytest.mark.parametrize("shape", RISE_SHAPES)
@pytest.mark.parametrize("case", RISE_CASES, ids=[c[0] for c in RISE_CASES])
def test_rising_scores_every_schedule(case, shape):
    """Keys scaled by 1 + 3 j / N along the sequence and a scale of 2 / sqrt(d):
    under the causal mask a row's running maximum rises on almost every key
    tile, so the lazy rescale's slow path (and, with key splits, the merge of
    groups or chunks whose maxima differ by far) runs in every launch shape;
    against the oracle, copies along the batch bitwise equal.  The weights
    concentrate on a few keys, so |O| approaches max |V| (about 4.5) instead
    of staying near the flat-softmax values the absolute O bounds are set
    for; the bound adds O's own rounding to the output type, a unit roundoff
    (2^-8 bf16, 2^-11 fp16) times |O|."""
    name, d, dt = case
    N = {"small": 300, "interleaved": 300, "phased": 300, "intra": 1100, "intra_long": 4300, "chunked": 4096}[shape]
    B, H = 1, ({64: 1, 128: 2}[d] if shape == "chunked" else 2)
    blocks = math.ceil(N / 128) * B * H
    R = copies(shape, blocks, d) if shape in ("small", "interleaved", "phased") else 1
    say("case rising scores %s %s: %d copies, %d workgroups" % (name, shape, R, R * blocks))
    inp = make_qkv(B, H, N, N, d, dt, "bhsd", seed=89)
    ramp = 1.0 + 3.0 * torch.arange(N, dtype=torch.float32) / N
    q, v = inp["q"], inp["v"]
    k = (inp["k"].float() * ramp[None, None, :, None]).to(inp["k"].dtype)  # the bits both sides get
    scale = 2.0 / math.sqrt(d)
    if shape == "chunked":
        assert fa.fa_fwd_splitk_workspace_bytes(B, H, N, N, d, True, (-1, -1)) > 0
    qg, kg, vg = (x.repeat(R, 1, 1, 1).to(DEV) for x in (q, k, v))
    o, lse = fa.attention_fwd(qg, kg, vg, causal=True, scale=scale, splitk=shape in ("small", "chunked"))
    # (intra_long: at d = 64 the six two-wave groups on 64-query blocks)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    o_ref, lse_ref = attention_fwd64(*(to_bhsd64(x) for x in (q, k, v)), scale, True)
    got_o = to_bhsd64(o[:B])
    got_l = lse[:B].numpy().astype(np.float64)
    assert np.isfinite(got_o).all() and np.isfinite(got_l).all()
    unit = {"fp16": 2.0 ** -11, "bf16": 2.0 ** -8}[dt]
    excess = np.abs(got_o - o_ref) - (TOL_O[dt] + unit * np.abs(o_ref))
    err_l = np.abs(got_l - lse_ref).max()
    say("  O max-abs err %.3e (max |O| %.2f), worst excess over the bound %.3e; LSE %.3e (LSE up to %.1f)"
        % (np.abs(got_o - o_ref).max(), np.abs(o_ref).max(), excess.max(), err_l, lse_ref.max()))
    assert excess.max() <= 0 and err_l <= TOL_LSE
    for r in range(1, R):
        assert torch.equal(o[r * B:(r + 1) * B].view(torch.int16), o[:B].view(torch.int16)), r
        assert torch.equal(lse[r * B:(r + 1) * B], lse[:B]), r
