"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle.

Tolerances (the parity bounds for these shapes, used unchanged here):
  O      max |gpu - oracle| <= 2e-3 (fp16), 1.6e-2 (bf16)
  LSE    max |gpu - oracle| <= 1e-3
  dQ/dK/dV  ||gpu - oracle||_F / ||oracle||_F <= 2e-2 per tensor
The oracle sees exactly the fp16/bf16 values the GPU gets, widened to fp64.
"""
import math
import sys

import numpy as np
import pytest
import torch

import exact_io_aware_02_amd as fa
from attn_inputs import WORKLOADS, make_qkv, sample_rows, to_bhsd64, workload_inputs
from oracle import attention_bwd64, attention_fwd64, attention_rows_fwd64

pytestmark = pytest.mark.gpu

TOL_O = {"fp16": 2e-3, "bf16": 1.6e-2}
TOL_LSE = 1e-3
TOL_GRAD = 2e-2
DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def gpu(t):
    return t.to(DEV)


def fwd_gpu(inp, causal, scale, layout):
    o, lse = fa.attention_fwd(gpu(inp["q"]), gpu(inp["k"]), gpu(inp["v"]), causal=causal, scale=scale,
                              layout=layout)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def bwd_gpu(inp, o, lse, causal, scale, layout):
    dq, dk, dv = fa.attention_bwd(gpu(inp["q"]), gpu(inp["k"]), gpu(inp["v"]), gpu(o), gpu(lse),
                                  gpu(inp["do"]), causal=causal, scale=scale, layout=layout)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def check_o(o_gpu, o_ref, dtype, layout, what=""):
    got = to_bhsd64(o_gpu, layout)
    assert np.isfinite(got).all(), "non-finite output " + what
    err = np.abs(got - o_ref).max() if o_ref.size else 0.0
    say("  O max-abs err %.3e (tol %.1e) %s" % (err, TOL_O[dtype], what))
    assert err <= TOL_O[dtype], what
    return err


def check_lse(lse_gpu, lse_ref, what=""):
    got = lse_gpu.numpy().astype(np.float64)
    assert np.isfinite(got).all()
    err = np.abs(got - lse_ref).max() if lse_ref.size else 0.0
    say("  LSE max-abs err %.3e %s" % (err, what))
    assert err <= TOL_LSE, what


def check_grad(g_gpu, g_ref, layout, name):
    got = to_bhsd64(g_gpu, layout)
    assert np.isfinite(got).all(), name + " non-finite"
    rn = np.linalg.norm(g_ref)
    if rn < 1e-6:
        say("  %s: reference is zero, max|gpu| = %.2e" % (name, np.abs(got).max()))
        assert np.abs(got).max() < 1e-3, name
        return
    rel = np.linalg.norm(got - g_ref) / rn
    rmax = np.abs(got - g_ref).max() / max(np.abs(g_ref).max(), 1e-30)
    say("  %s rel-F err %.3e  (max-err / max-ref %.3e)" % (name, rel, rmax))
    assert rel <= TOL_GRAD, name


def scale_of(d):
    return 1.0 / math.sqrt(d)


# ------------------------------------------------------------------ workloads

@pytest.mark.parametrize("name,causal", [
    ("fwd_b1h2_n128_d64_fp16_bhsd", False),
    ("fwd_b2h8_n512_d64_fp16_bhsd", False),
    ("fwd_b2h8_n512_d64_fp16_bhsd", True),
    ("fwd_causal_b2h16_n1024_d64_bf16_bshd", True),
])
def test_workload_forward(name, causal):
    w = WORKLOADS[name]
    say("case", name, "causal", causal)
    inp = workload_inputs(w)
    s = scale_of(w.d)
    o, lse = fwd_gpu(inp, causal, s, w.layout)
    ro, rl = attention_fwd64(*(to_bhsd64(inp[x], w.layout) for x in "qkv"), s, causal)
    check_o(o, ro, w.dtype, w.layout, name)
    check_lse(lse, rl, name)


def test_workload_train_step_fwd_bwd():
    w = WORKLOADS["train_causal_b2h8_n2048_d64_fp16_bhsd"]
    say("case", w.name)
    inp = workload_inputs(w)
    s = scale_of(w.d)
    o, lse = fwd_gpu(inp, True, s, w.layout)
    q, k, v, do = (to_bhsd64(inp[x], w.layout) for x in ("q", "k", "v", "do"))
    ro, rl = attention_fwd64(q, k, v, s, True)
    check_o(o, ro, w.dtype, w.layout, w.name)
    check_lse(lse, rl, w.name)
    dq, dk, dv = bwd_gpu(inp, o, lse, True, s, w.layout)
    rq, rk, rv = attention_bwd64(q, k, v, do, s, True)
    check_grad(dq, rq, w.layout, "dQ")
    check_grad(dk, rk, w.layout, "dK")
    check_grad(dv, rv, w.layout, "dV")


@pytest.fixture(scope="module")
def long_ctx():
    """The 16K workload, run once: forward, then backward with seeded dO."""
    w = WORKLOADS["fwd_causal_b1h16_n16384_d128_bf16_bhsd"]
    say("case", w.name)
    inp = workload_inputs(w)
    s = scale_of(w.d)
    o, lse = fwd_gpu(inp, True, s, w.layout)
    rng = np.random.default_rng(w.seed + 2000)
    inp["do"] = torch.from_numpy(rng.standard_normal(inp["q"].shape, dtype=np.float32)).to(torch.bfloat16)
    dq, dk, dv = bwd_gpu(inp, o, lse, True, s, w.layout)
    return w, inp, s, o, lse, (dq, dk, dv)


def test_long_context_repeat_runs_bitwise(long_ctx):
    """Thirty forward runs (the phased schedule of grids of 512+ workgroups)
    and ten backward runs of the 16K workload are bitwise identical to the
    first: no result depends on how the waves happen to interleave."""
    w, inp, s, o, lse, grads = long_ctx
    q, k, v, do = (gpu(inp[x]) for x in ("q", "k", "v", "do"))
    o0, l0 = gpu(o), gpu(lse)
    for i in range(30):
        o1, l1 = fa.attention_fwd(q, k, v, causal=True, scale=s, layout=w.layout)
        torch.cuda.synchronize()
        assert torch.equal(o1, o0) and torch.equal(l1, l0), "forward run %d differs" % i
    g0 = [gpu(g) for g in grads]
    for i in range(10):
        g1 = fa.attention_bwd(q, k, v, o0, l0, do, causal=True, scale=s, layout=w.layout)
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(g1, g0)), "backward run %d differs" % i


def test_long_context_sampled_rows(long_ctx):
    """256 seeded query rows per head (rows 0 and N-1 always), every head."""
    w, inp, s, o, lse, _ = long_ctx
    rows = sample_rows(w.B, w.H, w.N, 256, w.seed + 1000)
    q, k, v = (to_bhsd64(inp[x]) for x in "qkv")
    ro, rl = attention_rows_fwd64(q, k, v, s, True, rows)
    og = to_bhsd64(o)
    lg = lse.numpy().astype(np.float64)
    got_o = np.stack([np.stack([og[b, h][rows[b, h]] for h in range(w.H)]) for b in range(w.B)])
    got_l = np.stack([np.stack([lg[b, h][rows[b, h]] for h in range(w.H)]) for b in range(w.B)])
    err = np.abs(got_o - ro).max()
    say("  sampled O max-abs err %.3e, LSE err %.3e" % (err, np.abs(got_l - rl).max()))
    assert err <= TOL_O[w.dtype]
    assert np.abs(got_l - rl).max() <= TOL_LSE
    assert np.isfinite(og).all() and np.isfinite(lg).all()


def test_long_context_full_head_forward(long_ctx):
    """Every row of head 0 against the full oracle."""
    w, inp, s, o, lse, _ = long_ctx
    q, k, v = (to_bhsd64(inp[x][:, :1]) for x in "qkv")
    ro, rl = attention_fwd64(q, k, v, s, True)
    check_o(o[:, :1], ro, w.dtype, "bhsd", "head 0")
    check_lse(lse[:, :1], rl, "head 0")


def test_long_context_backward_one_head_and_invariants(long_ctx):
    w, inp, s, o, lse, (dq, dk, dv) = long_ctx
    h = 5
    q, k, v, do = (to_bhsd64(inp[x][:, h:h + 1]) for x in ("q", "k", "v", "do"))
    rq, rk, rv = attention_bwd64(q, k, v, do, s, True)
    check_grad(dq[:, h:h + 1], rq, "bhsd", "dQ[h5]")
    check_grad(dk[:, h:h + 1], rk, "bhsd", "dK[h5]")
    check_grad(dv[:, h:h + 1], rv, "bhsd", "dV[h5]")
    # every head: sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i (exact identities)
    gk = to_bhsd64(dk)
    gv = to_bhsd64(dv)
    gdo = to_bhsd64(inp["do"])
    assert np.isfinite(gk).all() and np.isfinite(gv).all() and np.isfinite(to_bhsd64(dq)).all()
    rel_k = np.abs(gk.sum(axis=2)).max() / np.abs(gk).sum(axis=2).max()
    rel_v = np.abs(gv.sum(axis=2) - gdo.sum(axis=2)).max() / np.abs(gdo.sum(axis=2)).max()
    say("  identities: |sum dK| / sum|dK| = %.2e, sum dV vs sum dO rel %.2e" % (rel_k, rel_v))
    assert rel_k < 2e-2 and rel_v < 2e-2


def test_long_context_head_shard_split(long_ctx):
    """One GPU's share of the 16K workload under 8-way head sharding (heads
    0-1) in the launch configuration the benchmark times: fa_fwd_splitk
    with its workspace (the key range of heavy query blocks cut over
    workgroups, partials merged in chunk order) and the small-grid backward
    (dQ's intra-workgroup key split, beside dK/dV on the side stream).
    Forward against the oracle on 256 seeded rows per head.  Backward with
    the full 16-head run's O and LSE, as the benchmark runs it (fa_bwd_ex
    with the workspace of fa_bwd_ex_workspace_bytes: each key block's query
    tiles in two runs, fp32 partials added in run order): dQ, dK, dV within
    fp32 reordering of the 16-head run; and with the statistics-only
    workspace (no dK/dV split) dK, dV bit for bit equal to that run's first
    two heads (the same workgroups)."""
    w, inp, s, o, lse, (dq, dk, dv) = long_ctx
    B, H, N, d = w.B, 2, w.N, w.d
    q, k, v, do = (gpu(inp[x][:, :H].contiguous()) for x in ("q", "k", "v", "do"))
    nws = fa.fa_fwd_splitk_workspace_bytes(B, H, N, N, d, True)
    say("case head shard: workspace %d bytes" % nws)
    assert nws > 0
    ws = torch.empty(nws, dtype=torch.uint8, device=DEV)
    o2 = torch.empty_like(q)
    l2 = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    fa.fa_fwd_splitk(q, k, v, o2, l2, s, True, ws)
    torch.cuda.synchronize()
    og, lg = to_bhsd64(o2.cpu()), l2.cpu().numpy().astype(np.float64)
    assert np.isfinite(og).all() and np.isfinite(lg).all()
    rows = sample_rows(B, H, N, 256, w.seed + 3000)
    ro, rl = attention_rows_fwd64(*(to_bhsd64(inp[x][:, :H]) for x in "qkv"), s, True, rows)
    got_o = np.stack([np.stack([og[b, h][rows[b, h]] for h in range(H)]) for b in range(B)])
    got_l = np.stack([np.stack([lg[b, h][rows[b, h]] for h in range(H)]) for b in range(B)])
    err_o, err_l = np.abs(got_o - ro).max(), np.abs(got_l - rl).max()
    say("  split forward: sampled O max-abs err %.3e, LSE err %.3e" % (err_o, err_l))
    assert err_o <= TOL_O[w.dtype] and err_l <= TOL_LSE
    oh, lh = gpu(o[:, :H].contiguous()), gpu(lse[:, :H].contiguous())
    big = fa.fa_bwd_ex_workspace_bytes(B, H, H, N, N, d, fa.FA_BF16)
    small = fa.fa_bwd_workspace_bytes(B, H, N, N, d, fa.FA_BF16)
    assert big > small  # the dK/dV split applies
    for tag, nbytes in (("split", big), ("unsplit dK/dV", small)):
        ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
        g2 = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
        fa.fa_bwd_ex(q, k, v, oh, lh, do, *g2, s, True, ws)
        torch.cuda.synchronize()
        dq2, dk2, dv2 = (g.cpu() for g in g2)
        if tag != "split":
            assert torch.equal(dk2, dk[:, :H]) and torch.equal(dv2, dv[:, :H]), "dK/dV differ from the 16-head run"
        for nm, x, r in (("dQ", dq2, dq), ("dK", dk2, dk), ("dV", dv2, dv)):
            a, rr = to_bhsd64(x), to_bhsd64(r[:, :H])
            rel = np.linalg.norm(a - rr) / np.linalg.norm(rr)
            say("  %s %s vs 16-head run: relative Frobenius %.2e" % (tag, nm, rel))
            assert rel <= 4e-3, (tag, nm)


# ------------------------------------------------------------------ sweeps

SIZES = [1, 2, 3, 17, 63, 64, 65, 127, 129, 255]


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_sweep_square(dtype, d, causal):
    for i, n in enumerate(SIZES):
        inp = make_qkv(2, 3, n, n, d, dtype, "bhsd", seed=100 + i, with_do=True)
        s = scale_of(d)
        say("case sweep n=%d d=%d %s causal=%s" % (n, d, dtype, causal))
        o, lse = fwd_gpu(inp, causal, s, "bhsd")
        q, k, v, do = (to_bhsd64(inp[x]) for x in ("q", "k", "v", "do"))
        ro, rl = attention_fwd64(q, k, v, s, causal)
        check_o(o, ro, dtype, "bhsd", "n=%d" % n)
        check_lse(lse, rl)
        dq, dk, dv = bwd_gpu(inp, o, lse, causal, s, "bhsd")
        rq, rk, rv = attention_bwd64(q, k, v, do, s, causal)
        check_grad(dq, rq, "bhsd", "dQ")
        check_grad(dk, rk, "bhsd", "dK")
        check_grad(dv, rv, "bhsd", "dV")


@pytest.mark.parametrize("nq,nk", [(17, 130), (130, 17), (1, 300), (300, 1), (64, 192), (257, 64)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("layout", ["bhsd", "bshd"])
def test_sweep_rectangular(nq, nk, causal, layout):
    for d, dtype in ((64, "fp16"), (128, "bf16")):
        say("case rect nq=%d nk=%d d=%d %s causal=%s %s" % (nq, nk, d, dtype, causal, layout))
        inp = make_qkv(1, 4, nq, nk, d, dtype, layout, seed=nq * 1000 + nk, with_do=True)
        s = scale_of(d)
        o, lse = fwd_gpu(inp, causal, s, layout)
        q, k, v, do = (to_bhsd64(inp[x], layout) for x in ("q", "k", "v", "do"))
        ro, rl = attention_fwd64(q, k, v, s, causal)
        check_o(o, ro, dtype, layout)
        check_lse(lse, rl)
        dq, dk, dv = bwd_gpu(inp, o, lse, causal, s, layout)
        rq, rk, rv = attention_bwd64(q, k, v, do, s, causal)
        check_grad(dq, rq, layout, "dQ")
        check_grad(dk, rk, layout, "dK")
        check_grad(dv, rv, layout, "dV")


@pytest.mark.parametrize("scale", [-0.125, 0.0, 0.9, 1e-3])
def test_scales(scale):
    """Any finite scale: negative (Q negated internally), zero (uniform
    weights), large and tiny."""
    inp = make_qkv(1, 2, 100, 100, 64, "fp16", seed=7, with_do=True)
    for causal in (False, True):
        say("case scale=%g causal=%s" % (scale, causal))
        o, lse = fwd_gpu(inp, causal, scale, "bhsd")
        q, k, v, do = (to_bhsd64(inp[x]) for x in ("q", "k", "v", "do"))
        ro, rl = attention_fwd64(q, k, v, scale, causal)
        check_o(o, ro, "fp16", "bhsd")
        check_lse(lse, rl)
        dq, dk, dv = bwd_gpu(inp, o, lse, causal, scale, "bhsd")
        rq, rk, rv = attention_bwd64(q, k, v, do, scale, causal)
        check_grad(dq, rq, "bhsd", "dQ")
        check_grad(dk, rk, "bhsd", "dK")
        check_grad(dv, rv, "bhsd", "dV")


def test_empty_inputs():
    for shape_q, shape_k in [((0, 2, 8, 64), (0, 2, 8, 64)), ((1, 0, 8, 64), (1, 0, 8, 64)),
                             ((1, 2, 0, 64), (1, 2, 8, 64))]:
        q = torch.zeros(shape_q, dtype=torch.float16, device=DEV)
        k = torch.randn(shape_k, dtype=torch.float16, device=DEV)
        o, lse = fa.attention_fwd(q, k, k, causal=True)
        assert o.shape == q.shape and lse.numel() == 0
    # no queries: dK = dV = 0
    q = torch.zeros((1, 2, 0, 64), dtype=torch.float16, device=DEV)
    k = torch.randn((1, 2, 40, 64), dtype=torch.float16, device=DEV)
    lse = torch.zeros((1, 2, 0), dtype=torch.float32, device=DEV)
    dq, dk, dv = fa.attention_bwd(q, k, k, q, lse, q, causal=False)
    torch.cuda.synchronize()
    assert float(dk.abs().max()) == 0.0 and float(dv.abs().max()) == 0.0


def test_non_default_stream():
    inp = make_qkv(2, 2, 333, 333, 128, "bf16", seed=11)
    s = scale_of(128)
    st = torch.cuda.Stream()
    q, k, v = gpu(inp["q"]), gpu(inp["k"]), gpu(inp["v"])
    torch.cuda.synchronize()
    with torch.cuda.stream(st):
        o, lse = fa.attention_fwd(q, k, v, causal=True, scale=s)
    st.synchronize()
    ro, rl = attention_fwd64(*(to_bhsd64(inp[x]) for x in "qkv"), s, True)
    check_o(o.cpu(), ro, "bf16", "bhsd")
    check_lse(lse.cpu(), rl)


# ------------------------------------------------------------------ invariants at real dtypes

@pytest.mark.parametrize("dtype,d", [("fp16", 64), ("bf16", 128)])
def test_closed_forms_on_gpu(dtype, d):
    td = torch.float16 if dtype == "fp16" else torch.bfloat16
    N = 300
    g = torch.Generator().manual_seed(5)
    v = torch.randn(1, 1, N, d, generator=g).to(td)
    q = torch.randn(1, 1, N, d, generator=g).to(td)
    s = scale_of(d)
    # all-equal keys: O_i = mean of visible V rows, lse_i = s q_i.k0 + log(count)
    k = torch.randn(1, 1, 1, d, generator=g).to(td).expand(1, 1, N, d).contiguous()
    for causal in (False, True):
        o, lse = fa.attention_fwd(gpu(q), gpu(k), gpu(v), causal=causal, scale=s)
        v64 = v.double()[0, 0].numpy()
        cnt = np.arange(1, N + 1) if causal else np.full(N, N)
        mean = np.cumsum(v64, 0) / cnt[:, None] if causal else np.broadcast_to(v64.mean(0), (N, d))
        err = np.abs(o.cpu().double()[0, 0].numpy() - mean).max()
        say("  all-equal keys causal=%s err %.2e" % (causal, err))
        assert err <= TOL_O[dtype]
        ql = s * (q.double()[0, 0].numpy() @ k.double()[0, 0, 0].numpy()) + np.log(cnt)
        assert np.abs(lse.cpu().double()[0, 0].numpy() - ql).max() <= TOL_LSE
        # causal row 0: O_0 = V_0 exactly up to output rounding
        if causal:
            assert torch.equal(o[0, 0, 0].cpu(), v[0, 0, 0])
    # dominant key: q_i = a e1, k_j* = a e1 (others 0), s a^2 = 50 -> O_i = V_j*
    a = math.sqrt(50 / s)
    qd = torch.zeros(1, 1, N, d); qd[..., 0] = a
    kd = torch.zeros(1, 1, N, d); kd[0, 0, 123, 0] = a
    qd, kd = qd.to(td), kd.to(td)
    o, _ = fa.attention_fwd(gpu(qd), gpu(kd), gpu(v), causal=False, scale=s)
    err = (o.cpu().double()[0, 0] - v.double()[0, 0, 123]).abs().max().item()
    say("  dominant key err %.2e" % err)
    assert err <= TOL_O[dtype]


def test_key_shift_invariance_on_gpu():
    """k_j + u: O unchanged, lse shifted by s q.u (u exactly representable)."""
    inp = make_qkv(1, 2, 200, 200, 64, "fp16", seed=9)
    s = scale_of(64)
    u = torch.zeros(1, 2, 1, 64, dtype=torch.float16)
    u[..., :8] = 0.25
    o1, l1 = fwd_gpu(inp, True, s, "bhsd")
    inp2 = dict(inp, k=(inp["k"].double() + u.double()).half())
    o2, l2 = fwd_gpu(inp2, True, s, "bhsd")
    q, k2, v = (to_bhsd64(inp2[x]) for x in "qkv")
    ro, rl = attention_fwd64(q, k2, v, s, True)
    check_o(o2, ro, "fp16", "bhsd")
    assert (o1.double() - o2.double()).abs().max().item() <= 2 * TOL_O["fp16"]


def test_deterministic_and_finite():
    w = WORKLOADS["fwd_causal_b2h16_n1024_d64_bf16_bshd"]
    inp = workload_inputs(w)
    q, k, v = gpu(inp["q"]), gpu(inp["k"]), gpu(inp["v"])
    o1, l1 = fa.attention_fwd(q, k, v, causal=True, layout="bshd")
    o2, l2 = fa.attention_fwd(q, k, v, causal=True, layout="bshd")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    do = torch.randn_like(q)
    g1 = fa.attention_bwd(q, k, v, o1, l1, do, causal=True, layout="bshd")
    g2 = fa.attention_bwd(q, k, v, o1, l1, do, causal=True, layout="bshd")
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
        assert torch.isfinite(a.float()).all()


def test_pages_accuracy_recipe():
    """The skill guide's accuracy check (Workflow 1, step 4): fp16 inputs of
    shape (1, 8, 512, 64), scale 1/8, max |difference| below 1e-3."""
    inp = make_qkv(1, 8, 512, 512, 64, "fp16", seed=21)
    o, _ = fwd_gpu(inp, False, 1.0 / 8.0, "bhsd")
    ro, _ = attention_fwd64(*(to_bhsd64(inp[x]) for x in "qkv"), 1.0 / 8.0, False)
    err = np.abs(to_bhsd64(o) - ro).max()
    say("  pages' recipe max diff %.3e" % err)
    assert err < 1e-3


def test_batch_offsets_beyond_32_bits():
    """Batch strides past 2^31 elements (64-bit offsets): q, k, v are views
    into one 8.6 GB buffer with batch stride 2^31 + 64; the result equals the
    contiguous copies' bit for bit, forward and backward."""
    say("case batch_offsets_beyond_32_bits")
    B, H, N, d = 2, 1, 256, 64
    S = (1 << 31) + 64
    buf = torch.empty(B * S, dtype=torch.float16, device=DEV)
    inp = make_qkv(B, H, N, N, d, "fp16", seed=41, with_do=True)
    views = []
    for i, name in enumerate(("q", "k", "v")):
        vw = torch.as_strided(buf, (B, H, N, d), (S, N * d, d, 1), storage_offset=i * N * d)
        vw.copy_(inp[name].to(DEV))
        views.append(vw)
    q, k, v = views
    do = inp["do"].to(DEV)
    o1, l1 = fa.attention_fwd(q, k, v, causal=True)
    g1 = fa.attention_bwd(q, k, v, o1, l1, do, causal=True)
    qc, kc, vc = (x.contiguous() for x in views)
    o2, l2 = fa.attention_fwd(qc, kc, vc, causal=True)
    g2 = fa.attention_bwd(qc, kc, vc, o2, l2, do, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    del buf, views, q, k, v
    torch.cuda.empty_cache()


def test_large_grid_sampled_rows():
    """32 x 32 (batch, head) pairs of 1024 causal fp16 tokens (8192 forward
    workgroups): sampled rows of two (b, h) pairs against the oracle."""
    say("case large_grid_sampled_rows")
    B, H, N, d = 32, 32, 1024, 64
    inp = make_qkv(B, H, N, N, d, "fp16", seed=43)
    q, k, v = (inp[x].to(DEV) for x in ("q", "k", "v"))
    o, lse = fa.attention_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    rows = sample_rows(1, 1, N, 64, seed=44)
    for b, h in ((0, 0), (B - 1, H - 1)):
        q64, k64, v64 = (to_bhsd64(inp[x][b:b + 1, h:h + 1]) for x in ("q", "k", "v"))
        ro, rl = attention_rows_fwd64(q64, k64, v64, 1 / 8.0, True, rows)
        go = o[b, h].cpu().double().numpy()[rows[0, 0]]
        gl = lse[b, h].cpu().double().numpy()[rows[0, 0]]
        eo = np.abs(go - ro[0, 0]).max()
        el = np.abs(gl - rl[0, 0]).max()
        say("  (b, h) = (%d, %d): O max-abs %.2e, LSE %.2e" % (b, h, eo, el))
        assert eo <= TOL_O["fp16"] and el <= TOL_LSE


@pytest.mark.parametrize("dtype,causal", [("bf16", False), ("fp16", True)])
def test_d64_full_chip_every_head(dtype, causal):
    """A d = 64 grid that fills the chip (4 x 32 heads of 1024 tokens: 1024
    forward workgroups, three per CU): every head against the oracle."""
    B, H, N, d = 4, 32, 1024, 64
    say("case d64_full_chip %s causal=%s" % (dtype, causal))
    inp = make_qkv(B, H, N, N, d, dtype, seed=47)
    o, lse = fwd_gpu(inp, causal, 1 / 8.0, "bhsd")
    q, k, v = (to_bhsd64(inp[x]) for x in ("q", "k", "v"))
    ro, rl = attention_fwd64(q, k, v, 1 / 8.0, causal)
    check_o(o, ro, dtype, "bhsd")
    check_lse(lse, rl)


@pytest.mark.parametrize("B,H,N,d,dt", [(2, 8, 1024, 64, "fp16"), (1, 4, 1000, 128, "bf16")])
def test_small_backward_side_stream(B, H, N, d, dt):
    """A backward whose dK/dV grid is under two waves of the chip runs dQ on
    the library's side stream.  Its results equal the three stages run one
    after another on the caller's stream, bit for bit, and so do replays of
    a captured graph of it, with eager work on the outputs between them."""
    say("case B%d H%d N%d d%d %s" % (B, H, N, d, dt))
    inp = make_qkv(B, H, N, N, d, dt, seed=5, with_do=True)
    q, k, v, do = (gpu(inp[x]) for x in ("q", "k", "v", "do"))
    s = 1.0 / math.sqrt(d)
    o, lse = fa.attention_fwd(q, k, v, causal=True, scale=s)
    code = fa.FA_FP16 if dt == "fp16" else fa.FA_BF16
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, N, d, code), dtype=torch.uint8, device=DEV)
    ref = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    for st in (fa.FA_BWD_PREP, fa.FA_BWD_DKDV, fa.FA_BWD_DQ):
        fa.fa_bwd_stages(q, k, v, o, lse, do, *ref, s, True, ws, st)
    got = [torch.empty_like(t) for t in ref]
    fa.fa_bwd(q, k, v, o, lse, do, *got, s, True, ws)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a, b)
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fa.fa_bwd(q, k, v, o, lse, do, *got, s, True, ws, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.fa_bwd(q, k, v, o, lse, do, *got, s, True, ws, torch.cuda.current_stream())
    for i in range(3):
        for t in got:
            t.fill_(float(i + 1))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b), "replay %d" % i


def test_small_backward_several_calls_in_one_graph():
    """Three small backwards captured in one graph, each on its own outputs
    and workspace: every call of the capture (not only the first) may fork
    dQ onto the side stream that the capture already holds.  Replays, with
    eager work on the outputs between them, equal the eager result bit for
    bit."""
    B, H, N, d = 2, 8, 1024, 64
    inp = make_qkv(B, H, N, N, d, "fp16", seed=9, with_do=True)
    q, k, v, do = (gpu(inp[x]) for x in ("q", "k", "v", "do"))
    s = 1.0 / math.sqrt(d)
    o, lse = fa.attention_fwd(q, k, v, causal=True, scale=s)
    nb = fa.fa_bwd_workspace_bytes(B, H, N, N, d, fa.FA_FP16)
    ref = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    for st in (fa.FA_BWD_PREP, fa.FA_BWD_DKDV, fa.FA_BWD_DQ):
        fa.fa_bwd_stages(q, k, v, o, lse, do, *ref, s, True, torch.empty(nb, dtype=torch.uint8, device=DEV), st)
    wss = [torch.empty(nb, dtype=torch.uint8, device=DEV) for _ in range(3)]
    outs = [[torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)] for _ in range(3)]
    fa.fa_bwd(q, k, v, o, lse, do, *outs[0], s, True, wss[0])  # creates the side stream outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(3):
            fa.fa_bwd(q, k, v, o, lse, do, *outs[i], s, True, wss[i], torch.cuda.current_stream())
    for r in range(3):
        for ts in outs:
            for t in ts:
                t.fill_(float(r + 1))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, ts in enumerate(outs):
            for a, b in zip(ts, ref):
                assert torch.equal(a, b), "replay %d call %d" % (r, i)


def test_small_backward_from_two_host_threads():
    """Two host threads run small backwards (side-stream path) on their own
    streams at the same time, 20 calls each; every result equals the
    single-threaded one bit for bit (the fork and join stay paired)."""
    import threading

    B, H, N, d = 2, 8, 1024, 64
    inp = make_qkv(B, H, N, N, d, "fp16", seed=6, with_do=True)
    q, k, v, do = (gpu(inp[x]) for x in ("q", "k", "v", "do"))
    s = 1.0 / math.sqrt(d)
    o, lse = fa.attention_fwd(q, k, v, causal=True, scale=s)
    ws0 = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, N, d, fa.FA_FP16), dtype=torch.uint8, device=DEV)
    ref = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    fa.fa_bwd(q, k, v, o, lse, do, *ref, s, True, ws0)  # the same (unsplit) workspace size as the workers'
    torch.cuda.synchronize()
    bad = []

    def worker(idx):
        torch.cuda.set_device(DEV)
        st = torch.cuda.Stream(device=DEV)
        ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, N, d, fa.FA_FP16), dtype=torch.uint8, device=DEV)
        outs = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
        st.wait_stream(torch.cuda.default_stream(DEV))
        for i in range(20):
            fa.fa_bwd(q, k, v, o, lse, do, *outs, s, True, ws, st)
            st.synchronize()
            if not all(torch.equal(a, b) for a, b in zip(outs, ref)):
                bad.append((idx, i))

    ts = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not bad, bad


def test_small_backward_captured_while_another_thread_runs_eagerly():
    """One thread captures a small backward (its dQ forks onto the library's
    side stream, which then belongs to that capture until it ends) while a
    second thread runs eager small backwards: the eager calls must keep off
    the captured side stream.  Both the eager results and replays of the
    graph equal the plain result bit for bit."""
    import threading

    B, H, N, d = 2, 8, 1024, 64
    inp = make_qkv(B, H, N, N, d, "fp16", seed=8, with_do=True)
    q, k, v, do = (gpu(inp[x]) for x in ("q", "k", "v", "do"))
    s = 1.0 / math.sqrt(d)
    o, lse = fa.attention_fwd(q, k, v, causal=True, scale=s)
    ws_a = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, N, d, fa.FA_FP16), dtype=torch.uint8, device=DEV)
    ref = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    fa.fa_bwd(q, k, v, o, lse, do, *ref, s, True, ws_a)  # also creates the side stream
    torch.cuda.synchronize()
    ws_b = torch.empty_like(ws_a)
    outs_a = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    outs_b = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    st_b = torch.cuda.Stream(device=DEV)
    captured, eager_done = threading.Event(), threading.Event()
    bad = []
    g = torch.cuda.CUDAGraph()

    def capturer():
        torch.cuda.set_device(DEV)
        with torch.cuda.graph(g, capture_error_mode="thread_local"):
            fa.fa_bwd(q, k, v, o, lse, do, *outs_a, s, True, ws_a, torch.cuda.current_stream())
            captured.set()
            eager_done.wait(timeout=60)

    def eager():
        torch.cuda.set_device(DEV)
        captured.wait(timeout=60)
        try:
            for i in range(5):
                fa.fa_bwd(q, k, v, o, lse, do, *outs_b, s, True, ws_b, st_b)
                st_b.synchronize()
                if not all(torch.equal(a, b) for a, b in zip(outs_b, ref)):
                    bad.append(("eager", i))
        finally:
            eager_done.set()

    ta, tb = threading.Thread(target=capturer), threading.Thread(target=eager)
    ta.start()
    tb.start()
    ta.join()
    tb.join()
    assert captured.is_set() and eager_done.is_set()
    for i in range(3):
        for t in outs_a:
            t.fill_(float(i + 1))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        if not all(torch.equal(a, b) for a, b in zip(outs_a, ref)):
            bad.append(("replay", i))
    assert not bad, bad


@pytest.mark.parametrize("B,H,N,dtype,layout", [
    (1, 72, 256, "fp16", "bhsd"),    # 72 key blocks of 256: one per head
    (1, 40, 300, "bf16", "bshd"),    # 80 blocks; the second one's pairs partly or wholly past Nk
    (1, 9, 2048, "bf16", "bhsd"),    # 72 blocks, fewer than the CUs: each block's query tiles in two runs
])
def test_causal_two_key_blocks(B, H, N, dtype, layout):
    """Causal d = 128 bands with at least 65 key blocks of 256 run the
    dK/dV kernel with two 32-key blocks per wave (smaller grids and windows
    run the single-block one): full tensors against the oracle."""
    d = 128
    say("case causal two-block B%d H%d N%d %s %s" % (B, H, N, dtype, layout))
    assert B * H * ((N + 255) // 256) >= 65
    inp = make_qkv(B, H, N, N, d, dtype, layout, seed=N + H, with_do=True)
    s = scale_of(d)
    o, lse = fwd_gpu(inp, True, s, layout)
    q, k, v, do = (to_bhsd64(inp[x], layout) for x in ("q", "k", "v", "do"))
    ro, rl = attention_fwd64(q, k, v, s, True)
    check_o(o, ro, dtype, layout)
    check_lse(lse, rl)
    dq, dk, dv = bwd_gpu(inp, o, lse, True, s, layout)
    rq, rk, rv = attention_bwd64(q, k, v, do, s, True)
    check_grad(dq, rq, layout, "dQ")
    check_grad(dk, rk, layout, "dK")
    check_grad(dv, rv, layout, "dV")
