"""Byte-exact GPU checks of the dropout keep mask and closed forms of the
sliding-window band (fa_fwd_ex / fa_bwd_ex through the C ABI).

Dropout keep decisions are integer compares of Philox bytes, drawn three
ways by the kernels: per lane (a query) in the forward, per (query, key
half) and transposed through LDS in the dK/dV kernel, and per lane again in
the dQ kernel.  Each is read out exactly here by inputs that make every
output element depend on one weight (the skill guide's Workflow 2, step 2:
flash_attn_func's dropout_p):

* forward: q = 0, so every admitted weight of row i is 1/count_i; V rows
  one-hot (key j -> column j - t d in pass t), so O[i, c] =
  keep(i, td + c) * s_keep / count_i, nonzero iff kept;
* dK/dV kernel, role A's draw (dV = W^T dO with W = P * keep * s_keep):
  q = k = 0 and dO rows one-hot (query i -> column i - t d), so
  dV[j, c] = W(td + c, j), nonzero iff kept;
* dK/dV kernel, role B's draw (dK = scale dS^T Q): k = 0, Q rows one-hot,
  all V rows e_0 and all dO rows e_0, so dP = 1, D_i = s_keep kappa_i with
  kappa_i the kept weight of row i, and dS_ij = P_ij s_keep (keep_ij -
  kappa_i): dK[j, c] = scale dS(td + c, j) is positive iff kept;
* dQ kernel's draw (dQ = scale dS K): q = 0, K rows one-hot, V and dO rows
  e_0: dQ[i, c] = scale dS(i, td + c), positive iff kept.

In the last two, rows whose every admitted weight is kept or dropped
(kappa_i in {0, 1}) carry no sign and are skipped.  Every read-out mask
must equal ``oracle.dropout_keep`` on every admitted (query, key) pair.

The window closed forms (same step, window_size = (left, right)): with all
keys equal, O_i is the mean of the admitted V rows and LSE_i =
scale q_i.k_0 + log(count_i); a row that admits no key has O = 0 and
LSE = -inf.
"""
import math
import sys

import numpy as np
import pytest
import torch

import exact_io_aware_02_amd as fa
from oracle import dropout_keep, dropout_threshold

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL_O = {torch.float16: 2e-3, torch.bfloat16: 1.6e-2}
TOL_LSE = 1e-3


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def admitted(Nq, Nk, causal, window):
    """Boolean [Nq, Nk]: query i admits key j (top-left causal; window
    bounds inclusive, a negative side unbounded)."""
    i = np.arange(Nq)[:, None]
    j = np.arange(Nk)[None, :]
    ok = np.ones((Nq, Nk), dtype=bool)
    if causal:
        ok &= j <= i
    left, right = window
    if left >= 0:
        ok &= j >= i - left
    if right >= 0:
        ok &= j <= i + right
    return ok


def run(q, k, v, do, causal, window, drop, scale):
    o, lse = fa.attention_fwd(q, k, v, causal=causal, scale=scale, window=window, dropout=drop)
    if do is None:
        torch.cuda.synchronize()
        return o, lse, None
    g = fa.attention_bwd(q, k, v, o, lse, do, causal=causal, scale=scale, window=window, dropout=drop)
    torch.cuda.synchronize()
    return o, lse, g


def onehot_rows(B, H, N, d, t, dtype, amp=1.0):
    """[B, H, N, d]: row n is amp * e_(n - t d) for t d <= n < (t+1) d, else 0."""
    x = torch.zeros(B, H, N, d, dtype=torch.float32)
    n = torch.arange(t * d, min(N, (t + 1) * d))
    x[:, :, n, n - t * d] = amp
    return x.to(dtype).to(DEV)


def e0_rows(B, H, N, d, dtype):
    x = torch.zeros(B, H, N, d, dtype=torch.float32)
    x[..., 0] = 1.0
    return x.to(dtype).to(DEV)


MASK_CASES = [
    # name, B, H, Nq, Nk, d, dtype, causal, window, (p, seed, offset)
    ("d64_fp16_seed_above_2p32", 2, 3, 200, 200, 64, torch.float16, False, (-1, -1), (0.5, (1 << 32) + 12345, 7)),
    ("d128_bf16_causal", 1, 2, 300, 300, 128, torch.bfloat16, True, (-1, -1), (0.5, (3 << 40) + 5, 123)),
    ("d64_bf16_causal_rect", 1, 2, 150, 230, 64, torch.bfloat16, True, (-1, -1), (0.25, 99, 0)),
    ("d128_fp16_window", 2, 2, 260, 260, 128, torch.float16, False, (40, 70), (0.5, 2024, (1 << 31) + 3)),
]


def _keep_ref(B, H, Nq, Nk, drop):
    p, seed, off = drop
    return np.stack([np.stack([dropout_keep(b, h, H, np.arange(Nq), Nk, p, seed, off) for h in range(H)])
                     for b in range(B)])


def _compare(name, got, ref, ok):
    bad = (got != ref) & ok[None, None]
    say("  %s: %d admitted entries, %d kept, %d mismatches" % (name, int(ok.sum()) * got.shape[0] * got.shape[1],
                                                                int((ref & ok[None, None]).sum()), int(bad.sum())))
    assert not bad.any(), "%s: first mismatch at %r" % (name, tuple(np.argwhere(bad)[0]))


@pytest.mark.parametrize("case", MASK_CASES, ids=[c[0] for c in MASK_CASES])
def test_dropout_mask_forward_bit_exact(case):
    name, B, H, Nq, Nk, d, dt, causal, window, drop = case
    say("case fwd mask %s" % name)
    ok = admitted(Nq, Nk, causal, window)
    cnt = ok.sum(1)
    ref = _keep_ref(B, H, Nq, Nk, drop)
    _, s_keep = dropout_threshold(drop[0])
    q = torch.zeros(B, H, Nq, d, dtype=dt, device=DEV)
    k = torch.zeros(B, H, Nk, d, dtype=dt, device=DEV)
    got = np.zeros((B, H, Nq, Nk), dtype=bool)
    for t in range(math.ceil(Nk / d)):
        v = onehot_rows(B, H, Nk, d, t, dt)
        o, _, _ = run(q, k, v, None, causal, window, drop, 1.0 / math.sqrt(d))
        on = o.float().cpu().numpy()
        c1 = min(Nk, (t + 1) * d) - t * d
        got[..., t * d:t * d + c1] = on[..., :c1] != 0
        # a kept weight is s_keep / count_i (to output rounding)
        want = np.where(ref[..., t * d:t * d + c1] & ok[None, None, :, t * d:t * d + c1],
                        s_keep / np.maximum(cnt, 1)[None, None, :, None], 0.0)
        assert np.abs(on[..., :c1] - want).max() <= 2.0 ** -7 * want.max(), "values of pass %d" % t
        assert np.all(on[..., c1:] == 0)
    _compare("forward", got, ref, ok)


@pytest.mark.parametrize("case", MASK_CASES, ids=[c[0] for c in MASK_CASES])
def test_dropout_mask_dkdv_role_a_bit_exact(case):
    """dV read-out: the dK/dV kernel's transposed keep bytes."""
    name, B, H, Nq, Nk, d, dt, causal, window, drop = case
    say("case dV mask %s" % name)
    ok = admitted(Nq, Nk, causal, window)
    ref = _keep_ref(B, H, Nq, Nk, drop)
    q = torch.zeros(B, H, Nq, d, dtype=dt, device=DEV)
    k = torch.zeros(B, H, Nk, d, dtype=dt, device=DEV)
    v = torch.randn(B, H, Nk, d, generator=torch.Generator().manual_seed(3)).to(dt).to(DEV)
    got = np.zeros((B, H, Nq, Nk), dtype=bool)
    for t in range(math.ceil(Nq / d)):
        do = onehot_rows(B, H, Nq, d, t, dt)
        _, _, (dq, dk, dv) = run(q, k, v, do, causal, window, drop, 1.0 / math.sqrt(d))
        g = dv.float().cpu().numpy()  # [B, H, Nk, d]: column c is query t d + c
        c1 = min(Nq, (t + 1) * d) - t * d
        got[:, :, t * d:t * d + c1, :] = np.swapaxes(g[..., :c1], 2, 3) != 0
    _compare("dV (role A)", got, ref, ok)


def _kappa(ref, ok):
    """Kept share of each row's (uniform) admitted weights."""
    cnt = ok.sum(1)
    return (ref & ok[None, None]).sum(-1) / np.maximum(cnt, 1)[None, None]


@pytest.mark.parametrize("case", MASK_CASES, ids=[c[0] for c in MASK_CASES])
def test_dropout_mask_dkdv_role_b_bit_exact(case):
    """dK read-out: the keep bytes the dK/dV kernel's role B applies to dS."""
    name, B, H, Nq, Nk, d, dt, causal, window, drop = case
    say("case dK mask %s" % name)
    ok = admitted(Nq, Nk, causal, window)
    ref = _keep_ref(B, H, Nq, Nk, drop)
    kap = _kappa(ref, ok)
    signed = (kap > 0) & (kap < 1)  # rows with a sign to read
    k = torch.zeros(B, H, Nk, d, dtype=dt, device=DEV)
    v = e0_rows(B, H, Nk, d, dt)
    do = e0_rows(B, H, Nq, d, dt)
    got = np.zeros((B, H, Nq, Nk), dtype=bool)
    for t in range(math.ceil(Nq / d)):
        q = onehot_rows(B, H, Nq, d, t, dt)
        _, _, (dq, dk, dv) = run(q, k, v, do, causal, window, drop, 1.0 / math.sqrt(d))
        g = dk.float().cpu().numpy()  # [B, H, Nk, d]: column c is query t d + c
        c1 = min(Nq, (t + 1) * d) - t * d
        got[:, :, t * d:t * d + c1, :] = np.swapaxes(g[..., :c1], 2, 3) > 0
    use = ok[None, None] & signed[..., None]
    bad = (got != ref) & use
    say("  dK (role B): %d signed entries, %d mismatches" % (int(use.sum()), int(bad.sum())))
    assert use.sum() > 0.8 * ok.sum() * B * H
    assert not bad.any(), "first mismatch at %r" % (tuple(np.argwhere(bad)[0]),)


@pytest.mark.parametrize("case", MASK_CASES, ids=[c[0] for c in MASK_CASES])
def test_dropout_mask_dq_bit_exact(case):
    """dQ read-out: the dQ kernel's per-lane keep bytes."""
    name, B, H, Nq, Nk, d, dt, causal, window, drop = case
    say("case dQ mask %s" % name)
    ok = admitted(Nq, Nk, causal, window)
    ref = _keep_ref(B, H, Nq, Nk, drop)
    kap = _kappa(ref, ok)
    signed = (kap > 0) & (kap < 1)
    q = torch.zeros(B, H, Nq, d, dtype=dt, device=DEV)
    v = e0_rows(B, H, Nk, d, dt)
    do = e0_rows(B, H, Nq, d, dt)
    got = np.zeros((B, H, Nq, Nk), dtype=bool)
    for t in range(math.ceil(Nk / d)):
        k = onehot_rows(B, H, Nk, d, t, dt)
        _, _, (dq, dk, dv) = run(q, k, v, do, causal, window, drop, 1.0 / math.sqrt(d))
        g = dq.float().cpu().numpy()  # [B, H, Nq, d]: column c is key t d + c
        c1 = min(Nk, (t + 1) * d) - t * d
        got[..., t * d:t * d + c1] = g[..., :c1] > 0
    use = ok[None, None] & signed[..., None]
    bad = (got != ref) & use
    say("  dQ: %d signed entries, %d mismatches" % (int(use.sum()), int(bad.sum())))
    assert use.sum() > 0.8 * ok.sum() * B * H
    assert not bad.any(), "first mismatch at %r" % (tuple(np.argwhere(bad)[0]),)


def test_dropout_mask_forward_phased_schedule_bit_exact():
    """A d = 128 grid of 1024 forward workgroups (the phased schedule):
    the mask of two (batch, head) pairs read out exactly."""
    B, H, N, d, dt = 2, 64, 1024, 128, torch.bfloat16
    drop = (0.5, (7 << 33) + 1, 11)
    say("case fwd mask phased B%d H%d N%d d%d" % (B, H, N, d))
    q = torch.zeros(B, H, N, d, dtype=dt, device=DEV)
    k = torch.zeros(B, H, N, d, dtype=dt, device=DEV)
    ok = admitted(N, N, True, (-1, -1))
    pairs = ((0, 0), (B - 1, H - 1))
    got = {bh: np.zeros((N, N), dtype=bool) for bh in pairs}
    for t in range(N // d):
        v = onehot_rows(B, H, N, d, t, dt)
        o, _, _ = run(q, k, v, None, True, (-1, -1), drop, 1.0 / math.sqrt(d))
        for (b, h) in pairs:
            got[(b, h)][:, t * d:(t + 1) * d] = o[b, h].float().cpu().numpy() != 0
    for (b, h) in pairs:
        ref = dropout_keep(b, h, H, np.arange(N), N, *drop)
        _compare("forward (%d, %d)" % (b, h), got[(b, h)][None, None], ref[None, None], ok)


# ------------------------------------------------------------ window closed forms

# (left, right) with edges inside a 32-key tile, on a tile boundary, across
# tiles, one-sided, and a band that leaves later rows empty when Nq > Nk
WINDOWS = [(0, 0), (5, 7), (31, 32), (32, 31), (64, 0), (100, -1), (-1, 45), (200, 3), (33, 95)]


@pytest.mark.parametrize("dt,d", [(torch.float16, 64), (torch.bfloat16, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_window_all_equal_keys_closed_form(dt, d, causal):
    """All keys equal: O_i = mean of the admitted V rows, LSE_i = scale
    q_i.k_0 + log(count_i); rows admitting no key: O = 0, LSE = -inf."""
    g = torch.Generator().manual_seed(17)
    for Nq, Nk in ((300, 300), (330, 200)):
        q = torch.randn(2, 2, Nq, d, generator=g).to(dt)
        k0 = torch.randn(1, 1, 1, d, generator=g).to(dt)
        k = k0.expand(2, 2, Nk, d).contiguous()
        v = torch.randn(2, 2, Nk, d, generator=g).to(dt)
        s = 1.0 / math.sqrt(d)
        v64 = v.double().numpy()
        qk = s * (q.double().numpy() @ k0.double().numpy()[0, 0, 0])  # [2, 2, Nq]
        for window in WINDOWS:
            say("case window %r causal=%s Nq=%d Nk=%d d=%d" % (window, causal, Nq, Nk, d))
            o, lse = fa.attention_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=s, window=window)
            torch.cuda.synchronize()
            ok = admitted(Nq, Nk, causal, window).astype(np.float64)
            cnt = ok.sum(1)
            mean = (ok @ v64) / np.maximum(cnt, 1)[:, None]  # [2, 2, Nq, d]
            go, gl = o.double().cpu().numpy(), lse.double().cpu().numpy()
            err = np.abs(go - mean).max()
            assert err <= TOL_O[dt], (window, err)
            full = cnt > 0
            want = qk + np.log(np.maximum(cnt, 1))
            el = np.abs(gl[..., full] - want[..., full]).max()
            assert el <= TOL_LSE, (window, el)
            assert np.all(np.isneginf(gl[..., ~full])) and np.all(go[..., ~full, :] == 0), window
