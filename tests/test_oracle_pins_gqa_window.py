"""Pins of the oracle's fewer-K/V-heads and sliding-window variants (CPU).

Readings pinned here (the pages show the features, not their semantics):
query head h uses K/V head h // (H / H_kv); a window (left, right) admits
keys i - left <= j <= i + right with negative meaning unbounded and causal
adding j <= i; a row with no admitted key has O = 0 and lse = -inf.
Independent references: torch's float64 SDPA with ``enable_gqa`` or an
explicit boolean mask (and its autograd), closed forms, scalar loops and
finite differences.
"""
import math

import numpy as np
import pytest
import torch

from grad_identities import identity_errors
from oracle import attention_bwd64, attention_fwd64, attention_rows_dq64, attention_rows_fwd64

RNG = np.random.default_rng(4321)  # reseeded per test (tests/conftest.py)


def rand(*shape):
    return RNG.standard_normal(shape)


def _t(x, grad=False):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.requires_grad_() if grad else t


def _mask(nq, nk, causal, left, right):
    """Boolean [nq, nk] admitted-key mask written with explicit loops."""
    m = np.zeros((nq, nk), dtype=bool)
    for i in range(nq):
        for j in range(nk):
            ok = True
            if causal and j > i:
                ok = False
            if left >= 0 and j < i - left:
                ok = False
            if right >= 0 and j > i + right:
                ok = False
            m[i, j] = ok
    return m


# ---------------------------------------------------------------- fewer K/V heads

@pytest.mark.parametrize("H,Hkv", [(4, 1), (4, 2), (6, 3), (3, 3)])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_matches_torch_enable_gqa(H, Hkv, causal):
    q, k, v = rand(2, H, 13, 8), rand(2, Hkv, 17, 8), rand(2, Hkv, 17, 8)
    s = 0.41
    o, lse = attention_fwd64(q, k, v, s, causal)
    ref = torch.nn.functional.scaled_dot_product_attention(_t(q), _t(k), _t(v), is_causal=causal, scale=s,
                                                           enable_gqa=True)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12)
    # lse against the heads expanded by torch's own repeat_interleave
    kr = torch.repeat_interleave(_t(k), H // Hkv, dim=1)
    sc = s * _t(q) @ kr.transpose(-1, -2)
    if causal:
        sc = sc.masked_fill(torch.ones(13, 17, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(sc, -1).numpy(), atol=1e-12)


@pytest.mark.parametrize("H,Hkv", [(4, 1), (6, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_bwd_matches_torch_autograd(H, Hkv, causal):
    q, k, v, do = rand(1, H, 11, 8), rand(1, Hkv, 11, 8), rand(1, Hkv, 11, 8), rand(1, H, 11, 8)
    s = 0.5
    tq, tk, tv = _t(q, True), _t(k, True), _t(v, True)
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=s, enable_gqa=True)
    out.backward(_t(do))
    dq, dk, dv = attention_bwd64(q, k, v, do, s, causal)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


def test_gqa_head_map_direction():
    """Distinguishes h // G from h % G: with two K/V heads whose values are
    the constants 0 and 1, query heads 0,1 must see 0 and heads 2,3 see 1."""
    q, k = rand(1, 4, 5, 4), rand(1, 2, 5, 4)
    v = np.zeros((1, 2, 5, 4))
    v[0, 1] = 1.0
    o, _ = attention_fwd64(q, k, v, 0.5, False)
    np.testing.assert_allclose(o[0, :2], 0.0, atol=1e-15)
    np.testing.assert_allclose(o[0, 2:], 1.0, atol=1e-14)


# ---------------------------------------------------------------- sliding window

def test_window_zero_zero_is_diagonal():
    """(left, right) = (0, 0): query i sees only key i, so O_i = V_i and
    lse_i = s q_i.k_i; queries past the last key see nothing (O = 0,
    lse = -inf)."""
    q, k, v = rand(1, 2, 9, 5), rand(1, 2, 7, 5), rand(1, 2, 7, 5)
    s = 0.6
    o, lse = attention_fwd64(q, k, v, s, False, window=(0, 0))
    for i in range(9):
        if i < 7:
            np.testing.assert_allclose(o[0, :, i], v[0, :, i], atol=1e-14)
            np.testing.assert_allclose(lse[0, :, i], s * np.sum(q[0, :, i] * k[0, :, i], -1), atol=1e-13)
        else:
            np.testing.assert_array_equal(o[0, :, i], 0.0)
            assert np.all(np.isneginf(lse[0, :, i]))


@pytest.mark.parametrize("left", [0, 1, 3, 6])
def test_window_causal_all_equal_keys(left):
    """Causal with a left window on equal keys: O_i is the mean of
    V[max(0, i - left) .. i] and lse_i = s q_i.k0 + log(count)."""
    N, d, s = 10, 4, 0.3
    q, v = rand(1, 1, N, d), rand(1, 1, N, d)
    k0 = rand(d)
    k = np.broadcast_to(k0, (1, 1, N, d)).copy()
    o, lse = attention_fwd64(q, k, v, s, True, window=(left, 7))  # right is moot under causal
    for i in range(N):
        lo = max(0, i - left)
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, lo:i + 1].mean(axis=0), atol=1e-13)
        np.testing.assert_allclose(lse[0, 0, i], s * q[0, 0, i] @ k0 + math.log(i + 1 - lo), atol=1e-13)


WINDOWS = [(2, 3, False), (0, 5, False), (4, 0, False), (-1, 2, False), (3, -1, False), (2, -1, True),
           (5, 5, True), (0, -1, True)]


@pytest.mark.parametrize("left,right,causal", WINDOWS)
@pytest.mark.parametrize("nq,nk", [(12, 12), (7, 15), (15, 7)])
def test_window_matches_torch_masked_sdpa(left, right, causal, nq, nk):
    q, k, v = rand(2, 2, nq, 8), rand(2, 2, nk, 8), rand(2, 2, nk, 8)
    s = 0.37
    o, lse = attention_fwd64(q, k, v, s, causal, window=(left, right))
    m = _mask(nq, nk, causal, left, right)
    live = m.any(axis=1)
    ref = torch.nn.functional.scaled_dot_product_attention(_t(q), _t(k), _t(v), attn_mask=_t(m), scale=s)
    np.testing.assert_allclose(o[:, :, live], ref.numpy()[:, :, live], atol=1e-12)
    np.testing.assert_array_equal(o[:, :, ~live], 0.0)
    sc = (s * _t(q) @ _t(k).transpose(-1, -2)).masked_fill(~_t(m), float("-inf"))
    np.testing.assert_allclose(lse[:, :, live], torch.logsumexp(sc, -1).numpy()[:, :, live], atol=1e-12)
    assert np.all(np.isneginf(lse[:, :, ~live]))


@pytest.mark.parametrize("left,right,causal", WINDOWS)
def test_window_bwd_matches_torch_autograd(left, right, causal):
    nq, nk = 10, 13
    q, k, v, do = rand(1, 2, nq, 6), rand(1, 2, nk, 6), rand(1, 2, nk, 6), rand(1, 2, nq, 6)
    s = 0.45
    m = _mask(nq, nk, causal, left, right)
    live = m.any(axis=1)
    tq, tk, tv = _t(q, True), _t(k, True), _t(v, True)
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=_t(m), scale=s)
    # rows with no admitted key are NaN in torch; they carry no gradient
    out = torch.where(_t(live)[None, None, :, None], out, torch.zeros((), dtype=out.dtype))
    out.backward(_t(do))
    dq, dk, dv = attention_bwd64(q, k, v, do, s, causal, window=(left, right))
    np.testing.assert_allclose(dq, np.nan_to_num(tq.grad.numpy()), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)
    np.testing.assert_array_equal(dq[:, :, ~live], 0.0)


def test_window_brute_force_loops():
    """Tiny case with scalar loops and math.exp, window (1, 2), non-causal."""
    Nq, Nk, d, s = 6, 5, 3, 0.8
    q, k, v = rand(1, 1, Nq, d), rand(1, 1, Nk, d), rand(1, 1, Nk, d)
    o, lse = attention_fwd64(q, k, v, s, False, window=(1, 2))
    for i in range(Nq):
        keys = [j for j in range(Nk) if i - 1 <= j <= i + 2]
        sc = [s * sum(q[0, 0, i, t] * k[0, 0, j, t] for t in range(d)) for j in keys]
        z = sum(math.exp(x) for x in sc)
        for t in range(d):
            ref = sum(math.exp(x) * v[0, 0, j, t] for x, j in zip(sc, keys)) / z
            assert abs(o[0, 0, i, t] - ref) < 1e-12
        assert abs(lse[0, 0, i] - math.log(z)) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_wide_window_is_no_window(causal):
    q, k, v = rand(1, 2, 9, 4), rand(1, 2, 11, 4), rand(1, 2, 11, 4)
    o0, l0 = attention_fwd64(q, k, v, 0.5, causal)
    o1, l1 = attention_fwd64(q, k, v, 0.5, causal, window=(11, 11))
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(l0, l1)


def test_window_rows_variant_matches_full():
    q, k, v = rand(1, 2, 20, 4), rand(1, 1, 20, 4), rand(1, 1, 20, 4)
    rows = np.stack([np.stack([RNG.choice(20, 5, replace=False) for _ in range(2)])])
    o, lse = attention_fwd64(q, k, v, 0.4, True, window=(3, -1))
    orow, lrow = attention_rows_fwd64(q, k, v, 0.4, True, rows, window=(3, -1))
    for h in range(2):
        np.testing.assert_allclose(orow[0, h], o[0, h][rows[0, h]], atol=1e-14)
        np.testing.assert_allclose(lrow[0, h], lse[0, h][rows[0, h]], atol=1e-14)


@pytest.mark.parametrize("window,causal", [((1, 1), False), ((2, -1), True)])
def test_window_gqa_bwd_finite_differences(window, causal):
    """Central differences of L = sum(O * dO) with two query heads on one
    K/V head and a window, h = 1e-6, every element."""
    s, n, d = 0.7, 5, 3
    q, k, v, do = rand(1, 2, n, d), rand(1, 1, n, d), rand(1, 1, n, d), rand(1, 2, n, d)
    dq, dk, dv = attention_bwd64(q, k, v, do, s, causal, window=window)

    def loss():
        o, _ = attention_fwd64(q, k, v, s, causal, window=window)
        return float(np.sum(o * do))

    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = loss()
            x[idx] = old - h
            lm = loss()
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        err = np.abs(num - g).max() / max(np.abs(num).max(), 1e-3)
        assert err < 1e-6, err


@pytest.mark.parametrize("window,causal", [((3, -1), True), ((2, 4), False), ((0, 0), False)])
def test_rows_dq_matches_full_gqa_window(window, causal):
    """Row-restricted dQ with fewer K/V heads and a window equals those rows
    of the full backward (including rows whose window is cut by the ends)."""
    q, do = rand(1, 4, 25, 8), rand(1, 4, 25, 8)
    k, v = rand(1, 2, 25, 8), rand(1, 2, 25, 8)
    rows = np.array([[[0, 24, 12], [1, 2, 3], [24, 23, 0], [7, 7, 19]]])
    dq, _, _ = attention_bwd64(q, k, v, do, 0.5, causal, window=window)
    got = attention_rows_dq64(q, k, v, do, 0.5, causal, rows, window=window)
    for h in range(4):
        np.testing.assert_allclose(got[0, h], dq[0, h][rows[0, h]], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("window,causal", [((1, 1), False), ((2, -1), True), ((0, 0), False), ((-1, 2), False)])
def test_gqa_window_bwd_outer_identities(window, causal):
    """The gradient identities per K/V head, its sums running over the query
    heads that use it (h // G), with windowed rows that admit no key (25
    queries on 17 keys: under (1, 1) and (0, 0) the last rows see none and
    contribute nothing)."""
    q, k, v, do = rand(2, 6, 25, 8), rand(2, 2, 17, 8), rand(2, 2, 17, 8), rand(2, 6, 25, 8)
    o, lse = attention_fwd64(q, k, v, 0.45, causal, window=window)
    dq, dk, dv = attention_bwd64(q, k, v, do, 0.45, causal, window=window)
    if window in ((1, 1), (0, 0)):
        assert np.isneginf(lse[:, :, -1]).all()
    err = identity_errors(q, k, v, do, o, dq, dk, dv)
    assert max(err.values()) < 1e-12, err
