"""Pins of the oracle's dropout (CPU).

The generator is Philox4x32-10 from its published definition (Salmon,
Moraes, Dror, Shaw, SC'11); it is pinned to the known-answer vectors that
accompany that paper's reference implementation, and to a scalar
re-implementation.  The element -> (counter, byte) convention is pinned by
scalar loops; the dropout arithmetic by p = 0, unbiasedness over seeds,
torch autograd through an explicit masked softmax, and finite differences.
"""
import numpy as np
import pytest
import torch

from grad_identities import identity_errors
from oracle import (attention_bwd64, attention_fwd64, attention_rows_dq64, dropout_keep, dropout_threshold,
                    philox4x32_10)

RNG = np.random.default_rng(2468)  # reseeded per test (tests/conftest.py)
M32 = 0xFFFFFFFF


def rand(*shape):
    return RNG.standard_normal(shape)


def philox_scalar(ctr, key):
    """Plain-int Philox4x32-10, written independently of the oracle's."""
    x = list(ctr)
    k0, k1 = key
    for r in range(10):
        if r:
            k0, k1 = (k0 + 0x9E3779B9) & M32, (k1 + 0xBB67AE85) & M32
        a = 0xD2511F53 * x[0]
        c = 0xCD9E8D57 * x[2]
        x = [(c >> 32) ^ x[1] ^ k0, c & M32, (a >> 32) ^ x[3] ^ k1, a & M32]
    return x


@pytest.mark.parametrize("ctr,key,want", [
    ((0, 0, 0, 0), (0, 0), (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((M32,) * 4, (M32, M32), (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
])
def test_philox_known_answers(ctr, key, want):
    assert tuple(int(w) for w in philox4x32_10(ctr, key)) == want
    assert tuple(philox_scalar(ctr, key)) == want


def test_philox_vectorised_matches_scalar():
    ctr = RNG.integers(0, 1 << 32, size=(200, 4), dtype=np.uint64)
    key = RNG.integers(0, 1 << 32, size=(200, 2), dtype=np.uint64)
    got = philox4x32_10(ctr, key)
    for n in range(200):
        assert list(got[n]) == philox_scalar([int(c) for c in ctr[n]], [int(k) for k in key[n]])


@pytest.mark.parametrize("p,thr", [(0.0, 0), (0.1, 26), (0.5, 128), (0.0019, 0), (0.002, 1), (0.999, 255)])
def test_threshold(p, thr):
    t, s = dropout_threshold(p)
    assert t == thr and s == 256.0 / (256 - thr)


@pytest.mark.parametrize("bad", [-0.1, 1.0, 1.5, float("nan")])
def test_threshold_rejects(bad):
    with pytest.raises(ValueError):
        dropout_threshold(bad)


def test_keep_mapping_by_scalar_loops():
    """Element (b, h, i, j): counter (2*(j>>5) + ((j>>2)&1), i, b*H+h, offset),
    key (seed lo, seed hi), byte j&3 of word (j>>3)&3, kept iff >= thr."""
    B, H, Nq, Nk, p, seed, off = 2, 3, 9, 70, 0.3, (7 << 40) + 12345, 99
    thr, _ = dropout_threshold(p)
    for b in range(B):
        for h in range(H):
            got = dropout_keep(b, h, H, np.arange(Nq), Nk, p, seed, off)
            for i in range(Nq):
                for j in range(Nk):
                    w = philox_scalar((2 * (j >> 5) + ((j >> 2) & 1), i, b * H + h, off),
                                      (seed & M32, seed >> 32))
                    byte = (w[(j >> 3) & 3] >> (8 * (j & 3))) & 0xFF
                    assert bool(got[i, j]) == (byte >= thr), (b, h, i, j)


def test_keep_fraction_and_independence():
    p = 0.37
    thr, _ = dropout_threshold(p)
    q = (256 - thr) / 256
    a = dropout_keep(0, 0, 2, np.arange(512), 2048, p, 42, 0)
    b = dropout_keep(0, 1, 2, np.arange(512), 2048, p, 42, 0)
    n = a.size
    sig = np.sqrt(q * (1 - q) / n)
    assert abs(a.mean() - q) < 6 * sig and abs(b.mean() - q) < 6 * sig
    agree = (a == b).mean()
    want = q * q + (1 - q) * (1 - q)
    assert abs(agree - want) < 6 * np.sqrt(want * (1 - want) / n)
    c = dropout_keep(0, 0, 2, np.arange(512), 2048, p, 42, 1)  # another offset: another mask
    assert abs((a == c).mean() - want) < 6 * np.sqrt(want * (1 - want) / n)


@pytest.mark.parametrize("causal", [False, True])
def test_p_zero_is_no_dropout(causal):
    q, k, v, do = rand(1, 2, 13, 8), rand(1, 1, 17, 8), rand(1, 1, 17, 8), rand(1, 2, 13, 8)
    o0, l0 = attention_fwd64(q, k, v, 0.4, causal)
    o1, l1 = attention_fwd64(q, k, v, 0.4, causal, dropout=(0.0, 5, 6))
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(l0, l1)
    for g0, g1 in zip(attention_bwd64(q, k, v, do, 0.4, causal), attention_bwd64(q, k, v, do, 0.4, causal,
                                                                                dropout=(0.0, 5, 6))):
        np.testing.assert_array_equal(g0, g1)


def test_unbiased_over_seeds():
    """The mean of the dropped output over many seeds approaches the
    undropped output (s_keep restores the expectation); lse never changes."""
    q, k, v = rand(1, 1, 6, 4), rand(1, 1, 40, 4), rand(1, 1, 40, 4)
    o0, l0 = attention_fwd64(q, k, v, 0.5, False)
    acc = np.zeros_like(o0)
    n = 600
    for seed in range(n):
        o, l = attention_fwd64(q, k, v, 0.5, False, dropout=(0.25, seed, 3))
        np.testing.assert_array_equal(l, l0)
        acc += o
    assert np.abs(acc / n - o0).max() < 0.05


@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (4, -1))])
def test_dropout_bwd_matches_torch_autograd(causal, window):
    """torch autograd through softmax(S) * keep * s_keep @ V with the same mask."""
    B, H, Hkv, N, d, s, p, seed, off = 1, 2, 1, 11, 6, 0.45, 0.3, 77, 5
    q, k, v, do = rand(B, H, N, d), rand(B, Hkv, N, d), rand(B, Hkv, N, d), rand(B, H, N, d)
    thr, sk = dropout_threshold(p)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, v))
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    allowed = np.ones((N, N), bool)
    if causal:
        allowed &= j <= i
    if window[0] >= 0:
        allowed &= j >= i - window[0]
    out = []
    for h in range(H):
        S = s * tq[0, h] @ tk[0, h // 2].T
        S = S.masked_fill(torch.from_numpy(~allowed), float("-inf"))
        keep = torch.from_numpy(dropout_keep(0, h, H, np.arange(N), N, p, seed, off).astype(np.float64))
        out.append((torch.softmax(S, -1) * keep * sk) @ tv[0, h // 2])
    torch.stack(out)[None].backward(torch.from_numpy(do))
    o, _ = attention_fwd64(q, k, v, s, causal, window=window, dropout=(p, seed, off))
    np.testing.assert_allclose(o, torch.stack(out)[None].detach().numpy(), atol=1e-12)
    dq, dk, dv = attention_bwd64(q, k, v, do, s, causal, window=window, dropout=(p, seed, off))
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


def test_dropout_bwd_finite_differences():
    s, n, d, dr = 0.7, 6, 3, (0.4, 1234, 9)
    q, k, v, do = rand(1, 1, n, d), rand(1, 1, n, d), rand(1, 1, n, d), rand(1, 1, n, d)
    dq, dk, dv = attention_bwd64(q, k, v, do, s, True, dropout=dr)

    def loss():
        o, _ = attention_fwd64(q, k, v, s, True, dropout=dr)
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


@pytest.mark.parametrize("causal", [False, True])
def test_rows_dq_matches_full_with_dropout(causal):
    """Row-restricted dQ under dropout (the rows' own keep bits, by global
    row index) equals those rows of the full backward."""
    q, k, v, do = rand(2, 3, 40, 8), rand(2, 3, 40, 8), rand(2, 3, 40, 8), rand(2, 3, 40, 8)
    drop = (0.3, (7 << 32) + 5, 3)
    rows = np.tile(np.array([0, 9, 33, 39]), (2, 3, 1))
    dq, _, _ = attention_bwd64(q, k, v, do, 0.35, causal, dropout=drop)
    got = attention_rows_dq64(q, k, v, do, 0.35, causal, rows, dropout=drop)
    for b in range(2):
        for h in range(3):
            np.testing.assert_allclose(got[b, h], dq[b, h][rows[b, h]], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (5, -1))])
def test_dropout_bwd_outer_identities(causal, window):
    """With dropout O and dV use the kept weights W = P keep s_keep and dS the
    kept dP, and the gradient identities still hold: sum_i dQ_i q_i^T =
    sum_j k_j dK_j^T, sum_i O_i dO_i^T = sum_j v_j dV_j^T, sum_j dK_j = 0
    (a keep mask applied to O but not to dV, or to dQ's dS but not to dK's,
    breaks one of them)."""
    q, k, v, do = rand(2, 4, 30, 8), rand(2, 2, 30, 8), rand(2, 2, 30, 8), rand(2, 4, 30, 8)
    drop = (0.3, (5 << 32) + 11, 7)
    o, _ = attention_fwd64(q, k, v, 0.5, causal, window=window, dropout=drop)
    dq, dk, dv = attention_bwd64(q, k, v, do, 0.5, causal, window=window, dropout=drop)
    err = identity_errors(q, k, v, do, o, dq, dk, dv)
    assert max(err.values()) < 1e-12, err
