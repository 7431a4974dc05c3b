"""Pins of the fp64 oracle to facts other than itself (CPU only).

The pages print no numeric worked example (see tests/golden/README.md), so
every pin is a closed form, an invariant, brute force on tiny inputs, an
independent re-derivation, a library special case, or finite differences.
Each is chosen so that a plausible slip in the oracle (dropped scale, wrong
mask direction, transposed operand, missing normaliser, wrong sign in dS)
fails at least one of them.
"""
import itertools
import math

import numpy as np
import pytest
import torch

from grad_identities import identity_errors
from oracle import attention_bwd64, attention_fwd64, attention_rows_dq64, attention_rows_fwd64

RNG = np.random.default_rng(1234)  # reseeded per test (tests/conftest.py)


def rand(*shape):
    return RNG.standard_normal(shape)


# ---------------------------------------------------------------- forward

def test_hand_worked_2x2():
    """Worked by hand: q = k = I_2, v = [[1,2],[3,4]], scale 1.
    Non-causal row 0 scores [1, 0]: weights e/(1+e), 1/(1+e).
    Causal row 0 sees only key 0; causal row 1 scores [0, 1]."""
    e = math.e
    q = np.eye(2)[None, None]
    k = np.eye(2)[None, None]
    v = np.array([[1.0, 2.0], [3.0, 4.0]])[None, None]
    o, lse = attention_fwd64(q, k, v, 1.0, False)
    np.testing.assert_allclose(o[0, 0, 0], [(e + 3) / (1 + e), (2 * e + 4) / (1 + e)], rtol=0, atol=1e-14)
    np.testing.assert_allclose(o[0, 0, 1], [(1 + 3 * e) / (1 + e), (2 + 4 * e) / (1 + e)], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], [math.log(1 + e)] * 2, rtol=0, atol=1e-14)
    o, lse = attention_fwd64(q, k, v, 1.0, True)
    np.testing.assert_allclose(o[0, 0, 0], [1.0, 2.0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(o[0, 0, 1], [(1 + 3 * e) / (1 + e), (2 + 4 * e) / (1 + e)], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], [1.0, math.log(1 + e)], rtol=0, atol=1e-14)


def test_scale_enters_once():
    """Doubling the scale equals doubling q (pins that scale multiplies q.k)."""
    q, k, v = rand(1, 2, 7, 5), rand(1, 2, 9, 5), rand(1, 2, 9, 5)
    o1, l1 = attention_fwd64(q, k, v, 0.7, False)
    o2, l2 = attention_fwd64(2 * q, k, v, 0.35, False)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_all_equal_keys(causal):
    """Every k_j equal: weights uniform over the visible keys, so O_i is the
    mean of those V rows and lse_i = s q_i.k0 + log(count)."""
    B, H, N, d, s = 2, 3, 11, 6, 0.37
    q, v = rand(B, H, N, d), rand(B, H, N, d)
    k0 = rand(B, H, 1, d)
    k = np.repeat(k0, N, axis=2)
    o, lse = attention_fwd64(q, k, v, s, causal)
    for i in range(N):
        cnt = i + 1 if causal else N
        np.testing.assert_allclose(o[:, :, i], v[:, :, :cnt].mean(axis=2), atol=1e-12)
        np.testing.assert_allclose(lse[:, :, i], s * np.sum(q[:, :, i] * k0[:, :, 0], -1) + math.log(cnt),
                                   atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_rows_sum_to_one(causal):
    """With V = ones every output element is sum_j P_ij, which must be 1."""
    q, k = rand(1, 2, 13, 4), rand(1, 2, 13, 4)
    o, _ = attention_fwd64(q, k, np.ones((1, 2, 13, 4)), 1.3, causal)
    np.testing.assert_allclose(o, 1.0, atol=1e-12)


def test_dominant_key():
    """q_i = a e1, k_j* = a e1, other keys 0: s a^2 >= 50 puts all weight on
    j*, so O_i = V_j* up to Nk * exp(-50) * max|V|."""
    N, d, a = 16, 64, 20.0
    s = 1.0 / 8.0  # 1/sqrt(64); s*a^2 = 50
    for jstar in (0, 5, N - 1):
        q = np.zeros((1, 1, N, d)); q[..., 0] = a
        k = np.zeros((1, 1, N, d)); k[0, 0, jstar, 0] = a
        v = rand(1, 1, N, d)
        o, lse = attention_fwd64(q, k, v, s, False)
        bound = N * math.exp(-50) * np.abs(v).max() * 2
        np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0, jstar], (N, d)), atol=bound)
        np.testing.assert_allclose(lse[0, 0], 50.0 + math.log1p((N - 1) * math.exp(-50)), atol=1e-12)


def test_causal_row0_and_single_key():
    """Causal row 0 sees only key 0: O_0 = V_0, lse_0 = s q0.k0.  With one
    key (non-causal) every row is V_0."""
    q, k, v = rand(2, 2, 9, 8), rand(2, 2, 9, 8), rand(2, 2, 9, 8)
    s = 0.25
    o, lse = attention_fwd64(q, k, v, s, True)
    np.testing.assert_allclose(o[:, :, 0], v[:, :, 0], atol=1e-14)
    np.testing.assert_allclose(lse[:, :, 0], s * np.sum(q[:, :, 0] * k[:, :, 0], -1), atol=1e-13)
    o1, lse1 = attention_fwd64(q, k[:, :, :1], v[:, :, :1], s, False)
    np.testing.assert_allclose(o1, np.broadcast_to(v[:, :, :1], o1.shape), atol=1e-14)
    np.testing.assert_allclose(lse1, s * np.einsum("bhnd,bhd->bhn", q, k[:, :, 0]), atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift(causal):
    """k_j -> k_j + u leaves O unchanged and shifts lse_i by s q_i.u."""
    q, k, v = rand(1, 2, 10, 5), rand(1, 2, 10, 5), rand(1, 2, 10, 5)
    u = rand(1, 2, 1, 5)
    s = 0.6
    o1, l1 = attention_fwd64(q, k, v, s, causal)
    o2, l2 = attention_fwd64(q, k + u, v, s, causal)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l2 - l1, s * np.einsum("bhnd,bhd->bhn", q, u[:, :, 0]), atol=1e-12)


def test_linear_in_v():
    q, k = rand(1, 1, 8, 4), rand(1, 1, 8, 4)
    v1, v2 = rand(1, 1, 8, 4), rand(1, 1, 8, 4)
    a, b = 1.7, -0.3
    o1, _ = attention_fwd64(q, k, v1, 0.5, True)
    o2, _ = attention_fwd64(q, k, v2, 0.5, True)
    o3, _ = attention_fwd64(q, k, a * v1 + b * v2, 0.5, True)
    np.testing.assert_allclose(o3, a * o1 + b * o2, atol=1e-12)


def test_permutation_equivariance():
    """Non-causal: permuting keys (with their values) changes nothing;
    permuting queries permutes the output rows."""
    q, k, v = rand(1, 1, 9, 4), rand(1, 1, 12, 4), rand(1, 1, 12, 4)
    pk = RNG.permutation(12)
    pq = RNG.permutation(9)
    o, l = attention_fwd64(q, k, v, 0.9, False)
    o2, l2 = attention_fwd64(q[:, :, pq], k[:, :, pk], v[:, :, pk], 0.9, False)
    np.testing.assert_allclose(o2, o[:, :, pq], atol=1e-12)
    np.testing.assert_allclose(l2, l[:, :, pq], atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_loops(causal):
    """Tiny case recomputed with scalar Python loops and math.exp."""
    Nq, Nk, d, s = 5, 7, 3, 0.8
    q, k, v = rand(1, 1, Nq, d), rand(1, 1, Nk, d), rand(1, 1, Nk, d)
    o, lse = attention_fwd64(q, k, v, s, causal)
    for i in range(Nq):
        keys = [j for j in range(Nk) if not (causal and j > i)]
        sc = [s * sum(q[0, 0, i, t] * k[0, 0, j, t] for t in range(d)) for j in keys]
        z = sum(math.exp(x) for x in sc)
        for t in range(d):
            ref = sum(math.exp(x) * v[0, 0, j, t] for x, j in zip(sc, keys)) / z
            assert abs(o[0, 0, i, t] - ref) < 1e-12
        assert abs(lse[0, 0, i] - math.log(z)) < 1e-12


def _online_softmax_tiled(q, k, v, s, causal, bm, bn):
    """Independent fp64 re-derivation of the method: Q split into row blocks,
    K/V streamed in column blocks, a running max m and sum l per row, the
    partial output rescaled whenever m grows (glossary article, "Online
    Softmax"), merged and normalised once at the end."""
    Nq, d = q.shape
    Nk = k.shape[0]
    o = np.zeros((Nq, d))
    lse = np.zeros(Nq)
    for i0 in range(0, Nq, bm):
        qi = q[i0:i0 + bm]
        rows = np.arange(i0, i0 + qi.shape[0])
        m = np.full(qi.shape[0], -np.inf)
        l = np.zeros(qi.shape[0])
        acc = np.zeros((qi.shape[0], d))
        for j0 in range(0, Nk, bn):
            kj, vj = k[j0:j0 + bn], v[j0:j0 + bn]
            sc = s * qi @ kj.T
            if causal:
                cols = np.arange(j0, j0 + kj.shape[0])
                sc = np.where(cols[None, :] > rows[:, None], -np.inf, sc)
            m_new = np.maximum(m, sc.max(axis=1))
            alpha = np.where(np.isneginf(m), 0.0, np.exp(m - np.where(np.isneginf(m_new), 0, m_new)))
            p = np.exp(sc - m_new[:, None])
            l = alpha * l + p.sum(axis=1)
            acc = alpha[:, None] * acc + p @ vj
            m = m_new
        o[i0:i0 + bm] = acc / l[:, None]
        lse[i0:i0 + bm] = m + np.log(l)
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
def test_tiled_online_softmax_matches(causal):
    q, k, v = rand(1, 1, 37, 8), rand(1, 1, 41, 8), rand(1, 1, 41, 8)
    o, lse = attention_fwd64(q, k, v, 0.35, causal)
    for bm, bn in [(1, 1), (4, 7), (16, 5), (64, 64), (3, 41)]:
        ot, lt = _online_softmax_tiled(q[0, 0], k[0, 0], v[0, 0], 0.35, causal, bm, bn)
        np.testing.assert_allclose(ot, o[0, 0], atol=1e-12)
        np.testing.assert_allclose(lt, lse[0, 0], atol=1e-12)


@pytest.mark.parametrize("causal,nq,nk", [(False, 17, 17), (True, 17, 17), (True, 9, 23), (True, 23, 9)])
def test_matches_torch_sdpa_fp64(causal, nq, nk):
    """Library special case: torch's CPU float64 SDPA (math backend)."""
    q, k, v = rand(2, 3, nq, 16), rand(2, 3, nk, 16), rand(2, 3, nk, 16)
    s = 0.29
    o, lse = attention_fwd64(q, k, v, s, causal)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=causal, scale=s)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12)
    sc = s * torch.from_numpy(q) @ torch.from_numpy(k).transpose(-1, -2)
    if causal:
        sc = sc.masked_fill(torch.ones(nq, nk, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(sc, -1).numpy(), atol=1e-12)


def test_rows_variant_matches_full():
    q, k, v = rand(2, 2, 30, 8), rand(2, 2, 30, 8), rand(2, 2, 30, 8)
    rows = np.stack([np.stack([RNG.choice(30, 6, replace=False) for _ in range(2)]) for _ in range(2)])
    for causal in (False, True):
        o, lse = attention_fwd64(q, k, v, 0.4, causal)
        orow, lrow = attention_rows_fwd64(q, k, v, 0.4, causal, rows)
        for b, h in itertools.product(range(2), range(2)):
            np.testing.assert_allclose(orow[b, h], o[b, h][rows[b, h]], atol=1e-14)
            np.testing.assert_allclose(lrow[b, h], lse[b, h][rows[b, h]], atol=1e-14)


# ---------------------------------------------------------------- backward

def _loss(q, k, v, do, s, causal):
    o, _ = attention_fwd64(q, k, v, s, causal)
    return float(np.sum(o * do))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(1, 1), (2, 3), (5, 4), (8, 8), (3, 7)])
def test_bwd_finite_differences(causal, n, d):
    """Central differences of L = sum(O * dO), h = 1e-6, every element."""
    s = 0.7
    q, k, v, do = rand(1, 1, n, d), rand(1, 1, n, d), rand(1, 1, n, d), rand(1, 1, n, d)
    dq, dk, dv = attention_bwd64(q, k, v, do, s, causal)
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(q, k, v, do, s, causal)
            x[idx] = old - h
            lm = _loss(q, k, v, do, s, causal)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        err = np.abs(num - g).max() / max(np.abs(num).max(), 1e-3)
        assert err < 1e-6, err


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_matches_torch_autograd(causal):
    q, k, v, do = rand(2, 2, 19, 8), rand(2, 2, 19, 8), rand(2, 2, 19, 8), rand(2, 2, 19, 8)
    s = 0.45
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=s)
    out.backward(torch.from_numpy(do))
    dq, dk, dv = attention_bwd64(q, k, v, do, s, causal)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_identities(causal):
    """Rows of dS sum to zero, so sum_j dK_j = 0; rows of P sum to one, so
    sum_j dV_j = sum_i dO_i.  Causal row 0's query gradient is zero (its
    softmax has a single entry)."""
    q, k, v, do = rand(1, 3, 21, 8), rand(1, 3, 21, 8), rand(1, 3, 21, 8), rand(1, 3, 21, 8)
    dq, dk, dv = attention_bwd64(q, k, v, do, 0.3, causal)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)
    if causal:
        np.testing.assert_allclose(dq[:, :, 0], 0.0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_outer_identities(causal):
    """sum_i dQ_i q_i^T = sum_j k_j dK_j^T (both scale sum_ij dS_ij k_j q_i^T)
    and sum_i O_i dO_i^T = sum_j v_j dV_j^T (both sum_ij P_ij v_j dO_i^T):
    they tie dK to dQ and dV to O with d x d equations per head (a scale
    applied to one gradient only, P for P^T in dV, or a dS sign slip in one
    of dQ and dK breaks them)."""
    q, k, v, do = rand(2, 2, 23, 8), rand(2, 2, 19, 8), rand(2, 2, 19, 8), rand(2, 2, 23, 8)
    o, _ = attention_fwd64(q, k, v, 0.4, causal)
    dq, dk, dv = attention_bwd64(q, k, v, do, 0.4, causal)
    err = identity_errors(q, k, v, do, o, dq, dk, dv)
    assert max(err.values()) < 1e-12, err


def test_outer_identities_under_output_rounding():
    """The GPU tests check these identities on 16-bit outputs at 2e-2.
    Rounding the oracle's inputs and outputs to bf16 moves them by about
    2.4e-3 (a causal head of 512 rows at d = 128, inputs x0.5 as in the
    16K workload), so the bound leaves room for the kernels' own rounding
    of P and dS."""
    def bf(x):
        return torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()

    q, k, v, do = (bf(0.5 * rand(1, 2, 512, 128)) for _ in range(4))
    s = 1.0 / math.sqrt(128)
    o, _ = attention_fwd64(q, k, v, s, True)
    dq, dk, dv = attention_bwd64(q, k, v, do, s, True)
    err = identity_errors(q, k, v, do, bf(o), bf(dq), bf(dk), bf(dv))
    assert max(err.values()) < 5e-3, err


def test_bwd_uses_rowsum_identity_consistently():
    """The kernel-side identity rowsum(P*dP) = dO.O: the oracle's gradients
    must equal those built from D = rowsum(dO*O) with the oracle's own O."""
    q, k, v, do = rand(1, 1, 12, 6), rand(1, 1, 12, 6), rand(1, 1, 12, 6), rand(1, 1, 12, 6)
    s = 0.55
    o, lse = attention_fwd64(q, k, v, s, True)
    D = np.sum(do * o, axis=-1)[0, 0]
    sc = s * q[0, 0] @ k[0, 0].T
    sc = np.where(np.triu(np.ones((12, 12), bool), 1), -np.inf, sc)
    p = np.exp(sc - lse[0, 0][:, None])
    ds = p * (do[0, 0] @ v[0, 0].T - D[:, None])
    dq, dk, _ = attention_bwd64(q, k, v, do, s, True)
    np.testing.assert_allclose(dq[0, 0], s * ds @ k[0, 0], atol=1e-12)
    np.testing.assert_allclose(dk[0, 0], s * ds.T @ q[0, 0], atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_rows_dq_matches_full(causal):
    """dQ restricted to chosen query rows equals those rows of the full
    backward's dQ (itself pinned to finite differences and torch autograd)."""
    q, k, v, do = rand(2, 2, 30, 8), rand(2, 2, 30, 8), rand(2, 2, 30, 8), rand(2, 2, 30, 8)
    rows = np.array([[[0, 5, 29], [3, 3, 17]], [[28, 1, 14], [0, 29, 2]]])
    dq, _, _ = attention_bwd64(q, k, v, do, 0.4, causal)
    got = attention_rows_dq64(q, k, v, do, 0.4, causal, rows)
    for b in range(2):
        for h in range(2):
            np.testing.assert_allclose(got[b, h], dq[b, h][rows[b, h]], rtol=1e-12, atol=1e-13)
