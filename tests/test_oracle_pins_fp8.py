"""Pins of the fp8 (e4m3fn) oracle and of its weight-rounding error model (CPU).

Independent references: torch's own float8_e4m3fn conversions (a library
routine), the OFP8 E4M3 values written out by hand, torch's float64 SDPA on
torch-decoded inputs, a closed-form homogeneity identity for the descale
factors, and a brute-force emulation of rounding the weights to e4m3fn
against which the error model's bound and standard deviation are checked.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention_fp8_fwd64, attention_fp8_rows_fwd64, e4m3fn_to_float64, fp8_rounding_model

RNG = np.random.default_rng(8080)  # reseeded per test (tests/conftest.py)


def fp8_inputs(B, H, Hkv, Nq, Nk, d, scale_in=1.0):
    """Random e4m3fn bytes (torch's round-to-nearest-even cast of normals)."""
    out = []
    for hh, n in ((H, Nq), (Hkv, Nk), (Hkv, Nk)):
        a = torch.from_numpy(RNG.standard_normal((B, hh, n, d)) * scale_in).to(torch.float8_e4m3fn)
        out.append(a.view(torch.uint8).numpy().copy())
    return out


def torch_decode(b):
    return torch.from_numpy(np.ascontiguousarray(b)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


# ---------------------------------------------------------------- the byte format

def test_decode_matches_torch_on_every_byte():
    b = np.arange(256, dtype=np.uint8)
    ours = e4m3fn_to_float64(b)
    ref = torch_decode(b)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


@pytest.mark.parametrize("byte,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x0f, 1.875 * 2.0 ** -6),
    (0x38, 1.0), (0x39, 1.125), (0x3f, 1.875), (0x40, 2.0), (0x1d, 1.625 * 2.0 ** -4), (0x77, 240.0),
    (0x7e, 448.0), (0xb8, -1.0), (0xfe, -448.0), (0x81, -(2.0 ** -9)),
])
def test_decode_closed_forms(byte, value):
    assert e4m3fn_to_float64(np.array([byte], dtype=np.uint8))[0] == value


def test_decode_special_patterns():
    v = e4m3fn_to_float64(np.array([0x7f, 0xff, 0x80], dtype=np.uint8))
    assert np.isnan(v[0]) and np.isnan(v[1])
    assert v[2] == 0.0 and np.signbit(v[2])


def test_decode_monotone_and_symmetric():
    pos = e4m3fn_to_float64(np.arange(0x7f, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    neg = e4m3fn_to_float64(np.arange(0x80, 0xff, dtype=np.uint8))
    assert np.array_equal(neg, -pos)


def test_decode_roundtrips_through_torch_cast():
    b = np.array([x for x in range(256) if x not in (0x7f, 0xff, 0x80)], dtype=np.uint8)
    back = torch.from_numpy(e4m3fn_to_float64(b)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(back, b)


# ---------------------------------------------------------------- attention on fp8 inputs

@pytest.mark.parametrize("H,Hkv,causal", [(2, 2, False), (4, 1, True), (4, 2, True)])
def test_fp8_attention_is_sdpa_of_decoded_inputs(H, Hkv, causal):
    q8, k8, v8 = fp8_inputs(2, H, Hkv, 37, 37, 32)
    scale = 0.3
    o, lse = attention_fp8_fwd64(q8, k8, v8, scale, causal)
    q, k, v = (torch.from_numpy(torch_decode(x)) for x in (q8, k8, v8))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=scale,
                                                           enable_gqa=Hkv != H)
    assert np.allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    G = H // Hkv
    s = scale * torch.einsum("bhqd,bhkd->bhqk", q, k.repeat_interleave(G, dim=1))
    if causal:
        s = s.masked_fill(torch.ones(37, 37, dtype=torch.bool).triu(1), -math.inf)
    assert np.allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)


def test_descale_factors_are_homogeneous():
    """O(a q, b k, c v; scale) = c O(q, k, v; a b scale); lse likewise with
    scale a b."""
    q8, k8, v8 = fp8_inputs(1, 3, 3, 40, 52, 64)
    a, b, c = 0.25, 3.0, -1.5
    o1, l1 = attention_fp8_fwd64(q8, k8, v8, 0.2, False, descale=(a, b, c))
    o0, l0 = attention_fp8_fwd64(q8, k8, v8, 0.2 * a * b, False)
    assert np.allclose(o1, c * o0, rtol=1e-13, atol=1e-13)
    assert np.allclose(l1, l0, rtol=1e-13, atol=1e-13)


def test_rows_variant_matches_full():
    q8, k8, v8 = fp8_inputs(1, 2, 1, 50, 50, 64)
    rows = np.array([[[0, 7, 49]], [[3, 4, 5]]]).reshape(1, 2, 3)
    o, lse = attention_fp8_fwd64(q8, k8, v8, 0.125, True, window=(10, -1), descale=(2.0, 0.5, 1.0))
    orr, lr = attention_fp8_rows_fwd64(q8, k8, v8, 0.125, True, rows, window=(10, -1), descale=(2.0, 0.5, 1.0))
    for h in range(2):
        assert np.array_equal(orr[0, h], o[0, h][rows[0, h]])
        assert np.array_equal(lr[0, h], lse[0, h][rows[0, h]])


# ---------------------------------------------------------------- the weight-rounding error model

def emulate_fp8_weights(q8, k8, v8, scale, causal, lag, window=(-1, -1)):
    """Brute-force stand-in for the kernel's arithmetic: weights
    p_j = 2^(log2(e) (s_j - s_max) + lag) rounded to e4m3fn by torch's cast,
    O = sum_j round(p_j) v_j / sum_j p_j, then rounded to bf16."""
    q, k, v = (e4m3fn_to_float64(x) for x in (q8, k8, v8))
    B, H, Nq, d = q.shape
    G = H // k.shape[1]
    Nk = k.shape[2]
    out = np.empty_like(q)
    for b in range(B):
        for h in range(H):
            s = scale * q[b, h] @ k[b, h // G].T
            for i in range(Nq):
                for j in range(Nk):
                    if (causal and j > i) or (window[0] >= 0 and j < i - window[0]):
                        s[i, j] = -np.inf
            smax = s.max(axis=1, keepdims=True)
            p = np.exp2(math.log2(math.e) * (s - smax) + lag)
            pr = torch.from_numpy(p).to(torch.float8_e4m3fn).to(torch.float64).numpy()
            o = pr @ v[b, h // G] / p.sum(axis=1, keepdims=True)
            out[b, h] = torch.from_numpy(o).to(torch.bfloat16).to(torch.float64).numpy()
    return out


@pytest.mark.parametrize("lag", [0.0, 2.5, 8.7])
@pytest.mark.parametrize("causal", [False, True])
def test_error_model_bounds_emulated_rounding(lag, causal):
    q8, k8, v8 = fp8_inputs(1, 2, 1, 64, 300, 64)
    scale = 1 / 8.0
    rows = np.tile(np.arange(64), (1, 2, 1))
    exact, _ = attention_fp8_fwd64(q8, k8, v8, scale, causal)
    bound, sigma = fp8_rounding_model(q8, k8, v8, scale, causal, rows)
    emu = emulate_fp8_weights(q8, k8, v8, scale, causal, lag)
    err = emu - exact
    assert np.all(np.abs(err) <= bound)
    # sigma = 0 only where nothing can round (a row's one admitted key with
    # a zero value): the error must be exactly 0 there
    flat = sigma == 0
    assert np.all(err[flat] == 0.0)
    z2 = np.mean((err[~flat] / sigma[~flat]) ** 2)
    # the uniform-rounding model is an upper bound in expectation; at lag 0
    # it is close (the row maximum, weight 1, rounds exactly, which short
    # causal rows feel most)
    assert z2 <= 1.2
    if lag == 0.0:
        assert z2 >= 0.4


def test_error_model_rejects_a_misaligned_value_row():
    """A plausible kernel defect (values paired with the neighbouring key)
    breaks both the bound and the statistical check."""
    q8, k8, v8 = fp8_inputs(1, 1, 1, 64, 200, 64)
    scale = 1 / 8.0
    rows = np.arange(64).reshape(1, 1, 64)
    exact, _ = attention_fp8_fwd64(q8, k8, v8, scale, False)
    bound, sigma = fp8_rounding_model(q8, k8, v8, scale, False, rows)
    wrong, _ = attention_fp8_fwd64(q8, k8, np.roll(v8, 1, axis=2), scale, False)
    err = wrong - exact
    assert np.any(np.abs(err) > bound)
    assert np.mean((err / sigma) ** 2) > 4.0


def test_error_model_rejects_coarser_weight_rounding():
    """Weights rounded to 2 mantissa bits (e5m2) instead of 3 fail the
    statistical check."""
    q8, k8, v8 = fp8_inputs(1, 2, 2, 64, 256, 64)
    scale = 1 / 8.0
    rows = np.tile(np.arange(64), (1, 2, 1))
    exact, _ = attention_fp8_fwd64(q8, k8, v8, scale, False)
    _, sigma = fp8_rounding_model(q8, k8, v8, scale, False, rows)
    q, k, v = (e4m3fn_to_float64(x) for x in (q8, k8, v8))
    s = scale * np.einsum("bhqd,bhkd->bhqk", q, k)
    p = np.exp(s - s.max(axis=-1, keepdims=True))
    pr = torch.from_numpy(p).to(torch.float8_e5m2).to(torch.float64).numpy()
    coarse = np.einsum("bhqk,bhkd->bhqd", pr, v) / p.sum(axis=-1)[..., None]
    assert np.mean(((coarse - exact) / sigma) ** 2) > 2.0
