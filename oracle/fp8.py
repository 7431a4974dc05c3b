"""fp64 reference of the fp8 (e4m3fn) forward, and the error model of its
fp8 weight rounding.

TEST INFRASTRUCTURE ONLY: the product path never imports this module.

What is computed, and where it is defined:

* The "Flash Attention" skill guide, Workflow 3 (FlashAttention-3's FP8 path),
  step 3: forward only, q, k and v cast to ``float8_e4m3fn`` before the call.
  The pages give no scaling convention and no accuracy figure.  Readings
  taken: the attention computed is exactly that of the values the fp8 bytes
  encode, each tensor multiplied by an optional per-tensor descale factor
  (1.0 for a plain cast); causal masking, fewer K/V heads and windows as in
  the 16-bit oracle.  So the reference output is ``attention_fwd64`` on the
  decoded, descaled inputs, in fp64.
* The byte format: OCP 8-bit Floating Point Specification (OFP8), E4M3
  ("fn": finite, no infinities).  Sign bit, 4 exponent bits with bias 7,
  3 mantissa bits; exponent field 0 holds subnormals m/8 * 2^-6; the bit
  patterns S.1111.111 are NaN; the largest finite value is 1.75 * 2^8 = 448.
* The error model (``fp8_rounding_model``) is not part of the method: it
  bounds what rounding the attention weights to e4m3fn before the P V
  product costs, so that a test can tell that rounding from a defect.
"""
import numpy as np

from .attention import _allowed, _as64, _check
from .attention import attention_fwd64, attention_rows_fwd64

__all__ = ["e4m3fn_to_float64", "attention_fp8_fwd64", "attention_fp8_rows_fwd64", "fp8_rounding_model"]


def e4m3fn_to_float64(b):
    """Decode OFP8 E4M3 bytes (uint8 array) to float64, element by element
    from the field definition."""
    b = np.asarray(b)
    if b.dtype != np.uint8:
        raise TypeError("expected uint8 bytes, got %s" % b.dtype)
    bi = b.astype(np.int64)
    sign = np.where(bi & 0x80, -1.0, 1.0)
    e = (bi >> 3) & 0xF
    m = (bi & 7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    mag = np.where(e == 0, sub, normal)
    mag = np.where((bi & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def _decoded(q8, k8, v8, descale):
    qd, kd, vd = (float(x) for x in descale)
    return e4m3fn_to_float64(q8) * qd, e4m3fn_to_float64(k8) * kd, e4m3fn_to_float64(v8) * vd


def attention_fp8_fwd64(q8, k8, v8, scale, causal, window=(-1, -1), descale=(1.0, 1.0, 1.0)):
    """(o, lse) in fp64 of attention on the decoded, descaled fp8 inputs.
    q8: uint8 [B, H, Nq, d]; k8, v8: uint8 [B, H_kv, Nk, d]."""
    q, k, v = _decoded(q8, k8, v8, descale)
    return attention_fwd64(q, k, v, scale, causal, window)


def attention_fp8_rows_fwd64(q8, k8, v8, scale, causal, rows, window=(-1, -1), descale=(1.0, 1.0, 1.0)):
    """The same restricted to query rows ``rows`` [B, H, R]."""
    q, k, v = _decoded(q8, k8, v8, descale)
    return attention_rows_fwd64(q, k, v, scale, causal, rows, window)


def fp8_rounding_model(q8, k8, v8, scale, causal, rows, window=(-1, -1), descale=(1.0, 1.0, 1.0)):
    """Bound and standard deviation of the error that rounding the weights
    to e4m3fn adds to O, per element of the query rows ``rows`` [B, H, R].

    The fp8 forward forms p_j = 2^(c s_j - m) with a running maximum m
    (m <= the row maximum, and p_j <= 448), rounds p_j to
    e4m3fn (round to nearest even) for the P V product and divides by
    l = sum_j p_j of the unrounded weights.  Writing L = sum_j exp(s_j -
    s_max) >= 1 and w_j = exp(s_j - s_max) / L (the exact weights):

    * |round(p) - p| <= 2^-4 p for p >= 2^-6 (3 mantissa bits, half a unit
      of 2^-3 relative) and <= 2^-10 for subnormal p (spacing 2^-9), hence
      <= 2^-4 p + 2^-10, and l >= L, so
      |dO| <= 2^-4 sum_j w_j |v_j| + 2^-10 sum_j |v_j| / L.
      ``bound`` adds the bf16 rounding of O (2^-8 |O|, above half a unit)
      and fp32 accumulation and score rounding (2^-9 + Nk 2^-23 relative to
      sum_j w_j |v_j|).
    * Modelling each rounding error as uniform over its spacing (2^(e-3) for
      p in [2^e, 2^(e+1)), 2^-9 below 2^-6), independent across keys, gives
      var(dO) = sum_j spacing_j^2 / 12 * v_j^2 / l^2.  Evaluated at m = the
      row maximum (p_j = w_j L, l = L) this is the largest it can be for
      any m in range: a larger p/l ratio spacing/l never grows.  ``sigma``
      adds the bf16 output rounding's variance, (2^-7 |O|)^2 / 12.

    Returns (bound, sigma), float64 [B, H, R, d].
    """
    q, k, v = _decoded(q8, k8, v8, descale)
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, Nq, d, G = _check(q, k, v)
    rows = np.asarray(rows, dtype=np.int64)
    R = rows.shape[2]
    Nk = k.shape[2]
    bound = np.empty((B, H, R, d))
    sigma = np.empty((B, H, R, d))
    for b in range(B):
        for h in range(H):
            r = rows[b, h]
            s = float(scale) * (q[b, h][r] @ k[b, h // G].T)
            ok = _allowed(r, Nk, causal, window)
            s = np.where(ok, s, -np.inf)
            smax = np.max(s, axis=1, keepdims=True)
            empty = ~np.isfinite(smax[:, 0])
            smax = np.where(np.isfinite(smax), smax, 0.0)
            p = np.exp(s - smax)  # masked: 0
            L = np.sum(p, axis=1, keepdims=True)
            L = np.where(L > 0, L, 1.0)
            w = p / L
            av = np.abs(v[b, h // G])
            A = w @ av
            C = ok.astype(np.float64) @ av
            o = w @ v[b, h // G]
            bd = 2.0 ** -4 * A + 2.0 ** -10 * C / L + 2.0 ** -8 * np.abs(o) + (2.0 ** -9 + Nk * 2.0 ** -23) * A
            # spacing of e4m3 at p: 2^(floor(log2 p) - 3) for normal p, 2^-9 below 2^-6
            with np.errstate(divide="ignore"):
                ex = np.floor(np.log2(np.where(p > 0, p, 1.0)))
            spacing = np.where(p >= 2.0 ** -6, np.exp2(ex - 3.0), 2.0 ** -9)
            spacing = np.where(ok, spacing, 0.0)
            var = (spacing ** 2 / 12.0) @ (v[b, h // G] ** 2) / L ** 2 + (2.0 ** -7 * o) ** 2 / 12.0
            bd[empty] = 0.0
            var[empty] = 0.0
            bound[b, h] = bd
            sigma[b, h] = np.sqrt(var)
    return bound, sigma
