"""The oracle's pins catch plausible mistakes in it (CPU).

Each mutant below is a copy of one or two oracle functions with one
plausible mistake planted (the oracle itself is untouched: the copies are
swapped in for the duration of one test).  Every pin of the pin module the
mistake concerns (``tests/test_oracle_pins.py``, ``..._gqa_window.py``,
``..._dropout.py``, ``..._fp8.py``) is then run against the mutated oracle; at least one
must fail.  A control run of each module with the unmodified oracle must
pass them all, which checks this harness itself.
"""
import importlib
import zlib

import numpy as np
import pytest

import oracle.attention as oa
import oracle.fp8 as of


PIN_MODULES = ("tests.test_oracle_pins", "tests.test_oracle_pins_gqa_window", "tests.test_oracle_pins_dropout",
               "tests.test_oracle_pins_fp8")


def _pins(module):
    """(name, callable, kwargs) for every pin of ``module``, its
    parametrizations written out."""
    pins = importlib.import_module(module)
    out = []
    for name in sorted(dir(pins)):
        fn = getattr(pins, name)
        if not name.startswith("test_") or not callable(fn):
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        cases = [{}]
        for m in marks:
            argnames = [a.strip() for a in m.args[0].split(",")] if isinstance(m.args[0], str) else list(m.args[0])
            new = []
            for c in cases:
                for values in m.args[1]:
                    vals = values if len(argnames) > 1 else (values,)
                    new.append({**c, **dict(zip(argnames, vals))})
            cases = new
        for c in cases:
            out.append(("%s%s" % (name, sorted(c.items()) if c else ""), fn, c))
    return pins, out


def _run_pins(module):
    """Names of the pins of ``module`` that fail (assertion or any error)."""
    pins, cases = _pins(module)
    failed = []
    for label, fn, kwargs in cases:
        pins.RNG = np.random.default_rng(zlib.crc32(label.encode()))
        try:
            with np.errstate(all="ignore"):
                fn(**kwargs)
        except Exception:  # noqa: BLE001 - any failure of the pin counts
            failed.append(label)
    return failed, len(cases)


# ---------------------------------------------------------------- the mutants

def _allowed_mask_reversed(rows, nk, causal, window):
    left, right = int(window[0]), int(window[1])
    keys = np.arange(nk)[None, :]
    i = np.asarray(rows)[:, None]
    ok = np.ones((len(rows), nk), dtype=bool)
    if causal:
        ok &= keys >= i  # planted: the mask points the wrong way
    if left >= 0:
        ok &= keys >= i - left
    if right >= 0:
        ok &= keys <= i + right
    return ok


def _softmax_rows_lse_without_max(s):
    m = np.max(s, axis=1, keepdims=True)
    empty = ~np.isfinite(m[:, 0])
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m)
    z = np.sum(e, axis=1, keepdims=True)
    p = e / np.where(z > 0, z, 1.0)
    with np.errstate(divide="ignore"):
        lse = np.log(z)[:, 0]  # planted: the maximum is not added back
    lse[empty] = -np.inf
    return p, lse


def _softmax_over_queries(s):
    m = np.max(s, axis=0, keepdims=True)  # planted: normalised down the columns
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m)
    z = np.sum(e, axis=0, keepdims=True)
    p = e / np.where(z > 0, z, 1.0)
    with np.errstate(divide="ignore"):
        lse = np.log(np.sum(np.exp(s - np.max(s, axis=1, keepdims=True)), axis=1)) + np.max(s, axis=1)
    return p, lse


def _scores_scale_twice(q2, k2, scale, causal, rows, window=(-1, -1)):
    s = scale * scale * (q2 @ k2.T)  # planted: the scale applied twice
    return np.where(oa._allowed(rows, k2.shape[0], causal, window), s, -np.inf)


def _bwd_mutant(kind):
    def bwd(q, k, v, do, scale, causal, window=(-1, -1), dropout=None):
        q, k, v, do = oa._as64(q), oa._as64(k), oa._as64(v), oa._as64(do)
        B, H, Nq, d, G = oa._check(q, k, v)
        Hkv = H // G
        scale = float(scale)
        dq = np.empty_like(q)
        dk = np.zeros_like(k)
        dv = np.zeros_like(v)
        rows = np.arange(Nq)
        for b in range(B):
            for h in range(H):
                hk = h % Hkv if kind == "head_map" else h // G
                qq, kk, vv, g = q[b, h], k[b, hk], v[b, hk], do[b, h]
                p, _ = oa._softmax_rows(oa._scores(qq, kk, scale, causal, rows, window))
                wgt = oa._dropped(p, b, h, H, rows, dropout)
                dvv = (wgt @ g) if kind == "dv_p_not_pt" else ((p if kind == "dv_no_mask" else wgt).T @ g)
                dp = g @ vv.T
                axis = 0 if kind == "ds_wrong_axis" else 1
                ds = p * (oa._dropped(dp, b, h, H, rows, dropout) - np.sum(wgt * dp, axis=axis, keepdims=True))
                dq[b, h] = (ds @ kk) if kind == "dq_no_scale" else scale * (ds @ kk)
                dkk = scale * (ds.T @ qq)
                if kind == "dk_perturbed":
                    dkk = dkk * (1 + 1e-6)
                if kind == "group_overwritten":
                    dk[b, hk], dv[b, hk] = dkk, dvv
                else:
                    dk[b, hk] += dkk
                    dv[b, hk] += dvv
        return dq, dk, dv
    return bwd


def _rows_dq_no_scale(q, k, v, do, scale, causal, rows, window=(-1, -1), dropout=None):
    return _REAL_ROWS_DQ(q, k, v, do, scale, causal, rows, window, dropout) / float(scale)  # planted


def _fwd_head_map_mod(q, k, v, scale, causal, window=(-1, -1), dropout=None):
    q, k, v = oa._as64(q), oa._as64(k), oa._as64(v)
    B, H, Nq, d, G = oa._check(q, k, v)
    Hkv = H // G
    o = np.empty((B, H, Nq, d))
    lse = np.empty((B, H, Nq))
    rows = np.arange(Nq)
    for b in range(B):
        for h in range(H):
            hk = h % Hkv  # planted: query head h reads K/V head h mod H_kv, not h / G
            p, lse[b, h] = oa._softmax_rows(oa._scores(q[b, h], k[b, hk], float(scale), causal, rows, window))
            o[b, h] = oa._dropped(p, b, h, H, rows, dropout) @ v[b, hk]
    return o, lse


def _allowed_window_edge(which):
    def allowed(rows, nk, causal, window):
        left, right = int(window[0]), int(window[1])
        keys = np.arange(nk)[None, :]
        i = np.asarray(rows)[:, None]
        ok = np.ones((len(rows), nk), dtype=bool)
        if causal:
            ok &= keys <= i
        if left >= 0:
            ok &= (keys > i - left) if which == "left" else (keys >= i - left)  # planted for "left"
        if right >= 0:
            ok &= (keys < i + right) if which == "right" else (keys <= i + right)  # planted for "right"
        return ok
    return allowed


def _keep_mutant(kind):
    def keep(b, h, H, rows, nk, p, seed, offset):
        thr, _ = oa.dropout_threshold(p)
        i = np.asarray(rows, dtype=np.uint64)[:, None]
        j = np.arange(nk, dtype=np.uint64)[None, :]
        ctr = np.stack(np.broadcast_arrays((j >> np.uint64(5)) * np.uint64(2) + ((j >> np.uint64(2)) & np.uint64(1)),
                                           i, np.uint64(b * H + h), np.uint64(offset)), axis=-1)
        seed = int(seed)
        key = (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
        if kind == "seed_halves_swapped":
            key = key[::-1]
        w = oa.philox4x32_10(ctr, key)
        word = np.take_along_axis(w, ((j >> np.uint64(3)) & np.uint64(3)).astype(np.int64)[..., None]
                                  .repeat(len(rows), axis=0), axis=-1)[..., 0]
        byte = (word >> ((j & np.uint64(3)) * np.uint64(8)).astype(np.uint32)) & np.uint32(0xFF)
        return (byte > thr) if kind == "strict_compare" else (byte >= thr)
    return keep


def _threshold_exact_scale(p):
    thr, _ = _REAL_THRESHOLD(p)
    return thr, 1.0 / (1.0 - float(np.float32(p)))  # planted: 1/(1-p) instead of 256/(256-thr)


def _philox_nine_rounds(ctr, key):
    c = np.asarray(ctr, dtype=np.uint64)
    k = np.asarray(key, dtype=np.uint64)
    x0, x1, x2, x3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0, k1 = k[..., 0], k[..., 1]
    m32 = np.uint64(0xFFFFFFFF)
    for r in range(9):  # planted: one round short
        if r > 0:
            k0 = (k0 + np.uint64(0x9E3779B9)) & m32
            k1 = (k1 + np.uint64(0xBB67AE85)) & m32
        p0 = np.uint64(0xD2511F53) * x0
        p1 = np.uint64(0xCD9E8D57) * x2
        x0, x1, x2, x3 = (p1 >> np.uint64(32)) ^ x1 ^ k0, p1 & m32, (p0 >> np.uint64(32)) ^ x3 ^ k1, p0 & m32
    return np.stack([x0, x1, x2, x3], axis=-1).astype(np.uint32)


def _e4m3_mutant(kind):
    def decode(b):
        b = np.asarray(b)
        bi = b.astype(np.int64)
        sign = 1.0 if kind == "no_sign" else np.where(bi & 0x80, -1.0, 1.0)
        e = (bi >> 3) & 0xF
        m = (bi & 7).astype(np.float64)
        normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - (8.0 if kind == "bias8" else 7.0))
        sub = ((1.0 + m / 8.0) if kind == "no_subnormals" else (m / 8.0)) * 2.0 ** -6
        mag = np.where(e == 0, sub, normal)
        if kind != "no_nan":
            mag = np.where((bi & 0x7F) == 0x7F, np.nan, mag)
        return sign * mag
    return decode


def _decoded_descales_swapped(q8, k8, v8, descale):
    qd, kd, vd = (float(x) for x in descale)
    return of.e4m3fn_to_float64(q8) * qd, of.e4m3fn_to_float64(k8) * vd, of.e4m3fn_to_float64(v8) * kd


_REAL_THRESHOLD = oa.dropout_threshold
_REAL_ROWS_DQ = oa.attention_rows_dq64
CORE, GQA_WINDOW, DROPOUT, FP8 = PIN_MODULES

# mutant: (pin module, [(oracle function, mutated copy), ...]); the
# functions are those of oracle.attention unless the name is one of
# oracle.fp8's
MUTANTS = {
    "causal mask reversed": (CORE, [("_allowed", _allowed_mask_reversed)]),
    "LSE without the row maximum": (CORE, [("_softmax_rows", _softmax_rows_lse_without_max)]),
    "softmax over the wrong axis": (CORE, [("_softmax_rows", _softmax_over_queries)]),
    "scale applied twice": (CORE, [("_scores", _scores_scale_twice)]),
    "dQ missing the scale": (CORE, [("attention_bwd64", _bwd_mutant("dq_no_scale"))]),
    "dV with P instead of P^T": (CORE, [("attention_bwd64", _bwd_mutant("dv_p_not_pt"))]),
    "dS row sum over the wrong axis": (CORE, [("attention_bwd64", _bwd_mutant("ds_wrong_axis"))]),
    "dK off by 1e-6 relative": (CORE, [("attention_bwd64", _bwd_mutant("dk_perturbed"))]),
    "rows dQ missing the scale": (CORE, [("attention_rows_dq64", _rows_dq_no_scale)]),
    "window left edge off by one": (GQA_WINDOW, [("_allowed", _allowed_window_edge("left"))]),
    "window right edge off by one": (GQA_WINDOW, [("_allowed", _allowed_window_edge("right"))]),
    "K/V head map h mod H_kv": (GQA_WINDOW, [("attention_fwd64", _fwd_head_map_mod),
                                             ("attention_bwd64", _bwd_mutant("head_map"))]),
    "group gradients overwritten, not summed": (GQA_WINDOW, [("attention_bwd64", _bwd_mutant("group_overwritten"))]),
    "dropout keeps byte > thr": (DROPOUT, [("dropout_keep", _keep_mutant("strict_compare"))]),
    "dropout seed halves swapped": (DROPOUT, [("dropout_keep", _keep_mutant("seed_halves_swapped"))]),
    "dropout scale 1/(1-p)": (DROPOUT, [("dropout_threshold", _threshold_exact_scale)]),
    "Philox one round short": (DROPOUT, [("philox4x32_10", _philox_nine_rounds)]),
    "dV without the dropout mask": (DROPOUT, [("attention_bwd64", _bwd_mutant("dv_no_mask"))]),
    "e4m3 exponent bias 8": (FP8, [("e4m3fn_to_float64", _e4m3_mutant("bias8"))]),
    "e4m3 subnormals decoded as normals": (FP8, [("e4m3fn_to_float64", _e4m3_mutant("no_subnormals"))]),
    "e4m3 0x7f not NaN": (FP8, [("e4m3fn_to_float64", _e4m3_mutant("no_nan"))]),
    "e4m3 sign bit ignored": (FP8, [("e4m3fn_to_float64", _e4m3_mutant("no_sign"))]),
    "fp8 K and V descales swapped": (FP8, [("_decoded", _decoded_descales_swapped)]),
}
FP8_FUNCTIONS = ("e4m3fn_to_float64", "_decoded")


@pytest.mark.parametrize("module", PIN_MODULES)
def test_pins_pass_on_the_oracle(module):
    failed, n = _run_pins(module)
    assert n >= 10  # the module's pins and their parametrizations were found
    assert failed == [], failed


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_planted_mistake(mutant, monkeypatch):
    module, swaps = MUTANTS[mutant]
    pins, _ = _pins(module)
    for attr, fn in swaps:
        target = of if attr in FP8_FUNCTIONS else oa
        assert hasattr(target, attr), attr
        monkeypatch.setattr(target, attr, fn)
        if hasattr(pins, attr):  # the pin module imported the function by name
            monkeypatch.setattr(pins, attr, fn)
    failed, n = _run_pins(module)
    print("%s: %d of %d pins fail" % (mutant, len(failed), n))
    assert failed, "no pin catches: " + mutant
