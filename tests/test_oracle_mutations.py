"""The oracle's pins catch plausible mistakes in it (CPU).

Each mutant below is a copy of one oracle function with one plausible
mistake planted (the oracle itself is untouched: the copy is swapped in for
the duration of one test).  Every pin of ``tests/test_oracle_pins.py`` is
then run against the mutated oracle; at least one must fail.  A control
run with the unmodified oracle must pass them all, which checks this
harness itself.
"""
import importlib
import zlib

import numpy as np
import pytest

import oracle.attention as oa


def _pins():
    """(name, callable) for every pin, parametrizations written out."""
    pins = importlib.import_module("tests.test_oracle_pins")
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


def _run_pins():
    """Names of the pins that fail (assertion or any error)."""
    pins, cases = _pins()
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
        scale = float(scale)
        dq = np.empty_like(q)
        dk = np.zeros_like(k)
        dv = np.zeros_like(v)
        rows = np.arange(Nq)
        for b in range(B):
            for h in range(H):
                qq, kk, vv, g = q[b, h], k[b, h // G], v[b, h // G], do[b, h]
                p, _ = oa._softmax_rows(oa._scores(qq, kk, scale, causal, rows, window))
                wgt = oa._dropped(p, b, h, H, rows, dropout)
                dv[b, h // G] += (wgt @ g) if kind == "dv_p_not_pt" else (wgt.T @ g)
                dp = g @ vv.T
                axis = 0 if kind == "ds_wrong_axis" else 1
                ds = p * (oa._dropped(dp, b, h, H, rows, dropout) - np.sum(wgt * dp, axis=axis, keepdims=True))
                dq[b, h] = (ds @ kk) if kind == "dq_no_scale" else scale * (ds @ kk)
                dkk = scale * (ds.T @ qq)
                dk[b, h // G] += dkk * (1 + 1e-6) if kind == "dk_perturbed" else dkk
        return dq, dk, dv
    return bwd


MUTANTS = {
    "causal mask reversed": ("_allowed", _allowed_mask_reversed),
    "LSE without the row maximum": ("_softmax_rows", _softmax_rows_lse_without_max),
    "softmax over the wrong axis": ("_softmax_rows", _softmax_over_queries),
    "scale applied twice": ("_scores", _scores_scale_twice),
    "dQ missing the scale": ("attention_bwd64", _bwd_mutant("dq_no_scale")),
    "dV with P instead of P^T": ("attention_bwd64", _bwd_mutant("dv_p_not_pt")),
    "dS row sum over the wrong axis": ("attention_bwd64", _bwd_mutant("ds_wrong_axis")),
    "dK off by 1e-6 relative": ("attention_bwd64", _bwd_mutant("dk_perturbed")),
}


def test_pins_pass_on_the_oracle():
    failed, n = _run_pins()
    assert n >= 30  # every parametrization of every pin was found
    assert failed == [], failed


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_planted_mistake(mutant, monkeypatch):
    attr, fn = MUTANTS[mutant]
    pins, _ = _pins()
    monkeypatch.setattr(oa, attr, fn)
    if hasattr(pins, attr):  # a pin module that imported the function by name
        monkeypatch.setattr(pins, attr, fn)
    failed, n = _run_pins()
    print("%s: %d of %d pins fail" % (mutant, len(failed), n))
    assert failed, "no pin catches: " + mutant
