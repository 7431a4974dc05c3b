"""Seeded synthetic inputs shared by the parity tests, the bench and smoke().

This module holds none of the attention arithmetic: it draws iid normal
numbers, rounds them to the kernel's storage dtype, and converts layouts.
Both the HIP path and the fp64 oracle receive exactly the same rounded
values (the oracle widens them to float64).

Recipe: numpy ``default_rng(seed)`` (PCG64) draws float32 ``standard_normal``
arrays in the workload's own memory layout, in the order q, k, v, then dO
when a backward is needed; an optional constant factor (0.5 for the 16K
workload, exact in binary) is applied in float32; the result is rounded to
fp16/bf16 with round-to-nearest-even (torch ``.to``), or to float8_e4m3fn
(torch's round-to-nearest-even cast) for the fp8 forward, whose pages cast
torch.randn tensors the same way.  The pages' workloads
are ``torch.randn`` tensors of fixed shapes ("Flash Attention" skill guide
quick start and Workflows 1-2; glossary article quick start), which these
stand in for.
"""
import numpy as np
import torch

__all__ = ["WORKLOADS", "Workload", "make_qkv", "to_bhsd64", "sample_rows", "torch_dtype"]


def torch_dtype(name):
    return {"fp16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[name]


class Workload:
    """One named problem: sizes, storage dtype, memory layout, masking."""

    def __init__(self, name, B, H, N, d, dtype, layout, causal, seed, in_scale=1.0, backward=False):
        self.name, self.B, self.H, self.N, self.d = name, B, H, N, d
        self.dtype, self.layout, self.causal, self.seed = dtype, layout, tuple(causal), seed
        self.in_scale, self.backward = in_scale, backward

    def __repr__(self):
        return "Workload(%s)" % self.name


# The five named workloads (the small-to-long-context shapes of the parity
# tests and the benchmark), each named by what it is.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("fwd_b1h2_n128_d64_fp16_bhsd", 1, 2, 128, 64, "fp16", "bhsd", (False,), 0),
        Workload("fwd_b2h8_n512_d64_fp16_bhsd", 2, 8, 512, 64, "fp16", "bhsd", (False, True), 1),
        Workload("fwd_causal_b2h16_n1024_d64_bf16_bshd", 2, 16, 1024, 64, "bf16", "bshd", (True,), 2),
        Workload("fwd_causal_b1h16_n16384_d128_bf16_bhsd", 1, 16, 16384, 128, "bf16", "bhsd", (True,), 3,
                 in_scale=0.5),
        Workload("train_causal_b2h8_n2048_d64_fp16_bhsd", 2, 8, 2048, 64, "fp16", "bhsd", (True,), 4,
                 backward=True),
    ]
}


def _shape(B, H, N, d, layout):
    if layout == "bhsd":
        return (B, H, N, d)
    if layout == "bshd":
        return (B, N, H, d)
    raise ValueError("layout must be 'bhsd' or 'bshd'")


def make_qkv(B, H, Nq, Nk, d, dtype, layout="bhsd", seed=0, in_scale=1.0, with_do=False, Hkv=None):
    """Draw q, k, v (and dO) as described in the module docstring.

    Returns a dict of contiguous CPU torch tensors in the requested layout:
    ``[B, H, N, d]`` for 'bhsd' or ``[B, N, H, d]`` for 'bshd'.  k and v get
    ``Hkv`` heads (default H).
    """
    rng = np.random.default_rng(seed)
    td = torch_dtype(dtype)
    hk = H if Hkv is None else Hkv
    out = {}
    for name, n, hh in (("q", Nq, H), ("k", Nk, hk), ("v", Nk, hk)) + ((("do", Nq, H),) if with_do else ()):
        a = rng.standard_normal(_shape(B, hh, n, d, layout), dtype=np.float32)
        if in_scale != 1.0:
            a *= np.float32(in_scale)
        out[name] = torch.from_numpy(a).to(td).contiguous()
    return out


def make_qkv_pooled(B, H, N, d, dtype, layout="bhsd", seed=0, pool_rows=1 << 16, with_do=False):
    """Inputs for grids too large to draw element by element in seconds.

    For each of q, k, v (then dO) in that order: a pool of ``pool_rows``
    rows drawn as in ``make_qkv`` (float32 standard normal, rounded to the
    dtype), then a seeded offset o per (b, h); row i of head (b, h) is pool
    row (o + i) mod pool_rows.  Heads hold distinct cyclic windows of the
    pool, so a head read in place of another gives other values.  Returns
    contiguous CPU tensors like ``make_qkv`` (K/V with H heads).
    """
    rng = np.random.default_rng(seed)
    td = torch_dtype(dtype)
    out = {}
    for name in ("q", "k", "v") + (("do",) if with_do else ()):
        pool = torch.from_numpy(rng.standard_normal((pool_rows, d), dtype=np.float32)).to(td)
        off = torch.from_numpy(rng.integers(0, pool_rows, size=(B, H)))
        idx = (off[:, :, None] + torch.arange(N)[None, None, :]) % pool_rows
        x = pool[idx]  # [B, H, N, d]
        if layout == "bshd":
            x = x.transpose(1, 2)
        out[name] = x.contiguous()
    return out


def workload_inputs(w, seed=None):
    """Inputs of a named workload (dO drawn only when it has a backward)."""
    return make_qkv(w.B, w.H, w.N, w.N, w.d, w.dtype, w.layout, w.seed if seed is None else seed,
                    w.in_scale, with_do=w.backward)


def fp8_bytes(t, layout="bhsd"):
    """The bytes of a float8_e4m3fn CPU tensor as a uint8 numpy array in
    [B, H, N, d] order."""
    a = t.detach().to("cpu").view(torch.uint8).numpy()
    if layout == "bshd":
        a = np.ascontiguousarray(a.transpose(0, 2, 1, 3))
    return a


def to_bhsd64(t, layout="bhsd"):
    """Widen a CPU tensor to a float64 numpy array in [B, H, N, d] order."""
    a = t.detach().to("cpu").to(torch.float64).numpy()
    if layout == "bshd":
        a = np.ascontiguousarray(a.transpose(0, 2, 1, 3))
    return a


def sample_rows(B, H, N, R, seed):
    """Seeded query-row sample per (b, h): rows 0 and N-1 always, plus R-2
    distinct uniform others.  Returns int64 [B, H, min(R, N)], sorted."""
    rng = np.random.default_rng(seed)
    R = min(R, N)
    out = np.empty((B, H, R), dtype=np.int64)
    for b in range(B):
        for h in range(H):
            if R == N:
                out[b, h] = np.arange(N)
                continue
            mid = rng.choice(np.arange(1, N - 1), size=R - 2, replace=False)
            out[b, h] = np.sort(np.concatenate([[0, N - 1], mid]))
    return out


__all__ += ["workload_inputs", "fp8_bytes", "make_qkv_pooled"]
