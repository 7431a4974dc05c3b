"""C-ABI boundary checks that need no GPU.

libfa.so must load, export every function include/fa.h declares, and reject
invalid arguments with the documented status codes before it makes any HIP
call.  Pointers passed here are fake (never dereferenced): every case fails
validation first.
"""
import ctypes
import os
import re

import pytest

import exact_io_aware_02_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(fa.lib_path()), reason="libfa.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert set(declared_functions()) == set(fa.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fa.lib_path())
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_exported_dynamic_symbols_are_c_names():
    """The symbols are unmangled C names in the dynamic symbol table."""
    import subprocess

    out = subprocess.run(["nm", "-D", "--defined-only", fa.lib_path()], capture_output=True, text=True).stdout
    names = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for name in declared_functions():
        assert name in names, name


def test_status_strings_and_version():
    assert fa.fa_abi_version() == 6
    assert fa.fa_status_string(0) == "FA_OK"
    assert fa.fa_status_string(1) == "FA_ERR_INVALID_ARG"
    assert fa.fa_status_string(2) == "FA_ERR_UNSUPPORTED"
    assert fa.fa_status_string(3) == "FA_ERR_DEVICE"
    assert fa.fa_status_string(4) == "FA_ERR_LAUNCH"
    assert fa.fa_status_string(99) == "FA_UNKNOWN_STATUS"


def test_workspace_bytes():
    n = fa.fa_bwd_workspace_bytes(2, 8, 2048, 2048, 64, 0)
    assert n >= 2 * 8 * 2048 * 4 and n % 256 == 0
    assert fa.fa_bwd_workspace_bytes(1, 1, 1, 1, 96, 0) == 0
    assert fa.fa_bwd_workspace_bytes(1, 1, 1, 1, 64, 7) == 0
    assert fa.fa_bwd_workspace_bytes(-1, 1, 1, 1, 64, 0) == 0


# --- forward validation -------------------------------------------------------

P = lambda a: ctypes.c_void_p(a)  # noqa: E731
A = 1 << 20  # fake, 16-byte aligned "device" addresses, far apart


def fwd(q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, B=1, H=1, Nq=16, Nk=16, d=64, scale=0.125, causal=0, dtype=0):
    lib = fa.load_library()
    return lib.fa_fwd(P(q), P(k), P(v), P(o), P(lse), B, H, Nq, Nk, d, scale, causal, dtype, None)


def fwd_strided(strides, **kw):
    lib = fa.load_library()
    I3 = ctypes.c_int64 * 3
    s = [I3(*x) for x in strides]
    a = dict(q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, B=1, H=1, Nq=16, Nk=16, d=64, scale=0.125, causal=0, dtype=0)
    a.update(kw)
    return lib.fa_fwd_strided(P(a["q"]), P(a["k"]), P(a["v"]), P(a["o"]), P(a["lse"]), a["B"], a["H"], a["Nq"],
                              a["Nk"], a["d"], a["scale"], a["causal"], a["dtype"], *s, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), fa.FA_ERR_INVALID_ARG),
    (dict(k=0), fa.FA_ERR_INVALID_ARG),
    (dict(v=0), fa.FA_ERR_INVALID_ARG),
    (dict(o=0), fa.FA_ERR_INVALID_ARG),
    (dict(lse=0), fa.FA_ERR_INVALID_ARG),
    (dict(q=A + 2), fa.FA_ERR_INVALID_ARG),          # misaligned
    (dict(lse=5 * A + 2), fa.FA_ERR_INVALID_ARG),    # misaligned lse
    (dict(B=-1), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=0), fa.FA_ERR_INVALID_ARG),             # softmax over no keys
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=32), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=2), fa.FA_ERR_UNSUPPORTED),          # fp32 / unknown
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(o=A), fa.FA_ERR_INVALID_ARG),              # o aliases q
    (dict(o=A + 1024), fa.FA_ERR_INVALID_ARG),       # o overlaps q
    (dict(lse=4 * A + 64), fa.FA_ERR_INVALID_ARG),   # lse overlaps o
])
def test_fwd_rejects(kw, code):
    assert fwd(**kw) == code
    assert fa.fa_last_error_message() != ""


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(Nq=0), dict(Nq=0, Nk=0)])
def test_fwd_empty_is_ok_without_touching_pointers(kw):
    assert fwd(q=0, k=0, v=0, o=0, lse=0, **kw) == fa.FA_OK


def test_fwd_strided_rejects_bad_strides():
    good = [(16 * 64, 16 * 64, 64)] * 4
    bad_mult = [(16 * 64, 16 * 64, 68)] + good[1:]
    assert fwd_strided(bad_mult) == fa.FA_ERR_INVALID_ARG
    neg = [(16 * 64, 16 * 64, -64)] + good[1:]
    assert fwd_strided(neg) == fa.FA_ERR_INVALID_ARG
    overlap_rows = [(16 * 64, 16 * 64, 32)] + good[1:]
    assert fwd_strided(overlap_rows) == fa.FA_ERR_INVALID_ARG
    huge = [(0, 0, 1 << 28)] + good[1:]
    assert fwd_strided(huge) == fa.FA_ERR_INVALID_ARG  # per-head extent > 2^31 elements


BH2 = dict(B=2, H=2, Nq=16, Nk=16)
DENSE = (2 * 16 * 64, 16 * 64, 64)   # BHSD, B=H=2, N=16, d=64
BSHD = (16 * 2 * 64, 64, 2 * 64)


@pytest.mark.parametrize("o_st", [
    (0, 16 * 64, 64),          # every batch on one slice
    (2 * 16 * 64, 0, 64),      # every head on one slice
    (16 * 64, 16 * 64, 64),    # batch and head share a stride
    (2 * 16 * 64, 512, 64),    # head slices interleave with rows
    (64, 192, 128),            # [N][H][B] order, but the head stride lands inside the rows
])
def test_fwd_rejects_self_overlapping_output(o_st):
    """Two (b, h, row) elements of o at one address would be written by two
    workgroups; only inputs may broadcast with such strides."""
    assert fwd_strided([DENSE] * 3 + [o_st], **BH2) == fa.FA_ERR_INVALID_ARG
    assert "one address" in fa.fa_last_error_message()


@pytest.mark.parametrize("q_st", [(0, 16 * 64, 64), (0, 0, 64), (16 * 64, 16 * 64, 64)])
def test_fwd_inputs_may_broadcast(q_st):
    """A zero or shared stride is fine on an input: the call gets past
    validation (the device check fails where no device exists)."""
    if _gpu_visible():
        pytest.skip("a valid call would run on the device")
    assert fwd_strided([q_st, DENSE, DENSE, DENSE], **BH2) == fa.FA_ERR_DEVICE


@pytest.mark.parametrize("o_st", [DENSE, BSHD, (4 * 16 * 64, 2 * 16 * 64, 128)])  # dense, BSHD, padded
def test_fwd_accepts_non_overlapping_outputs(o_st):
    if _gpu_visible():
        pytest.skip("a valid call would run on the device")
    assert fwd_strided([DENSE] * 3 + [o_st], **BH2) == fa.FA_ERR_DEVICE


def bwd_strided(out_st, ws_bytes=1 << 16):
    lib = fa.load_library()
    I3 = ctypes.c_int64 * 3
    st = [I3(*DENSE)] * 5 + [I3(*x) for x in out_st]
    return lib.fa_bwd_strided(P(A), P(2 * A), P(3 * A), P(4 * A), P(5 * A), P(6 * A), P(7 * A), P(8 * A), P(9 * A),
                              2, 2, 16, 16, 64, 0.125, 1, 0, *st, P(10 * A), ws_bytes, None)


@pytest.mark.parametrize("which", [0, 1, 2])
def test_bwd_rejects_self_overlapping_gradient(which):
    out = [DENSE] * 3
    out[which] = (2 * 16 * 64, 0, 64)
    assert bwd_strided(out) == fa.FA_ERR_INVALID_ARG
    assert ("dq", "dk", "dv")[which] + ": strides" in fa.fa_last_error_message()


def test_bwd_accepts_bshd_gradients():
    if _gpu_visible():
        pytest.skip("a valid call would run on the device")
    assert bwd_strided([BSHD] * 3) == fa.FA_ERR_DEVICE


def test_sizes_beyond_the_row_bound_are_rejected():
    """B*H*max(Nq, Nk) above 2^48 rows: every byte count stays far from
    64-bit overflow (the LSE and workspaces are B*H*N-sized)."""
    B, H, N = 1 << 20, 1 << 10, 1 << 20           # 2^50 rows
    assert fwd(q=0, k=0, v=0, o=0, lse=0, B=B, H=H, Nq=N, Nk=N) == fa.FA_ERR_INVALID_ARG
    assert "2^48" in fa.fa_last_error_message()
    assert fa.fa_bwd_workspace_bytes(B, H, N, N, 64, 0) == 0
    assert fa.fa_bwd_ex_workspace_bytes(B, H, H, N, N, 64, 0) == 0
    assert fa.fa_fwd_splitk_workspace_bytes(B, H, N, N, 64, 1) == 0
    # at the bound itself the queries still answer
    assert fa.fa_bwd_workspace_bytes(1 << 17, 1 << 10, 1 << 21, 1, 64, 0) == 2 * (1 << 48) * 4


# --- backward validation ------------------------------------------------------

def bwd(ws=10 * A, ws_bytes=1 << 16, dq=7 * A, dk=8 * A, dv=9 * A, d=64, Nq=16, Nk=16, dtype=0):
    lib = fa.load_library()
    return lib.fa_bwd(P(A), P(2 * A), P(3 * A), P(4 * A), P(5 * A), P(6 * A), P(dq), P(dk), P(dv),
                      1, 1, Nq, Nk, d, 0.125, 1, dtype, P(ws), ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(ws=0), fa.FA_ERR_INVALID_ARG),
    (dict(ws_bytes=4), fa.FA_ERR_INVALID_ARG),        # too small
    (dict(ws=10 * A + 16), fa.FA_ERR_INVALID_ARG),    # workspace not 256-aligned
    (dict(dq=A), fa.FA_ERR_INVALID_ARG),              # dq aliases q
    (dict(dk=7 * A), fa.FA_ERR_INVALID_ARG),          # dk aliases dq
    (dict(ws=9 * A), fa.FA_ERR_INVALID_ARG),          # workspace aliases dv
    (dict(d=80), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=5), fa.FA_ERR_UNSUPPORTED),
    (dict(Nk=0), fa.FA_ERR_INVALID_ARG),
])
def test_bwd_rejects(kw, code):
    assert bwd(**kw) == code


def test_bwd_stages_rejects_bad_mask():
    lib = fa.load_library()
    I3 = ctypes.c_int64 * 3
    st = [I3(16 * 64, 16 * 64, 64)] * 8
    for stages in (0, 8, -1, 16):
        r = lib.fa_bwd_stages(P(A), P(2 * A), P(3 * A), P(4 * A), P(5 * A), P(6 * A), P(7 * A), P(8 * A), P(9 * A),
                              1, 1, 16, 16, 64, 0.125, 1, 0, *st, P(10 * A), 1 << 16, stages, None)
        assert r == fa.FA_ERR_INVALID_ARG, stages


def test_python_binding_rejects_fp32():
    import torch

    q = torch.zeros(1, 1, 8, 64)
    with pytest.raises(fa.FaError) as e:
        fa.attention_fwd(q, q, q)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED


def _gpu_visible():
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_gpu_visible(), reason="only meaningful where no HIP device exists")
def test_valid_call_without_device_reports_device_error():
    """Arguments are valid, so the call reaches the device check, which fails
    here; nothing is launched."""
    assert fwd() == fa.FA_ERR_DEVICE


# --- fewer K/V heads and sliding window (fa_fwd_ex / fa_bwd_ex) ---------------

def fwd_ex(H=4, Hkv=2, wl=-1, wr=-1, causal=0, Nq=16, Nk=16, dropout=0.0):
    lib = fa.load_library()
    I3 = ctypes.c_int64 * 3
    sq = I3(H * Nq * 64, Nq * 64, 64)
    sk = I3(Hkv * Nk * 64, Nk * 64, 64)
    return lib.fa_fwd_ex(P(A), P(2 * A), P(3 * A), P(4 * A), P(5 * A), 1, H, Hkv, Nq, Nk, 64, 0.125, causal, wl, wr,
                         dropout, 7, 0, 0, sq, sk, sk, sq, None)


def bwd_ex(H=4, Hkv=2, wl=-1, wr=-1, causal=0, dk=8 * A, stages=fa.FA_BWD_ALL, dropout=0.0):
    lib = fa.load_library()
    I3 = ctypes.c_int64 * 3
    sq = I3(H * 16 * 64, 16 * 64, 64)
    sk = I3(Hkv * 16 * 64, 16 * 64, 64)
    st = [sq, sk, sk, sq, sq, sq, sk, sk]
    return lib.fa_bwd_ex(P(A), P(2 * A), P(3 * A), P(4 * A), P(5 * A), P(6 * A), P(7 * A), P(dk), P(9 * A),
                         1, H, Hkv, 16, 16, 64, 0.125, causal, wl, wr, dropout, 7, 0, 0, *st, P(10 * A), 1 << 16,
                         stages, None)


@pytest.mark.parametrize("H,Hkv", [(4, 3), (4, 0), (4, -2), (3, 6)])
def test_ex_rejects_heads_that_do_not_divide(H, Hkv):
    assert fwd_ex(H=H, Hkv=Hkv) == fa.FA_ERR_INVALID_ARG
    assert "H_kv" in fa.fa_last_error_message()
    assert bwd_ex(H=H, Hkv=Hkv) == fa.FA_ERR_INVALID_ARG


def test_ex_validates_kv_tensors_with_kv_heads():
    # dk overlapping dv is detected with the K/V head count's extent
    assert bwd_ex(H=4, Hkv=2, dk=9 * A - 64) == fa.FA_ERR_INVALID_ARG
    assert bwd_ex(stages=0) == fa.FA_ERR_INVALID_ARG


@pytest.mark.skipif(_gpu_visible(), reason="only meaningful where no HIP device exists")
@pytest.mark.parametrize("wl,wr,causal", [(-1, -1, 0), (0, 0, 0), (5, -7, 1), (-3, 2, 0), (1 << 30, 1 << 30, 0)])
def test_ex_accepts_any_window(wl, wr, causal):
    """Any window value is valid (negative: that side unbounded), so a valid
    call reaches the device check."""
    assert fwd_ex(wl=wl, wr=wr, causal=causal) == fa.FA_ERR_DEVICE
    assert bwd_ex(wl=wl, wr=wr, causal=causal) == fa.FA_ERR_DEVICE


@pytest.mark.parametrize("p", [-0.1, 1.0, 2.0, float("nan"), float("inf")])
def test_ex_rejects_bad_dropout(p):
    assert fwd_ex(dropout=p) == fa.FA_ERR_INVALID_ARG
    assert "dropout" in fa.fa_last_error_message()
    assert bwd_ex(dropout=p) == fa.FA_ERR_INVALID_ARG


@pytest.mark.skipif(_gpu_visible(), reason="only meaningful where no HIP device exists")
@pytest.mark.parametrize("p", [0.0, 0.1, 0.5, 0.999])
def test_ex_accepts_dropout(p):
    assert fwd_ex(dropout=p) == fa.FA_ERR_DEVICE
    assert bwd_ex(dropout=p) == fa.FA_ERR_DEVICE


# --- fp8 forward (fa_fwd_fp8) ---------------------------------------------------

def fwd_fp8(H=4, Hkv=2, Nq=16, Nk=16, d=64, scale=0.125, descale=(1.0, 1.0, 1.0), sq=None, sk=None, so=None,
            q=A, o=4 * A):
    lib = fa.load_library()
    I3 = ctypes.c_int64 * 3
    sq = I3(*(sq or (H * Nq * d, Nq * d, d)))
    sk = I3(*(sk or (Hkv * Nk * d, Nk * d, d)))
    so = I3(*(so or (H * Nq * d, Nq * d, d)))
    return lib.fa_fwd_fp8(P(q), P(2 * A), P(3 * A), P(o), P(5 * A), 1, H, Hkv, Nq, Nk, d, scale, 1, -1, -1,
                          *descale, sq, sk, sk, so, None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(H=4, Hkv=3), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(descale=(1.0, float("inf"), 1.0)), fa.FA_ERR_INVALID_ARG),
    (dict(descale=(float("nan"), 1.0, 1.0)), fa.FA_ERR_INVALID_ARG),
    (dict(scale=1e30, descale=(1e10, 1e10, 1.0)), fa.FA_ERR_INVALID_ARG),
    # fp8 rows must stay 16-byte aligned: strides in multiples of 16 bytes
    (dict(sq=(4 * 16 * 64, 16 * 64, 72)), fa.FA_ERR_INVALID_ARG),
    (dict(sk=(2 * 16 * 64, 16 * 64 + 8, 64)), fa.FA_ERR_INVALID_ARG),
    (dict(q=A + 8), fa.FA_ERR_INVALID_ARG),
    # o is bf16: 8-element strides are fine there, 4 are not
    (dict(so=(4 * 16 * 64, 16 * 64, 68)), fa.FA_ERR_INVALID_ARG),
    # o overlapping q (q's extent counted in bytes)
    (dict(o=A + 4 * 16 * 64 - 16), fa.FA_ERR_INVALID_ARG),
])
def test_fwd_fp8_rejects(kw, code):
    assert fwd_fp8(**kw) == code


def test_fwd_fp8_empty_is_ok():
    assert fwd_fp8(Nq=0) == fa.FA_OK


@pytest.mark.skipif(_gpu_visible(), reason="only meaningful where no HIP device exists")
@pytest.mark.parametrize("kw", [dict(), dict(d=128), dict(sq=(4 * 16 * 80, 16 * 80, 80)),
                                dict(o=A + 4 * 16 * 64), dict(scale=-0.5, descale=(2.0, -3.0, 0.25))])
def test_fwd_fp8_valid_call_reaches_device_check(kw):
    assert fwd_fp8(**kw) == fa.FA_ERR_DEVICE


def test_python_fp8_binding_checks_dtypes():
    import torch

    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(fa.FaError) as e:
        fa.attention_fwd_fp8(q, q, q)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED


def split_extra(S, B, Hkv, Nk, d):
    """Bytes the split dK/dV stage adds to the workspace: S fp32 partial
    sums of dK and of dV."""
    return 2 * S * B * Hkv * Nk * d * 4


def test_ex_workspace_bytes():
    base = fa.fa_bwd_workspace_bytes(1, 16, 16384, 16384, 128, fa.FA_BF16)
    # equal heads: nothing extra when the dK/dV grid gives every CU a
    # workgroup (64 key blocks of 256 keys x 16 heads)...
    assert fa.fa_bwd_ex_workspace_bytes(1, 16, 16, 16384, 16384, 128, fa.FA_BF16) == base
    # ...two runs per key block when it does not (64 x 2 = 128 < 256 CUs)
    assert fa.fa_bwd_ex_workspace_bytes(1, 2, 2, 16384, 16384, 128, fa.FA_BF16) == \
        fa.fa_bwd_workspace_bytes(1, 2, 16384, 16384, 128, fa.FA_BF16) + split_extra(2, 1, 2, 16384, 128)
    # ...at d = 64 below the 512 workgroups the chip holds (B2 H8 N2048: 16 x 16)...
    assert fa.fa_bwd_ex_workspace_bytes(2, 8, 8, 2048, 2048, 64, fa.FA_FP16) == \
        fa.fa_bwd_workspace_bytes(2, 8, 2048, 2048, 64, fa.FA_FP16) + split_extra(2, 2, 8, 2048, 64)
    # ...but not below 2048 keys, nor from a full chip on (d = 128: 256; d = 64: 512)
    assert fa.fa_bwd_ex_workspace_bytes(1, 2, 2, 1024, 1024, 128, fa.FA_BF16) == \
        fa.fa_bwd_workspace_bytes(1, 2, 1024, 1024, 128, fa.FA_BF16)
    assert fa.fa_bwd_ex_workspace_bytes(1, 4, 4, 16384, 16384, 128, fa.FA_BF16) == \
        fa.fa_bwd_workspace_bytes(1, 4, 16384, 16384, 128, fa.FA_BF16)
    assert fa.fa_bwd_ex_workspace_bytes(1, 3, 3, 16384, 16384, 128, fa.FA_BF16) == \
        fa.fa_bwd_workspace_bytes(1, 3, 16384, 16384, 128, fa.FA_BF16) + split_extra(2, 1, 3, 16384, 128)
    assert fa.fa_bwd_ex_workspace_bytes(1, 4, 4, 16384, 16384, 64, fa.FA_BF16) == \
        fa.fa_bwd_workspace_bytes(1, 4, 16384, 16384, 64, fa.FA_BF16)
    # 16 query heads on 2 K/V heads at 16K, d = 128 (256 keys per dK/dV
    # workgroup): 64 key blocks x 2 = 128 workgroups, split 8 ways to reach 1024
    big = fa.fa_bwd_ex_workspace_bytes(1, 16, 2, 16384, 16384, 128, fa.FA_BF16)
    assert big == base + split_extra(8, 1, 2, 16384, 128)
    # d = 64 (128 keys per workgroup): 128 x 2 = 256 workgroups, split 4 ways
    base64 = fa.fa_bwd_workspace_bytes(1, 16, 16384, 16384, 64, fa.FA_BF16)
    assert fa.fa_bwd_ex_workspace_bytes(1, 16, 2, 16384, 16384, 64, fa.FA_BF16) == \
        base64 + split_extra(4, 1, 2, 16384, 64)
    # a problem that already fills the chip is not split
    assert fa.fa_bwd_ex_workspace_bytes(8, 64, 8, 16384, 16384, 128, fa.FA_BF16) == \
        fa.fa_bwd_workspace_bytes(8, 64, 16384, 16384, 128, fa.FA_BF16)
    # invalid sizes give 0
    assert fa.fa_bwd_ex_workspace_bytes(1, 16, 3, 128, 128, 128, fa.FA_BF16) == 0
    assert fa.fa_bwd_ex_workspace_bytes(1, 16, 2, 128, 128, 96, fa.FA_BF16) == 0


@pytest.mark.skipif(_gpu_visible(), reason="only meaningful where no HIP device exists")
def test_ex_accepts_either_workspace_size():
    """The split workspace is optional: the statistics-only size stays valid."""
    lib = fa.load_library()
    I3 = ctypes.c_int64 * 3
    H, Hkv, N = 8, 2, 64
    sq = I3(H * N * 64, N * 64, 64)
    sk = I3(Hkv * N * 64, N * 64, 64)
    st = [sq, sk, sk, sq, sq, sq, sk, sk]
    for nbytes in (fa.fa_bwd_workspace_bytes(1, H, N, N, 64, 0), fa.fa_bwd_ex_workspace_bytes(1, H, Hkv, N, N, 64, 0)):
        assert lib.fa_bwd_ex(P(A), P(2 * A), P(3 * A), P(4 * A), P(5 * A), P(6 * A), P(7 * A), P(8 * A), P(9 * A),
                             1, H, Hkv, N, N, 64, 0.125, 1, -1, -1, 0.0, 0, 0, 0, *st, P(10 * A), nbytes,
                             fa.FA_BWD_ALL, None) == fa.FA_ERR_DEVICE


# --- key-split forward (fa_fwd_splitk) ------------------------------------------

def _plan_model(B, H, Nq, Nk, d, causal, wl=-1, wr=-1):
    """The chunk plan restated: 128-query blocks, 32-key tiles; grids of at
    most 512 blocks; with W the key tiles of one head's blocks and
    S = floor(F * 256 / (B H)) the resident workgroups per head (F = 4 at
    d = 64, else 3), the chunk length starts at max(8, ceil(W / S)) and
    grows by max(1, chunk // 32) while the chunks exceed S and it is below
    the longest block; the plan is dropped unless chunk + 32 (chunk + 96
    with more than 256 blocks) <= the unsplit critical path (the longest
    block's tiles divided by 3, rounded up, when the grid has at most 256
    blocks and that block 32+ tiles); a block of n tiles has
    ceil(n / chunk) chunks (1 if n = 0); the workspace holds
    (d + 2) * 128 floats per chunk of a block with two or more."""
    wl = -1 if wl < 0 or wl >= Nq else wl
    wr = 0 if causal else (-1 if wr < 0 or wr >= Nk else wr)
    n_qt = -(-Nq // 128)
    if n_qt * B * H > 512:
        return 0
    tiles = []
    for qb in range(n_qt):
        kend, j0 = Nk, 0
        if wl >= 0 or wr >= 0:
            qlast = min(qb * 128 + 128, Nq) - 1
            if wr >= 0:
                kend = min(Nk, qlast + wr + 1)
            if wl >= 0:
                j0 = max(0, qb * 128 - wl) // 32
        tiles.append(max(j0, -(-kend // 32)) - j0)
    per_bh = max(1, (4 if d == 64 else 3) * 256 // (B * H))
    chunks = lambda c: sum(max(1, -(-n // c)) for n in tiles)  # noqa: E731
    chunk = max(8, -(-sum(tiles) // per_bh))
    while chunk < max(tiles) and chunks(chunk) > per_bh:
        chunk += max(1, chunk // 32)
    most = max(tiles)
    ks = 3
    unsplit = -(-most // ks) if n_qt * B * H <= 256 and most >= 32 else most
    if chunk + (32 if n_qt * B * H <= 256 else 96) > unsplit:
        return 0
    P = sum(c for c in (max(1, -(-n // chunk)) for n in tiles) if c > 1)
    return 0 if P == 0 else -(-(B * H * P * 128 * (d + 2) * 4) // 256) * 256


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal,wl,wr", [
    (2, 8, 2048, 2048, 64, 1, -1, -1),      # the training-step workload
    (1, 2, 16384, 16384, 128, 1, -1, -1),   # 2 heads of 16K (one GPU of 8 under head sharding)
    (2, 16, 1024, 1024, 64, 1, -1, -1),
    (2, 8, 512, 512, 64, 0, -1, -1),
    (1, 2, 128, 128, 64, 0, -1, -1),        # one block of 4 tiles: nothing to split
    (1, 16, 16384, 16384, 128, 1, -1, -1),  # 2048 blocks: fills the chip
    (1, 4, 3000, 2000, 128, 0, 300, 40),    # a window (rows past 2040 admit no key)
    (3, 1, 5000, 7000, 64, 1, -1, -1),
    (1, 4, 16384, 16384, 128, 1, -1, -1),   # 512 blocks, long rows: chunks kept
    (1, 16, 4096, 4096, 128, 1, -1, -1),    # 512 blocks, short rows: dropped
    (1, 8, 8192, 8192, 128, 1, -1, -1),
])
def test_fwd_splitk_workspace_bytes(B, H, Nq, Nk, d, causal, wl, wr):
    assert fa.fa_fwd_splitk_workspace_bytes(B, H, Nq, Nk, d, causal, (wl, wr)) == \
        _plan_model(B, H, Nq, Nk, d, causal, wl, wr)


def test_fwd_splitk_workspace_examples():
    # 16 blocks of 4 .. 64 tiles per head: the intra-workgroup split's run
    # (22 tiles) beats any chunking, so no workspace
    assert fa.fa_fwd_splitk_workspace_bytes(2, 8, 2048, 2048, 64, 1) == 0
    # 2 heads of 128 blocks of 4 .. 512 tiles, 384 resident workgroups per
    # head: chunks of at most 115 tiles
    assert fa.fa_fwd_splitk_workspace_bytes(1, 2, 16384, 16384, 128, 1) > 0
    assert fa.fa_fwd_splitk_workspace_bytes(1, 16, 16384, 16384, 128, 1) == 0
    assert fa.fa_fwd_splitk_workspace_bytes(1, 1, 1, 1, 96, 0) == 0
    # 512 blocks (two per CU for some): chunks only for long rows
    assert fa.fa_fwd_splitk_workspace_bytes(1, 4, 16384, 16384, 128, 1) > 0
    assert fa.fa_fwd_splitk_workspace_bytes(1, 16, 4096, 4096, 128, 1) == 0


S = 1 << 30  # fake addresses far enough apart for tensors of up to 1 GiB


def fwd_splitk(ws=10 * S, ws_bytes=1 << 30, B=1, H=2, N=16384, d=128, causal=1):
    lib = fa.load_library()
    I3 = ctypes.c_int64 * 3
    st = I3(H * N * d, N * d, d)
    return lib.fa_fwd_splitk(P(S), P(2 * S), P(3 * S), P(4 * S), P(5 * S), B, H, H, N, N, d, 0.125, causal, -1, -1,
                             0.0, 0, 0, 0, st, st, st, st, P(ws), ws_bytes, None)


@pytest.mark.parametrize("kw", [
    dict(ws=0),                       # needed, NULL
    dict(ws_bytes=1024),              # too small
    dict(ws=10 * S + 128),            # not 256-byte aligned
    dict(ws=4 * S + 256),             # overlaps o
])
def test_fwd_splitk_rejects_bad_workspace(kw):
    assert fwd_splitk(**kw) == fa.FA_ERR_INVALID_ARG
    assert "workspace" in fa.fa_last_error_message()


@pytest.mark.skipif(_gpu_visible(), reason="only meaningful where no HIP device exists")
def test_fwd_splitk_valid_call_reaches_device_check():
    assert fwd_splitk() == fa.FA_ERR_DEVICE
    # sizes that need no workspace accept NULL
    assert fwd_splitk(ws=0, ws_bytes=0, B=1, H=16, N=16384, d=128) == fa.FA_ERR_DEVICE
