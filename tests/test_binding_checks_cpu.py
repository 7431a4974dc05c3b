"""The Python binding checks every tensor against q's and k's sizes before it
calls the library (CPU only; no library call is reached).

The library takes every extent from (B, H, Nq, Nk, d), so a v, dO, dQ, dK
or dV smaller than those sizes, an lse that is not fp32 [B, H, Nq], a
mixed fp16/bf16 set, a non-contiguous tensor passed to a contiguous entry
point, or a tensor off the device would make the kernels read or write
outside an allocation.  Each case here must raise FaError with
FA_ERR_INVALID_ARG, naming the offending tensor, before any pointer is
passed on.  The tensors are CPU tensors: the device check comes last, so
every other check is reached first.
"""
import pytest
import torch

import exact_io_aware_02_amd as fa

B, H, HKV, NQ, NK, D = 2, 4, 2, 16, 24, 64
F16, BF16 = torch.float16, torch.bfloat16


def T(*shape, dtype=F16):
    return torch.zeros(shape, dtype=dtype)


def fwd_set(dtype=F16, hk=H):
    return dict(q=T(B, H, NQ, D, dtype=dtype), k=T(B, hk, NK, D, dtype=dtype), v=T(B, hk, NK, D, dtype=dtype),
                o=T(B, H, NQ, D, dtype=dtype), lse=T(B, H, NQ, dtype=torch.float32))


def bwd_set(dtype=F16, hk=H):
    s = fwd_set(dtype, hk)
    s.update(do=T(B, H, NQ, D, dtype=dtype), dq=T(B, H, NQ, D, dtype=dtype), dk=T(B, hk, NK, D, dtype=dtype),
             dv=T(B, hk, NK, D, dtype=dtype), ws=T(1 << 16, dtype=torch.uint8))
    return s


def call_fwd(s):
    fa.fa_fwd(s["q"], s["k"], s["v"], s["o"], s["lse"], 0.125, True)


def call_fwd_ex(s):
    fa.fa_fwd_ex(s["q"], s["k"], s["v"], s["o"], s["lse"], 0.125, True)


def call_bwd(s):
    fa.fa_bwd(s["q"], s["k"], s["v"], s["o"], s["lse"], s["do"], s["dq"], s["dk"], s["dv"], 0.125, True, s["ws"])


def call_bwd_ex(s):
    fa.fa_bwd_ex(s["q"], s["k"], s["v"], s["o"], s["lse"], s["do"], s["dq"], s["dk"], s["dv"], 0.125, True,
                 s["ws"])


def call_bwd_stages(s):
    fa.fa_bwd_stages(s["q"], s["k"], s["v"], s["o"], s["lse"], s["do"], s["dq"], s["dk"], s["dv"], 0.125, True,
                     s["ws"], fa.FA_BWD_ALL)


def expect_invalid(fn, s, word):
    with pytest.raises(fa.FaError) as e:
        fn(s)
    assert e.value.status == fa.FA_ERR_INVALID_ARG, str(e.value)
    assert word in str(e.value), str(e.value)


FWD_BREAKS = [
    ("v fewer rows", lambda s: s.update(v=T(B, H, NK - 8, D)), "v"),
    ("v fewer heads", lambda s: s.update(v=T(B, H // 2, NK, D)), "v"),
    ("o fewer rows", lambda s: s.update(o=T(B, H, NQ - 1, D)), "o"),
    ("lse fp16", lambda s: s.update(lse=T(B, H, NQ)), "lse"),
    ("lse short", lambda s: s.update(lse=T(B, H, NQ - 1, dtype=torch.float32)), "lse"),
    ("lse strided", lambda s: s.update(lse=T(B, H, 2 * NQ, dtype=torch.float32)[:, :, ::2]), "lse"),
    ("k bf16", lambda s: s.update(k=T(B, H, NK, D, dtype=BF16)), "k"),
    ("v bf16", lambda s: s.update(v=T(B, H, NK, D, dtype=BF16)), "v"),
    ("o bf16", lambda s: s.update(o=T(B, H, NQ, D, dtype=BF16)), "o"),
    ("k other d", lambda s: s.update(k=T(B, H, NK, 128), v=T(B, H, NK, 128)), "k"),
    ("k other batch", lambda s: s.update(k=T(B + 1, H, NK, D), v=T(B + 1, H, NK, D)), "k"),
    ("k 3-d", lambda s: s.update(k=T(H, NK, D)), "4-D"),
]


@pytest.mark.parametrize("name,brk,word", FWD_BREAKS, ids=[b[0] for b in FWD_BREAKS])
@pytest.mark.parametrize("fn", [call_fwd, call_fwd_ex], ids=["fa_fwd", "fa_fwd_ex"])
def test_forward_rejects(fn, name, brk, word):
    s = fwd_set()
    brk(s)
    expect_invalid(fn, s, word)


def test_fa_fwd_needs_equal_heads_and_contiguous():
    s = fwd_set(hk=HKV)
    expect_invalid(call_fwd, s, "k")
    s = fwd_set()
    s["q"] = T(B, NQ, H, D).transpose(1, 2)  # a BSHD view: not contiguous BHSD
    expect_invalid(call_fwd, s, "contiguous")


def test_forward_valid_set_stops_at_device():
    for fn in (call_fwd, call_fwd_ex):
        expect_invalid(fn, fwd_set(), "HIP device")
    expect_invalid(call_fwd_ex, fwd_set(hk=HKV), "HIP device")


BWD_BREAKS = [
    ("dout fewer rows", lambda s: s.update(do=T(B, H, NQ - 4, D)), "dout"),
    ("dq fewer rows", lambda s: s.update(dq=T(B, H, NQ - 4, D)), "dq"),
    ("dk fewer rows", lambda s: s.update(dk=T(B, H, NK - 4, D)), "dk"),
    ("dv fewer rows", lambda s: s.update(dv=T(B, H, NK - 4, D)), "dv"),
    ("dv other d", lambda s: s.update(dv=T(B, H, NK, 128)), "dv"),
    ("dout bf16", lambda s: s.update(do=T(B, H, NQ, D, dtype=BF16)), "do"),
    ("dk bf16", lambda s: s.update(dk=T(B, H, NK, D, dtype=BF16)), "dk"),
    ("lse fp16", lambda s: s.update(lse=T(B, H, NQ)), "lse"),
    ("v fewer rows", lambda s: s.update(v=T(B, H, NK - 8, D)), "v"),
    ("workspace strided", lambda s: s.update(ws=T(1 << 17, dtype=torch.uint8)[::2]), "workspace"),
]


@pytest.mark.parametrize("name,brk,word", BWD_BREAKS, ids=[b[0] for b in BWD_BREAKS])
@pytest.mark.parametrize("fn", [call_bwd, call_bwd_ex, call_bwd_stages], ids=["fa_bwd", "fa_bwd_ex", "fa_bwd_stages"])
def test_backward_rejects(fn, name, brk, word):
    s = bwd_set()
    brk(s)
    expect_invalid(fn, s, word)


def test_fa_bwd_needs_contiguous_outputs():
    s = bwd_set()
    s["dq"] = T(B, NQ, H, D).transpose(1, 2)
    expect_invalid(call_bwd, s, "contiguous")


def test_bwd_ex_kv_gradients_take_kv_heads():
    s = bwd_set(hk=HKV)
    s["dk"] = T(B, H, NK, D)  # shaped like q's heads instead of k's
    expect_invalid(call_bwd_ex, s, "dk")
    expect_invalid(call_bwd_ex, bwd_set(hk=HKV), "HIP device")


def test_fp8_forward_rejects():
    q8 = T(B, H, NQ, D, dtype=torch.float8_e4m3fn)
    k8 = T(B, HKV, NK, D, dtype=torch.float8_e4m3fn)
    o = T(B, H, NQ, D, dtype=BF16)
    lse = T(B, H, NQ, dtype=torch.float32)
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd_fp8(q8, k8, k8[:, :, :-1], o, lse, 0.1, True)
    assert e.value.status == fa.FA_ERR_INVALID_ARG and "v" in str(e.value)
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd_fp8(q8, k8, k8, o[:, :, :-1], lse, 0.1, True)
    assert e.value.status == fa.FA_ERR_INVALID_ARG and "o" in str(e.value)
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd_fp8(q8, k8, k8, o, lse.half(), 0.1, True)
    assert e.value.status == fa.FA_ERR_INVALID_ARG and "lse" in str(e.value)
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd_fp8(q8, k8, k8, o, lse, 0.1, True)
    assert e.value.status == fa.FA_ERR_INVALID_ARG and "HIP device" in str(e.value)
