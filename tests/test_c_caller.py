"""The C ABI from a plain C program (``tests/c_caller/fa_caller.c``).

* ``include/fa.h`` compiles on its own as strict C99 and as C++11, with
  every warning an error.
* The program, built with gcc against libfa.so, reports the same version,
  status strings, workspace sizes and argument rejections as the library
  does through the Python binding (CPU).
* On a GPU it allocates its own device memory, runs fa_fwd and fa_bwd on
  seeded fp16 inputs of the B2 H8 N512 d64 causal shape and writes the
  results back: they match the fp64 oracle within the parity tolerances and
  the Python binding's results bit for bit (same kernels, same launches).
"""
import math
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

import exact_io_aware_02_amd as fa
from attn_inputs import make_qkv, to_bhsd64

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_caller", "fa_caller.c")
INC = os.path.join(ROOT, "include")
ROCM = "/opt/rocm"

pytestmark = pytest.mark.skipif(
    shutil.which("gcc") is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h"))
    or not os.path.exists(fa.lib_path()),
    reason="gcc, the HIP headers or libfa.so missing")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def build_caller(tmp_path):
    libdir = os.path.dirname(os.path.abspath(fa.lib_path()))
    libname = os.path.basename(fa.lib_path())
    assert libname.startswith("lib") and libname.endswith(".so")
    exe = str(tmp_path / "fa_caller")
    cmd = ["gcc", "-std=c99", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", INC, SRC, "-o", exe,
           "-L", libdir, "-l" + libname[3:-3], "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + libdir, "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


@pytest.mark.parametrize("compiler,std", [("gcc", "-std=c99"), ("g++", "-std=c++11")])
def test_header_compiles_strictly(tmp_path, compiler, std):
    if shutil.which(compiler) is None:
        pytest.skip(compiler + " missing")
    src = tmp_path / ("h.c" if compiler == "gcc" else "h.cc")
    src.write_text('#include "fa.h"\nint main(void) { return fa_abi_version() > 0 ? 0 : 1; }\n')
    r = subprocess.run([compiler, std, "-pedantic", "-Wall", "-Wextra", "-Werror", "-fsyntax-only", "-I", INC,
                        str(src)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr


def _gpu_visible():
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


def test_c_caller_checks_match_the_binding(tmp_path):
    exe = build_caller(tmp_path)
    r = subprocess.run([exe, "check"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    got = dict(line.split("=", 1) for line in r.stdout.split() if "=" in line)
    assert int(got["version"]) == fa.fa_abi_version()
    for st in (0, 1, 2, 3, 4, 99):
        assert got["status%d" % st] == fa.fa_status_string(st)
    assert int(got["bwd_workspace"]) == fa.fa_bwd_workspace_bytes(2, 8, 2048, 2048, 64, fa.FA_FP16)
    assert int(got["bwd_ex_workspace"]) == fa.fa_bwd_ex_workspace_bytes(1, 16, 2, 16384, 16384, 128, fa.FA_BF16)
    assert int(got["splitk_workspace"]) == fa.fa_fwd_splitk_workspace_bytes(1, 2, 16384, 16384, 128, 1)
    assert int(got["null_q"]) == fa.FA_ERR_INVALID_ARG and got["message"] == "1"
    assert int(got["d96"]) == fa.FA_ERR_UNSUPPORTED
    assert int(got["o_aliases_q"]) == fa.FA_ERR_INVALID_ARG
    assert int(got["empty"]) == fa.FA_OK
    if _gpu_visible():
        assert got.get("device") == "present"
    else:
        assert int(got["valid_without_device"]) == fa.FA_ERR_DEVICE


@pytest.mark.gpu
def test_c_caller_runs_forward_and_backward(tmp_path):
    import torch

    from oracle import attention_bwd64, attention_fwd64

    B, H, N, d, causal = 2, 8, 512, 64, True
    scale = 1.0 / math.sqrt(d)
    say("case C caller B%d H%d N%d d%d fp16 causal" % (B, H, N, d))
    exe = build_caller(tmp_path)
    inp = make_qkv(B, H, N, N, d, "fp16", seed=1, with_do=True)
    src, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        np.array([B, H, N, d, fa.FA_FP16, int(causal)], dtype=np.int32).tofile(f)
        np.array([scale], dtype=np.float32).tofile(f)
        for x in ("q", "k", "v", "do"):
            inp[x].contiguous().view(torch.int16).numpy().tofile(f)
    r = subprocess.run([exe, "run", str(src), str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    n, rows = B * H * N * d, B * H * N
    raw = np.fromfile(out, dtype=np.uint8)
    assert raw.size == 2 * n + 4 * rows + 3 * 2 * n
    as16 = lambda b: torch.from_numpy(b.view(np.int16).copy()).view(torch.float16).reshape(B, H, N, d)  # noqa: E731
    o = as16(raw[:2 * n])
    lse = raw[2 * n:2 * n + 4 * rows].view(np.float32).reshape(B, H, N)
    grads = [as16(raw[2 * n + 4 * rows + i * 2 * n:2 * n + 4 * rows + (i + 1) * 2 * n]) for i in range(3)]

    # the oracle
    q, k, v, do = (to_bhsd64(inp[x]) for x in ("q", "k", "v", "do"))
    o_ref, lse_ref = attention_fwd64(q, k, v, scale, causal)
    refs = attention_bwd64(q, k, v, do, scale, causal)
    err_o = np.abs(to_bhsd64(o) - o_ref).max()
    err_l = np.abs(lse.astype(np.float64) - lse_ref).max()
    say("  O max-abs %.3e, LSE %.3e" % (err_o, err_l))
    assert err_o <= 2e-3 and err_l <= 1e-3
    for nm, g, ref in zip(("dQ", "dK", "dV"), grads, refs):
        rel = np.linalg.norm(to_bhsd64(g) - ref) / np.linalg.norm(ref)
        say("  %s rel-F %.3e" % (nm, rel))
        assert rel <= 2e-2, nm

    # the same kernels through the Python binding: bit for bit
    dev = "cuda:0"
    qd, kd, vd, dod = (inp[x].to(dev) for x in ("q", "k", "v", "do"))
    o2 = torch.empty_like(qd)
    l2 = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    fa.fa_fwd(qd, kd, vd, o2, l2, scale, causal)
    g2 = [torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)]
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, N, d, fa.FA_FP16), dtype=torch.uint8, device=dev)
    fa.fa_bwd(qd, kd, vd, o2, l2, dod, *g2, scale, causal, ws)
    torch.cuda.synchronize()
    assert torch.equal(o2.cpu().view(torch.int16), o.view(torch.int16))
    assert np.array_equal(l2.cpu().numpy(), lse)
    for a, b in zip(g2, grads):
        assert torch.equal(a.cpu().view(torch.int16), b.view(torch.int16))
