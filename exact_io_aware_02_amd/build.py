"""Build libfa.so (gfx950) in-tree with hipcc.

    python -m exact_io_aware_02_amd.build            # build
    python -m exact_io_aware_02_amd.build --asm DIR  # also keep the gfx950 assembly

Cross-compiles without a GPU.  The library lands next to this file, where
the binding loads it from.
"""
import argparse
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfa.so")
SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_fwd_fp8.hip", "fa_bwd.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    # keep the compiler from emitting packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; ROCm is required to build libfa.so")
    return exe


def build(asm_dir=None, verbose=False):
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (r.returncode, err))
    if err and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
        for s in SOURCES:
            if not s.endswith(".hip"):
                continue
            out = os.path.join(asm_dir, s.replace(".hip", ".s"))
            acmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "--cuda-device-only", "-S",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-I" + os.path.join(ROOT, "include"), os.path.join(CSRC, s), "-o", out]
            subprocess.run(acmd, check=True, capture_output=True)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None, help="directory for gfx950 assembly listings")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    print(build(a.asm, a.verbose))
