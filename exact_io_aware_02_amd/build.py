"""Build libfa.so (gfx950) in-tree with hipcc.

    python -m exact_io_aware_02_amd.build             # build
    python -m exact_io_aware_02_amd.build --asm DIR   # also keep the gfx950 assembly
    python -m exact_io_aware_02_amd.build --sanitize OUT.so
        # the same library with AddressSanitizer and UndefinedBehaviorSanitizer
        # in the host code (argument validation, dispatch), written to OUT.so;
        # device code is built as usual.  Load it with the ASan runtime
        # preloaded (sanitizer_env() gives the environment).

Cross-compiles without a GPU.  Each source is compiled to an object in
parallel, then linked; the library lands next to this file, where the
binding loads it from.
"""
import argparse
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfa.so")
SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_fwd_fp8.hip", "fa_bwd.hip"]
ARCH = "gfx950"

COMMON_FLAGS = [
    "--offload-arch=" + ARCH,
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # keep the compiler from emitting packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]
OPT_FLAGS = ["-O3"]
# host code only: the device code of a sanitized build is the normal one
SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined"]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; ROCm is required to build libfa.so")
    return exe


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError("hipcc failed (%d): %s\n%s" % (r.returncode, " ".join(cmd), err))
    return err


def _compile_and_link(out, flags, link_flags=(), verbose=False):
    with tempfile.TemporaryDirectory(prefix="fa_build_") as tmpd:
        def one(src):
            obj = os.path.join(tmpd, src + ".o")
            cmd = [hipcc()] + COMMON_FLAGS + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            return obj, _run(cmd)

        with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
            results = list(ex.map(one, SOURCES))
        tmp = out + ".tmp"
        cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC"] + list(link_flags) + \
              [o for o, _ in results] + ["-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        err = _run(cmd)
        if verbose:
            for _, e in results:
                if e:
                    print(e, file=sys.stderr)
            if err:
                print(err, file=sys.stderr)
        os.replace(tmp, out)
    return out


def build(asm_dir=None, verbose=False):
    _compile_and_link(LIB, OPT_FLAGS, verbose=verbose)
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
        for s in SOURCES:
            if not s.endswith(".hip"):
                continue
            out = os.path.join(asm_dir, s.replace(".hip", ".s"))
            acmd = [hipcc()] + COMMON_FLAGS + OPT_FLAGS + ["--cuda-device-only", "-S", os.path.join(CSRC, s),
                                                           "-o", out]
            subprocess.run(acmd, check=True, capture_output=True)
    return LIB


def asan_runtime():
    """Path of the ASan runtime shared library of the HIP compiler's clang."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "lib", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("ASan runtime not found")
    return path


def build_sanitized(out, verbose=False):
    """libfa.so with ASan + UBSan in its host code, written to ``out``."""
    return _compile_and_link(out, SANITIZE_FLAGS, ["-Xarch_host", "-fsanitize=address",
                                                   "-Xarch_host", "-fsanitize=undefined"], verbose)


def sanitizer_env(lib):
    """Environment for a process that loads the sanitized ``lib``."""
    env = dict(os.environ)
    env["EXACT_IO_AWARE_FA_LIB"] = lib
    env["LD_PRELOAD"] = asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None, help="directory for gfx950 assembly listings")
    ap.add_argument("--sanitize", default=None, metavar="OUT", help="build the ASan/UBSan host variant to OUT")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    if a.sanitize:
        print(build_sanitized(os.path.abspath(a.sanitize), a.verbose))
    else:
        print(build(a.asm, a.verbose))
