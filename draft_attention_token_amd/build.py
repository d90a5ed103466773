"""Build libspecprefill.so for gfx950 with hipcc (in-tree), and the small
measurement library libspbench.so (a plain streaming read) that bench.py
uses next to it.

Usage: python -m draft_attention_token_amd.build
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libspecprefill.so")
BENCH_SRC = os.path.join(PKG, "bench", "read_peak.hip")
BENCH_OUT = os.path.join(PKG, "libspbench.so")
OBJDIR = os.path.join(PKG, "_build")

ARCH = os.environ.get("SP_OFFLOAD_ARCH", "gfx950")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", f"-I{INCLUDE}", f"-I{CSRC}",
    # Keep the compiler from emitting packed fp32 arithmetic.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc() -> str:
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.sep not in c or os.path.exists(c):
            return c
    return "hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link the shared libraries. Always rebuilds."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs) + 1)) as ex:
        bench_obj = ex.submit(_compile, BENCH_SRC)
        objs = list(ex.map(_compile, srcs))
        bench_obj = bench_obj.result()
    _link(objs, OUT)
    _link([bench_obj], BENCH_OUT)
    if verbose:
        print(f"built {OUT} and {BENCH_OUT}")
    return OUT


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer: every flag after
# -Xarch_host, so only the host half of each HIP source is instrumented (the
# device code is built as usual).
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]


def build_sanitized(out_dir: str) -> str:
    """libspecprefill.so with its host code built under ASan + UBSan, into
    out_dir (for the host-side checks; load it with the ASan runtime
    preloaded, see sanitizer_runtime())."""
    objdir = os.path.join(out_dir, "obj")
    os.makedirs(objdir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))

    def one(src):
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        r = subprocess.run([_hipcc(), *FLAGS, *SANITIZE, "-c", src, "-o", obj],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}{r.stderr}")
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(one, srcs))
    out = os.path.join(out_dir, "libspecprefill.so")
    r = subprocess.run([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libsan",
                        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                        *objs, "-o", out], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("sanitized link failed:\n" + r.stdout + r.stderr)
    return out


def sanitizer_runtime() -> str:
    """Path of the ASan shared runtime of hipcc's clang (it carries UBSan's
    handlers too)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(_hipcc())), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                       text=True, check=True)
    return r.stdout.strip()


if __name__ == "__main__":
    build(verbose=True)
