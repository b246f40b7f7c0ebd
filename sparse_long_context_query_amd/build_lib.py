"""Compiles the HGA HIP library (libhga.so) for gfx950 in-tree.

    python -m sparse_long_context_query_amd.build_lib      (or build())

Every source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled (-Xclang -target-feature -Xclang -packed-fp32-ops).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libhga.so")
SOURCES = ["hga_api.cpp", "hga_select.hip", "hga_fwd.hip", "hga_bwd.hip", "hga_decode.hip",
           "hga_tier.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HGA library)")


COMMON = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I" + INCLUDE, "-I" + CSRC]


# Host-only AddressSanitizer + UndefinedBehaviorSanitizer (the device code is
# built as usual): every -fsanitize= sits right after -Xarch_host.
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def sanitizer_runtime() -> str:
    """clang's shared ASan runtime (to preload into a process that loads a
    sanitized library), or '' when absent."""
    base = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "llvm",
                        "lib", "clang")
    if not os.path.isdir(base):
        base = "/opt/rocm/llvm/lib/clang"
    for ver in sorted(os.listdir(base)) if os.path.isdir(base) else []:
        cand = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(cand):
            return cand
    return ""


def _compile(src: str, objdir: str, extra=()) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + COMMON + list(extra) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, sanitize: bool = False, out: str = LIB) -> str:
    """Compiles every source for gfx950 and links `out` (default: the
    package's libhga.so).  sanitize=True instruments the host code with ASan
    and UBSan (for CPU checks of the host-side validation; load it with the
    runtime from sanitizer_runtime() preloaded)."""
    objdir = os.path.join(PKG, "_build_san" if sanitize else "_build")
    os.makedirs(objdir, exist_ok=True)
    extra = SANITIZE_HOST if sanitize else []
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, objdir, extra), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    if sanitize:
        cmd += ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-shared-libasan"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
