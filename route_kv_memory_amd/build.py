"""Build the FastMKA HIP library (``libmka.so``) for gfx950 with hipcc.

Usage: ``python -m route_kv_memory_amd.build`` (or ``build()`` from Python).
Every source is recompiled on each call; objects go to ``_build/`` beside the
package and the shared library into the package directory, where the binding
loads it from.

``build(sanitize=True)`` (``python -m route_kv_memory_amd.build --sanitize``)
builds a second library, ``_build/sanitize/libmka.so``, whose host code is
instrumented with AddressSanitizer and UndefinedBehaviorSanitizer (the
device code is not: the sanitizer flags apply to the host compilation only,
``-Xarch_host``).  It is for host-side tests of the C ABI on the CPU: load it
with the binding's ``MKA_LIB`` variable and the sanitizer runtime
(``sanitizer_runtime()``) preloaded.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmka.so")

SOURCES = ["mka_api.hip", "gemm.hip", "route.hip", "ema.hip", "l3.hip", "fuse.hip", "attn.hip",
           "decode.hip", "probe.hip", "backward.hip", "attn_bwd.hip"]

ARCH = os.environ.get("MKA_OFFLOAD_ARCH", "gfx950")

# Packed fp32 VALU ops are disabled: the kernels are written with scalar float
# arithmetic and must not be lowered to v_pk_{add,mul,fma}_f32.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


# Host-only sanitizers: each -fsanitize= follows -Xarch_host, so no device
# code is instrumented.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-fno-omit-frame-pointer", "-shared-libsan"]
SANITIZE_DIR = os.path.join(BUILD, "sanitize")


def sanitizer_runtime() -> str:
    """The ASan runtime to preload into a process that loads the sanitized library."""
    hipcc = _hipcc()
    res = subprocess.run([hipcc, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path):
        raise RuntimeError("the clang ASan runtime was not found")
    return path


def _compile(hipcc: str, src: str, out_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc, *HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
    return obj


def build(verbose: bool = True, sanitize: bool = False) -> str:
    """Compile every kernel source and link ``libmka.so``; returns its path.
    ``sanitize``: the host-sanitized library under ``_build/sanitize/`` instead."""
    hipcc = _hipcc()
    out_dir = SANITIZE_DIR if sanitize else BUILD
    extra = SANITIZE_FLAGS if sanitize else []
    lib = os.path.join(SANITIZE_DIR, "libmka.so") if sanitize else LIB
    os.makedirs(out_dir, exist_ok=True)
    workers = min(len(SOURCES), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(lambda s: _compile(hipcc, s, out_dir, extra), SOURCES))
    tmp = lib + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}", file=sys.stderr)
    return lib


if __name__ == "__main__":
    build(sanitize="--sanitize" in sys.argv[1:])
