"""Build libkda.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950.

    python -m gated_delta_rule_76_amd.build [-v]

Every source is compiled for gfx950 only, with packed-fp32 VALU instructions
disabled (-Xclang -target-feature -Xclang -packed-fp32-ops).  The shared
library lands in gated_delta_rule_76_amd/lib/libkda.so.

A second library, lib/libkda_hostsan.so, links the same kernel objects with
the C ABI layer (kda_api.cpp: argument validation and dispatch) built with
the host AddressSanitizer and UndefinedBehaviorSanitizer (-Xarch_host, so the
device code is untouched).  The ABI tests load it, with the sanitizer runtime
preloaded, through KDA_LIBRARY (tests/test_abi_sanitized.py).
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(PKG, "lib")
LIB = os.path.join(OUT_DIR, "libkda.so")
OBJ_DIR = os.path.join(ROOT, "_build")
SAN_LIB = os.path.join(OUT_DIR, "libkda_hostsan.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]

SOURCES = ["kda_api.cpp", "kda_decode.hip", "kda_prefill.hip", "kda_backward.hip"]
ARCH = "gfx950"


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe) and shutil.which(exe) is None:
        raise RuntimeError("hipcc not found; the KDA library needs ROCm's hipcc")
    return exe


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument",
            "-I", INCLUDE, "-I", CSRC]


def _compile(src, verbose, extra=(), suffix=".o"):
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + suffix)
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc()] + common_flags() + lang + list(extra) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out, verbose, extra=()):
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs + list(extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


def build(verbose=False):
    """Compile every source and link lib/libkda.so and the host-sanitized
    lib/libkda_hostsan.so; returns the path of lib/libkda.so."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    os.makedirs(OUT_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES) + 1) as ex:
        jobs = [ex.submit(_compile, s, verbose) for s in SOURCES]
        san = ex.submit(_compile, "kda_api.cpp", verbose, ["-O1", "-g"] + SAN_FLAGS, ".san.o")
        objs = [j.result() for j in jobs]
        san_obj = san.result()
    _link(objs, LIB, verbose)
    _link([san_obj] + [o for o in objs if not o.endswith("kda_api.cpp.o")], SAN_LIB, verbose,
          SAN_FLAGS + ["-shared-libsan"])
    return LIB


def sanitizer_runtime():
    """Path of the clang AddressSanitizer runtime that lib/libkda_hostsan.so
    needs preloaded (the one shipped with ROCm's clang), or None."""
    import glob
    hits = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))),
                                         "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
