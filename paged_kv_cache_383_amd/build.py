"""Compile the HIP sources into paged_kv_cache_383_amd/lib/libpagedkv.so for gfx950.

Runs hipcc directly (cross-compiles without a GPU).  Packed-fp32 instructions
are disabled for the device code: the compiler would otherwise form
v_pk_{add,mul,fma}_f32 from ordinary float code.  The feature is a cc1 option
(-Xclang) that hipcc's driver cannot route to the device pass alone
(-Xarch_device and -Xarch_gfx950 both refuse -Xclang), so it reaches the x86
host pass too, which ignores it with one line per source file.  build() drops
exactly that line from the compiler's output and prints every other warning.

A sha256 over the sources, the headers and the compile flags is written beside
the library (libpagedkv.so.sha256).  ensure_built() rebuilds whenever the
library is missing or that fingerprint differs, so a stale binary is never
loaded by the tests, the benchmark or the smoke run.
"""
from __future__ import annotations

import glob
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libpagedkv.so")
STAMP_PATH = LIB_PATH + ".sha256"
SOURCES = ["api.hip", "kv_write.hip", "decode.hip", "decode_noalloc.hip", "copy_blocks.hip", "step.hip",
           "prefill.hip", "read_probe.hip", "mfma_probe.hip", "block_pool.cpp"]
ARCH = "gfx950"
# The host pass's notice about the device-only feature above; nothing else is filtered.
_HOST_FEATURE_NOTICE = "'-packed-fp32-ops' is not a recognized feature for this target"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def compile_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]


def fingerprint() -> str:
    """sha256 over every source and header the library is built from, and the compile flags."""
    h = hashlib.sha256()
    files = sorted(set([os.path.join(CSRC, s) for s in SOURCES] + glob.glob(os.path.join(CSRC, "*.h"))
                       + glob.glob(os.path.join(INCLUDE, "*.h"))))
    for p in files:
        h.update(os.path.relpath(p, ROOT).encode())
        with open(p, "rb") as f:
            h.update(f.read())
    h.update(" ".join(compile_flags()).replace(ROOT, "").encode())
    return h.hexdigest()


def is_current() -> bool:
    if not (os.path.exists(LIB_PATH) and os.path.exists(STAMP_PATH)):
        return False
    with open(STAMP_PATH) as f:
        return f.read().strip() == fingerprint()


def _report(text: str):
    lines = [ln for ln in text.splitlines() if _HOST_FEATURE_NOTICE not in ln]
    if any(ln.strip() for ln in lines):
        sys.stderr.write("\n".join(lines) + "\n")


def build(verbose: bool = False) -> str:
    os.makedirs(LIB_DIR, exist_ok=True)
    tmp = LIB_PATH + ".tmp"
    stamp = fingerprint()
    cmd = [hipcc(), *compile_flags(), "-shared", *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    _report(res.stdout + res.stderr)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, LIB_PATH)
    with open(STAMP_PATH, "w") as f:
        f.write(stamp + "\n")
    return LIB_PATH


SAN_LIB_PATH = os.path.join(LIB_DIR, "libpagedkv_hostsan.so")      # default output of build_host_sanitized


def build_host_sanitized(out_path: str = SAN_LIB_PATH) -> str:
    """The same library with AddressSanitizer and UndefinedBehaviorSanitizer on its host code only (every
    -fsanitize flag goes to the host pass; the gfx950 code is built as usual).  For CPU tests of the host
    paths: argument validation, the block pool and the batch planner.  Load it with the sanitizer runtime
    preloaded (asan_runtime()) and PKV_LIBRARY pointing at it."""
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-shared-libsan",
                "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f if f != "-O3" else "-O1" for f in compile_flags()] + ["-g"] + host_san
    cmd = [hipcc(), *flags, "-shared", *[os.path.join(CSRC, s) for s in SOURCES], "-o", out_path + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    _report(res.stdout + res.stderr)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(out_path + ".tmp", out_path)
    return out_path


def asan_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (it carries the UBSan runtime too)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "lib", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = shutil.which("clang") or "clang"
    res = subprocess.run([clang, "-print-resource-dir"], capture_output=True, text=True, check=True)
    lib = os.path.join(res.stdout.strip(), "lib", "linux", "libclang_rt.asan-x86_64.so")
    if not os.path.exists(lib):
        raise RuntimeError(f"AddressSanitizer runtime not found at {lib}")
    return lib


def ensure_built() -> str:
    """The library, rebuilt first if it is missing or was built from other sources or flags."""
    if not is_current():
        build()
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
