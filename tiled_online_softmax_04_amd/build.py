"""Builds libfa.so (the HIP kernels and their C ABI) for gfx950, in-tree.

    python -m tiled_online_softmax_04_amd.build
    python -m tiled_online_softmax_04_amd.build --sanitized   # host code under ASan/UBSan
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libfa.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["fa_api.hip", "fa_prefill.hip", "fa_prefill_fp8.hip", "fa_decode.hip", "fa_merge.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 instructions stay off: the compiler must not form v_pk_*_f32.
# No kernel value is ever NaN by design (padding and out-of-range rows are
# zeroed by index before any arithmetic), so max/min need no NaN canonicalising.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Wall", "-Wno-unused-function",
         "-fno-honor-nans",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # the host pass does not know the gfx950-only feature flag; that warning is harmless
        lines = [ln for ln in text.splitlines()
                 if "packed-fp32-ops' is not a recognized feature" not in ln]
        if lines and (verbose or p.returncode != 0):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, *objs,
           "-Wl,-rpath,/opt/rocm/lib"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


SAN_DIR = os.path.join(BUILD_DIR, "san")
SAN_OUT = os.path.join(SAN_DIR, "libfa_san.so")
# Host code only: the device pass of a .hip file is never instrumented.
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all"]


def sanitizer_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (UBSan's handlers
    are part of it); a process that loads the sanitized library preloads it."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang")
    out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True, check=True).stdout.strip()
    if not os.path.isabs(out) or not os.path.exists(out):
        raise RuntimeError(f"no shared AddressSanitizer runtime found ({out!r})")
    return out


def build_sanitized() -> str:
    """libfa.so with the C ABI layer (fa_api.hip: argument checks, dispatch and
    error reporting) compiled with AddressSanitizer and UndefinedBehaviorSanitizer
    on its host code; the kernel objects are those of build().  Written to
    _build/san/libfa_san.so, never over the product library."""
    objs = [os.path.join(BUILD_DIR, s.replace(".hip", ".o")) for s in SOURCES[1:]]
    if not all(os.path.exists(o) for o in objs):
        build()
    os.makedirs(SAN_DIR, exist_ok=True)
    api_obj = os.path.join(SAN_DIR, "fa_api.o")
    flags = [f for f in FLAGS if f != "-O3"] + SAN_FLAGS
    r = subprocess.run([HIPCC, *flags, "-c", os.path.join(CSRC, "fa_api.hip"), "-o", api_obj],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for the sanitized fa_api.hip:\n" + r.stdout + r.stderr)
    # The sanitizer symbols stay undefined here; the preloaded runtime supplies them.
    tmp = SAN_OUT + ".tmp"
    subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, api_obj, *objs,
                    "-Wl,-rpath,/opt/rocm/lib"], check=True)
    os.replace(tmp, SAN_OUT)
    return SAN_OUT


if __name__ == "__main__":
    if "--sanitized" in sys.argv:
        print(build_sanitized())
    else:
        print(build(verbose="-v" in sys.argv))
