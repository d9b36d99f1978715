"""Builds liblq.so (the HIP kernels and their C ABI) for gfx950, in-tree.

    python -m recurrent_state_quant_lq_amd.build

Each csrc/*.hip file is compiled by hipcc to an object under _build/, then
linked into recurrent_state_quant_lq_amd/liblq.so.  Packed-FP32 instructions
are disabled for all device code.

build(sanitize=True) compiles the host code (argument checks, dispatch) with
AddressSanitizer and UndefinedBehaviorSanitizer, device code unchanged, into
_build_san/liblq_san.so.  The binding loads it when LQ_LIB names it; the
process must preload clang's ASan runtime (sanitizer_runtime()).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblq.so")
BUILD_SAN = os.path.join(PKG, "_build_san")
LIB_SAN = os.path.join(BUILD_SAN, "liblq_san.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-variable"]
# host pass only (each sanitizer option right after -Xarch_host)
SAN_FLAGS = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
             "-Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer").split()


def _compile(src: str, verbose: bool, sanitize: bool = False) -> str:
    obj = os.path.join(BUILD_SAN if sanitize else BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *(SAN_FLAGS if sanitize else []), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only feature name: drop that line
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = LIB_SAN if sanitize else LIB
    os.makedirs(BUILD_SAN if sanitize else BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, sanitize), srcs))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def sanitizer_runtime() -> str:
    """LD_PRELOAD value for a process that loads liblq_san.so: the ASan
    runtime of the compiler hipcc drives (it carries the UBSan handlers)."""
    clang = os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "bin", "clang")
    res = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isfile(path):
        raise RuntimeError(f"no ASan runtime found next to {clang}")
    return path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
