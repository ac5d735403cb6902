"""Build libnq.so for gfx950 with hipcc (in-tree; run `python -m sub_bit_weight_amd.build`)."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libnq.so")
ARCH = os.environ.get("NQ_OFFLOAD_ARCH", "gfx950")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-I", INCLUDE, "-I", CSRC,
    # keep the compiler from emitting packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # single-lane atomics only: the atomic optimizer would turn a counter fetch
    # into a wave reduction whose result is waited for at once
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


# Host code only (the gfx950 code is built as usual): AddressSanitizer and
# UndefinedBehaviorSanitizer for the argument checks and planners, which run on
# the CPU.  Load the result with the clang runtime preloaded, e.g.
#   ASAN_OPTIONS=detect_leaks=0 UBSAN_OPTIONS=halt_on_error=1 \
#   LD_PRELOAD=$(/opt/rocm/llvm/bin/clang -print-file-name=libclang_rt.asan-x86_64.so) \
#   NQ_LIBRARY=sub_bit_weight_amd/_build/san/libnq_hostsan.so python -m pytest tests/test_abi.py
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
SAN_BUILD = os.path.join(BUILD, "san")
SAN_LIB = os.path.join(SAN_BUILD, "libnq_hostsan.so")


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(SAN_BUILD if sanitize else BUILD, os.path.basename(src).replace(".hip", ".o"))
    cmd = [hipcc(), *COMMON, *(HOST_SANITIZE if sanitize else []), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, host_sanitize: bool = False) -> str:
    os.makedirs(SAN_BUILD if host_sanitize else BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, host_sanitize), srcs))
    out = SAN_LIB if host_sanitize else LIB
    tmp = out + ".tmp"
    if host_sanitize:  # the sanitizer runtimes come from the preloaded shared runtime
        link = ["-shared-libsan", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    else:  # -z defs: an unresolved symbol (e.g. a kernel never instantiated) fails the link
        link = ["-Wl,-z,defs"]
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *link, *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True, host_sanitize="--host-sanitize" in sys.argv[1:])
    sys.exit(0)
