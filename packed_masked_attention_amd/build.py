"""Build libpma.so (gfx950) in-tree with hipcc.

Every source under csrc/ is compiled for gfx950 only, with packed fp32
instructions disabled, and linked into packed_masked_attention_amd/libpma.so.
Run as ``python -m packed_masked_attention_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libpma.so")
BUILD_DIR = os.path.join(ROOT, "_build")
# host code under AddressSanitizer + UndefinedBehaviorSanitizer (device code
# unchanged), for the CPU tests of the host-side checks: libpma_san.so
SAN_LIB = os.path.join(HERE, "libpma_san.so")
SAN_BUILD_DIR = os.path.join(ROOT, "_build_san")
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-I", os.path.join(ROOT, "include"),
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-command-line-argument"]


# Per-source options.  flash_fwd.hip: LLVM's max-ILP machine scheduler orders
# the softmax and the fragment reads between the pinned MFMA/DMA groups better
# than the default occupancy-driven one (same registers, no spills; measured
# 1-4% faster at 4096-32768 keys).
EXTRA = {"flash_fwd.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(SAN_BUILD_DIR if sanitize else BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    extra = EXTRA.get(os.path.basename(src), []) + (SAN_HOST if sanitize else [])
    subprocess.run([HIPCC, *COMMON, *extra, *lang, "-c", src, "-o", obj], check=True)
    return obj


def build(jobs: int = 8, sanitize: bool = False) -> str:
    """libpma.so; with sanitize, libpma_san.so whose host code runs under
    ASan + UBSan (the sanitizer runtime comes from the process: the CPU test
    run preloads clang's shared ASan runtime)."""
    out_dir = SAN_BUILD_DIR if sanitize else BUILD_DIR
    out = SAN_LIB if sanitize else LIB
    os.makedirs(out_dir, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, sanitize), srcs))
    tmp = out + ".tmp%d" % os.getpid()
    link = [] if sanitize else ["-Wl,--no-undefined"]
    subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *link, *objs, "-o", tmp],
                   check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(sanitize="--sanitize" in sys.argv))
    sys.exit(0)
