"""Build libroute.so for gfx950 with hipcc.

Each ``csrc/*.hip`` file is compiled to an object under ``_build/`` (in
parallel) and the objects are linked into ``libroute.so`` next to this file.
Run ``python -m token_routing_speculation_amd.build`` or call ``build()``.

``build_host_asan()`` (``--host-asan``) builds a second copy under
``_build_asan/`` whose host code (argument checks, launch set-up, the host
side of the prefetch DMA) carries AddressSanitizer; the device code is
compiled as usual. It is loaded through the ROUTE_LIBRARY variable with the
clang AddressSanitizer runtime preloaded, on a machine without a GPU.
"""

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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libroute.so")
BUILD_ASAN = os.path.join(ROOT, "_build_asan")
LIB_ASAN = os.path.join(BUILD_ASAN, "libroute_asan.so")
# host-only sanitizer flags: each one behind -Xarch_host, so device code is untouched
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    # keep hipcc from forming packed binary32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand):
        raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")
    return cand


def _compile(src: str, out_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(out_dir, os.path.basename(src).replace(".hip", ".o"))
    cmd = [hipcc(), *HIP_FLAGS, *extra, f"-I{INCLUDE}", f"-I{CSRC}", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every HIP source and link libroute.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found")
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)), 16)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


def asan_runtime() -> str | None:
    """The clang AddressSanitizer runtime shipped with ROCm's compiler, if any."""
    root = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    for base in (os.path.join(root, "llvm"), os.path.join(root, "lib", "llvm"), "/opt/rocm/llvm"):
        hits = sorted(glob.glob(os.path.join(base, "lib", "clang", "*", "lib", "linux",
                                             "libclang_rt.asan-x86_64.so")))
        if hits:
            return hits[-1]
    return None


def build_host_asan(jobs: int | None = None) -> str:
    """libroute_asan.so: the same sources with AddressSanitizer on the host code."""
    os.makedirs(BUILD_ASAN, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)), 16)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda f: _compile(f, BUILD_ASAN, ["-g", *HOST_ASAN]), srcs))
    tmp = LIB_ASAN + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, *HOST_ASAN,
           "-Xarch_host", "-shared-libsan", "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB_ASAN)
    return LIB_ASAN


if __name__ == "__main__":
    if "--host-asan" in sys.argv[1:]:
        print(build_host_asan())
    else:
        build(verbose=True)
    sys.exit(0)
