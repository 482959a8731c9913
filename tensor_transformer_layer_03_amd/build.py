"""Build libtplayer.so (the HIP kernels + C ABI) for gfx950 with hipcc.

Usage: python -m tensor_transformer_layer_03_amd.build [--jobs N] [--asan]
Compiles every source in csrc/ to an object under _build/ (in parallel) and
links the shared library next to this file. Always recompiles.

--asan builds libtplayer_asan.so instead (objects under _build_asan/): the
same sources with AddressSanitizer on the host code only (device code is
built as usual), for the CPU tests of the C ABI's host-side validation. A
process loading it must preload the ASan runtime (asan_runtime()).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtplayer.so")
BUILD_ASAN = os.path.join(HERE, "_build_asan")
LIB_ASAN = os.path.join(HERE, "libtplayer_asan.so")
ARCH = "gfx950"
# AddressSanitizer on the host pass only (each -fsanitize right after -Xarch_host)
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep fp32 arithmetic off the packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=fast", "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libtplayer.so)")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def asan_runtime() -> str:
    """Path of the clang ASan runtime that a process loading LIB_ASAN preloads."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "lib", "llvm", "bin", "clang")
    for cand in (clang, "/opt/rocm/llvm/bin/clang", shutil.which("clang") or ""):
        if cand and os.path.exists(cand):
            r = subprocess.run([cand, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
            path = r.stdout.strip()
            if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
                return path
    raise RuntimeError("clang ASan runtime (libclang_rt.asan-x86_64.so) not found")


# Per-source flags. The attention kernels keep their MFMA accumulators in
# VGPRs: with the compiler's default the softmax rescale and the loop-carried
# outputs were copied between AGPRs and VGPRs on every key tile (about 128
# extra VALU moves per tile at head size 128), and the forward needed 340
# registers instead of 252.
SOURCE_FLAGS = {"attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, asan: bool = False) -> str:
    obj = os.path.join(BUILD_ASAN if asan else BUILD, os.path.basename(src) + ".o")
    extra = SOURCE_FLAGS.get(os.path.basename(src), [])
    cmd = [hipcc(), *FLAGS, *extra, *(ASAN_FLAGS if asan else []), "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int | None = None, verbose: bool = False, asan: bool = False) -> str:
    out_dir, lib = (BUILD_ASAN, LIB_ASAN) if asan else (BUILD, LIB)
    os.makedirs(out_dir, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2) // 2), 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, asan), srcs))
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", *(["-shared-libasan"] + ASAN_FLAGS if asan else []),
           "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--asan", action="store_true")
    args = ap.parse_args()
    build(args.jobs, verbose=True, asan=args.asan)
    sys.exit(0)
