"""Compile the HIP sources under csrc/ into libwise.so (gfx950), in-tree.

    python -m block_sparse_attention_wise_amd.build [--jobs N] [--sanitize-host]

Every source is compiled with hipcc for gfx950 only, with packed-fp32 vector
instructions disabled, then linked into a shared library next to this file.
--sanitize-host builds _build/asan/libwise_asan.so instead: the same library
with its host code under AddressSanitizer (device code unchanged), to be loaded
with the sanitizer runtime preloaded.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libwise.so")
SOURCES = ["attn_bf16.hip", "attn_f32.hip", "support.hip", "wise_abi.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in VGPRs: the online-softmax rescale touches them
    # with VALU ops, and AGPR-resident accumulators cost copies every block
    "-mllvm", "--amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-command-line-argument",
]


# host code only: each sanitizer flag goes to the host compilation
ASAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
ASAN_LIB = os.path.join(BUILD, "asan", "libwise_asan.so")


def _compile(src: str, out_dir: str = BUILD, extra: tuple = ()) -> str:
    obj = os.path.join(out_dir, src + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(jobs: int | None = None, verbose: bool = False, sanitize_host: bool = False) -> str:
    out_dir = os.path.join(BUILD, "asan") if sanitize_host else BUILD
    lib = ASAN_LIB if sanitize_host else LIB
    extra = tuple(ASAN_HOST_FLAGS) if sanitize_host else ()
    os.makedirs(out_dir, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, out_dir, extra), SOURCES))
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--sanitize-host", action="store_true")
    args = ap.parse_args()
    build(args.jobs, verbose=True, sanitize_host=args.sanitize_host)
    sys.exit(0)
