"""Build libtaylor_attn.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Every source is compiled with hipcc for gfx950 only.  Packed float32 vector
instructions are disabled for device code (-packed-fp32-ops); hipcc's host pass
warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libtaylor_attn.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["taylor_abi.cpp", "taylor_decode.hip", "taylor_prefill.hip", "taylor_prefill_n3.hip",
           "taylor_prefill_n3_c128.hip", "taylor_prefill_fb.hip", "taylor_prefill_small.hip",
           "softmax_attn.hip", "taylor_decode_bf16.hip",
           "taylor_hybrid.hip", "taylor_debug.hip"]
# per-source extra flags: the 64-token n = 3 prefill is scheduled for
# instruction-level parallelism (measured faster for it, slower for 128 tokens);
# the n <= 2 prefill and the softmax kernels keep matrix-core results in
# ordinary vector registers (by default the compiler places them in the
# accumulation registers and copies every one back with a vector instruction)
VGPR_MFMA = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
MAX_ILP = ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]
EXTRA = {"taylor_prefill_n3.hip": MAX_ILP, "taylor_prefill_n3_c128.hip": MAX_ILP,
         "softmax_attn.hip": VGPR_MFMA, "taylor_prefill_small.hip": VGPR_MFMA}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", CSRC, "-I", INCLUDE]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, "-x", "hip", *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
