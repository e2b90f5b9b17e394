"""Build librht_ufp4.so (HIP kernels + C ABI) in-tree for gfx950.

Run as `python -m rht_bit_block_amd.build` or through __graft_entry__.build().
Objects are compiled in parallel; the library is written next to this file.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB_NAME = "librht_ufp4.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["api.cpp", "quant.hip", "quant_e1m2.hip", "quant_int4.hip", "quant_e2m1.hip", "quant_e4m3.hip",
           "gemm.hip", "gemm_rd.hip", "gemm_mx.hip", "misc.hip", "noalloc.hip"]

# -ffp-contract=off: every fp32 operation that decides an output bit is an
# explicit round-to-nearest op; no silent fma contraction.
# packed-fp32-ops disabled: no v_pk_{add,mul,fma}_f32 are generated.
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
    "-Wall", "-Wno-unused-function",
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-6000:]}")
    return obj


def build(verbose=True):
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr[-4000:])
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("built", LIB_PATH, file=sys.stderr)
    return LIB_PATH


if __name__ == "__main__":
    build()
