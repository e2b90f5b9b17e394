r"""Build librht_ufp4.so (HIP kernels + C ABI) in-tree for gfx950.

Run as `python -m rht_bit_block_amd.build` or through __graft_entry__.build().
Objects are compiled in parallel; the library is written next to this file.

`python -m rht_bit_block_amd.build --sanitize` builds a second library,
_build/sanitize/librht_ufp4.so, whose host code (argument validation, launch
set-up) is instrumented with AddressSanitizer and UndefinedBehaviorSanitizer
(device code unchanged).  It is for CPU runs of the ABI tests only, with the
compiler's own sanitizer runtime preloaded (it carries the UBSan handlers too)
and Python's small-object allocator off (so host arrays get redzones):
  PYTHONMALLOC=malloc UFP4_LIBRARY=_build/sanitize/librht_ufp4.so \
  LD_PRELOAD=$(/opt/rocm/llvm/bin/clang -print-file-name=libclang_rt.asan-x86_64.so) \
  ASAN_OPTIONS=detect_leaks=0:halt_on_error=1 UBSAN_OPTIONS=halt_on_error=1 \
  python -m pytest tests/test_abi.py tests/test_binding_checks.py
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


# Host-side sanitizers only: each flag goes to the host compilation.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def _compile(src, out_dir=BUILD_DIR, extra=()):
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *CFLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-6000:]}")
    return obj


def build(verbose=True, sanitize=False):
    out_dir = os.path.join(BUILD_DIR, "sanitize") if sanitize else BUILD_DIR
    lib_path = os.path.join(out_dir, LIB_NAME) if sanitize else LIB_PATH
    extra = SANITIZE if sanitize else ()
    os.makedirs(out_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, out_dir, extra), SOURCES))
    tmp = lib_path + ".tmp"
    # a sanitized shared library leaves the runtime to the process (preloaded)
    cmd = [_hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr[-4000:])
    os.replace(tmp, lib_path)
    if verbose:
        print("built", lib_path, file=sys.stderr)
    if not sanitize:
        build_test_helpers(verbose)
    return lib_path


def build_test_helpers(verbose=True):
    """tests/libufp4_hwcheck.so: GPU checks of arithmetic identities the
    kernels rely on (a test library, not part of the product)."""
    src = os.path.join(ROOT, "tests", "hw_identities.hip")
    out = os.path.join(ROOT, "tests", "libufp4_hwcheck.so")
    tmp = out + ".tmp"
    cmd = [_hipcc(), *CFLAGS, "-shared", src, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for tests/hw_identities.hip:\n" + r.stderr[-4000:])
    os.replace(tmp, out)
    if verbose:
        print("built", out, file=sys.stderr)


if __name__ == "__main__":
    build(sanitize="--sanitize" in sys.argv[1:])
