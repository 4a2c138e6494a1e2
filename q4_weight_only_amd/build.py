"""Build libjq4k.so (gfx950) in-tree from csrc/ with hipcc.

Every HIP source is compiled with packed-fp32 instruction selection switched
off; the library links only the HIP runtime.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libjq4k.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["api.hip", "gemv.hip", "gemm.hip", "gemm_ws.hip", "gemm_big.hip", "gemm_rw.hip", "gemm_skinny.hip",
           "kv_convert.hip", "rmsnorm.hip", "exports.hip", "probes.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(HERE, "..", "include"),
]


# Per-source flags.  gemm_rw.hip orders its matrix, vector and LDS
# instructions with scheduling-group barriers; the post-register-allocation
# scheduler would reorder them again (runs of 16 matrix instructions, then
# dozens of vector ones with the matrix cores idle), so it is off there.
EXTRA_FLAGS = {"gemm_rw.hip": ["-mllvm", "--disable-post-ra"]}


def _compile(src, verbose):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    if verbose and errs.strip():
        print(errs, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
