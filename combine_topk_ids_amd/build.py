"""Build libmoe_ep.so (the C ABI of include/moe_ep.h) for gfx950 with hipcc, in-tree."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["routing.hip", "dispatch_ll.hip", "movement.hip", "gemm.hip", "gemm_stream.hip", "gemm_fp8.hip", "router.hip", "fp8.hip", "api.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-Wall",
         # code object v5: loadable by the HIP runtime torch ships as well as by /opt/rocm's
         "-mcode-object-version=5",
         # packed fp32 instructions stay off (see the kernels' build notes)
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
LIB = os.path.join(HERE, "libmoe_ep.so")


def _compile(src: str, outdir: str, verbose: bool) -> str:
    obj = os.path.join(outdir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    outdir = os.path.join(HERE, "_build")
    os.makedirs(outdir, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, outdir, verbose), SOURCES))
    cmd = [HIPCC, "--offload-arch=gfx950", "-mcode-object-version=5", "-shared", "-fPIC", *objs, "-o",
           LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
