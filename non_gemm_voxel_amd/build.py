"""Build libngv.so (HIP for gfx950) in-tree: non_gemm_voxel_amd/libngv.so.

Every .hip file under csrc/ is compiled with hipcc for gfx950 and linked into
one shared library whose exported symbols are the C ABI of include/ngv.h.
Packed fp32 instructions are switched off (-packed-fp32-ops); the compiler
would otherwise form them from plain float code.
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libngv.so")
ARCH = os.environ.get("NGV_OFFLOAD_ARCH", "gfx950")

FLAGS = ["-std=c++17", "-O3", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas", "-Wno-unused-command-line-argument",
         f"-I{INCLUDE}", f"-I{CSRC}"]


def _compile(src, verbose):
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = ["hipcc"] + FLAGS + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    return obj, warn


def build(verbose=False, jobs=None):
    os.makedirs(OBJ, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, verbose), srcs))
    for _, warn in results:
        if warn and verbose:
            print(warn, flush=True)
    objs = [o for o, _ in results]
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-fvisibility=hidden"] + objs + \
        ["-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
