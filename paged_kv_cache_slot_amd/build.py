"""Builds libpa.so for gfx950 with hipcc, in this package folder.

Every HIP source is compiled with packed-fp32 code generation switched off
(`-Xclang -target-feature -Xclang -packed-fp32-ops`); hipcc's host pass warns
that it does not know that feature, which is harmless.

Host-only C++ sources (the block manager) are compiled by the host compiler
and linked into the same library; `bm_bench`, the block manager's host
benchmark executable, is linked from the same object.
"""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpa.so")
BM_BENCH = os.path.join(HERE, "bm_bench")
OBJDIR = os.path.join(HERE, "_build")

SOURCES = ["pa_api.hip", "store_kvcache.hip", "decode.hip", "prefill.hip", "sampler.hip"]
HOST_SOURCES = ["block_manager.cpp"]
CXX = os.environ.get("CXX", "g++")
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", f"-I{INCLUDE}"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src):
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    return obj


def _compile_host(src):
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [CXX, *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 or r.stderr.strip():
        raise RuntimeError(f"{CXX} failed on {src}:\n{r.stderr}")
    return obj


def build(verbose=False):
    """Compiles every source and links libpa.so; returns the library path."""
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = [(_compile, s) for s in SOURCES] + [(_compile_host, s) for s in HOST_SOURCES]
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = list(ex.map(lambda j: j[0](j[1]), jobs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    # The block manager's host benchmark (run by bench.py), linked statically
    # against the same object file.
    host_objs = [o for o in objs if os.path.basename(o) in
                 {os.path.splitext(h)[0] + ".o" for h in HOST_SOURCES}]
    cmd = [CXX, *HOST_FLAGS, os.path.join(CSRC, "bm_bench.cpp"), *host_objs, "-o",
           BM_BENCH + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 or r.stderr.strip():
        raise RuntimeError(f"{CXX} failed on bm_bench.cpp:\n{r.stderr}")
    os.replace(BM_BENCH + ".tmp", BM_BENCH)
    if verbose:
        print(LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
