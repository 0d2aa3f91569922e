"""Build libpkv.so (HIP kernels for gfx950 + C-ABI + host allocator) in-tree.

    python -m paged_kv_cache_448_amd.build

Objects go to <repo>/_build/, the library to paged_kv_cache_448_amd/libpkv.so.
Every HIP source is compiled with packed-fp32 instructions disabled.
"""
import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpkv.so")

SOURCES = ["api.cpp", "alloc.cpp", "kv_append.hip", "decode_simt.hip", "decode_mfma.hip", "decode_fp8.hip", "prefill_mfma.hip", "merge.hip", "noalloc.hip"]
ARCH = os.environ.get("PKV_OFFLOAD_ARCH", "gfx950")
COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [_hipcc(), "-x", "hip", f"--offload-arch={ARCH}", *COMMON, "-c", path, "-o", obj]
    else:
        cmd = [_hipcc(), *COMMON, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; drop that line
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    return obj, err


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(_compile, SOURCES))
    for obj, err in results:
        if verbose and err.strip():
            print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", tmp, *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
