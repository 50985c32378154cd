"""Build libbfq.so (the HIP kernels + C-ABI) for gfx950 with hipcc, in-tree.

Usage: python -m block_scaled_w8a8_amd.build   (or call build()).
Object files go to <repo>/_build/bfq/; the library lands next to this file so the Python
binding and the tile table (tables/gfx950.json) are found beside it.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ_DIR = os.path.join(REPO, "_build", "bfq")
LIB_PATH = os.path.join(HERE, "libbfq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["quant.hip", "gemm_std.hip", "gemm_swapab.hip", "moe.hip", "probe.hip", "api.cpp",
           "tile_table.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I" + os.path.join(REPO, "include")]
# Device code: gfx950 only; fp32 division/sqrt correctly rounded (the quantizers' x / scale
# must be the IEEE quotient); packed-fp32 instructions disabled.
DEVICE = ["-x", "hip", "--offload-arch=" + ARCH, "-fhip-fp32-correctly-rounded-divide-sqrt",
          "-ffp-contract=fast", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    flags = COMMON + DEVICE
    cmd = [HIPCC, *flags, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l
                    and "is not a recognized feature" not in l)
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int = 8) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp, *objs, "-ldl"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


# A build whose host code (argument validation, tile selection, the tile-table parser) runs
# under AddressSanitizer and UndefinedBehaviorSanitizer; the device code is the same. Loaded
# through BFQ_LIBRARY by a process that preloads the sanitizer runtime (sanitizer_runtime());
# the CPU tests run against it (tests/test_sanitizers.py). It lives in the build folder, not
# beside the package (no GPU run loads it), so its loader names the tile table with
# BFQ_TILE_TABLE (TABLE_PATH).
ASAN_LIB_PATH = os.path.join(REPO, "_build", "sanitize", "libbfq_asan.so")
TABLE_PATH = os.path.join(HERE, "tables", "gfx950.json")
HOST_SOURCES = ("api.cpp", "tile_table.cpp")
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-O1"]
def sanitizer_runtime() -> str:
    """The clang AddressSanitizer runtime matching hipcc (it carries the UBSan handlers)."""
    import glob
    hits = glob.glob(os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "lib", "llvm", "lib",
                                  "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("no clang AddressSanitizer runtime found next to hipcc")
    return sorted(hits)[-1]


def build_sanitized(jobs: int = 8) -> str:
    """libbfq_asan.so: the host sources built with -fsanitize=address,undefined, linked with
    the kernel objects of the regular build (compiled first if they are missing)."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    objs = []
    todo = []
    for src in SOURCES:
        obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
        if src in HOST_SOURCES:
            obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".asan.o")
            cmd = [HIPCC, *COMMON, *DEVICE, *SANITIZE, "-c", os.path.join(CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stderr}")
        elif not os.path.exists(obj):
            todo.append(src)
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(_compile, todo))
    os.makedirs(os.path.dirname(ASAN_LIB_PATH), exist_ok=True)
    tmp = ASAN_LIB_PATH + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp, *objs, "-ldl",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-shared-libsan"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, ASAN_LIB_PATH)
    return ASAN_LIB_PATH


if __name__ == "__main__":
    print(build())
