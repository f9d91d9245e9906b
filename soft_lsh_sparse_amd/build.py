"""Build libsocket_lsh.so (HIP, gfx950) in-tree.

Usage: python -m soft_lsh_sparse_amd.build   (or call build_library()).
Each csrc/*.hip file is compiled separately (in parallel) with hipcc for
--offload-arch=gfx950 and the objects are linked into one shared library
next to this file. Packed float32 instructions are disabled on purpose.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_NAME = "libsocket_lsh.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = "gfx950"

COMMON_FLAGS = [
    "-O3",
    "-std=c++17",
    f"--offload-arch={ARCH}",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


# Per-source additions. hash_keys.hip: the tile counter's answer is read a
# tile after the request; the atomic optimizer would combine the request
# across lanes and wait for the answer at once.
FILE_FLAGS = {
    "hash_keys.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"],
}


def _hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build the library")
    return path


def _compile(src: str, obj: str) -> None:
    cmd = [_hipcc(), *COMMON_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    # hipcc's host pass does not know the packed-fp32 feature; that warning is
    # expected and harmless, anything else is surfaced.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    extra = [ln for ln in (r.stderr or "").splitlines() if ln.strip() and noise not in ln]
    if extra:
        sys.stderr.write("\n".join(extra) + "\n")


def build_library(verbose: bool = True) -> str:
    """Compile every csrc/*.hip and link LIB_PATH. Always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD_DIR, os.path.basename(s)[:-4] + ".o") for s in sources]
    workers = max(1, min(len(sources), os.cpu_count() or 1, 8))
    with cf.ThreadPoolExecutor(workers) as ex:
        list(ex.map(_compile, sources, objs))
    tmp = LIB_PATH + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(sources)} sources")
    return LIB_PATH


if __name__ == "__main__":
    build_library()
