"""Build libmlstm.so (HIP for gfx950) in-tree.

    python -m linear_recurrent_sequence_amd.build

Compiles every ``csrc/*.hip`` translation unit with hipcc for gfx950 (in
parallel, objects under ``_build/`` at the repository root) and links them
into ``linear_recurrent_sequence_amd/libmlstm.so``.  Always recompiles.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libmlstm.so")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from emitting packed float32 VALU ops
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmlstm)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build(verbose=False, extra_flags=()):
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.basename(src)[:-4] + ".o")
        cmd = [hipcc, *CFLAGS, *extra_flags, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
        # hipcc's host pass warns that it does not know the packed-fp32 feature
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("built", LIB_PATH, flush=True)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
