"""Build libtreedraft.so for gfx950 with hipcc (in-tree, next to this file).

Every .hip source under csrc/ is compiled to an object in _build/ in
parallel and linked into one shared library.  Packed-fp32 instructions are
disabled for the device code (-packed-fp32-ops).
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtreedraft.so")
ARCH = os.environ.get("TD_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # matrix-core accumulators in ordinary VGPRs: the online softmax
         # rescales them with vector ALU ops, which cannot address AGPRs
         "-mllvm", "-amdgpu-mfma-vgpr-form=1", "-Wall",
         "-Wno-unused-function"]


# Per-source additions.  The attention kernels compare and take maxima of
# scores that are never NaN (masked keys are -inf): without NaN semantics a
# maximum is one instruction, not a canonicalisation and a maximum.
EXTRA = {"tree_attn.hip": ["-fno-honor-nans"]}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device feature name: drop that notice
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip() and verbose:
        print(err, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
