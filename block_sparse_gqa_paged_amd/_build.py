"""Compile libpa.so (HIP, gfx950) in place: block_sparse_gqa_paged_amd/libpa.so.

Each .hip source compiles to an object in parallel, then one shared-library link. Flags:
  --offload-arch=gfx950  CDNA4 code objects only
  -O3 -fPIC -std=c++17
  -Xclang -target-feature -Xclang -packed-fp32-ops   no packed fp32 instructions in device code
  -mllvm -amdgpu-mfma-vgpr-form                      MFMA operands and results in VGPRs
The host pass warns that it does not know that feature; the warning is harmless.
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpa.so")
OBJ_DIR = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # MFMA accumulators in VGPRs: avoids AGPR<->VGPR copies around the softmax rescale
         "-mllvm", "-amdgpu-mfma-vgpr-form"]


def _compile(src, verbose):
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    if errs.strip() and verbose:
        print(errs, flush=True)
    return obj


def build(verbose=False, jobs=None):
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
