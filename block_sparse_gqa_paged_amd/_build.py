"""Compile libpa.so (HIP, gfx950) in place: block_sparse_gqa_paged_amd/libpa.so.

Each .hip source compiles to an object in parallel, then one shared-library link. Flags:
  --offload-arch=gfx950  CDNA4 code objects only
  -O3 -fPIC -std=c++17
  -Xclang -target-feature -Xclang -packed-fp32-ops   no packed fp32 instructions in device code
  -mllvm -amdgpu-mfma-vgpr-form                      MFMA operands and results in VGPRs
The host pass warns that it does not know that feature; the warning is harmless.
build(sanitize=True, out=...) builds the host code with ASan/UBSan (a CPU check, not the product).
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


# AddressSanitizer and UndefinedBehaviorSanitizer on the host code only (argument checks,
# workspace layout, launch sizing): each flag goes to the host pass; device code is built as
# usual. A process loading that build must preload clang's ASan runtime (asan_runtime()).
SAN_FLAGS = []
for _f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer"):
    SAN_FLAGS += ["-Xarch_host", _f]


def _compile(src, verbose, obj_dir=None, extra=()):
    obj = os.path.join(obj_dir or OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + list(extra) + ["-c", src, "-o", obj]
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


def build(verbose=False, jobs=None, sanitize=False, out=None):
    """Compile every csrc/*.hip and link libpa.so (default in place). sanitize=True builds the
    host code with ASan/UBSan into out (a path outside the package: never the product build)."""
    if sanitize and not out:
        raise ValueError("a sanitized build needs its own output path")
    lib = out or LIB
    obj_dir = os.path.join(os.path.dirname(lib), "_san_obj") if sanitize else OBJ_DIR
    os.makedirs(obj_dir, exist_ok=True)
    extra = SAN_FLAGS + ["-g"] if sanitize else []
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, obj_dir, extra), srcs))
    tmp = lib + ".tmp"
    link_extra = SAN_FLAGS + ["-shared-libsan"] if sanitize else []
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + link_extra + ["-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


def asan_runtime():
    """clang's AddressSanitizer runtime (it also carries the UBSan handlers), to preload into a
    process that loads a sanitized build."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
        return path
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise FileNotFoundError("clang ASan runtime not found")
    return found[-1]


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
