"""Build the CPU oracle (test infrastructure) into oracle/liboracle.so with gcc.

-ffp-contract=off keeps the float32 rotary products from being fused; no -ffast-math, no
threads. Run as ``python oracle/build.py`` or through ``__graft_entry__.build()``.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


# AddressSanitizer and UndefinedBehaviorSanitizer build (host code; a CPU check of the oracle):
# every undefined-behaviour report aborts. A process loading it must preload gcc's libasan.
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
            "-g"]


def build(verbose=False, sanitize=False, out=None):
    """Compile oracle.c into out (default oracle/liboracle.so); sanitize=True adds ASan/UBSan."""
    lib = out or LIB
    cmd = (["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
            "-Wall", "-Wextra"] + (SANITIZE if sanitize else []) +
           ["-o", lib + ".tmp", SRC, "-lm"])
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


def asan_runtime():
    """gcc's AddressSanitizer runtime, to preload into a process that loads the sanitized build."""
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
