"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer: the oracle (gcc) running its
own pins, and libpa's host code (hipcc, sanitizers on the host pass only) running the host ABI
checks (argument validation, workspace sizing, the no-allocation entry point's size check). Each
runs in a subprocess that preloads its sanitizer runtime and loads the sanitized build in place
of the normal one; leak checks are off (the interpreter itself does not free everything at
exit), and any address or undefined-behaviour report fails the run."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")

SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run(preload, setup, files, timeout):
    code = (f"import sys\nsys.path.insert(0, {ROOT!r})\nsys.path.insert(0, {TESTS!r})\n"
            f"{setup}\nimport pytest\n"
            f"sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu'] + "
            f"{files!r}))\n")
    env = dict(os.environ, LD_PRELOAD=preload, **SAN_ENV)
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=timeout)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    return out


def test_oracle_pins_under_asan_ubsan(tmp_path):
    from oracle import build
    lib = build.build(sanitize=True, out=str(tmp_path / "liboracle_san.so"))
    files = [os.path.join(TESTS, f) for f in ("test_oracle_fp16.py", "test_oracle_append.py",
                                              "test_oracle_attention.py",
                                              "test_oracle_sparse.py")]
    out = _run(build.asan_runtime(), f"import oracle\noracle._LIB_PATH = {lib!r}", files, 900)
    assert " passed" in out


def test_host_abi_under_asan_ubsan(tmp_path):
    if not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    from block_sparse_gqa_paged_amd import _build
    lib = _build.build(sanitize=True, out=str(tmp_path / "libpa_san.so"))
    files = [os.path.join(TESTS, "test_abi_host.py")]
    out = _run(_build.asan_runtime(),
               f"import block_sparse_gqa_paged_amd as pa\npa.LIB_PATH = {lib!r}", files, 900)
    assert " passed" in out
