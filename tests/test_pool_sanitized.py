"""The C++ block pool under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

pool.cpp is pure host C++ (hash maps, a linked free queue, index arithmetic), so it is
built a second time with g++ -fsanitize=address,undefined into a host-only library, and the
pool-against-the-oracle-model suites are run against that build in a child process
(PKV_LIBRARY selects it; the sanitiser runtimes are preloaded because the interpreter is
not built with them). Any out-of-bounds access, use after free or undefined operation
aborts the child, so the test fails on the first one. Leak checking is off: the
interpreter itself does not free everything at exit.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_28_amd", "csrc")
SUITES = ["tests/test_pool_host.py::test_pool_matches_oracle_model",
          "tests/test_pool_host.py::test_exhaustion_is_atomic_and_counted",
          "tests/test_pool_host.py::test_invalid_pool_arguments",
          "tests/test_pool_host.py::test_seventeen_tokens_take_two_blocks",
          "tests/test_pool_host.py::test_seventeen_tokens_at_other_block_sizes",
          "tests/test_pool_prefix_host.py::test_prefix_cache_fork_and_copy_on_write_match_the_model",
          "tests/test_churn_pool.py"]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_pool_suites_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = str(tmp_path / "libpkv_pool_san.so")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-shared", "-fPIC",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    os.path.join(CSRC, "pool.cpp"), "-o", lib], check=True)
    env = dict(os.environ, PKV_LIBRARY=lib, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *SUITES], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    tail = (r.stdout[-3000:] + r.stderr[-3000:])
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr + r.stdout, tail
