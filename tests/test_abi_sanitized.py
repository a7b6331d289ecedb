"""The C ABI's host code under AddressSanitizer and UBSan, without a GPU.

msa_api.hip (argument checks, workspace planning, error paths, the noalloc
scratch bookkeeping) is rebuilt with the sanitizers on its host code only
(build.build_sanitized; the device code and the other objects are the normal
build), loaded through MSA_LIBRARY with the clang ASan runtime preloaded, and
every test of test_abi.py runs against it in a child process.  Any heap or
stack error, or any undefined behaviour (signed overflow, bad shifts, misaligned
or null accesses...), aborts the child and fails this test.
"""
import os
import shutil
import subprocess
import sys

import pytest

from block_sparse_attention_idx_amd import build

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.timeout(900)
def test_abi_tests_pass_under_asan_and_ubsan():
    if not os.path.exists(build.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc is not available")
    lib = build.build_sanitized()
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_" in syms and "__ubsan_" in syms, "the host code was not instrumented"
    env = dict(os.environ)
    env.update(LD_PRELOAD=build.asan_runtime(), MSA_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",  # the Python process itself leaks by design
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_abi.py")],
                       env=env, capture_output=True, text=True, timeout=850, cwd=os.path.dirname(HERE))
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, out
    assert " passed" in r.stdout, out
