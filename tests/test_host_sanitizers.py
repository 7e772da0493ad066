"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

The C ABI layer (abi.cpp: argument validation, workspace sizing, strides and
overlap checks) is rebuilt with host-side sanitizers and the oracle (oracle.c)
with clang's; a child process with the sanitizer runtime preloaded runs the
ABI validation tests and the oracle's pins against those builds.  Any invalid
memory access or undefined behaviour aborts the child, which fails this test.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RUNTIME = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
CHILD_TESTS = ["tests/test_abi_cpu.py", "tests/test_oracle_score.py", "tests/test_oracle_refine.py",
               "tests/test_oracle_select.py", "tests/test_oracle_h2o.py",
               "tests/test_oracle_select_layer.py", "tests/test_oracle_nestedkv.py"]


@pytest.mark.skipif(not RUNTIME, reason="clang AddressSanitizer runtime not found")
def test_abi_validation_and_oracle_under_asan_ubsan():
    import oracle
    from token_scoring_top_amd import build
    hk_san = build.build_sanitized()
    orc_san = oracle.build_sanitized()
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": RUNTIME[-1],
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "HUBKV_LIB": hk_san,
        "HUBKV_ORACLE_LIB": orc_san,
        "OMP_NUM_THREADS": "1",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *CHILD_TESTS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-4000:] + "\n" + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr, out
