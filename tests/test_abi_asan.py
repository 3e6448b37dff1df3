"""The C ABI's host-side argument validation under AddressSanitizer: capi.hip's host code is rebuilt with ASan
(device code unchanged) and tests/test_abi_cpu.py runs against that build in a child process that preloads the ASan
runtime. Every call there fails validation or returns before any HIP call, so no GPU is needed; an out-of-bounds
access or use-after-free in the validation code aborts the child with an ASan report."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_validation_is_clean_under_asan():
    from transformer_attention_causal_amd import build as b
    try:
        lib = b.build_asan()
        rt = b.asan_runtime()
    except RuntimeError as e:
        pytest.skip(f"no ASan toolchain: {e}")
    nm = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True)
    assert "__asan_" in nm.stdout, "the ASan build carries no ASan instrumentation"
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", ATTN_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "AddressSanitizer" not in r.stderr
    assert " passed" in r.stdout
