"""The C ABI's host-side code under AddressSanitizer (CPU only): the library is
rebuilt with its host code instrumented (device code unchanged) whenever a
source is newer than that build, and tests/test_abi.py runs against it in a
child process with the sanitizer runtime preloaded, so that an out-of-bounds or
use-after-free access in the argument validation, workspace sizing or status
paths aborts the run."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _asan_library():
    from block_sparse_attention_wise_amd import build as B
    sources = [os.path.join(B.CSRC, f) for f in os.listdir(B.CSRC)] + [os.path.join(ROOT, "include", "wise.h")]
    newest = max(os.path.getmtime(f) for f in sources)
    if not os.path.exists(B.ASAN_LIB) or os.path.getmtime(B.ASAN_LIB) < newest:
        B.build(sanitize_host=True)
    return B.ASAN_LIB


def test_abi_validation_under_address_sanitizer():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in this ROCm installation")
    lib = _asan_library()
    # the build is instrumented: its host code calls into the sanitizer runtime
    nm = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True)
    if nm.returncode == 0:
        assert "__asan_" in nm.stdout, "the host-sanitizer build carries no instrumentation"
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               WISE_ABI_TEST_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout and "AddressSanitizer" not in r.stderr
