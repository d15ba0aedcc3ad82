"""The CPU ABI checks (tests/test_abi.py) again, against a build of the
library whose host code carries AddressSanitizer and UndefinedBehaviorSanitizer
(device code unchanged): every validation path runs with out-of-bounds,
use-after-free and undefined-behaviour detection on."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCLANG = "/opt/rocm/llvm/bin/clang"


def _asan_runtime():
    if not os.path.exists(HIPCLANG):
        return None
    out = subprocess.run([HIPCLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                         text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def test_abi_checks_under_host_sanitizers():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no ASan runtime in this toolchain")
    sys.path.insert(0, ROOT)
    from head_latent_attention_16_amd import build as B

    lib = B.build(sanitize=True)
    env = dict(os.environ, MLA_LIB_PATH=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
