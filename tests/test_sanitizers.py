"""The host code of liblinattn.so and the oracle under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only; builds in _build/san, see
tests/sanitizers.py): the ABI tests and the oracle pins must pass with every
instrumented access checked."""
import os
import shutil

import pytest

from tests import sanitizers


@pytest.mark.skipif(not os.path.exists(sanitizers.HIPCC) or sanitizers.clang_asan_runtime() is None,
                    reason="hipcc or the clang ASan runtime is not available")
def test_library_host_code_under_asan_ubsan():
    r = sanitizers.run_library_checks(sanitizers.build_library())
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not available")
def test_oracle_under_asan_ubsan():
    r = sanitizers.run_oracle_checks(sanitizers.build_oracle())
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout
