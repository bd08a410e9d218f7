"""Host-side checks of the C ABI on the CPU (no GPU visible):

* the ABI tests (tests/test_abi.py: every validation path of every entry
  point) against a build whose host code runs under AddressSanitizer and
  UndefinedBehaviorSanitizer (rank_key_sparse_amd.build_sanitized), in a
  subprocess with the ASan runtime preloaded; any sanitizer report fails;
* a valid call on a host where no GPU can run it reports LOKI_ERR_HIP (a
  failed launch mapped to a status, no crash), with and without LOKI_DEBUG.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _no_gpu():
    import torch
    return torch.cuda.device_count() == 0  # counting devices does not initialise a GPU


pytestmark = pytest.mark.skipif(not _no_gpu(), reason="host-only checks: run where no GPU is visible")


def test_abi_tests_under_host_sanitizers():
    from rank_key_sparse_amd import build_sanitized as bs
    lib = bs.build_sanitized()
    env = dict(os.environ, LD_PRELOAD=bs.asan_runtime(), ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", LOKI_LIBRARY=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    report = r.stdout + r.stderr
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-4000:]
    assert r.returncode == 0, report[-4000:]


_CALL = """
import ctypes, sys
sys.path.insert(0, {root!r})
import rank_key_sparse_amd as rks
lib = rks.load_library()
A, A2 = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x20000)
print(lib.loki_project_keys(A, A, A2, 1, 1, 16, 64, 1, None),
      lib.loki_bench_copy(A, A2, ctypes.c_size_t(64), None))
"""


@pytest.mark.parametrize("debug", ["0", "1"])
def test_failed_launch_is_a_status(debug):
    env = dict(os.environ, LOKI_DEBUG=debug)
    r = subprocess.run([sys.executable, "-c", _CALL.format(root=ROOT)], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.split() == ["8", "8"]  # LOKI_ERR_HIP from both calls
