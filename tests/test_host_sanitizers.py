"""The C ABI's host code under AddressSanitizer + UndefinedBehaviorSanitizer
(CPU only): libmla is rebuilt with both sanitizers on its host pass and the
host-side ABI tests run against it in a child process with the sanitizer
runtime preloaded.  A deliberately undersized host buffer must be reported,
which shows the instrumentation is live."""
import os
import subprocess
import sys

import pytest

from sparse_mla_attention_decode_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

RUN_TESTS = """
import sys
sys.path.insert(0, {root!r})
import sparse_mla_attention_decode_amd as M
M.load_library({lib!r})
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", {tests!r}]))
"""

# the host plan writes num_parts records of 32 bytes: hand it one record too few
OVERFLOW = """
import sys
sys.path.insert(0, {root!r})
import numpy as np
import sparse_mla_attention_decode_amd as M
M.load_library({lib!r})
s = M.make_shape(4, 1, 128, 2048, 64 * 64, num_parts=8, split_granularity=32, fixed_overhead=0)
meta = np.zeros(7 * 8, np.int32)
prefix = np.zeros(5, np.int32)
M.mla_plan_sched_meta_host(s, meta.ctypes.data, prefix.ctypes.data)
print("no report")
"""


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    try:
        rt = B.sanitizer_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = str(tmp_path_factory.mktemp("asan") / "libmla_asan.so")
    B.build_sanitized(lib)
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report_store" in nm and "__ubsan_handle" in nm          # instrumented host code
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return lib, env


def _child(code, env):
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=600)


def test_host_abi_tests_clean_under_sanitizers(sanitized):
    lib, env = sanitized
    r = _child(RUN_TESTS.format(root=ROOT, lib=lib, tests=os.path.join(ROOT, "tests", "test_abi_host.py")), env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "passed" in out and "ERROR: AddressSanitizer" not in out and "runtime error" not in out


def test_sanitizer_reports_an_undersized_buffer(sanitized):
    lib, env = sanitized
    r = _child(OVERFLOW.format(root=ROOT, lib=lib), env)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, (r.stdout + r.stderr)[-3000:]
