"""The library's host code (argument validation, workspace sizing and carving,
launch set-up) built with AddressSanitizer and UndefinedBehaviorSanitizer and
run through the CPU ABI suite.  Device code is built as usual and no kernel
runs here: every call in that suite is rejected on the host, before any HIP
call.  A report from either sanitizer aborts the child process and fails the
test.  A planted out-of-bounds read of a host array shows the sanitizers live."""
import os
import subprocess
import sys

import pytest

from reconstruction_lact_chunk_amd import build_lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OPTS = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:verify_asan_link_order=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}

RUN_SUITE = """
import sys
sys.path.insert(0, {root!r})
from reconstruction_lact_chunk_amd import binding as B
B._lib = B.load_library({lib!r})
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", "tests/test_abi.py"]))
"""

# zm_ttt_chunked reads offsets[0 .. n_chunks]: an array one entry short makes it
# read past the end (a malloc'd NumPy buffer, so ASan sees it).  With a zero-byte
# workspace the call ends with ZM_ERR_WORKSPACE if nothing is reported.
PLANTED = """
import ctypes, sys
import numpy as np
sys.path.insert(0, {root!r})
from reconstruction_lact_chunk_amd import binding as B
L = B.load_library({lib!r})
d = B.Desc(8, 128, 256, B.BF16, 1, 0, 1024)
offs = np.array([0, 1, 2], dtype=np.int64)
G = ctypes.c_void_p(1 << 20)
st = L.zm_ttt_chunked(ctypes.byref(d), 0, 3, offs.ctypes.data_as(ctypes.c_void_p), None, 1,
                      G, G, G, G, G, G, G, G, G, 0, None)
print("status", st)
"""


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    try:
        runtime = build_lib.sanitizer_runtime()
    except RuntimeError as e:  # pragma: no cover
        pytest.skip(str(e))
    out = tmp_path_factory.mktemp("san") / "libzmttt_san.so"
    lib = build_lib.build(out=str(out), host_sanitize=True)
    return lib, dict(os.environ, LD_PRELOAD=runtime, **OPTS)


def _run(code, env):
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=900)


def test_abi_suite_clean_under_host_asan_ubsan(sanitized):
    lib, env = sanitized
    r = _run(RUN_SUITE.format(root=ROOT, lib=lib), env)
    log = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, log
    assert "AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, log


def test_sanitizers_report_a_planted_host_overread(sanitized):
    lib, env = sanitized
    r = _run(PLANTED.format(root=ROOT, lib=lib), env)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stdout + r.stderr[-3000:]
