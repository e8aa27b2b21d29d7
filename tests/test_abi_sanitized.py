"""The C-ABI checks (tests/test_abi.py) again, in a child process whose libxs.so is the host-side
AddressSanitizer + UndefinedBehaviorSanitizer build (paged_kv_decode_xs_amd/build.py,
build_host_sanitized): argument validation, the thread-local error string and the graph
descriptor checks run under both sanitizers, which abort the child on the first report. CPU only:
nothing here launches a kernel."""

import os
import subprocess
import sys

import pytest

from paged_kv_decode_xs_amd import build as xb_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _fresh() -> bool:
    lib = xb_build.SAN_LIB
    if not os.path.exists(lib):
        return False
    t = os.path.getmtime(lib)
    srcs = xb_build.sources() + [os.path.join(xb_build.INCLUDE, "xs", "xs.h")]
    srcs += [os.path.join(xb_build.CSRC, f) for f in os.listdir(xb_build.CSRC) if f.endswith(".h")]
    return all(os.path.getmtime(s) <= t for s in srcs)


@pytest.fixture(scope="module")
def sanitized_library():
    try:
        xb_build.hipcc()
        xb_build.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    if not _fresh():
        xb_build.build_host_sanitized()
    return xb_build.SAN_LIB


def test_abi_suite_under_asan_and_ubsan(sanitized_library):
    env = xb_build.sanitizer_env()
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "tests/test_abi.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout[-3000:] + r.stderr[-3000:])
    assert "AddressSanitizer" not in tail and "runtime error" not in tail, tail
    assert r.returncode == 0, tail
    assert " passed" in r.stdout


def test_sanitized_build_is_instrumented(sanitized_library):
    out = subprocess.run(["nm", "-D", sanitized_library], capture_output=True, text=True).stdout
    assert "__asan_report" in out and "__ubsan_handle" in out
