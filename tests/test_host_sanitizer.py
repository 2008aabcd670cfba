"""The host side of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer: the CPU ABI and binding tests run again in a
fresh Python that loads the host-sanitized build (host code only, no device
code) with the ASan runtime preloaded.  Any invalid access or undefined
behaviour in argument validation, descriptor checks, byte counts or
workspace sizing aborts that process."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def hostsan_lib():
    from compressed_index_matmul_amd import build
    try:
        build.asan_runtime()
    except (RuntimeError, OSError) as e:
        pytest.skip(f"no ASan runtime: {e}")
    return build.build_hostsan()


def test_abi_under_host_sanitizers(hostsan_lib):
    from compressed_index_matmul_amd import build
    env = build.hostsan_env()
    probe = ("import ctypes, compressed_index_matmul_amd as vq; "
             "assert vq.LIB_PATH.endswith('libvqmm_hostsan.so'); vq.lib(); "
             "ctypes.CDLL(None).__asan_address_is_poisoned; print('asan runtime active')")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "asan runtime active" in r.stdout, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_abi.py", "tests/test_binding_checks.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
