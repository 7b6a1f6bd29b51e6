"""The host side of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer: builds libtpcol_san.so (host code instrumented,
every undefined-behaviour finding fatal) and runs the CPU ABI tests against
it in a child process with the ASan runtime preloaded."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def san_env():
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc is not installed")
    from megatron_tensor_transformer_col_amd import _build_sanitized as bs
    lib = bs.build()
    env = dict(os.environ)
    env.update(LD_PRELOAD=bs.asan_runtime(), TPCOL_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    return env, lib


def test_sanitized_library_is_the_one_loaded(san_env):
    env, lib = san_env
    code = ("import megatron_tensor_transformer_col_amd as tp; tp.lib(); "
            "m = open('/proc/self/maps').read(); "
            "print('san' if 'libtpcol_san.so' in m else 'plain', 'asan' if 'libclang_rt.asan' in m else 'noasan')")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    assert r.stdout.split() == ["san", "asan"], r.stdout


def test_abi_tests_pass_under_sanitizers(san_env):
    env, _ = san_env
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
