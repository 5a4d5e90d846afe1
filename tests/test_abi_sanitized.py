"""The C ABI checks of test_abi.py again, against the library built with
AddressSanitizer on its host code (validation, size arithmetic, status strings,
the static-scratch bookkeeping), in a child process with the sanitizer runtime
preloaded. No GPU: every call fails validation before any launch."""

import os
import subprocess
import sys

import pytest

from causal_attention_attn_amd import build as _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def asan_env():
    try:
        runtime = _build.asan_runtime()
    except RuntimeError as e:
        pytest.fail(str(e))
    if not os.path.exists(_build.ASAN_LIB):
        _build.build_asan()
    env = dict(os.environ)
    env.update(LD_PRELOAD=runtime, ATTN_LIBRARY=_build.ASAN_LIB,
               # the interpreter itself is not instrumented and keeps memory to the end
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=23")
    return env


def _child(args, env):
    return subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=300)


def test_sanitized_library_is_the_one_loaded(asan_env):
    code = ("import causal_attention_attn_amd as a; a.load(); "
            "m = open('/proc/self/maps').read(); "
            "print('asan-runtime' if 'libclang_rt.asan' in m else 'no-runtime'); "
            "print('asan-lib' if 'libattn_asan.so' in m else 'other-lib'); "
            "print(a.attn_status_string(3))")
    res = _child(["-c", code], asan_env)
    assert res.returncode == 0, res.stderr[-2000:]
    assert res.stdout.split()[:2] == ["asan-runtime", "asan-lib"], res.stdout


def test_abi_checks_pass_under_address_sanitizer(asan_env):
    res = _child(["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                  os.path.join("tests", "test_abi.py")], asan_env)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in res.stdout
