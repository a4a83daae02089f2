"""The C ABI's host code under AddressSanitizer, UndefinedBehaviorSanitizer and libstdc++
assertions: api.cpp is rebuilt with them (device code unchanged) and tests/test_abi.py runs
against that build in a child process with the sanitizer runtime preloaded. Every validation
path those tests reach (null pointers, sizes out of range, misalignment, workspace sizes, the
error text) then runs instrumented; a sanitizer report or an assertion fails the child."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_under_host_sanitizers(tmp_path):
    from whisper_asr_encoder_amd import build
    try:
        build.hipcc()
        rt = build.sanitizer_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = build.build_sanitized(str(tmp_path / "san"))
    env = dict(os.environ, LD_PRELOAD=rt, EDDA_LIBRARY=lib, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    probe = ("import sys; sys.path.insert(0, %r); from whisper_asr_encoder_amd import _lib; _lib.load(); "
             "maps = open('/proc/self/maps').read(); "
             "assert 'libedda_san.so' in maps and 'libclang_rt.asan' in maps, 'sanitized build not loaded'; "
             "print('loaded', _lib.LIB_PATH)" % ROOT)
    r = subprocess.run([sys.executable, "-c", probe], env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")], env=env, cwd=ROOT, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:] + r.stderr[-3000:])
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
    assert " passed" in r.stdout
