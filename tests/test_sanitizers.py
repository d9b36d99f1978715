"""The oracle's CPU pins and the library's host-side argument checks, re-run
under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Each case builds the sanitizer variant of the library, then runs the
corresponding test files in a child process that preloads the sanitizer
runtime and loads that variant.  Any sanitizer report aborts the child, so
the case passes only if every test passes with no report.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.dirname(os.path.abspath(__file__))


def _run_under(preload: str, extra_env: dict, files: list, kexpr: str = "") -> subprocess.CompletedProcess:
    env = dict(os.environ)
    env.update(extra_env)
    env["LD_PRELOAD"] = preload
    # CPython keeps its arenas to the end of the process: leak reports are noise here
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    # -s: a sanitizer report ends the process; uncaptured, it reaches stderr
    cmd = [sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider", "-m", "not gpu", *files]
    if kexpr:
        cmd += ["-k", kexpr]
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def _check(res: subprocess.CompletedProcess):
    out = res.stdout + res.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "runtime error:" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in res.stdout


def test_oracle_pins_under_asan_ubsan():
    from oracle import build as ob
    lib = ob.build(sanitize=True)
    files = [os.path.join(TESTS, f) for f in
             ("test_oracle_codec.py", "test_oracle_window.py", "test_oracle_recurrence.py")]
    # torch is not loaded under the preloaded runtime; its two library pins run unsanitized
    _check(_run_under(ob.sanitizer_runtime(), {"LQ_ORACLE_LIB": lib}, files, "not torch"))


def test_host_argument_checks_under_asan_ubsan():
    from recurrent_state_quant_lq_amd import build as hb
    lib = hb.build(sanitize=True)
    _check(_run_under(hb.sanitizer_runtime(), {"LQ_LIB": lib}, [os.path.join(TESTS, "test_abi.py")]))
