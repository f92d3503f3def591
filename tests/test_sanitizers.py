"""Host-side sanitizer runs (CPU only, no GPU).

The library's host code (argument checks, workspace layouts, the ABI) is
built with AddressSanitizer and UndefinedBehaviorSanitizer on its host pass
(_build.build(sanitize=True)) and the ABI tests run against that build; the
C oracle is built with gcc's AddressSanitizer and UndefinedBehaviorSanitizer
and its pins run against it.  Each run is a child pytest process with the
matching sanitizer runtime preloaded; it must pass with no sanitizer report.
"""
import importlib.util
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer", "SUMMARY: UndefinedBehavior")


def _load_build():
    spec = importlib.util.spec_from_file_location(
        "_specverify_build_san", os.path.join(ROOT, "lossless_draft_verification_amd", "_build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _run(tests, env_extra, timeout=900):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    out = r.stdout + r.stderr
    return r.returncode, out


def _child_loads(code, env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0"
    return subprocess.check_output([sys.executable, "-c", code], cwd=ROOT, env=env, text=True).strip()


def test_library_host_code_under_asan_ubsan(tmp_path):
    b = _load_build()
    lib = b.build(sanitize=True, path=str(tmp_path / "libspecverify_san.so"))
    env = {"SPEC_LIBRARY": lib, "LD_PRELOAD": b.asan_runtime()}
    # the child really runs the sanitized build, with the runtime active
    seen = _child_loads("import ctypes, lossless_draft_verification_amd as L; "
                        "print(L.library_path(), hasattr(ctypes.CDLL(None), '__asan_init'))", env)
    assert seen == f"{lib} True", seen
    rc, out = _run(["tests/test_abi.py"], env)
    assert rc == 0 and not any(k in out for k in REPORTS), out[-4000:]
    assert "passed" in out


def test_oracle_under_asan_ubsan(tmp_path):
    lib = oracle.build(str(tmp_path / "liboracle_san.so"), sanitize=True)
    asan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    tests = ["tests/test_oracle_greedy.py", "tests/test_oracle_softmax.py", "tests/test_oracle_ragged.py",
             "tests/test_oracle_draw_fallbacks.py", "tests/test_oracle_philox.py"]
    env = {"SPEC_ORACLE_LIBRARY": lib, "LD_PRELOAD": asan}
    seen = _child_loads("import ctypes, oracle; print(oracle.default().path, "
                        "hasattr(ctypes.CDLL(None), '__asan_init'))", env)
    assert seen == f"{lib} True", seen
    rc, out = _run(tests, env)
    assert rc == 0 and not any(k in out for k in REPORTS), out[-4000:]
    assert "passed" in out
