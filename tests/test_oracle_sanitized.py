"""The oracle's pins, re-run against an AddressSanitizer + UndefinedBehavior-
Sanitizer build of the same C source (host code only; the colibri pull
request's KV8 commit reports its codec tests clean under ASan/UBSan, and the
oracle is held to the same bar: no out-of-bounds access, no use of
uninitialised or freed memory, no signed overflow or bad shift, anywhere the
pins reach).

The sanitized library is built into a temporary directory and loaded by a
child pytest process through KVQ_ORACLE_LIB, with the sanitizer runtimes
preloaded (Python itself is not instrumented, so leak checking is off).
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = ["tests/test_oracle_codec.py", "tests/test_oracle_attention.py", "tests/test_oracle_blocks.py",
             "tests/test_oracle_tq.py", "tests/test_golden_page_facts.py"]
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.fixture(scope="module")
def sanitized_env(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    sys.path.insert(0, ROOT)
    from oracle import build
    lib = build.build(SAN_FLAGS, out=str(tmp_path_factory.mktemp("asan") / "liboracle_asan.so"))
    env = dict(os.environ)
    env.update({"KVQ_ORACLE_LIB": lib, "LD_PRELOAD": f"{asan} {ubsan}", "ASAN_OPTIONS": "detect_leaks=0",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1", "OMP_NUM_THREADS": "4"})
    return env


def test_sanitized_build_is_the_one_loaded(sanitized_env):
    """The child process loads the sanitized build, with the ASan runtime in it."""
    code = ("import ctypes, oracle; oracle.lib(); "
            "assert oracle._LIB_PATH.endswith('liboracle_asan.so'), oracle._LIB_PATH; "
            "ctypes.CDLL(None).__asan_report_load1; print('ok')")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=sanitized_env, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stderr[-2000:]


def test_oracle_pins_clean_under_asan_ubsan(sanitized_env):
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        *PIN_FILES], cwd=ROOT, env=sanitized_env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout[-3000:] + r.stderr[-3000:])
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail
