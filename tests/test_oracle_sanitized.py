"""The oracle's pins run against a build of the oracle with AddressSanitizer
and UndefinedBehaviorSanitizer (host code only, gcc), so an out-of-bounds
access, a signed overflow or a bad shift in the checker itself fails the
suite instead of silently corrupting expected values.

Each run is a child process: the sanitizer runtimes are preloaded into a fresh
interpreter, and EPDC_ORACLE_LIB points the oracle module at the sanitized
copy.  A canary first shows that the setup does catch an overflow.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "epdc_oracle.c")
PIN_FILES = ["test_oracle_route.py", "test_oracle_quant.py", "test_oracle_combine.py",
             "test_oracle_dedup.py"]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("the environment already preloads a library; the sanitizer runtime would "
                    "have to take its place")
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc has no sanitizer runtimes here")
    lib = str(tmp_path_factory.mktemp("san") / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-Wall", "-ffp-contract=off",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", "-shared", "-fPIC", SRC, "-o", lib, "-lm"],
                   check=True)
    env = dict(os.environ, EPDC_ORACLE_LIB=lib, LD_PRELOAD=f"{asan} {ubsan}",
               ASAN_OPTIONS="detect_leaks=0", PYTHONDONTWRITEBYTECODE="1")
    return env


def test_canary_overflow_is_caught(sanitized):
    """oracle_route handed a count array one entry short must abort."""
    code = (
        "import ctypes, numpy as np, os\n"
        "lib = ctypes.CDLL(os.environ['EPDC_ORACLE_LIB'])\n"
        "T, K, E, R = 4, 2, 8, 2\n"
        "idx = np.full(T * K, E - 1, np.int32)\n"
        "cnt = np.zeros(E - 1, np.int32)\n"          # one short
        "eo = np.zeros(E + 1, np.int32); ro = np.zeros(R + 1, np.int32)\n"
        "rc = np.zeros(R, np.int32); so = np.zeros(T * K, np.int32); sp = np.zeros(T * K, np.int32)\n"
        "P = lambda a: a.ctypes.data_as(ctypes.c_void_p)\n"
        "lib.oracle_route.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p] * 7\n"
        "lib.oracle_route(T, K, E, R, P(idx), P(cnt), P(eo), P(ro), P(rc), P(so), P(sp))\n"
        "print('not caught')\n")
    r = subprocess.run([sys.executable, "-c", code], env=sanitized, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0 and "not caught" not in r.stdout
    assert "AddressSanitizer" in r.stderr


def test_pins_pass_under_sanitizers(sanitized):
    files = [os.path.join(ROOT, "tests", f) for f in PIN_FILES]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu"] + files, cwd=ROOT, env=sanitized, capture_output=True,
                       text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "failed" not in r.stdout, tail
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, tail
