"""The library used from C alone: tests/c/abi_parity.c (C99, the library's
header and the HIP runtime's C API, no Python in the loop) runs dispatch and
combine for several configurations and compares every output byte with the
oracle, linked into the same program.  The host-only part (sizes, argument
errors, kernel names) runs on the CPU."""
import importlib.util
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def _binary():
    spec = importlib.util.spec_from_file_location("c_build", os.path.join(HERE, "c", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    if mod.is_stale():
        mod.build()
    return mod.BIN


def test_c_consumer_host_checks():
    r = subprocess.run([_binary(), "--cpu"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host checks ok" in r.stdout


@pytest.mark.gpu
def test_c_consumer_parity():
    print("C consumer: dispatch + combine through the C ABI against the oracle", flush=True)
    r = subprocess.run([_binary()], capture_output=True, text=True, timeout=300)
    print(r.stdout[-2000:], flush=True)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "all cases bit-exact" in r.stdout
