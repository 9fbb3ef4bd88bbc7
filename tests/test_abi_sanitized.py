"""The host side of libepdc.so (argument checks, configuration rules,
workspace layout) under AddressSanitizer and UndefinedBehaviorSanitizer: the
library is rebuilt with its host pass instrumented (device code as usual),
the CPU boundary tests run against that build in a child process with the
sanitizer runtime preloaded, and a canary built the same way shows that an
out-of-bounds write is caught.  CPU only; no GPU work is launched.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

from combine_routing_histogram_amd import build as hip_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BOUNDARY_TESTS = ["tests/test_abi.py", "tests/test_abi_config_fuzz.py"]
SAN = "address,undefined"


def _host_sanitized(cmd):
    """hipcc flags that instrument the host pass only."""
    out = []
    for f in ("-fsanitize=" + SAN, "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"):
        out += ["-Xarch_host", f]
    return cmd[:1] + out + cmd[1:]


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    if shutil.which("hipcc") is None:
        pytest.skip("no hipcc")
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("the environment already preloads a library; the sanitizer runtime would "
                    "have to take its place")
    rts = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rts:
        pytest.skip("no clang sanitizer runtime")
    d = tmp_path_factory.mktemp("abi_san")
    lib = str(d / "libepdc_san.so")
    r = subprocess.run(_host_sanitized(hip_build.hipcc_command(lib)), capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    canary_src = d / "canary.hip"
    canary_src.write_text(
        "#include <cstdlib>\n"
        "extern \"C\" int canary(int n) {\n"
        "    int *p = static_cast<int *>(std::malloc(sizeof(int) * n));\n"
        "    for (int i = 0; i <= n; ++i) p[i] = i;  // one past the end\n"
        "    int s = p[0];\n"
        "    std::free(p);\n"
        "    return s;\n"
        "}\n")
    canary = str(d / "libcanary.so")
    cmd = hip_build.hipcc_command(canary, str(canary_src))
    r = subprocess.run(_host_sanitized(cmd), capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, LD_PRELOAD=rts[-1], ASAN_OPTIONS="detect_leaks=0",
               PYTHONDONTWRITEBYTECODE="1")
    return {"lib": lib, "canary": canary, "env": env, "dir": d}


def test_canary_overflow_is_caught(sanitized):
    code = ("import ctypes, sys\n"
            f"l = ctypes.CDLL({sanitized['canary']!r})\n"
            "l.canary(8)\n"
            "print('not caught')\n")
    r = subprocess.run([sys.executable, "-c", code], env=sanitized["env"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0 and "not caught" not in r.stdout
    assert "AddressSanitizer" in r.stderr


def test_boundary_tests_pass_under_sanitizers(sanitized):
    runner = sanitized["dir"] / "run.py"
    runner.write_text(
        "import sys\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "from combine_routing_histogram_amd import binding\n"
        f"binding.LIB_PATH = {sanitized['lib']!r}\n"
        "import pytest\n"
        "rc = pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu'] + sys.argv[1:])\n"
        "assert binding.lib()._name == binding.LIB_PATH\n"
        "sys.exit(rc)\n")
    files = [os.path.join(ROOT, f) for f in BOUNDARY_TESTS]
    r = subprocess.run([sys.executable, str(runner)] + files, cwd=ROOT, env=sanitized["env"],
                       capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "failed" not in r.stdout, tail
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, tail
