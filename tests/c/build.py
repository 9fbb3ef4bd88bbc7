"""Compile the C consumer test program (abi_parity.c) with gcc: C99, the
library's header, the HIP runtime's C API, linked against the built
libepdc.so and the oracle's liboracle.so (run-time paths set to where they
were built).  Host code only; no GPU code is compiled here.

    python tests/c/build.py
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_parity.c")
BIN = os.path.join(HERE, "abi_parity")
LIB_DIR = os.path.join(ROOT, "combine_routing_histogram_amd")
ORACLE_DIR = os.path.join(ROOT, "oracle")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def command(out: str = BIN) -> list:
    return ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
            SRC, "-o", out,
            os.path.join(LIB_DIR, "libepdc.so"), os.path.join(ORACLE_DIR, "liboracle.so"),
            f"-Wl,-rpath,{LIB_DIR}", f"-Wl,-rpath,{ORACLE_DIR}",
            "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]


def is_stale() -> bool:
    if not os.path.exists(BIN):
        return True
    t = os.path.getmtime(BIN)
    deps = [SRC, os.path.join(ROOT, "include", "epdc.h"), os.path.join(LIB_DIR, "libepdc.so"),
            os.path.join(ORACLE_DIR, "liboracle.so")]
    return any(os.path.exists(d) and os.path.getmtime(d) > t for d in deps)


def build(verbose: bool = False) -> str:
    cmd = command(BIN + ".tmp")
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed ({r.returncode}):\n{r.stdout}{r.stderr}")
    os.replace(BIN + ".tmp", BIN)
    return BIN


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
