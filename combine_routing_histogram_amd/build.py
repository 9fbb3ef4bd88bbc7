"""Build the gfx950 HIP libraries in place with hipcc: libepdc.so (the
dispatch/combine path) and libepdc_probe.so (the HBM rate probes the
benchmark compares it with).

Flags: -O3 without fast-math (IEEE fp32 division, denormals kept), and the
packed-fp32 instructions disabled for device code: hipcc would otherwise form
v_pk_{add,mul,fma}_f32 from ordinary float code, and this project keeps those
out of its kernels.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "epdc.hip")
DEPS = [SRC, os.path.join(PKG, "csrc", "epdc_kernels.hpp"), os.path.join(ROOT, "include", "epdc.h")]
LIB = os.path.join(PKG, "libepdc.so")
PROBE_SRC = os.path.join(PKG, "csrc", "hbm_probe.hip")
PROBE_DEPS = [PROBE_SRC, os.path.join(ROOT, "include", "epdc_probe.h"),
              os.path.join(ROOT, "include", "epdc.h")]
PROBE_LIB = os.path.join(PKG, "libepdc_probe.so")
ARCH = "gfx950"


def hipcc_command(out: str, src: str = SRC) -> list:
    return [
        "hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Wall", "-Wno-unused-command-line-argument",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        src, "-o", out,
    ]


def _compile(src: str, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = hipcc_command(tmp, src)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only feature; that warning is expected
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msg}")
    if verbose and msg.strip():
        print(msg, file=sys.stderr)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile libepdc.so and libepdc_probe.so (always; a few seconds)."""
    _compile(SRC, LIB, verbose)
    _compile(PROBE_SRC, PROBE_LIB, verbose)
    _write_build_info()
    return LIB


def _write_build_info() -> None:
    """Record the git revision the library was built at (build_info.json,
    not tracked), so a run on a copy of the tree without .git can say it."""
    import json
    info = {"git": None, "dirty": None}
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "--short=12", "HEAD"],
                           capture_output=True, text=True, timeout=10)
        if r.returncode == 0:
            info["git"] = r.stdout.strip()
            d = subprocess.run(["git", "-C", ROOT, "status", "--porcelain", "--untracked-files=no"],
                               capture_output=True, text=True, timeout=10)
            info["dirty"] = bool(d.stdout.strip()) if d.returncode == 0 else None
    except (OSError, subprocess.SubprocessError):
        pass
    with open(os.path.join(PKG, "build_info.json"), "w") as fh:
        json.dump(info, fh)


def is_stale() -> bool:
    for lib, deps in ((LIB, DEPS), (PROBE_LIB, PROBE_DEPS)):
        if not os.path.exists(lib):
            return True
        t = os.path.getmtime(lib)
        if any(os.path.getmtime(d) > t for d in deps):
            return True
    return False


if __name__ == "__main__":
    print(build(verbose=True))
