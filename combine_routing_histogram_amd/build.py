"""Build the gfx950 HIP library libepdc.so in place with hipcc.

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
ARCH = "gfx950"


def hipcc_command(out: str) -> list:
    return [
        "hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Wall", "-Wno-unused-command-line-argument",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        SRC, "-o", out,
    ]


def build(verbose: bool = False) -> str:
    """Compile libepdc.so (always; a few seconds)."""
    tmp = LIB + ".tmp"
    cmd = hipcc_command(tmp)
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
    os.replace(tmp, LIB)
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
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(d) > t for d in DEPS)


if __name__ == "__main__":
    print(build(verbose=True))
