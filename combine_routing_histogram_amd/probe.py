"""ctypes binding of libepdc_probe.so (include/epdc_probe.h): the streaming
read, write and copy kernels the benchmark uses to measure the card's HBM
rates.  Arguments are device addresses, sizes and a hipStream_t as integers;
a non-SUCCESS status raises.  Not part of the dispatch/combine path.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import List

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_PATH = os.path.join(PKG, "libepdc_probe.so")
HEADER = os.path.join(ROOT, "include", "epdc_probe.h")

P = ctypes.c_void_p
SZ = ctypes.c_size_t
U32 = ctypes.c_uint32
I32 = ctypes.c_int32

_SIGNATURES = {
    "epdc_probe_read": (I32, [P, SZ, U32, P, P]),
    "epdc_probe_write": (I32, [P, SZ, U32, P]),
    "epdc_probe_copy": (I32, [P, P, SZ, P]),
    "epdc_probe_last_error": (ctypes.c_char_p, []),
}

_lib = None


def lib():
    """Load libepdc_probe.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; build it with "
                           "`python -m combine_routing_histogram_amd.build`")
    l = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        f = getattr(l, name)
        f.restype = res
        f.argtypes = args
    _lib = l
    return l


def header_entry_points() -> List[str]:
    """Names of the functions include/epdc_probe.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\**\s*(epdc_probe_[a-z_]+)\s*\(",
                                 text, flags=re.M)))


def _check(status: int) -> None:
    if status != 0:
        msg = lib().epdc_probe_last_error().decode()
        raise RuntimeError(f"epdc_probe status {status}: {msg}")


def read(src: int, nbytes: int, magic: int, flag: int, stream: int) -> None:
    _check(lib().epdc_probe_read(src, nbytes, magic, flag, stream))


def write(dst: int, nbytes: int, value: int, stream: int) -> None:
    _check(lib().epdc_probe_write(dst, nbytes, value, stream))


def copy(src: int, dst: int, nbytes: int, stream: int) -> None:
    _check(lib().epdc_probe_copy(src, dst, nbytes, stream))
