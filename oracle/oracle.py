"""CPU oracle for MoE dispatch/combine -- TEST INFRASTRUCTURE ONLY.

Thin numpy/ctypes front end of ``epdc_oracle.c`` (plain C loops, single
thread; a second build of the same source with OpenMP runs the loops over
tokens on all host cores, selected with ``use_openmp``).  Only ``tests/``, the smoke check and the benchmark's CPU-baseline
leg may import this module; the product path never does, and the HIP library
shares no code with it.  See the C file's header for the passages of the MORI
pages each step follows.

The composition below follows the order the pages' dispatch implies: count
the routing, scan it to expert and rank offsets, give every (token, k) pair a
row, then copy (or quantize once per token and copy) the token's row and its
weights/scales/indices rows to every row it owns.  Combine gathers the K rows
of each token back and sums them with their weights in fp32.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "epdc_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_OMP_LIB_PATH = os.path.join(_HERE, "liboracle_omp.so")
_libs = {}
_variant = "plain"

GCC_CMD = ["gcc", "-O2", "-std=c11", "-Wall", "-Wno-unknown-pragmas", "-ffp-contract=off",
           "-shared", "-fPIC", _SRC]


def _build_one(path: str, extra) -> str:
    tmp = path + ".tmp"
    subprocess.run(GCC_CMD + list(extra) + ["-o", tmp, "-lm"], check=True)
    os.replace(tmp, path)
    return path


def build() -> str:
    """Compile the oracle library in place (plain gcc, no fast-math), and
    the OpenMP build of the same source beside it."""
    _build_one(_OMP_LIB_PATH, ["-fopenmp"])
    return _build_one(_LIB_PATH, [])


def use_openmp(on: bool = True) -> int:
    """Route every oracle call to the OpenMP build (on) or the plain
    single-thread build (off).  Returns the threads the token loops use."""
    global _variant
    _variant = "openmp" if on else "plain"
    return int(_load().oracle_num_threads())


def _stale(path: str) -> bool:
    return not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC)


def _load():
    lib = _libs.get(_variant)
    if lib is not None:
        return lib
    if _variant == "openmp":
        path = _OMP_LIB_PATH
        if _stale(path):
            _build_one(path, ["-fopenmp"])
    else:
        # EPDC_ORACLE_LIB: a separately built copy of the oracle (the mutation
        # and sanitizer tests build copies and run the pins against them)
        path = os.environ.get("EPDC_ORACLE_LIB")
        if not path:
            path = _LIB_PATH
            if _stale(path):
                _build_one(path, [])
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    L = ctypes.c_long
    lib.oracle_route.argtypes = [I, I, I, I, P, P, P, P, P, P, P]
    lib.oracle_route.restype = I
    lib.oracle_scatter_rows.argtypes = [I, I, P, P, L, P]
    lib.oracle_scatter_rows.restype = None
    lib.oracle_quant_fp8.argtypes = [I, I, P, P, P]
    lib.oracle_quant_fp8.restype = I
    lib.oracle_quant_mxfp4.argtypes = [I, I, P, P, P]
    lib.oracle_quant_mxfp4.restype = I
    lib.oracle_combine.argtypes = [I, I, I, P, P, P, P, P]
    lib.oracle_combine.restype = None
    lib.oracle_combine_push.argtypes = [I, I, I, I, P, P, P, P, P, P, P]
    lib.oracle_route_units.argtypes = [I, I, I, I, P, P, P, P, P]
    lib.oracle_route_units.restype = I
    lib.oracle_gather_rows.argtypes = [I, P, P, L, P]
    lib.oracle_units_to_experts.argtypes = [L, P, P, P, L, P]
    lib.oracle_experts_to_units.argtypes = [I, I, I, P, P, P, P, P, P]
    lib.oracle_combine_units.argtypes = [I, I, I, P, P, P, P, P]
    lib.oracle_e4m3_encode_array.argtypes = [L, P, P]
    lib.oracle_e2m1_encode_array.argtypes = [L, P, P]
    lib.oracle_f32_to_bf16_array.argtypes = [L, P, P]
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = I
    _libs[_variant] = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


# ---- scalar encoders (array forms) -----------------------------------------

def e4m3_encode(v) -> np.ndarray:
    v = _c(v, np.float32).ravel()
    out = np.empty(v.size, np.uint8)
    _load().oracle_e4m3_encode_array(v.size, _ptr(v), _ptr(out))
    return out


def e2m1_encode(v) -> np.ndarray:
    v = _c(v, np.float64).ravel()
    out = np.empty(v.size, np.uint8)
    _load().oracle_e2m1_encode_array(v.size, _ptr(v), _ptr(out))
    return out


def f32_to_bf16(v) -> np.ndarray:
    v = _c(v, np.float32).ravel()
    out = np.empty(v.size, np.uint16)
    _load().oracle_f32_to_bf16_array(v.size, _ptr(v), _ptr(out))
    return out


# ---- routing: histogram, exclusive scan, stable slots ------------------------

def route(indices: np.ndarray, num_experts: int, num_ranks: int) -> Dict[str, np.ndarray]:
    """Histogram, exclusive scan and stable slots for int32 indices [T,K]."""
    idx = _c(indices, np.int32)
    T, K = idx.shape
    E, R = int(num_experts), int(num_ranks)
    n = T * K
    cnt = np.zeros(E, np.int32)
    expert_off = np.zeros(E + 1, np.int32)
    rank_off = np.zeros(R + 1, np.int32)
    recv_count = np.zeros(R, np.int32)
    slot_of = np.zeros(n, np.int32)
    src = np.full(n, -1, np.int32)
    invalid = _load().oracle_route(T, K, E, R, _ptr(idx), _ptr(cnt), _ptr(expert_off),
                                   _ptr(rank_off), _ptr(recv_count), _ptr(slot_of), _ptr(src))
    if invalid < 0:
        raise ValueError("oracle_route: bad arguments")
    n_valid = n - invalid
    return {"cnt": cnt, "expert_off": expert_off, "rank_off": rank_off,
            "recv_count": recv_count, "slot_of": slot_of,
            "src_token_pos": src[:n_valid].copy(), "invalid": invalid, "n_valid": n_valid}


# ---- row copies ----------------------------------------------------------------

def scatter_rows(src_rows: np.ndarray, slot_of: np.ndarray, topk: int, n_rows: int) -> np.ndarray:
    """dst[slot_of[t*K+k]] = src_rows[t]; src_rows any dtype [T, ...]."""
    src = np.ascontiguousarray(src_rows)
    T = src.shape[0]
    row_bytes = src.nbytes // T if T else src.itemsize
    dst = np.zeros((n_rows,) + src.shape[1:], dtype=src.dtype)
    so = _c(slot_of, np.int32)
    _load().oracle_scatter_rows(T, int(topk), _ptr(so), _ptr(src), row_bytes, _ptr(dst))
    return dst


# ---- quantization ---------------------------------------------------------------

def quant_fp8(x_bf16: np.ndarray):
    """bf16 bits [T,H] -> (E4M3 codes uint8 [T,H], fp32 scales [T,H/128])."""
    x = _c(x_bf16, np.uint16)
    T, H = x.shape
    q = np.empty((T, H), np.uint8)
    s = np.empty((T, H // 128), np.float32)
    if _load().oracle_quant_fp8(T, H, _ptr(x), _ptr(q), _ptr(s)) != 0:
        raise ValueError("hidden must be a multiple of 128")
    return q, s


def quant_mxfp4(x_bf16: np.ndarray):
    """bf16 bits [T,H] -> (packed E2M1 uint8 [T,H/2], E8M0 scales uint8 [T,H/32])."""
    x = _c(x_bf16, np.uint16)
    T, H = x.shape
    q = np.empty((T, H // 2), np.uint8)
    s = np.empty((T, H // 32), np.uint8)
    if _load().oracle_quant_mxfp4(T, H, _ptr(x), _ptr(q), _ptr(s)) != 0:
        raise ValueError("hidden must be a multiple of 32")
    return q, s


# ---- whole dispatch / combine --------------------------------------------------

def dispatch(x: np.ndarray, weights: Optional[np.ndarray], indices: np.ndarray,
             num_experts: int, num_ranks: int, quant: str = "none",
             scales: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Reference dispatch.

    ``x``: bf16 bits uint16 [T,H], or (quant "none" only) any byte rows [T,P]
    to be carried unchanged.  ``scales``: optional per-token rows to carry
    (quant "none" only).  Returns the received rows for the n_valid valid
    pairs, in slot order: ``out``, ``out_weights``, ``out_scales``,
    ``out_indices``, plus the routing (``recv_count``, ``expert_off``,
    ``rank_off``, ``slot_of``, ``src_token_pos``).
    """
    idx = _c(indices, np.int32)
    T, K = idx.shape
    r = route(idx, num_experts, num_ranks)
    n = r["n_valid"]
    so = r["slot_of"]
    if quant == "none":
        payload, sc = x, scales
    elif quant == "fp8_e4m3_b128":
        if scales is not None:
            raise ValueError("scales are produced by quantization")
        payload, sc = quant_fp8(x)
    elif quant == "mxfp4_b32":
        if scales is not None:
            raise ValueError("scales are produced by quantization")
        payload, sc = quant_mxfp4(x)
    else:
        raise ValueError(quant)
    out = dict(r)
    out["out"] = scatter_rows(payload, so, K, n)
    out["out_indices"] = scatter_rows(idx, so, K, n)
    out["out_weights"] = None if weights is None else scatter_rows(_c(weights, np.float32), so, K, n)
    out["out_scales"] = None if sc is None else scatter_rows(sc, so, K, n)
    return out


def combine(inp: np.ndarray, weights: Optional[np.ndarray], slot_of: np.ndarray,
            tokens: int, topk: int):
    """Reference combine: bf16 bits [N,H] (received layout) -> (bf16 bits [T,H], fp32 [T,K])."""
    x = _c(inp, np.uint16)
    H = x.shape[1]
    so = _c(slot_of, np.int32)
    w = None if weights is None else _c(weights, np.float32)
    out = np.empty((tokens, H), np.uint16)
    out_w = np.empty((tokens, topk), np.float32)
    _load().oracle_combine(int(tokens), H, int(topk), _ptr(so), _ptr(x), _ptr(w),
                           _ptr(out), _ptr(out_w))
    return out, out_w


# ---- scatter combine ------------------------------------------------------------

def combine_push(inp: np.ndarray, weights: Optional[np.ndarray], src_token_pos: np.ndarray,
                 slot_of: np.ndarray, tokens: int, topk: int):
    """Scatter combine: each received row, weighted in fp32, pushed to its
    pair's staging row; each token adds its staging rows in k order.
    Returns (bf16 bits [T,H], fp32 [T,K], the fp32 staging rows [T*K,H])."""
    x = _c(inp, np.uint16)
    H = x.shape[1]
    src = _c(src_token_pos, np.int32)
    so = _c(slot_of, np.int32)
    w = None if weights is None else _c(weights, np.float32)
    staging = np.zeros((tokens * topk, H), np.float32)
    out = np.empty((tokens, H), np.uint16)
    out_w = np.empty((tokens, topk), np.float32)
    _load().oracle_combine_push(src.size, int(tokens), H, int(topk), _ptr(src), _ptr(so), _ptr(x),
                                _ptr(w), _ptr(staging), _ptr(out), _ptr(out_w))
    return out, out_w, staging


# ---- rank-deduplicated dispatch and the standard-MoE conversion ------------------

def route_units(indices: np.ndarray, num_experts: int, num_ranks: int) -> Dict[str, np.ndarray]:
    """One unit per (token, destination rank): unit_cnt [R] (rows per rank),
    unit_off [R+1], unit_of [T*K] (-1 for an invalid expert), unit_src [U]."""
    idx = _c(indices, np.int32)
    T, K = idx.shape
    R = int(num_ranks)
    cnt = np.zeros(R, np.int32)
    off = np.zeros(R + 1, np.int32)
    unit_of = np.zeros(T * K, np.int32)
    src = np.zeros(T * min(K, R), np.int32)
    U = _load().oracle_route_units(T, K, int(num_experts), R, _ptr(idx), _ptr(cnt), _ptr(off),
                                   _ptr(unit_of), _ptr(src))
    if U < 0:
        raise ValueError("oracle_route_units: bad arguments")
    return {"unit_cnt": cnt, "unit_off": off, "unit_of": unit_of, "unit_src": src[:U].copy(),
            "units": U}


def gather_rows(src_rows: np.ndarray, unit_src: np.ndarray) -> np.ndarray:
    """dst[u] = src_rows[unit_src[u]]."""
    src = np.ascontiguousarray(src_rows)
    T = src.shape[0]
    row_bytes = src.nbytes // T if T else src.itemsize
    us = _c(unit_src, np.int32)
    dst = np.zeros((us.size,) + src.shape[1:], dtype=src.dtype)
    _load().oracle_gather_rows(us.size, _ptr(us), _ptr(src), row_bytes, _ptr(dst))
    return dst


def dispatch_dedup(x: np.ndarray, weights: Optional[np.ndarray], indices: np.ndarray,
                   num_experts: int, num_ranks: int, quant: str = "none",
                   scales: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Reference rank-deduplicated dispatch: the token's row (quantized once
    per token when asked) and its weights/scales/indices rows, once per unit.
    Also returns the pair routing (``slot_of`` ...) the conversion uses."""
    idx = _c(indices, np.int32)
    out = dict(route(idx, num_experts, num_ranks))
    u = route_units(idx, num_experts, num_ranks)
    out.update(u)
    if quant == "none":
        payload, sc = x, scales
    elif quant == "fp8_e4m3_b128":
        payload, sc = quant_fp8(x)
    elif quant == "mxfp4_b32":
        payload, sc = quant_mxfp4(x)
    else:
        raise ValueError(quant)
    us = u["unit_src"]
    out["recv_count"] = u["unit_cnt"]
    out["out"] = gather_rows(payload, us)
    out["out_indices"] = gather_rows(idx, us)
    out["out_weights"] = None if weights is None else gather_rows(_c(weights, np.float32), us)
    out["out_scales"] = None if sc is None else gather_rows(sc, us)
    return out


def units_to_experts(unit_rows: np.ndarray, slot_of: np.ndarray, unit_of: np.ndarray,
                     n_rows: int) -> np.ndarray:
    """Standard-MoE conversion of unit rows [U, ...] into expert-layout rows [n_rows, ...]."""
    src = np.ascontiguousarray(unit_rows)
    U = src.shape[0]
    row_bytes = src.nbytes // U if U else src.itemsize
    so = _c(slot_of, np.int32)
    uo = _c(unit_of, np.int32)
    dst = np.zeros((n_rows,) + src.shape[1:], dtype=src.dtype)
    _load().oracle_units_to_experts(so.size, _ptr(so), _ptr(uo), _ptr(src), row_bytes, _ptr(dst))
    return dst


def experts_to_units(inp: np.ndarray, weights: Optional[np.ndarray], unit_src: np.ndarray,
                     unit_of: np.ndarray, slot_of: np.ndarray, topk: int) -> np.ndarray:
    """Weighted sum of each unit's expert rows: bf16 bits [N,H] -> bf16 bits [U,H]."""
    x = _c(inp, np.uint16)
    H = x.shape[1]
    us = _c(unit_src, np.int32)
    w = None if weights is None else _c(weights, np.float32)
    out = np.empty((us.size, H), np.uint16)
    _load().oracle_experts_to_units(us.size, H, int(topk), _ptr(us), _ptr(_c(unit_of, np.int32)),
                                    _ptr(_c(slot_of, np.int32)), _ptr(x), _ptr(w), _ptr(out))
    return out


def combine_units(partial: np.ndarray, unit_weights: Optional[np.ndarray], unit_of: np.ndarray,
                  tokens: int, topk: int):
    """Sum of each token's unit rows (ascending rank): bf16 bits [U,H] ->
    (bf16 bits [T,H], fp32 [T,K] weights read back from the unit rows)."""
    x = _c(partial, np.uint16)
    H = x.shape[1]
    w = None if unit_weights is None else _c(unit_weights, np.float32)
    out = np.empty((tokens, H), np.uint16)
    out_w = np.empty((tokens, topk), np.float32)
    _load().oracle_combine_units(int(tokens), H, int(topk), _ptr(_c(unit_of, np.int32)), _ptr(x),
                                 _ptr(w), _ptr(out), _ptr(out_w))
    return out, out_w
