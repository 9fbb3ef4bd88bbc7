"""Benchmark: MoE dispatch + combine on one MI355X.

One step = one dispatch (routing histogram, scan, stable slots, scatter of the
rows with their weights / indices, quantized on the fly where the workload
asks) followed by one combine (gather + fp32 weighted top-k sum).  The
headline workload is DeepSeek-V3-shaped: 4096 tokens x hidden 7168, bf16,
top-8 of 256 experts (Zipf 1.1 routing), 8 virtual ranks, and its combine
consumes the dispatch output (identity experts).  Inputs are resident in HBM
before any timed region.  Prints one JSON line.

Protocol of the headline figure (value, ms_per_step):
  * before every step (warm-up and timed alike) a 512 MiB scratch buffer is
    written, which evicts the 4 MB L2s and the 256 MB MALL; the write is
    outside the timed region;
  * HIP events on the launch stream bracket the dispatch and the combine
    separately; a step's time is their sum;
  * value = tokens / median step time over --steps (>= 20) timed steps;
  * every timed step's outputs (counts, source positions, payload, carried
    rows, produced scales, combine output and weights) are compared bit for
    bit with the CPU oracle's on the same inputs before the next step runs.
Secondary figures under their own keys: `warm` (steps back to back, no
flush: part of each kernel's data is still in the MALL from the step
before), `clean_flush` (512 MiB read instead of written before each step, so
the MALL holds no dirty lines of other data), `kernels` (per-kernel HIP
events in a further pass under the headline protocol), `workloads` (the
FP8, MXFP4, decode and pre-quantized-FP8 workloads under the headline
protocol, each with parity on every timed step), `cpu_baseline` (the oracle,
plain C, on one thread and with OpenMP over tokens on all host cores,
median of 3 whole steps each), `ceilings` (HBM read, write and copy rates of
streaming probe kernels over 4 GiB, and each kernel's read and written bytes
priced at those rates against its measured time).

roofline: the kernel with the most time in the per-kernel pass; algorithmic
bytes per launch / its mean event duration, against 8000 GB/s.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E, AMD's published figure
HEADLINE = "deepseek_v3_bf16"
EXTRA_WORKLOADS = ["deepseek_v3_fp8", "qwen3_moe_mxfp4", "decode_bf16", "deepseek_v3_raw_fp8"]
FLUSH_BYTES = 512 << 20


def log(msg: str) -> None:
    print(f"bench: {msg}", file=sys.stderr, flush=True)


# ---- algorithmic bytes ----------------------------------------------------------------

def row_sizes(w):
    """(input row bytes the scatter reads per token, payload P and scale Q
    bytes per received row).  Raw workloads read and carry their byte row and
    its scale row unchanged."""
    H = w.hidden
    if w.raw_row_bytes:
        return w.raw_row_bytes + w.scale_row_bytes, w.raw_row_bytes, w.scale_row_bytes
    P, Q = {"none": (2 * H, 0), "fp8_e4m3_b128": (H, 4 * H // 128),
            "mxfp4_b32": (H // 2, H // 32)}[w.quant]
    return 2 * H, P, Q


def alg_bytes_units(kernel: str, w, units: int) -> int:
    """Algorithmic bytes of the rank-deduplicated path's launches, for U =
    `units` unit rows (one per (token, destination rank)):
      dispatch scatter:   read x (2H; a raw row and its scales: P + Q) +
                          weights and indices (8K) per token;
                          write U rows (P + Q + 8K carried), slot_of,
                          src_token_pos and unit_of (12K) per token, unit_src (4U)
      units_to_experts:   read U rows (P + Q + 8K) and unit_src; read unit_of
                          and slot_of (8K per token); write N rows (P + Q + 8K)
      experts_to_units:   read N rows (2H) + one weight each (4N), the pair
                          arrays (8N) and unit_src (4U); write U rows (2H)
      combine_units:      read U rows (2H) + unit_of (4K per token); write T
                          rows (2H) and their K weights read back (8K)
    """
    T, H, K = w.tokens, w.hidden, w.topk
    N = T * K
    U = units
    X, P, Q = row_sizes(w)
    if kernel.startswith("k_scatter"):
        return T * (X + 8 * K + 12 * K) + U * (P + Q + 8 * K + 4)
    if kernel == "k_units_to_experts":
        return U * (P + Q + 8 * K + 4) + 8 * N + N * (P + Q + 8 * K)
    if kernel == "k_experts_to_units":
        return N * (2 * H + 4 + 8) + U * (4 + 2 * H)
    if kernel == "k_combine_units":
        return U * 2 * H + T * (4 * K + 2 * H + 8 * K)
    if kernel == "k_route_rank":
        return 8 * N * 2
    raise ValueError(kernel)


def alg_bytes(kernel: str, w) -> int:
    """Algorithmic bytes one launch of `kernel` must move for workload w.

    Per token (N = T*K pairs, P/Q = payload/scale bytes per received row):
      scatter: read the row (2H; a raw row and its scales: P + Q) + weights
               and indices (8K); write K rows
               (K*(P+Q)), each slot's weight and index rows (8K^2), slot_of
               and src_token_pos (8K)
      combine: read K rows (2KH) + slot_of and the K weights (8K); write
               the row (2H) and its K weights (4K)
      route:   read the indices (4K); write the in-tile ranks (4K); the scan
               of its last block only touches the small tile table (counted
               as 0)
    """
    T, H, K = w.tokens, w.hidden, w.topk
    X, P, Q = row_sizes(w)
    if kernel.startswith("k_scatter"):
        per = X + 8 * K + K * (P + Q) + 8 * K * K + 8 * K
    elif kernel == "k_combine":
        per = 2 * K * H + 8 * K + 2 * H + 4 * K
    elif kernel == "k_combine_push":
        # read each received row (2H) and its weight and pair (8); write the
        # fp32 products to the pair's staging row (4H)
        per = K * (2 * H + 8 + 4 * H)
    elif kernel == "k_combine_reduce":
        # read the K staging rows (4KH) + slot_of and weights (8K); write the
        # row (2H) and its K weights (4K)
        per = 4 * K * H + 8 * K + 2 * H + 4 * K
    elif kernel == "k_route_rank":
        per = 8 * K
    elif kernel == "k_check_indices":
        return 0
    else:
        raise ValueError(kernel)
    return per * T


def alg_read_write(kernel: str, w):
    """alg_bytes(kernel, w) split into (bytes read, bytes written), for the
    pair path's launches (route, scatter, gather combine)."""
    T, H, K = w.tokens, w.hidden, w.topk
    X, P, Q = row_sizes(w)
    if kernel.startswith("k_scatter"):
        return T * (X + 8 * K), T * (K * (P + Q) + 8 * K * K + 8 * K)
    if kernel == "k_combine":
        return T * (2 * K * H + 8 * K), T * (2 * H + 4 * K)
    if kernel == "k_route_rank":
        return T * 4 * K, T * 4 * K
    raise ValueError(kernel)


def scatter_kernel(w) -> str:
    return {"none": "k_scatter_copy", "fp8_e4m3_b128": "k_scatter_fp8",
            "mxfp4_b32": "k_scatter_mxfp4"}[w.quant]


def step_alg_bytes(w, path: str, combine: str, units) -> int:
    """The method's bytes for one step: x read once, K row copies written, K
    rows read back, one row written, plus the small per-pair arrays (the
    route's own index read and rank array are workspace traffic, not
    counted)."""
    sk = scatter_kernel(w)
    if path == "dedup":
        return sum(alg_bytes_units(k, w, units) for k in
                   (sk, "k_units_to_experts", "k_experts_to_units", "k_combine_units"))
    if combine == "scatter":
        return alg_bytes(sk, w) + alg_bytes("k_combine_push", w) + alg_bytes("k_combine_reduce", w)
    return alg_bytes(sk, w) + alg_bytes("k_combine", w)


# ---- records of what was measured ------------------------------------------------------

def kernel_source_hash() -> str:
    from combine_routing_histogram_amd.profiling import kernel_source_hash as h
    return h()


def file_hash(path: str) -> str:
    try:
        with open(path, "rb") as fh:
            return hashlib.sha256(fh.read()).hexdigest()[:16]
    except OSError:
        return None


def revision() -> dict:
    """Git revision of the tree (when .git is present), else the one the
    library was built at (build_info.json written by the build)."""
    rev = {"git": None, "built_at_git": None}
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "--short=12", "HEAD"],
                           capture_output=True, text=True, timeout=10)
        if r.returncode == 0:
            rev["git"] = r.stdout.strip()
    except (OSError, subprocess.SubprocessError):
        pass
    info = os.path.join(ROOT, "combine_routing_histogram_amd", "build_info.json")
    if os.path.exists(info):
        try:
            rev["built_at_git"] = json.load(open(info)).get("git")
        except (OSError, ValueError):
            pass
    return rev


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


# ---- the oracle: expected outputs and the CPU baseline ------------------------------------

def oracle_step(w, inp, path: str, combine: str) -> dict:
    """One whole step in the oracle: the arrays the GPU step must reproduce."""
    from oracle import oracle  # test infrastructure: expected values and the CPU leg only

    identity = w.combine_input == "identity"
    T, K = inp["indices"].shape
    if path == "dedup":
        d = oracle.dispatch_dedup(inp["x"], inp["weights"], inp["indices"], w.experts, w.ranks,
                                  quant=w.quant, scales=inp.get("scales"))
        n = d["n_valid"]
        e_out = oracle.units_to_experts(d["out"], d["slot_of"], d["unit_of"], n)
        e_w = oracle.units_to_experts(d["out_weights"], d["slot_of"], d["unit_of"], n)
        c_in = e_out if identity else inp["combine_input"]
        part = oracle.experts_to_units(c_in, e_w, d["unit_src"], d["unit_of"], d["slot_of"], K)
        y, y_w = oracle.combine_units(part, d["out_weights"], d["unit_of"], T, K)
        return {"recv": d["recv_count"], "payload": d["out"], "y": y, "y_w": y_w,
                "rows": d["units"], "scales": d["out_scales"]}
    d = oracle.dispatch(inp["x"], inp["weights"], inp["indices"], w.experts, w.ranks,
                        quant=w.quant, scales=inp.get("scales"))
    c_in = d["out"] if identity else inp["combine_input"]
    if combine == "scatter":
        y, y_w, _ = oracle.combine_push(c_in, d["out_weights"], d["src_token_pos"],
                                        d["slot_of"], T, K)
    else:
        y, y_w = oracle.combine(c_in, d["out_weights"], d["slot_of"], T, K)
    return {"recv": d["recv_count"], "payload": d["out"], "weights": d["out_weights"],
            "indices": d["out_indices"], "scales": d["out_scales"],
            "src_pos": d["src_token_pos"], "y": y, "y_w": y_w, "rows": d["n_valid"]}


def _same(a: dict, b: dict) -> bool:
    import numpy as np

    for k in a:
        x, y = a[k], b.get(k)
        if x is None or y is None:
            if (x is None) != (y is None):
                return False
            continue
        if not np.array_equal(np.ascontiguousarray(x).view(np.uint8),
                              np.ascontiguousarray(y).view(np.uint8)):
            return False
    return True


def cpu_baseline(w, inp, reps: int, path: str, combine: str, builds=(False, True)):
    """The oracle timed on whole steps: the plain single-thread build, then
    the same source built with OpenMP over tokens on all host cores; median
    of `reps` steps each (time.perf_counter, a monotonic clock).  Returns the
    baseline record and the first leg's outputs, which the GPU's timed steps
    are checked against."""
    from oracle import oracle  # test infrastructure: used by this leg only

    legs, expected, same = [], None, None
    for omp in builds:
        threads = oracle.use_openmp(omp)
        times, res = [], None
        for _ in range(reps):
            t0 = time.perf_counter()
            res = oracle_step(w, inp, path, combine)
            times.append(time.perf_counter() - t0)
        med = statistics.median(times)
        legs.append({"value": w.tokens / med, "unit": "tokens/s", "cores": threads,
                     "median_s": med, "times_s": times,
                     "build": "gcc -O2 -fopenmp" if omp else "gcc -O2 (plain)"})
        if expected is None:
            expected = res
        else:
            same = _same(expected, res)
    oracle.use_openmp(False)
    best = legs[-1]
    base = {"value": best["value"], "unit": "tokens/s", "cores": best["cores"],
            "host_cores": os.cpu_count(), "kind": "oracle",
            "sample": f"median of {reps} whole {'rank-deduplicated ' if path == 'dedup' else ''}"
                      f"dispatch+combine steps of {w.name} ({w.tokens} tokens each) per leg; "
                      f"legs: plain C on 1 thread, the same source with OpenMP over tokens",
            "legs": legs}
    if same is not None:
        base["openmp_result_identical"] = same
    return base, expected


# ---- the GPU side ---------------------------------------------------------------------------

# 512 MiB fills queued ahead of a back-to-back block of steps (about 70 us each)
BACK_TO_BACK_GATE_FILLS = 16


class HipEvent:
    """A HIP event of the process's HIP runtime (the one torch loaded),
    created with hipEventDisableSystemFence: recording it takes the
    timestamp without the system-scope release (an L2 write-back) that a
    default timing event performs, which would otherwise add its own cost
    between the two kernels it separates.  Timing only; never used to make
    device memory visible to the host."""
    _hip = None
    FLAGS = 0x20000000   # hipEventDisableSystemFence

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            import ctypes
            path = next((l.split()[-1] for l in open("/proc/self/maps")
                         if "libamdhip64" in l), "libamdhip64.so.7")
            h = ctypes.CDLL(path)
            P = ctypes.c_void_p
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(P), ctypes.c_uint]
            h.hipEventRecord.argtypes = [P, P]
            h.hipEventSynchronize.argtypes = [P]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), P, P]
            h.hipEventDestroy.argtypes = [P]
            cls._hip = h
        return cls._hip

    def __init__(self):
        import ctypes
        self._ct = ctypes
        self.ev = ctypes.c_void_p()
        if self._lib().hipEventCreateWithFlags(ctypes.byref(self.ev), self.FLAGS) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream):
        if self._lib().hipEventRecord(self.ev, stream.cuda_stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def synchronize(self):
        if self._lib().hipEventSynchronize(self.ev) != 0:
            raise RuntimeError("hipEventSynchronize failed")

    def elapsed_time(self, end) -> float:
        ms = self._ct.c_float()
        if self._lib().hipEventElapsedTime(self._ct.byref(ms), self.ev, end.ev) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.ev:
            self._hip.hipEventDestroy(self.ev)


class Bench:
    """One workload on the GPU: op, resident inputs, expected outputs on the
    device, and the step / check / timing loops."""

    def __init__(self, w, dev, path="pair", combine="gather", graph=False, events="nofence",
                 combine_hint="auto"):
        import numpy as np
        import torch

        from combine_routing_histogram_amd import workloads as wl
        from combine_routing_histogram_amd.op import (EpDispatchCombineConfig,
                                                      EpDispatchCombineOp)
        self.torch = torch
        self.w, self.dev, self.path, self.combine_kind = w, dev, path, combine
        self.new_event = (HipEvent if events == "nofence" else
                          (lambda: torch.cuda.Event(enable_timing=True)))
        t0 = time.perf_counter()
        self.inp = wl.make_inputs(w)
        log(f"{w.name}: inputs drawn in {time.perf_counter() - t0:.1f} s")

        def to_bf16(bits):
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

        inp = self.inp
        self.raw = w.raw_row_bytes > 0
        self.x = torch.from_numpy(inp["x"]).to(dev) if self.raw else to_bf16(inp["x"])
        self.sc = torch.from_numpy(inp["scales"]).to(dev) if self.raw else None
        self.idx = torch.from_numpy(inp["indices"]).to(dev)
        self.wts = torch.from_numpy(inp["weights"]).to(dev)
        self.identity = w.combine_input == "identity"
        self.c_in = None if self.identity else to_bf16(inp["combine_input"])
        self.op = EpDispatchCombineOp(
            EpDispatchCombineConfig(w.tokens, w.hidden, w.topk, w.experts, w.ranks,
                                    quant=w.quant, raw_row_bytes=w.raw_row_bytes,
                                    scale_row_bytes=w.scale_row_bytes), dev)
        # the combine of identity experts reads the rows the dispatch has just
        # written: say so (only how its output is stored changes)
        self.recent = self.identity if combine_hint == "auto" else combine_hint == "recent"
        self.op.set_combine_hint(recent_input=self.recent)
        self.expected = None
        self.graph = None
        self._scratch = None
        if graph:
            self._capture()

    # the two phases of a step; check() reads their results from the op's buffers
    def dispatch(self):
        if self.path == "dedup":
            self.op.dispatch_dedup(self.x, self.wts, self.sc, self.idx)
            self.op.units_to_experts()
        else:
            self.op.dispatch(self.x, self.wts, self.sc, self.idx)

    def combine(self):
        op = self.op
        if self.path == "dedup":
            e_out = op.received_payload()
            e_w = op._out_weights
            op.experts_to_units(e_out if self.identity else self.c_in, e_w)
            u_w = op._unit_buffers()["weights"]
            return op.combine_units(None, u_w)
        out = op.received_payload()
        comb = op.combine_scatter if self.combine_kind == "scatter" else op.combine
        return comb(out if self.identity else self.c_in, op._out_weights, op._out_indices)

    def step(self):
        if self.graph is not None:
            self.graph.replay()
            return
        self.dispatch()
        self.combine()

    def _capture(self):
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream(self.dev))
        with torch.cuda.stream(side):
            self.dispatch()
            self.combine()
        torch.cuda.current_stream(self.dev).wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.dispatch()
            self.combine()
        torch.cuda.synchronize()
        self.graph = g

    def set_expected(self, ref: dict) -> None:
        """Upload the oracle's outputs once; check() compares on the device."""
        import numpy as np
        torch = self.torch

        def dev_bytes(a):
            if a is None:
                return None
            a = np.ascontiguousarray(a)
            return torch.from_numpy(a.view(np.uint8).reshape(-1)).to(self.dev)
        self.rows = int(ref["rows"])
        self.expected = {k: dev_bytes(v) for k, v in ref.items() if k != "rows"}

    def got(self) -> dict:
        op, n, T = self.op, self.rows, self.w.tokens
        y, y_w = op._combined[:T], op._combined_weights[:T]
        if self.path == "dedup":
            ub = op._unit_buffers()
            return {"recv": ub["recv"], "payload": ub["out"][:n],
                    "scales": None if ub["scales"] is None else ub["scales"][:n],
                    "y": y, "y_w": y_w}
        return {"recv": op._recv_count, "payload": op._out[:n],
                "weights": op._out_weights[:n], "indices": op._out_indices[:n],
                "scales": None if op._out_scales is None else op._out_scales[:n],
                "src_pos": op.get_dispatch_src_token_pos()[:n], "y": y, "y_w": y_w}

    def check(self) -> list:
        """Names of the outputs that differ from the oracle's (empty: bit-exact)."""
        torch = self.torch
        got = self.got()
        bad = []
        for k, exp in self.expected.items():
            if exp is None:
                continue
            g = got.get(k)
            if g is None or not torch.equal(g.contiguous().view(torch.uint8).reshape(-1), exp):
                bad.append(k)
        return bad

    def make_flush(self, mode: str):
        torch = self.torch
        if mode == "none":
            return lambda i: None
        if self._scratch is None:
            self._scratch = torch.zeros(FLUSH_BYTES // 4, dtype=torch.int32, device=self.dev)
        scratch = self._scratch
        if mode == "write":
            return lambda i: scratch.fill_(i)           # 512 MiB written by a fill kernel
        if mode == "read":
            return lambda i: scratch.sum()              # 512 MiB read by a reduction
        raise ValueError(mode)

    def timed(self, steps: int, warmup: int, flush_mode: str, check: bool):
        """Per-step dispatch and combine times (ms) from HIP events on the
        launch stream.  With a flush: flush before every step, parity after
        every timed step (the next flush evicts what the check read).  With
        none: the steps run back to back and the last step is checked."""
        torch = self.torch
        flush = self.make_flush(flush_mode)
        stream = torch.cuda.current_stream(self.dev)
        back_to_back = flush_mode == "none"
        if back_to_back:
            # Back to back, a small step takes less GPU time than the host
            # needs to launch it, and the events would time the host's launch
            # rate.  So the warm-up and timed steps are queued behind about
            # 1 ms of fills: the host has launched them all before the GPU
            # reaches them, and the GPU sets the pace.  The fills only touch
            # the scratch buffer; the warm-up steps run after them.
            gate = self.make_flush("write")
            for i in range(BACK_TO_BACK_GATE_FILLS):
                gate(i)
        for i in range(warmup):
            flush(i)
            self.step()
        if not back_to_back:
            torch.cuda.synchronize()
        events, mismatches = [], []
        for i in range(steps):
            flush(i)
            e = [self.new_event() for _ in range(3)]
            e[0].record(stream)
            if self.graph is not None:
                self.graph.replay()
            else:
                self.dispatch()
                e[1].record(stream)
                self.combine()
            e[2].record(stream)
            events.append(e)
            if not back_to_back:
                e[2].synchronize()
                if check:
                    bad = self.check()
                    if bad:
                        mismatches.append((i, bad))
        torch.cuda.synchronize()
        if back_to_back and check:
            bad = self.check()
            if bad:
                mismatches.append((steps - 1, bad))
        ts = [e[0].elapsed_time(e[2]) for e in events]
        td = tc = []
        if self.graph is None:
            td = [e[0].elapsed_time(e[1]) for e in events]
            tc = [e[1].elapsed_time(e[2]) for e in events]
        return td, tc, ts, mismatches

    def kernel_pass(self, steps: int, flush_mode: str) -> dict:
        """Per-kernel HIP events (recorded by the library around each launch)."""
        torch = self.torch
        flush = self.make_flush(flush_mode)
        if flush_mode == "none":
            gate = self.make_flush("write")   # as in timed(): the GPU sets the pace
            for i in range(BACK_TO_BACK_GATE_FILLS):
                gate(i)
            self.step()
        self.op.profile_begin(16 * steps)
        for i in range(steps):
            flush(i)
            self.dispatch()
            self.combine()
        torch.cuda.synchronize()
        return self.op.profile_end()


def summary(v: list) -> dict:
    if not v:
        return None
    us = [x * 1e3 for x in v]
    return {"median_us": statistics.median(us), "mean_us": statistics.fmean(us),
            "min_us": min(us), "max_us": max(us)}


def kernel_table(prof: dict, w, units) -> dict:
    out = {}
    for name, (ms, n) in prof.items():
        b = alg_bytes_units(name, w, units) if units is not None else alg_bytes(name, w)
        avg = ms / n
        out[name] = {"launches": n, "avg_us": avg * 1e3, "alg_bytes": b,
                     "gbps": b / (avg * 1e-3) / 1e9 if b else None,
                     "frac": b / (avg * 1e-3) / 1e9 / HBM_PEAK_GBPS if b else None}
    return out


def measure(bench: Bench, steps: int, warmup: int, flush_mode: str, check: bool,
            step_bytes: int) -> dict:
    td, tc, ts, bad = bench.timed(steps, warmup, flush_mode, check)
    if bench.graph is None:
        per_step = [a + b for a, b in zip(td, tc)]
    else:
        per_step = ts
    med = statistics.median(per_step)
    return {"flush": {"write": "512 MiB written before each step",
                      "read": "512 MiB read before each step",
                      "none": "none (steps back to back)"}[flush_mode],
            "steps": steps, "warmup": warmup,
            "ms_per_step": med, "ms_per_step_mean": statistics.fmean(per_step),
            "tokens_per_s": bench.w.tokens / (med * 1e-3),
            "step_gbps": step_bytes / (med * 1e-3) / 1e9,
            "step_frac_of_hbm_peak": step_bytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "dispatch": summary(td), "combine": summary(tc),
            "parity": None if not check else (
                (f"bit-exact on all {steps} timed steps" if flush_mode != "none" else
                 f"bit-exact on the last of {steps} back-to-back steps") if not bad else
                f"MISMATCH on {len(bad)} of {steps} timed steps, first at step {bad[0][0]}: "
                f"{', '.join(bad[0][1])}")}


def layers_measure(benches, steps: int, warmup: int, check: bool, step_bytes: int) -> dict:
    """Several independent layers (each its own inputs, op and buffers) stepped
    in turn with no flush: every layer's inputs have been pushed out of the
    caches by the other layers' traffic, and the caches hold the previous
    layer's data, as in a model that runs its MoE layers one after another.
    Per-layer step = dispatch + combine by HIP events; the median over all
    layer steps.  Each layer's last step is checked against the oracle."""
    torch = benches[0].torch
    stream = torch.cuda.current_stream(benches[0].dev)
    gate = benches[0].make_flush("write")     # as in Bench.timed: the GPU sets the pace
    for i in range(BACK_TO_BACK_GATE_FILLS):
        gate(i)
    for _ in range(warmup):
        for b in benches:
            b.step()
    events = []
    for _ in range(steps):
        for b in benches:
            e = [b.new_event() for _ in range(3)]
            e[0].record(stream)
            b.dispatch()
            e[1].record(stream)
            b.combine()
            e[2].record(stream)
            events.append(e)
    torch.cuda.synchronize()
    bad = []
    if check:
        for li, b in enumerate(benches):
            m = b.check()
            if m:
                bad.append((li, m))
    td = [e[0].elapsed_time(e[1]) for e in events]
    tc = [e[1].elapsed_time(e[2]) for e in events]
    per_step = [a + c for a, c in zip(td, tc)]
    med = statistics.median(per_step)
    tokens = benches[0].w.tokens
    return {"layers": len(benches), "steps": steps, "warmup": warmup,
            "flush": "none (layers in turn, each with its own inputs and buffers)",
            "ms_per_step": med, "ms_per_step_mean": statistics.fmean(per_step),
            "tokens_per_s": tokens / (med * 1e-3),
            "step_gbps": step_bytes / (med * 1e-3) / 1e9,
            "step_frac_of_hbm_peak": step_bytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "dispatch": summary(td), "combine": summary(tc),
            "parity": None if not check else (
                f"bit-exact on the last step of each of {len(benches)} layers" if not bad else
                f"MISMATCH in layer {bad[0][0]}: {', '.join(bad[0][1])}")}


PROBE_BYTES = 4 << 30  # 16x the 256 MB last-level cache: the probes see HBM, not the cache


def hbm_rates(torch, dev, reps: int = 5, launches: int = 4) -> dict:
    """HBM read, write and 1:1 copy rates from the streaming probe kernels
    (libepdc_probe.so) over 4 GiB buffers: the median over `reps` event
    pairs, each around `launches` back-to-back launches."""
    from combine_routing_histogram_amd import probe

    a = torch.zeros(PROBE_BYTES, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream().cuda_stream

    def rate(fn, moved: int) -> float:
        fn()
        times = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(launches):
                fn()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / launches)
        return moved / (statistics.median(times) * 1e-3) / 1e9

    # `a` is all zeros, so its words never XOR to the magic 1
    read = rate(lambda: probe.read(a.data_ptr(), PROBE_BYTES, 1, flag.data_ptr(), st),
                PROBE_BYTES)
    write = rate(lambda: probe.write(b.data_ptr(), PROBE_BYTES, 0, st), PROBE_BYTES)
    copy = rate(lambda: probe.copy(a.data_ptr(), b.data_ptr(), PROBE_BYTES, st),
                2 * PROBE_BYTES)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    del a, b
    torch.cuda.empty_cache()
    return {"read_gbps": read, "write_gbps": write, "copy_gbps": copy,
            "buffer_bytes": PROBE_BYTES, "reps": reps, "launches_per_rep": launches}


def mix_seconds_per_gb(read_frac: float, rates: dict) -> float:
    """Time per GB of a stream whose fraction `read_frac` of the bytes are
    reads, interpolated linearly between the probes' write-only (0), 1:1
    copy (0.5) and read-only (1) rates."""
    tw, tc, tr = (1 / rates["write_gbps"], 1 / rates["copy_gbps"], 1 / rates["read_gbps"])
    if read_frac <= 0.5:
        return tw + (tc - tw) * 2 * read_frac
    return tc + (tr - tc) * (2 * read_frac - 1)


def kernel_ceilings(rates: dict, w, states: dict) -> dict:
    """Each route, scatter and combine kernel's bytes priced at the probes'
    rates, two ways:
      bound_us     = read bytes / read rate + written bytes / write rate (the
                     two directions one after the other with no interference
                     between them: a floor no mixed stream reaches);
      mix_bound_us = all bytes at the rate mix_seconds_per_gb gives for the
                     kernel's read fraction (reads and writes interleaved as
                     in the probes' copy);
    and frac_<state> / frac_mix_<state> = bound / the kernel's mean event
    time in each cache state."""
    out = {}
    names = set()
    for ks in states.values():
        names.update(ks or {})
    for k in sorted(names):
        try:
            r, wr = alg_read_write(k, w)
        except ValueError:
            continue
        bound = r / rates["read_gbps"] / 1e3 + wr / rates["write_gbps"] / 1e3
        mix = (r + wr) * mix_seconds_per_gb(r / (r + wr), rates) / 1e3
        rec = {"read_bytes": r, "write_bytes": wr, "bound_us": bound, "mix_bound_us": mix}
        for state, ks in states.items():
            if ks and k in ks:
                rec[f"frac_{state}"] = bound / ks[k]["avg_us"]
                rec[f"frac_mix_{state}"] = mix / ks[k]["avg_us"]
        out[k] = rec
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20,
                    help="timed steps of the headline protocol (median over them)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--path", choices=["pair", "dedup"], default="pair",
                    help="pair: dispatch / combine with one row per (token, k) (default); "
                         "dedup: rank-deduplicated dispatch, conversion to the expert layout, "
                         "conversion back and unit combine")
    ap.add_argument("--combine", choices=["gather", "scatter"], default="gather",
                    help="pair path only: gather combine (default) or scatter (push) combine")
    ap.add_argument("--combine-hint", choices=["auto", "cold", "recent"], default="auto",
                    help="what the op is told about combine's input: auto = recent when the "
                         "combine reads the dispatch output (identity experts), else cold")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph and replay it in the timed loops "
                         "(phases are then not timed separately)")
    ap.add_argument("--flush", choices=["write", "read", "none"], default="write",
                    help="what happens before each step of the headline protocol")
    ap.add_argument("--events", choices=["nofence", "default"], default="nofence",
                    help="phase events: HIP events without the system-scope release "
                         "(default), or torch's default timing events")
    ap.add_argument("--warm-steps", type=int, default=20,
                    help="steps of the secondary back-to-back pass (0 = skip)")
    ap.add_argument("--clean-steps", type=int, default=20,
                    help="steps of the secondary pass with a 512 MiB read before each (0 = skip)")
    ap.add_argument("--kernel-steps", type=int, default=20,
                    help="steps of the per-kernel event pass (0 = skip)")
    ap.add_argument("--layers", type=int, default=4,
                    help="also step this many independent copies of the workload (own inputs, "
                         "op and buffers) in turn with no flush, as a model's successive MoE "
                         "layers (0 = skip)")
    ap.add_argument("--extras", choices=["default", "none"], default="default",
                    help="with the headline workload: also measure " + ", ".join(EXTRA_WORKLOADS))
    ap.add_argument("--extra-steps", type=int, default=20)
    ap.add_argument("--cpu-reps", type=int, default=3,
                    help="whole oracle steps per CPU leg of the headline (median); 0 = only "
                         "one OpenMP oracle step, for the expected outputs")
    ap.add_argument("--no-check", action="store_true",
                    help="skip the per-step parity check (e.g. under a profiler)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (a known-size "
                         "kernel for scaling rocprofv3 byte counters)")
    ap.add_argument("--ceilings", "--device-copy", dest="ceilings", type=int, default=1,
                    help="also measure the HBM read, write and copy rates with the probe "
                         "kernels and price each kernel at them (0 = skip; --device-copy is "
                         "the older name)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(destination ranks are segments of one HBM buffer). Run with --gpus 1.",
              file=sys.stderr)
        return 2
    if args.steps < 1:
        print("--steps must be >= 1", file=sys.stderr)
        return 2

    import torch

    from combine_routing_histogram_amd import workloads as wl

    w = wl.WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    log(f"{w.name} T={w.tokens} H={w.hidden} K={w.topk} E={w.experts} R={w.ranks} "
        f"path={args.path} combine={args.combine} on {getattr(props, 'gcnArchName', '?')}")
    check = not args.no_check

    if args.calibration_copy_mib > 0:
        n = args.calibration_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    b = Bench(w, dev, args.path, args.combine, graph=args.graph, events=args.events,
              combine_hint=args.combine_hint)
    cpu = None
    if check or args.cpu_reps > 0:
        t0 = time.perf_counter()
        if args.cpu_reps > 0:
            cpu, ref = cpu_baseline(w, b.inp, args.cpu_reps, args.path, args.combine)
        else:
            cpu, ref = cpu_baseline(w, b.inp, 1, args.path, args.combine, builds=(True,))
        b.set_expected(ref)
        del ref
        log(f"oracle done in {time.perf_counter() - t0:.1f} s")

    units = None
    if args.path == "dedup":
        b.dispatch()
        torch.cuda.synchronize()
        units = int(b.op.get_unit_routing()[0][-1])
    step_bytes = step_alg_bytes(w, args.path, args.combine, units)

    log(f"headline protocol: {args.warmup} warm-up + {args.steps} timed steps, flush "
        f"{args.flush}")
    head = measure(b, args.steps, args.warmup, args.flush, check, step_bytes)
    log(f"headline: {head['ms_per_step'] * 1e3:.1f} us/step, parity {head['parity']}")
    kernels = None
    if args.kernel_steps > 0:
        kernels = kernel_table(b.kernel_pass(args.kernel_steps, args.flush), w, units)
    warm = clean = None
    if args.warm_steps > 0:
        warm = measure(b, args.warm_steps, args.warmup, "none", check, step_bytes)
        if args.kernel_steps > 0:
            warm["kernels"] = kernel_table(b.kernel_pass(args.kernel_steps, "none"), w, units)
        log(f"warm: {warm['ms_per_step'] * 1e3:.1f} us/step")
    if args.clean_steps > 0:
        clean = measure(b, args.clean_steps, args.warmup, "read", check, step_bytes)
        log(f"clean flush: {clean['ms_per_step'] * 1e3:.1f} us/step")
    rates = hbm_rates(torch, dev) if args.ceilings else None
    if rates:
        log(f"HBM probes: read {rates['read_gbps']:.0f} GB/s, write {rates['write_gbps']:.0f} "
            f"GB/s, copy {rates['copy_gbps']:.0f} GB/s")

    # roofline: the kernel with the most time under the headline protocol
    roof = None
    if kernels:
        dom = max(kernels, key=lambda k: kernels[k]["avg_us"] * kernels[k]["launches"])
        dk = kernels[dom]
        roof = {"bound": "hbm", "kernel": dom, "achieved": dk["gbps"], "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": dk["frac"],
                "traffic": None if args.path == "dedup" else load_traffic(dom, w.name),
                "avg_us": dk["avg_us"], "state": head["flush"]}
        if dom == "k_combine" and head["combine"]:
            # the same kernel timed by the phase events of the timed steps
            ph = head["combine"]["mean_us"]
            roof["achieved_timed_phase"] = dk["alg_bytes"] / (ph * 1e-6) / 1e9

    ceilings = None
    if rates is not None:
        ceilings = dict(rates, kernels=None)
        if args.path == "pair" and args.combine == "gather":
            ceilings["kernels"] = kernel_ceilings(
                rates, w, {"headline": kernels, "warm": (warm or {}).get("kernels")})
            if roof and roof["kernel"] in ceilings["kernels"]:
                c = ceilings["kernels"][roof["kernel"]]
                # the same kernel against what this card's HBM delivers for its mix
                roof["vs_measured_hbm"] = {k: c[k] for k in (
                    "bound_us", "mix_bound_us", "frac_headline", "frac_mix_headline")}

    recent = b.recent
    b.op = None
    del b
    torch.cuda.empty_cache()

    layers = None
    if args.layers > 0 and args.path == "pair" and args.combine == "gather" and not args.graph:
        import dataclasses
        lbs = []
        for li in range(args.layers):
            # each layer its own draw (another seed) and its own op and buffers
            lw = dataclasses.replace(w, seed=w.seed + 7919 * (li + 1))
            lb = Bench(lw, dev, events=args.events, combine_hint=args.combine_hint)
            if check:
                _, ref = cpu_baseline(lw, lb.inp, 1, "pair", "gather", builds=(True,))
                lb.set_expected(ref)
                del ref
            lbs.append(lb)
        layers = layers_measure(lbs, args.steps, args.warmup, check, step_bytes)
        log(f"{args.layers} layers in turn: {layers['ms_per_step'] * 1e3:.1f} us/step, "
            f"parity {layers['parity']}")
        for lb in lbs:
            lb.op = None
        del lbs
        torch.cuda.empty_cache()

    extras = None
    if args.extras == "default" and w.name == HEADLINE and args.path == "pair" \
            and args.combine == "gather" and not args.graph:
        extras = {}
        for name in EXTRA_WORKLOADS:
            ew = wl.WORKLOADS[name]
            eb = Bench(ew, dev, events=args.events)
            e_cpu = None
            if check:
                # one OpenMP oracle step: its outputs are the expected values
                e_cpu, ref = cpu_baseline(ew, eb.inp, 1, "pair", "gather", builds=(True,))
                eb.set_expected(ref)
                del ref
            sb = step_alg_bytes(ew, "pair", "gather", None)
            r = measure(eb, args.extra_steps, args.warmup, args.flush, check, sb)
            r["cpu_baseline"] = e_cpu
            r["config"] = {"tokens": ew.tokens, "hidden": ew.hidden, "topk": ew.topk,
                           "experts": ew.experts, "ranks": ew.ranks, "quant": ew.quant,
                           "routing": f"{ew.routing}{ew.zipf_s or ''}",
                           "raw_row_bytes": ew.raw_row_bytes,
                           "combine_input": ew.combine_input}
            r["step_alg_bytes"] = sb
            if args.kernel_steps > 0:
                r["kernels"] = kernel_table(eb.kernel_pass(args.kernel_steps, args.flush),
                                            ew, None)
                if rates:
                    r["ceilings"] = kernel_ceilings(rates, ew, {"headline": r["kernels"]})
            # the same workload in the two other cache states (step figures only)
            if args.clean_steps > 0:
                r["clean_flush"] = measure(eb, args.clean_steps, args.warmup, "read", check, sb)
            if args.warm_steps > 0:
                r["warm"] = measure(eb, args.warm_steps, args.warmup, "none", check, sb)
            extras[name] = r
            log(f"{name}: {r['ms_per_step'] * 1e3:.1f} us/step, parity {r['parity']}"
                + (f"; clean flush {r['clean_flush']['ms_per_step'] * 1e3:.1f}"
                   if "clean_flush" in r else "")
                + (f"; warm {r['warm']['ms_per_step'] * 1e3:.1f}" if "warm" in r else ""))
            eb.op = None
            del eb
            torch.cuda.empty_cache()

    rev = revision()
    raw = w.raw_row_bytes > 0
    result = {
        "metric": ("dispatch+combine tokens/s and achieved HBM GB/s (% peak), 4096x7168 top-8"
                   if w.name == HEADLINE else
                   f"dispatch+combine tokens/s and achieved HBM GB/s (% peak), {w.name}")
                  + (" [rank-deduplicated dispatch + standard-MoE conversion]"
                     if args.path == "dedup" else "")
                  + (" [scatter combine]" if args.combine == "scatter" and args.path == "pair"
                     else ""),
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("u8 rows + fp32 scales carried, bf16 fp32-accumulated combine" if raw else
                  {"none": "bf16", "fp8_e4m3_b128": "bf16->e4m3 (fp32 scales), fp32 combine",
                   "mxfp4_b32": "bf16->e2m1 (e8m0 scales), fp32 combine"}[w.quant]),
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.tokens, "hidden": w.hidden, "topk": w.topk,
                   "experts": w.experts, "ranks": w.ranks,
                   "routing": f"{w.routing}{w.zipf_s or ''}", "quant": w.quant,
                   "input": (f"pre-quantized rows of {w.raw_row_bytes} B + "
                             f"{w.scale_row_bytes} B of fp32 scales, carried" if raw
                             else "bf16 rows"),
                   "combine_input": "identity (dispatch output)" if w.combine_input == "identity"
                   else "independent N(0,1) bf16 rows",
                   "combine_hint": "recent input" if recent else "cold input",
                   "graph_mode": "hip graph replay" if args.graph else "eager",
                   "path": args.path, "combine": args.combine, "unit_rows": units,
                   "protocol": (f"{head['flush']}; hipEvents ({args.events}) around dispatch "
                                f"and combine; median of {args.steps} steps; parity every "
                                f"timed step"),
                   "gpu": props.name, "gpu_arch": getattr(props, "gcnArchName", None),
                   "revision": rev["git"], "built_at_revision": rev["built_at_git"],
                   "kernel_source_sha256_16": kernel_source_hash(),
                   "library_sha256_16": file_hash(os.path.join(
                       ROOT, "combine_routing_histogram_amd", "libepdc.so"))},
        "step_alg_bytes": step_bytes,
        "step_gbps": head["step_gbps"],
        "step_frac_of_hbm_peak": head["step_frac_of_hbm_peak"],
        "phases": {"dispatch": head["dispatch"], "combine": head["combine"]},
        "roofline": roof,
        "kernels": kernels,
        "warm": warm,
        "layers": layers,
        "clean_flush": clean,
        "ceilings": ceilings,
        "workloads": extras,
        "cpu_baseline": cpu,
        "parity": head["parity"] if check else "skipped",
    }
    print(json.dumps(result), flush=True)
    failed = [r["parity"] for r in [head, warm, clean] + list((extras or {}).values())
              if r and r.get("parity") and r["parity"].startswith("MISMATCH")]
    if cpu is not None and cpu.get("openmp_result_identical") is False:
        failed.append("openmp oracle differs from the plain oracle")
    return 1 if failed else 0


if __name__ == "__main__":
    sys.exit(main())
