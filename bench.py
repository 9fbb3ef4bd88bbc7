"""Benchmark: MoE dispatch + combine on one MI355X.

One step = one dispatch (routing histogram, scan, stable slots, scatter of the
bf16 rows with their weights/indices) followed by one combine (gather + fp32
weighted top-k sum) of the dispatched rows (identity experts), by default on
the DeepSeek-V3-shaped workload: 4096 tokens x hidden 7168, top-8 of 256
experts (Zipf 1.1 routing), 8 virtual ranks.  --workload picks another one
(the quantizing workloads, and the one whose FP8 rows were quantized before
dispatch and are carried as bytes with their scales, combine an independent
bf16 expert output).
Inputs are resident in HBM before the timed region.  Prints one JSON line.

value = tokens/s of whole steps.  roofline: the kernel with the most time,
algorithmic bytes per launch / its mean duration from HIP events recorded on
the launch stream around each kernel during the timed steps.
copy_ceiling: a plain 512 MiB device copy timed in the same run, as the
practical HBM ceiling for mixed read/write traffic, and the step's fraction
of it.
cold_cache: per-kernel event times of a further pass in which writing a
512 MiB scratch buffer before every step evicts L2 and the MALL (the timed loop reuses its buffers,
so part of each kernel's data is still cached from the step before).
cpu_baseline: the CPU oracle (plain C, single thread) on the same workload;
its last step is also compared bit for bit with the GPU's last timed step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E, AMD's published figure


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
    if kernel == "k_route_scan":
        return 0
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
               only touches the small tile table (counted as 0)
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
    elif kernel == "k_route_scan":
        return 0
    else:
        raise ValueError(kernel)
    return per * T


def kernel_source_hash() -> str:
    from combine_routing_histogram_amd.profiling import kernel_source_hash as h
    return h()


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


def cpu_baseline(w, inp, budget_s: float, gpu_payload, gpu_scales, gpu_combined,
                 dedup: bool = False):
    """Time the oracle (plain C, one thread) on whole steps of the workload,
    and compare its last step with the GPU's last timed step (payload bytes,
    produced scales, combine output)."""
    import numpy as np

    from oracle import oracle  # test infrastructure, used only by this leg

    identity = w.combine_input == "identity"
    reps, t0 = 0, time.perf_counter()
    while True:
        if not dedup:
            d = oracle.dispatch(inp["x"], inp["weights"], inp["indices"], w.experts, w.ranks,
                                quant=w.quant, scales=inp.get("scales"))
            c_in = d["out"] if identity else inp["combine_input"]
            y, _ = oracle.combine(c_in, d["out_weights"], d["slot_of"], w.tokens, w.topk)
        else:
            d = oracle.dispatch_dedup(inp["x"], inp["weights"], inp["indices"], w.experts,
                                      w.ranks, quant=w.quant, scales=inp.get("scales"))
            n = d["n_valid"]
            e_out = oracle.units_to_experts(d["out"], d["slot_of"], d["unit_of"], n)
            e_w = oracle.units_to_experts(d["out_weights"], d["slot_of"], d["unit_of"], n)
            c_in = e_out if identity else inp["combine_input"]
            part = oracle.experts_to_units(c_in, e_w, d["unit_src"], d["unit_of"], d["slot_of"],
                                           w.topk)
            y, _ = oracle.combine_units(part, d["out_weights"], d["unit_of"], w.tokens, w.topk)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 50:
            break
    n = d["units"] if dedup else d["n_valid"]
    same = (np.array_equal(gpu_payload[:n], d["out"].view(np.uint8).reshape(n, -1))
            and np.array_equal(gpu_combined, y))
    if d["out_scales"] is not None:
        same = same and np.array_equal(gpu_scales[:n], d["out_scales"].view(np.uint8).reshape(n, -1))
    base = {"value": w.tokens * reps / el, "unit": "tokens/s", "cores": 1,
            "host_cores": os.cpu_count(), "kind": "oracle",
            "sample": f"{reps} whole {'rank-deduplicated ' if dedup else ''}"
                      f"dispatch+combine steps of {w.name} "
                      f"({w.tokens} tokens each), {el:.1f} s"}
    return base, ("bit-exact" if same else "MISMATCH")


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="deepseek_v3_bf16")
    ap.add_argument("--path", choices=["pair", "dedup"], default="pair",
                    help="pair: dispatch / combine with one row per (token, k) (default); "
                         "dedup: rank-deduplicated dispatch, conversion to the expert layout, "
                         "conversion back and unit combine")
    ap.add_argument("--combine", choices=["gather", "scatter"], default="gather",
                    help="pair path only: gather combine (default) or scatter (push) combine")
    ap.add_argument("--kernel-events", choices=["timed", "separate"], default="separate",
                    help="record the per-kernel events in the timed steps, or (default) in a "
                         "second pass of the same number of steps right after them: each "
                         "event record costs about 3.5 us of GPU time, which would inflate "
                         "the step time")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph and replay it in the timed loop "
                         "(the per-kernel event pass stays eager)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before the steps "
                         "(a known-size kernel for scaling rocprofv3 byte counters)")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="steps of an extra per-kernel event pass in which writing a 512 MiB "
                         "scratch buffer before each step evicts L2 and the MALL (0 = skip)")
    ap.add_argument("--copy-ceiling", type=int, default=1,
                    help="also time a plain 512 MiB device copy as the practical HBM ceiling "
                         "(0 = skip)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="time budget of the CPU-oracle baseline (0 = skip)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(destination ranks are segments of one HBM buffer). Run with --gpus 1.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from combine_routing_histogram_amd import workloads as wl
    from combine_routing_histogram_amd.op import EpDispatchCombineConfig, EpDispatchCombineOp

    w = wl.WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    print(f"bench: {w.name} T={w.tokens} H={w.hidden} K={w.topk} E={w.experts} R={w.ranks}",
          file=sys.stderr, flush=True)

    def to_bf16(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    inp = wl.make_inputs(w)
    raw = w.raw_row_bytes > 0
    x = torch.from_numpy(inp["x"]).to(dev) if raw else to_bf16(inp["x"])
    sc = torch.from_numpy(inp["scales"]).to(dev) if raw else None
    idx = torch.from_numpy(inp["indices"]).to(dev)
    wts = torch.from_numpy(inp["weights"]).to(dev)
    identity = w.combine_input == "identity"
    c_in = None if identity else to_bf16(inp["combine_input"])
    op = EpDispatchCombineOp(EpDispatchCombineConfig(w.tokens, w.hidden, w.topk, w.experts,
                                                     w.ranks, quant=w.quant,
                                                     raw_row_bytes=w.raw_row_bytes,
                                                     scale_row_bytes=w.scale_row_bytes), dev)

    dedup = args.path == "dedup"

    def step():
        if not dedup:
            out, out_w, _, out_idx, _ = op.dispatch(x, wts, sc, idx)
            comb = op.combine_scatter if args.combine == "scatter" else op.combine
            return comb(out if identity else c_in, out_w, out_idx)
        _, u_w, _, _, _ = op.dispatch_dedup(x, wts, sc, idx)
        e_out, e_w, _, _, _ = op.units_to_experts()
        op.experts_to_units(e_out if identity else c_in, e_w)
        return op.combine_units(None, u_w)

    if args.calibration_copy_mib > 0:
        n = args.calibration_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    units = int(op.get_unit_routing()[0][-1]) if dedup else None
    timed_step = step
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream(dev).wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            g_out = step()
        torch.cuda.synchronize()

        def timed_step():
            graph.replay()
            return g_out
        for _ in range(args.warmup):
            timed_step()
        torch.cuda.synchronize()
    print(f"bench: warmup {args.warmup} done; timing {args.steps} steps", file=sys.stderr,
          flush=True)

    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    timed_events = args.kernel_events == "timed" and not args.graph
    if timed_events:
        op.profile_begin(8 * args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        y, y_w = timed_step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if not timed_events:
        op.profile_begin(8 * args.steps)
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
    prof = op.profile_end()
    ms_step_events = ev0.elapsed_time(ev1) / args.steps

    # Cold-cache pass: the timed loop reuses the same buffers every step, so
    # part of each kernel's input or output is still in the 256 MB MALL from
    # the step before.  Here writing a 512 MiB scratch buffer (outside the
    # kernel events) before every step leaves L2 and the MALL full of other,
    # dirty lines, as a layer with other work in between would find them.
    cold = None
    if args.cold_steps > 0:
        scratch = torch.empty(256 << 20, dtype=torch.int16, device=dev)
        op.profile_begin(8 * args.cold_steps)
        for i in range(args.cold_steps):
            scratch.fill_(i)          # writes 512 MiB with a fill kernel
            step()
        torch.cuda.synchronize()
        cold = op.profile_end()
        del scratch
    ms_step = wall * 1e3 / args.steps
    tokens_per_s = w.tokens / (ms_step * 1e-3)

    def kbytes(name):
        return alg_bytes_units(name, w, units) if dedup else alg_bytes(name, w)

    kernels = {}
    for name, (ms, n) in prof.items():
        b = kbytes(name)
        avg = ms / n
        kernels[name] = {"launches": n, "avg_us": avg * 1e3, "alg_bytes": b,
                         "gbps": b / (avg * 1e-3) / 1e9 if b else None,
                         "frac": b / (avg * 1e-3) / 1e9 / HBM_PEAK_GBPS if b else None}
    # practical ceiling: a plain 512 MiB device-to-device copy (read + write)
    copy_gbps = None
    if args.copy_ceiling:
        a_buf = torch.empty(256 << 20, dtype=torch.int16, device=dev)
        b_buf = torch.empty_like(a_buf)
        for _ in range(3):
            b_buf.copy_(a_buf)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(10):
            b_buf.copy_(a_buf)
        c1.record()
        torch.cuda.synchronize()
        copy_gbps = 2 * a_buf.numel() * 2 / (c0.elapsed_time(c1) / 10 * 1e-3) / 1e9
        del a_buf, b_buf

    cold_kernels = None
    if cold is not None:
        cold_kernels = {}
        for name, (ms, n) in cold.items():
            b = kbytes(name)
            avg = ms / n
            cold_kernels[name] = {"avg_us": avg * 1e3,
                                  "frac": b / (avg * 1e-3) / 1e9 / HBM_PEAK_GBPS if b else None}
    dom = max(kernels, key=lambda k: kernels[k]["avg_us"] * kernels[k]["launches"])
    dk = kernels[dom]
    # the method's bytes: x read once, K row copies written, K rows read back, one row
    # written, plus the small per-pair arrays (the route's own index read and rank array
    # are workspace traffic, not counted)
    scatter_name = {"none": "k_scatter_copy", "fp8_e4m3_b128": "k_scatter_fp8",
                    "mxfp4_b32": "k_scatter_mxfp4"}[w.quant]
    if dedup:
        step_bytes = sum(kbytes(k) for k in (scatter_name, "k_units_to_experts",
                                              "k_experts_to_units", "k_combine_units"))
    elif args.combine == "scatter":
        step_bytes = (alg_bytes(scatter_name, w) + alg_bytes("k_combine_push", w)
                      + alg_bytes("k_combine_reduce", w))
    else:
        step_bytes = alg_bytes(scatter_name, w) + alg_bytes("k_combine", w)
    traffic = None if dedup else load_traffic(dom, w.name)

    result = {
        "metric": ("dispatch+combine tokens/s and achieved HBM GB/s (% peak), 4096x7168 top-8"
                   if w.name == "deepseek_v3_bf16" else
                   f"dispatch+combine tokens/s and achieved HBM GB/s (% peak), {w.name}")
                  + (" [rank-deduplicated dispatch + standard-MoE conversion]" if dedup else "")
                  + (" [scatter combine]" if args.combine == "scatter" and not dedup else ""),
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("u8 rows + fp32 scales carried, bf16 fp32-accumulated combine" if raw else
                  {"none": "bf16", "fp8_e4m3_b128": "bf16->e4m3 (fp32 scales), fp32 combine",
                   "mxfp4_b32": "bf16->e2m1 (e8m0 scales), fp32 combine"}[w.quant]),
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.tokens, "hidden": w.hidden, "topk": w.topk,
                   "experts": w.experts, "ranks": w.ranks, "routing": f"{w.routing}{w.zipf_s or ''}",
                   "quant": w.quant,
                   "input": (f"pre-quantized rows of {w.raw_row_bytes} B + "
                             f"{w.scale_row_bytes} B of fp32 scales, carried" if raw
                             else "bf16 rows"),
                   "combine_input": "identity (dispatch output)" if identity
                   else "independent N(0,1) bf16 rows",
                   "graph_mode": "hip graph replay" if args.graph else "eager",
                   "path": args.path,
                   "combine": args.combine,
                   "unit_rows": units,
                   "gpu": torch.cuda.get_device_name(dev)},
        "step_alg_bytes": step_bytes,
        "step_gbps": step_bytes / (ms_step * 1e-3) / 1e9,
        "step_frac_of_hbm_peak": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "copy_ceiling": None if copy_gbps is None else {
            "kernel": "512 MiB device-to-device copy (torch copy_)", "gbps": copy_gbps,
            "step_frac_of_copy": step_bytes / (ms_step * 1e-3) / 1e9 / copy_gbps},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": dk["gbps"],
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": dk["frac"],
                     "traffic": traffic,
                     # the same kernel against the device copy measured in this run
                     "frac_of_copy": None if copy_gbps is None or not dk["gbps"]
                     else dk["gbps"] / copy_gbps},
        "kernels": kernels,
        "ms_per_step_events": ms_step_events,
        "kernel_events": args.kernel_events,
        "cold_cache": None if cold_kernels is None else {
            "flush_mib": 512, "steps": args.cold_steps, "kernels": cold_kernels,
            "kernel_sum_us": sum(v["avg_us"] for v in cold_kernels.values())},
    }
    parity = "skipped"
    result["cpu_baseline"] = None
    if args.cpu_seconds > 0:
        if dedup:
            payload = op.received_unit_payload().view(torch.uint8).cpu().numpy()
            scales = op.received_unit_scales(raw)
            scales = None if scales is None else scales.view(torch.uint8).cpu().numpy()
        else:
            payload = op.received_payload().view(torch.uint8).cpu().numpy()
            scales = op.received_scales(raw)
            scales = None if scales is None else scales.view(torch.uint8).cpu().numpy()
        combined = y.view(torch.int16).cpu().numpy().view(np.uint16)
        result["cpu_baseline"], parity = cpu_baseline(w, inp, args.cpu_seconds, payload, scales,
                                                      combined, dedup)
    result["parity"] = parity
    print(json.dumps(result), flush=True)
    return 0 if parity != "MISMATCH" else 1


if __name__ == "__main__":
    sys.exit(main())
