"""Seeded sweep of random valid configurations through every entry point,
each compared with the oracle bit for bit: pair dispatch and gather
combine, the scatter combine, routing replay, and the rank-deduplicated
dispatch with both conversions and the unit combine.  Shapes, payload kinds,
routing skew, invalid ids, missing weights and ragged token counts are drawn
per case, so tile and segment boundaries land in many different places.

EPDC_SWEEP_CASES=N runs N seeds instead of 24, starting at EPDC_SWEEP_FIRST
(default 0); seeds from 24 on also draw, for about a third of the cases,
700-6000 tokens (many routing tiles, so the table is scanned by the last
rank block).  Seeds 0-2499 were run once.
"""
import os

import numpy as np
import pytest
import torch

from combine_routing_histogram_amd import workloads as wl
from combine_routing_histogram_amd.op import EpDispatchCombineConfig, EpDispatchCombineOp
from oracle import oracle

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def b8(t):
    return t.contiguous().view(torch.uint8).cpu().numpy()


def u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def rows(a, n):
    """Byte view of the first n rows of a numpy array (empty when n == 0)."""
    return a.view(np.uint8).reshape(n, -1) if n else np.zeros((0, 0), np.uint8)


def same(got_t, ref, n, msg=""):
    if n == 0:
        return
    np.testing.assert_array_equal(b8(got_t[:n]).reshape(n, -1), rows(ref, n), err_msg=msg)


def draw_case(rng):
    quant = rng.choice(["none", "none", "fp8_e4m3_b128", "mxfp4_b32", "raw"])
    R = int(rng.choice([1, 2, 3, 4, 8]))
    E = R * int(rng.integers(1, 513 // R if R > 1 else 513))
    E = min(E, 512 - 512 % R)
    K = int(rng.integers(1, 17))
    if quant == "fp8_e4m3_b128":
        H = 128 * int(rng.integers(1, 20))
    elif quant == "mxfp4_b32":
        H = 128 * int(rng.integers(1, 20))      # scale rows in whole 4-byte words
    else:
        H = 8 * int(rng.integers(1, 300))
    T = int(rng.integers(0, 700))
    T_max = T + int(rng.integers(0, 50))
    return dict(quant=quant, R=R, E=E, K=K, H=H, T=T, T_max=max(T_max, 1),
                weighted=bool(rng.random() < 0.8), invalid=bool(rng.random() < 0.3),
                skew=float(rng.choice([0.0, 1.1, 1.5])))


SWEEP_CASES = int(os.environ.get("EPDC_SWEEP_CASES", "24"))
SWEEP_FIRST = int(os.environ.get("EPDC_SWEEP_FIRST", "0"))


@pytest.mark.parametrize("seed", range(SWEEP_FIRST, SWEEP_FIRST + SWEEP_CASES))
def test_random_configurations(seed):
    rng = np.random.default_rng(5000 + seed)
    c = draw_case(rng)
    if seed >= 24 and rng.random() < 0.35:   # the extended sweep: larger batches too
        c["T"] = int(rng.integers(700, 6000))
        c["T_max"] = c["T"] + int(rng.integers(0, 50))
    print(f"sweep seed={seed} {c}", flush=True)
    T, H, K, E, R = c["T"], c["H"], c["K"], c["E"], c["R"]
    raw = c["quant"] == "raw"
    quant = "none" if raw else c["quant"]
    if c["skew"] > 0 and K <= E:
        idx = wl.draw_topk(rng, T, E, K, "zipf", c["skew"])
    else:
        idx = rng.integers(0, E, (T, K)).astype(np.int32)
    if c["invalid"] and T > 0:
        n_bad = int(rng.integers(1, 4))
        for _ in range(n_bad):
            idx[rng.integers(0, T), rng.integers(0, K)] = rng.choice([-1, E, 1 << 30])
    wts = wl.softmax_weights(rng, T, K) if c["weighted"] else None
    scales = None
    if raw:
        x = rng.integers(0, 256, (T, 16 * int(rng.integers(1, 60))), dtype=np.uint8)
        scales = rng.standard_normal((T, int(rng.integers(1, 9)))).astype(np.float32)
        cfg = EpDispatchCombineConfig(c["T_max"], H, K, E, R, raw_row_bytes=x.shape[1],
                                      scale_row_bytes=scales[0].nbytes if T else 4)
        x_d = torch.from_numpy(x).to(DEV)
    else:
        x = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
        cfg = EpDispatchCombineConfig(c["T_max"], H, K, E, R, quant=quant)
        x_d = bf16_dev(x)
    if raw and T == 0:
        scales = np.zeros((0, 1), np.float32)
    op = EpDispatchCombineOp(cfg, DEV)
    idx_d = torch.from_numpy(np.ascontiguousarray(idx)).to(DEV)
    w_d = None if wts is None else torch.from_numpy(wts).to(DEV)
    s_d = None if scales is None else torch.from_numpy(scales).to(DEV)
    c_in = wl.f32_to_bf16_bits(rng.standard_normal((T * K, H)).astype(np.float32))
    c_in_d = bf16_dev(c_in) if T * K else torch.zeros((1, H), dtype=torch.bfloat16, device=DEV)

    # pair dispatch, gather and scatter combine
    out, out_w, out_s, out_i, recv = op.dispatch(x_d, w_d, s_d, idx_d)
    ref = oracle.dispatch(x, wts, idx, E, R, quant=quant, scales=scales)
    n = ref["n_valid"]
    torch.cuda.synchronize()
    np.testing.assert_array_equal(recv.cpu().numpy(), ref["recv_count"])
    same(out, ref["out"], n, "payload")
    same(out_i, ref["out_indices"], n, "indices")
    if wts is not None:
        same(out_w, ref["out_weights"], n, "weights")
    if ref["out_scales"] is not None:
        same(out_s, ref["out_scales"], n, "scales")
    np.testing.assert_array_equal(op.get_dispatch_src_token_pos()[:n].cpu().numpy(),
                                  ref["src_token_pos"])
    ry, ry_w = oracle.combine(c_in, ref["out_weights"], ref["slot_of"], T, K)
    # the gather combine under both input hints (each hint picks its own launch
    # form and stores), then the scatter combine
    for comb, recent in ((op.combine, False), (op.combine, True), (op.combine_scatter, False)):
        op.set_combine_hint(recent_input=recent)
        y, y_w = comb(c_in_d, out_w, out_i)
        torch.cuda.synchronize()
        same(y, ry, T, f"{comb.__name__} (recent={recent})")
        same(y_w, ry_w, T, f"{comb.__name__} weights (recent={recent})")
        y.view(torch.uint8).fill_(0x5A)
    op.set_combine_hint(recent_input=False)

    # routing replay with a new payload
    if raw:
        x2 = rng.integers(0, 256, x.shape, dtype=np.uint8)
        x2_d = torch.from_numpy(x2).to(DEV)
    else:
        x2 = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
        x2_d = bf16_dev(x2)
    out2 = op.dispatch_replay(x2_d, w_d, s_d)[0]
    torch.cuda.synchronize()
    ref2 = oracle.dispatch(x2, wts, idx, E, R, quant=quant, scales=scales)
    same(out2, ref2["out"], n, "replay")

    # rank-deduplicated dispatch, conversions, unit combine
    u_out, u_w, _, _, u_recv = op.dispatch_dedup(x_d, w_d, s_d, idx_d)
    d = oracle.dispatch_dedup(x, wts, idx, E, R, quant=quant, scales=scales)
    U = d["units"]
    torch.cuda.synchronize()
    np.testing.assert_array_equal(u_recv.cpu().numpy(), d["unit_cnt"])
    same(u_out, d["out"], U, "unit rows")
    e_out, e_w, e_s, e_i, _ = op.units_to_experts()
    torch.cuda.synchronize()
    same(e_out, ref["out"], n, "converted payload")
    same(e_i, ref["out_indices"], n, "converted indices")
    part = op.experts_to_units(c_in_d, e_w)
    y3, y3_w = op.combine_units(None, u_w)
    torch.cuda.synchronize()
    rpart = oracle.experts_to_units(c_in, ref["out_weights"], d["unit_src"], d["unit_of"],
                                    d["slot_of"], K)
    same(part, rpart, U, "unit partials")
    ry3, ry3_w = oracle.combine_units(rpart, d["out_weights"], d["unit_of"], T, K)
    same(y3, ry3, T, "unit combine")
    same(y3_w, ry3_w, T, "unit combine weights")
    assert op.device_error() == int(ref["invalid"] > 0)
