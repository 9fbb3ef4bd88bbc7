"""Scatter (push) combine on the GPU against the CPU oracle (reading of
"Choosing an EP API and backend", "EP paths" table, FlyDSL row: gather /
scatter combine).  The pushed products and their order are the gather
combine's, so the output must equal the oracle's combine bit for bit; the
staging rows are checked against the oracle's push step.
"""
import numpy as np
import pytest
import torch

from combine_routing_histogram_amd import binding as B
from combine_routing_histogram_amd import workloads as wl
from combine_routing_histogram_amd.op import EpDispatchCombineConfig, EpDispatchCombineOp
from oracle import oracle

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)


def log(msg):
    print(msg, flush=True)


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def run_push(x, weights, idx, E, R, c_in=None, check_staging=False, quant="none"):
    T, K = idx.shape
    H = x.shape[1] if c_in is None else c_in.shape[1]
    op = EpDispatchCombineOp(EpDispatchCombineConfig(T, H, K, E, R, quant=quant), DEV)
    w_d = None if weights is None else torch.from_numpy(weights).to(DEV)
    out, out_w, _, out_i, _ = op.dispatch(bf16_dev(x), w_d, None, torch.from_numpy(idx).to(DEV))
    ref = oracle.dispatch(x, weights, idx, E, R, quant=quant)
    if c_in is None:
        c_in_host, c_in_d = ref["out"], out
    else:
        c_in_host, c_in_d = c_in, bf16_dev(c_in)
    y, y_w = op.combine_scatter(c_in_d, out_w, out_i)
    torch.cuda.synchronize()
    ry, ry_w = oracle.combine(c_in_host, ref["out_weights"], ref["slot_of"], T, K)
    np.testing.assert_array_equal(u16(y), ry, err_msg="scatter combine")
    np.testing.assert_array_equal(y_w.cpu().numpy().view(np.uint32), ry_w.view(np.uint32),
                                  err_msg="scatter combine weights")
    if check_staging:
        _, _, st = oracle.combine_push(c_in_host, ref["out_weights"], ref["src_token_pos"],
                                       ref["slot_of"], T, K)
        got = op._staging[:T * K].cpu().numpy()
        valid = ref["slot_of"] >= 0
        np.testing.assert_array_equal(got[valid].view(np.uint32), st[valid].view(np.uint32),
                                      err_msg="staging rows")
    # the gather combine on the same rows agrees
    y2, _ = op.combine(c_in_d, out_w, out_i)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(u16(y2), u16(y))
    return op


@pytest.mark.parametrize("name", ["deepseek_v3_bf16", "decode_bf16", "deepseek_v3_fp8",
                                  "qwen3_moe_mxfp4"])
def test_push_combine_workloads(name):
    w = wl.WORKLOADS[name]
    log(f"push combine {name}")
    inp = wl.make_inputs(w, with_combine_input=True)
    c_in = inp["combine_input"] if w.combine_input == "independent" else None
    run_push(inp["x"], inp["weights"], inp["indices"], w.experts, w.ranks, c_in=c_in,
             quant=w.quant)


@pytest.mark.parametrize("T,H,K,E,R", [
    (200, 64, 3, 16, 4),        # runtime K
    (150, 200, 16, 512, 8),     # largest K and E; ragged rows
    (300, 8200, 8, 64, 8),      # long rows: several segments plus a tail
])
def test_push_combine_shapes_and_staging(T, H, K, E, R):
    log(f"push combine shape T={T} H={H} K={K}")
    rng = np.random.default_rng(T + H + K)
    idx = wl.draw_topk(rng, T, E, K, "zipf", 1.2)
    idx[3, 0], idx[T - 1, K - 1] = -1, E       # pairs without a row
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    run_push(x, wl.softmax_weights(rng, T, K), idx, E, R, check_staging=True)


def test_push_combine_unweighted_and_states():
    log("push combine unweighted")
    rng = np.random.default_rng(91)
    T, H, K, E, R = 120, 128, 4, 32, 4
    idx = wl.draw_topk(rng, T, E, K, "uniform")
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    run_push(x, None, idx, E, R)
    op = EpDispatchCombineOp(EpDispatchCombineConfig(T, H, K, E, R), DEV)
    with pytest.raises(B.EpdcError) as ei:
        op.combine_scatter(bf16_dev(np.zeros((T * K, H), np.uint16)))
    assert ei.value.status == B.EPDC_ERR_BAD_STATE
