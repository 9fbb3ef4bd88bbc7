"""Rank-deduplicated dispatch and the standard-MoE conversion on the GPU
against the CPU oracle (reading of "Choosing an EP API and backend", "EP
paths" table: one row per (token, destination rank), expanded into the expert
layout on the receiving side and summed back per unit).

Everything integer or byte-valued is compared bit for bit, and so are the
unit partial sums and the unit combine, since both sides add in the same
order with separate fp32 multiply and add.
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


def bytes_of(t):
    return t.contiguous().view(torch.uint8).cpu().numpy()


def u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def run_dedup(x, weights, indices, E, R, quant="none", hidden=None, scales=None, raw_row_bytes=0,
              c_in=None, max_tokens=None):
    T, K = indices.shape
    H = hidden if hidden is not None else x.shape[1]
    cfg = EpDispatchCombineConfig(max_tokens or T, H, K, E, R, quant=quant,
                                  raw_row_bytes=raw_row_bytes,
                                  scale_row_bytes=0 if scales is None else scales[0].nbytes)
    op = EpDispatchCombineOp(cfg, DEV)
    x_d = (torch.from_numpy(np.ascontiguousarray(x)).to(DEV) if raw_row_bytes else bf16_dev(x))
    w_d = None if weights is None else torch.from_numpy(np.ascontiguousarray(weights)).to(DEV)
    s_d = None if scales is None else torch.from_numpy(np.ascontiguousarray(scales)).to(DEV)
    idx_d = torch.from_numpy(np.ascontiguousarray(indices)).to(DEV)
    out, out_w, out_s, out_i, recv = op.dispatch_dedup(x_d, w_d, s_d, idx_d)
    torch.cuda.synchronize()

    ref = oracle.dispatch_dedup(x, weights, indices, E, R, quant=quant, scales=scales)
    U = ref["units"]
    np.testing.assert_array_equal(recv.cpu().numpy(), ref["unit_cnt"], err_msg="recv_count")
    uo, uof, usrc = op.get_unit_routing()
    np.testing.assert_array_equal(uo.cpu().numpy(), ref["unit_off"], err_msg="unit_off")
    np.testing.assert_array_equal(uof.cpu().numpy(), ref["unit_of"], err_msg="unit_of")
    np.testing.assert_array_equal(usrc[:U].cpu().numpy(), ref["unit_src"], err_msg="unit_src")
    np.testing.assert_array_equal(bytes_of(out[:U]), ref["out"].view(np.uint8).reshape(U, -1),
                                  err_msg="unit payload")
    np.testing.assert_array_equal(out_i[:U].cpu().numpy(), ref["out_indices"],
                                  err_msg="unit indices")
    if weights is not None:
        np.testing.assert_array_equal(out_w[:U].cpu().numpy().view(np.uint32),
                                      ref["out_weights"].view(np.uint32), err_msg="unit weights")
    if ref["out_scales"] is not None:
        np.testing.assert_array_equal(bytes_of(out_s[:U]),
                                      ref["out_scales"].view(np.uint8).reshape(U, -1),
                                      err_msg="unit scales")
    # the pair routing is recorded too
    eo, ro, so = op.get_routing()
    np.testing.assert_array_equal(eo.cpu().numpy(), ref["expert_off"], err_msg="expert_off")
    np.testing.assert_array_equal(ro.cpu().numpy(), ref["rank_off"], err_msg="rank_off")
    np.testing.assert_array_equal(so.cpu().numpy(), ref["slot_of"], err_msg="slot_of")
    n = ref["n_valid"]
    np.testing.assert_array_equal(op.get_dispatch_src_token_pos()[:n].cpu().numpy(),
                                  ref["src_token_pos"], err_msg="src_token_pos")

    # standard-MoE conversion: exactly the pair dispatch
    pair = oracle.dispatch(x, weights, indices, E, R, quant=quant, scales=scales)
    e_out, e_w, e_s, e_i, _ = op.units_to_experts()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bytes_of(e_out[:n]), pair["out"].view(np.uint8).reshape(n, -1),
                                  err_msg="converted payload")
    np.testing.assert_array_equal(e_i[:n].cpu().numpy(), pair["out_indices"],
                                  err_msg="converted indices")
    if weights is not None:
        np.testing.assert_array_equal(e_w[:n].cpu().numpy().view(np.uint32),
                                      pair["out_weights"].view(np.uint32),
                                      err_msg="converted weights")
    if pair["out_scales"] is not None:
        np.testing.assert_array_equal(bytes_of(e_s[:n]),
                                      pair["out_scales"].view(np.uint8).reshape(n, -1),
                                      err_msg="converted scales")

    # the way back: expert rows -> weighted unit sums -> token sums
    if c_in is None:
        assert quant == "none" and not raw_row_bytes
        c_in_host, c_in_d = pair["out"], e_out
    else:
        c_in_host, c_in_d = c_in, bf16_dev(c_in)
    wts_rows = pair["out_weights"]
    part = op.experts_to_units(c_in_d, e_w)
    torch.cuda.synchronize()
    ref_part = oracle.experts_to_units(c_in_host, wts_rows, ref["unit_src"], ref["unit_of"],
                                       ref["slot_of"], K)
    np.testing.assert_array_equal(u16(part[:U]), ref_part, err_msg="unit partial sums")
    uw = None if weights is None else out_w
    y, y_w = op.combine_units(None, uw)
    torch.cuda.synchronize()
    ry, ry_w = oracle.combine_units(ref_part, ref["out_weights"], ref["unit_of"], T, K)
    np.testing.assert_array_equal(u16(y), ry, err_msg="unit combine")
    np.testing.assert_array_equal(y_w.cpu().numpy().view(np.uint32), ry_w.view(np.uint32),
                                  err_msg="unit combine weights")
    # and the gather combine still works on the converted expert rows
    y2, _ = op.combine(c_in_d, e_w, e_i)
    torch.cuda.synchronize()
    ry2, _ = oracle.combine(c_in_host, wts_rows, ref["slot_of"], T, K)
    np.testing.assert_array_equal(u16(y2), ry2, err_msg="gather combine after dedup")
    assert op.device_error() == int(ref["invalid"] > 0)
    return op, ref


@pytest.mark.parametrize("T", [100, 2000, 4096])    # 800 pairs: one tile; 16000; headline
def test_dedup_bf16(T):
    log(f"dedup bf16 T={T}")
    inp = wl.make_inputs(wl.WORKLOADS["deepseek_v3_bf16"], tokens=T)
    run_dedup(inp["x"], inp["weights"], inp["indices"], 256, 8)


@pytest.mark.parametrize("T,quant,H", [(300, "fp8_e4m3_b128", 7168), (100, "fp8_e4m3_b128", 7168),
                                       (700, "mxfp4_b32", 4096)])
def test_dedup_quantized(T, quant, H):
    log(f"dedup {quant} T={T}")
    rng = np.random.default_rng(T + 51)
    K, E, R = 8, 256 if H == 7168 else 128, 8
    idx = wl.draw_topk(rng, T, E, K, "zipf", 1.2)
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    w = wl.softmax_weights(rng, T, K)
    c_in = wl.f32_to_bf16_bits(rng.standard_normal((T * K, H)).astype(np.float32))
    run_dedup(x, w, idx, E, R, quant=quant, c_in=c_in)


@pytest.mark.parametrize("T", [513, 100])
def test_dedup_raw_rows_scales_invalid_ids(T):
    log(f"dedup raw T={T}")
    rng = np.random.default_rng(61)
    K, E, R = 8, 64, 4
    raw = rng.integers(0, 256, (T, 1024), dtype=np.uint8)
    sc = rng.standard_normal((T, 12)).astype(np.float32)
    idx = wl.draw_topk(rng, T, E, K, "uniform")
    idx[7, 3], idx[T - 1, 0], idx[T // 2, 7] = -1, E, 1 << 30
    w = wl.softmax_weights(rng, T, K)
    c_in = wl.f32_to_bf16_bits(rng.standard_normal((T * K, 128)).astype(np.float32))
    _, ref = run_dedup(raw, w, idx, E, R, hidden=128, raw_row_bytes=1024, scales=sc, c_in=c_in)
    assert ref["invalid"] == 3


@pytest.mark.parametrize("T,H,K,E,R", [
    (64, 64, 1, 4, 1),         # one rank: every token one unit
    (90, 200, 3, 9, 9),        # one expert per rank: units are the distinct ids
    (300, 128, 16, 512, 8),    # K > R: at most 8 units per token
    (1500, 256, 6, 96, 3),     # several tiles, E not a power of two
    (40, 8200, 5, 20, 4),      # long rows: several chunks plus a tail
])
def test_dedup_shapes(T, H, K, E, R):
    log(f"dedup shape T={T} H={H} K={K} E={E} R={R}")
    rng = np.random.default_rng(T * 3 + K)
    idx = rng.integers(0, E, (T, K)).astype(np.int32)        # duplicates allowed
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    w = wl.softmax_weights(rng, T, K)
    run_dedup(x, w, idx, E, R)


def test_dedup_no_weights_and_ragged_capacity():
    log("dedup no weights")
    rng = np.random.default_rng(71)
    T, H, K, E, R = 333, 256, 4, 32, 8
    idx = wl.draw_topk(rng, T, E, K, "zipf", 1.3)
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    run_dedup(x, None, idx, E, R, max_tokens=1000)


def test_dedup_replay_and_states():
    log("dedup replay and states")
    rng = np.random.default_rng(81)
    T, H, K, E, R = 400, 512, 8, 64, 8
    idx = wl.draw_topk(rng, T, E, K, "zipf", 1.1)
    x1 = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    x2 = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    w1, w2 = wl.softmax_weights(rng, T, K), wl.softmax_weights(rng, T, K)
    op = EpDispatchCombineOp(EpDispatchCombineConfig(T, H, K, E, R), DEV)
    x_d = bf16_dev(x1)
    # no rank-deduplicated dispatch yet: the conversions refuse
    for call in (lambda: op.units_to_experts(), lambda: op.experts_to_units(x_d),
                 lambda: op.combine_units(), op.get_unit_routing):
        with pytest.raises(B.EpdcError) as ei:
            call()
        assert ei.value.status == B.EPDC_ERR_BAD_STATE
    op.dispatch(x_d, None, None, torch.from_numpy(idx).to(DEV))
    with pytest.raises(B.EpdcError) as ei:
        op.units_to_experts()
    assert ei.value.status == B.EPDC_ERR_BAD_STATE

    op.dispatch_dedup(x_d, torch.from_numpy(w1).to(DEV), None, torch.from_numpy(idx).to(DEV))
    out, out_w, _, _, _ = op.dispatch_replay(bf16_dev(x2), torch.from_numpy(w2).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.dispatch_dedup(x2, w2, idx, E, R)
    U = ref["units"]
    np.testing.assert_array_equal(u16(out[:U]), ref["out"], err_msg="replayed unit rows")
    np.testing.assert_array_equal(out_w[:U].cpu().numpy().view(np.uint32),
                                  ref["out_weights"].view(np.uint32), err_msg="replayed weights")

    op.reset()
    with pytest.raises(B.EpdcError):
        op.units_to_experts()
    # zero tokens: counts and offsets are zero, the conversions do nothing
    op.dispatch_dedup(x_d[:0], None, None, torch.from_numpy(idx[:0]).to(DEV))
    uo, _, _ = op.get_unit_routing()
    torch.cuda.synchronize()
    assert uo.cpu().tolist() == [0] * (R + 1)
    assert op._unit_buffers()["recv"].cpu().tolist() == [0] * R
    op.units_to_experts()
    y, yw = op.combine_units()
    assert y.shape == (0, H) and yw.shape == (0, K)


@pytest.mark.parametrize("T,H,K", [
    (128, 4096, 8),    # 512 vectors per row: 8 segments of 64
    (100, 4104, 8),    # 513 vectors: 8 segments of 65, the last one 58
    (128, 7168, 8),    # the decode shape: 8 segments of 112
    (60, 8200, 6),     # 1025 vectors: 16 segments of 65
])
def test_dedup_xcd_local_layout(T, H, K):
    """Small bf16 batches run the four kernels of the deduplicated path in
    segments of a multiple of 8 per row, in XCD order; ragged segment counts
    and widths, plus the replay of the unit rows."""
    log(f"dedup xcd-local T={T} H={H} K={K}")
    rng = np.random.default_rng(T + H)
    E, R = 64, 8
    idx = wl.draw_topk(rng, T, E, K, "zipf", 1.1)
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    w = wl.softmax_weights(rng, T, K)
    op, ref = run_dedup(x, w, idx, E, R)
    x2 = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    op.dispatch_dedup(bf16_dev(x), torch.from_numpy(w).to(DEV), None, torch.from_numpy(idx).to(DEV))
    out = op.dispatch_replay(bf16_dev(x2), torch.from_numpy(w).to(DEV))[0]
    torch.cuda.synchronize()
    ref2 = oracle.dispatch_dedup(x2, w, idx, E, R)
    U = ref2["units"]
    np.testing.assert_array_equal(u16(out[:U]), ref2["out"], err_msg="replayed unit rows")
