"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bit-exact for everything integer or byte-valued (counts, offsets, slots,
source positions, carried rows, bf16 payload, FP8/FP4 codes and scales).
Combine: within the bf16 tolerance (|g - o| <= max(1 ulp, 8e-3 |o|,
2^-20 sum|w x|)); it is also checked bit-exact, since both sides add the K
products in the same order with separate fp32 multiply and add.
"""
import functools

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


def bits16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bytes_of(t):
    return t.contiguous().view(torch.uint8).cpu().numpy()


def u8rows(a):
    """Host array as bytes, one row per leading index (also for zero rows)."""
    a = np.ascontiguousarray(a)
    return a.view(np.uint8).reshape(a.shape[0], int(np.prod(a.shape[1:], dtype=np.int64)) *
                                    a.itemsize)


@functools.lru_cache(maxsize=2)
def inputs_for(name, tokens=None):
    w = wl.WORKLOADS[name]
    return wl.make_inputs(w, tokens=tokens, with_combine_input=True)


def tolerance_ok(got_bits, ref_bits, abs_sum=None):
    g = wl.bf16_bits_to_f32(got_bits).astype(np.float64)
    o = wl.bf16_bits_to_f32(ref_bits).astype(np.float64)
    ulp = np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(o), 2.0 ** -126))).astype(np.int64) - 7)
    tol = np.maximum(ulp, 8e-3 * np.abs(o))
    if abs_sum is not None:
        tol = np.maximum(tol, 2.0 ** -20 * abs_sum)
    return np.abs(g - o) <= tol


def run_case(x, weights, indices, E, R, quant="none", max_tokens=None, hidden=None,
             combine_input=None, scales=None, raw_row_bytes=0, weights_none=False):
    """Dispatch + combine on the GPU and in the oracle; compare; return both."""
    T, K = indices.shape
    H = hidden if hidden is not None else x.shape[1]
    cfg = EpDispatchCombineConfig(max_tokens if max_tokens is not None else T, H, K, E, R,
                                  quant=quant, raw_row_bytes=raw_row_bytes,
                                  scale_row_bytes=0 if scales is None else scales[0].nbytes)
    op = EpDispatchCombineOp(cfg, DEV)
    if raw_row_bytes:
        x_d = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    else:
        x_d = bf16_dev(x)
    idx_d = torch.from_numpy(np.ascontiguousarray(indices)).to(DEV)
    w_d = None if weights_none else torch.from_numpy(np.ascontiguousarray(weights)).to(DEV)
    sc_d = None if scales is None else torch.from_numpy(np.ascontiguousarray(scales)).to(DEV)
    out, out_w, out_sc, out_idx, recv = op.dispatch(x_d, w_d, sc_d, idx_d)
    torch.cuda.synchronize()

    ref = oracle.dispatch(x, None if weights_none else weights, indices, E, R, quant=quant,
                          scales=scales)
    n = ref["n_valid"]
    eo, ro, so = op.get_routing()
    np.testing.assert_array_equal(recv.cpu().numpy(), ref["recv_count"], err_msg="recv_count")
    np.testing.assert_array_equal(eo.cpu().numpy(), ref["expert_off"], err_msg="expert_off")
    np.testing.assert_array_equal(ro.cpu().numpy(), ref["rank_off"], err_msg="rank_off")
    np.testing.assert_array_equal(so.cpu().numpy(), ref["slot_of"], err_msg="slot_of")
    np.testing.assert_array_equal(op.get_dispatch_src_token_pos()[:n].cpu().numpy(),
                                  ref["src_token_pos"], err_msg="src_token_pos")
    np.testing.assert_array_equal(bytes_of(out[:n]), u8rows(ref["out"]),
                                  err_msg="payload")
    np.testing.assert_array_equal(out_idx[:n].cpu().numpy(), ref["out_indices"],
                                  err_msg="out_indices")
    if not weights_none:
        np.testing.assert_array_equal(out_w[:n].cpu().numpy().view(np.uint32),
                                      ref["out_weights"].view(np.uint32), err_msg="out_weights")
    if ref["out_scales"] is not None:
        np.testing.assert_array_equal(bytes_of(out_sc[:n]),
                                      u8rows(ref["out_scales"]),
                                      err_msg="out_scales")

    # combine: identity expert (the dispatch output) for bf16, else the given rows
    if combine_input is None:
        assert quant == "none" and not raw_row_bytes
        c_in_host = ref["out"]
        c_in = out
    else:
        c_in_host = combine_input
        c_in = bf16_dev(combine_input)
    y, y_w = op.combine(c_in, out_w, out_idx)
    torch.cuda.synchronize()
    ry, ry_w = oracle.combine(c_in_host, ref["out_weights"], ref["slot_of"], T, K)
    gy = bits16(y)
    ok = tolerance_ok(gy, ry)
    assert ok.all(), f"combine: {np.size(ok) - ok.sum()} elements outside the bf16 tolerance"
    np.testing.assert_array_equal(gy, ry, err_msg="combine not bit-identical")
    np.testing.assert_array_equal(y_w.cpu().numpy().view(np.uint32), ry_w.view(np.uint32),
                                  err_msg="combine weights")
    assert op.device_error() == int((ref["invalid"] > 0))
    return op, ref


# ---- the workloads at their full sizes ---------------------------------------------

@pytest.mark.parametrize("name", ["tiny_bf16", "decode_sparse_bf16", "decode_bf16",
                                  "deepseek_v3_bf16", "deepseek_v3_fp8", "qwen3_moe_mxfp4",
                                  "deepseek_v3_raw_fp8"])
def test_workload_parity(name):
    w = wl.WORKLOADS[name]
    log(f"workload {name}: T={w.tokens} H={w.hidden} K={w.topk} E={w.experts} R={w.ranks} "
        f"quant={w.quant} raw_row_bytes={w.raw_row_bytes}")
    inp = inputs_for(name)
    c_in = inp["combine_input"] if w.combine_input == "independent" else None
    run_case(inp["x"], inp["weights"], inp["indices"], w.experts, w.ranks, quant=w.quant,
             combine_input=c_in, hidden=w.hidden, raw_row_bytes=w.raw_row_bytes,
             scales=inp.get("scales"))


# ---- ragged and edge cases ----------------------------------------------------------------

@pytest.mark.parametrize("tokens", [1, 3, 127, 1000, 4095])
def test_ragged_token_counts(tokens):
    """num_tokens below capacity; tiles and waves end mid-way."""
    w = wl.WORKLOADS["deepseek_v3_bf16"]
    log(f"ragged tokens={tokens}")
    inp = inputs_for("deepseek_v3_bf16", tokens)
    run_case(inp["x"], inp["weights"], inp["indices"], w.experts, w.ranks, max_tokens=w.tokens)


def test_zero_tokens():
    log("zero tokens")
    cfg = EpDispatchCombineConfig(64, 256, 4, 16, 4)
    op = EpDispatchCombineOp(cfg, DEV)
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros((0, 4), dtype=torch.int32, device=DEV)
    w = torch.zeros((0, 4), dtype=torch.float32, device=DEV)
    _, _, _, _, recv = op.dispatch(x, w, None, idx)
    eo, ro, so = op.get_routing()
    torch.cuda.synchronize()
    assert recv.cpu().tolist() == [0, 0, 0, 0]
    assert eo.cpu().tolist() == [0] * 17 and ro.cpu().tolist() == [0] * 5
    y, yw = op.combine(torch.zeros((1, 256), dtype=torch.bfloat16, device=DEV))
    assert y.shape == (0, 256) and yw.shape == (0, 4)


@pytest.mark.parametrize("T", [300, 200])   # 1200 pairs: two routing tiles; 800: routed inline
def test_invalid_expert_ids_get_no_slot(T):
    log(f"invalid ids T={T}")
    rng = np.random.default_rng(21)
    H, K, E, R = 64, 4, 16, 4
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    idx = rng.integers(0, E, (T, K)).astype(np.int32)
    idx[5, 2], idx[100, 0], idx[T - 1, 3] = -1, E, 1 << 30
    wts = rng.random((T, K)).astype(np.float32)
    op, ref = run_case(x, wts, idx, E, R)
    assert ref["invalid"] == 3
    assert op.device_error() == 0   # the flag was cleared by the read inside run_case


@pytest.mark.parametrize("T", [700, 300])   # 2100 pairs: three tiles; 900: routed inline
def test_all_pairs_one_expert_and_empty_ranks(T):
    log(f"one expert T={T}")
    rng = np.random.default_rng(22)
    H, K, E, R = 128, 3, 32, 8
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    idx = np.full((T, K), 9, np.int32)                  # duplicates within a token too
    wts = rng.random((T, K)).astype(np.float32)
    _, ref = run_case(x, wts, idx, E, R)
    assert ref["recv_count"].tolist() == [0, 0, T * K, 0, 0, 0, 0, 0]


@pytest.mark.parametrize("T,H,K,E,R", [
    (50, 64, 1, 1, 1),          # one expert, one rank, K = 1
    (33, 8, 2, 4, 2),           # one 16-byte vector per row
    (97, 200, 3, 10, 5),        # 25 vectors per row: ragged against 64 lanes
    (40, 8200, 5, 20, 4),       # 1025 vectors: several chunks plus a tail; generic combine
    (300, 128, 16, 512, 8),     # largest K and E
    (2500, 256, 6, 96, 3),      # several routing tiles, E not a power of two
])
def test_shapes(T, H, K, E, R):
    log(f"shape T={T} H={H} K={K} E={E} R={R}")
    rng = np.random.default_rng(T * 7 + H)
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    idx = wl.draw_topk(rng, T, E, K, "uniform")
    wts = wl.softmax_weights(rng, T, K)
    run_case(x, wts, idx, E, R)


def test_unweighted_combine_and_no_weights():
    log("no weights")
    rng = np.random.default_rng(23)
    T, H, K, E, R = 200, 256, 4, 16, 2
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    idx = wl.draw_topk(rng, T, E, K, "zipf", 1.2)
    run_case(x, None, idx, E, R, weights_none=True)


@pytest.mark.parametrize("T", [513, 100])   # 4104 pairs: five tiles; 800: routed inline
def test_raw_rows_and_carried_scales(T):
    """Already-quantized payloads are carried as bytes with their scales."""
    log(f"raw carry T={T}")
    rng = np.random.default_rng(24)
    K, E, R = 8, 256, 8
    raw = rng.integers(0, 256, (T, 7168), dtype=np.uint8)
    sc = rng.standard_normal((T, 56)).astype(np.float32)
    idx = wl.draw_topk(rng, T, E, K, "zipf", 1.1)
    wts = wl.softmax_weights(rng, T, K)
    c_in = wl.f32_to_bf16_bits(rng.standard_normal((T * K, 256)).astype(np.float32))
    run_case(raw, wts, idx, E, R, hidden=256, raw_row_bytes=7168, scales=sc, combine_input=c_in)


def _edge_rows(H, block, rng):
    vals = []
    tiny = np.float32(2.0) ** -133
    for b in range(H // block):
        kind = b % 8
        if kind == 0:
            v = np.zeros(block, np.float32)
        elif kind == 1:
            v = -np.zeros(block, np.float32)
            v[3] = -tiny
        elif kind == 2:
            v = np.full(block, tiny, np.float32) * rng.integers(1, 100, block)
        elif kind == 3:
            v = rng.standard_normal(block).astype(np.float32) * 1e-30
        elif kind == 4:
            v = rng.standard_normal(block).astype(np.float32) * 3e4
        elif kind == 5:
            v = np.linspace(-448, 448, block).astype(np.float32)
        elif kind == 6:
            v = rng.standard_normal(block).astype(np.float32)
            v[rng.integers(0, block)] = 1e3
        else:
            v = np.round(rng.standard_normal(block) * 8).astype(np.float32) / 8
        vals.append(v)
    return np.concatenate(vals)


@pytest.mark.parametrize("quant,block", [("fp8_e4m3_b128", 128), ("mxfp4_b32", 32)])
def test_quant_edge_values(quant, block):
    """Zero and -0 blocks, bf16 subnormals, tiny and huge scales, ties."""
    log(f"quant edges {quant}")
    rng = np.random.default_rng(25)
    T, H, K, E, R = 64, 1024, 2, 8, 2
    x = np.stack([_edge_rows(H, block, rng) for _ in range(T)])
    xb = wl.f32_to_bf16_bits(x)
    idx = wl.draw_topk(rng, T, E, K, "uniform")
    wts = wl.softmax_weights(rng, T, K)
    c_in = wl.f32_to_bf16_bits(rng.standard_normal((T * K, H)).astype(np.float32))
    run_case(xb, wts, idx, E, R, quant=quant, combine_input=c_in)


def test_fp8_exhaustive_code_points():
    """Every E4M3 code's value and every midpoint, scaled into blocks whose
    amax is 448 * s, so x / s hits the code points and ties exactly."""
    log("fp8 code points")
    pos = []
    for c in range(127):
        e, m = c >> 3, c & 7
        pos.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    pos = np.array(pos)
    pts = np.concatenate([pos, (pos[:-1] + pos[1:]) / 2])
    pts = np.concatenate([pts, -pts])
    per = 127
    n_blocks = -(-pts.size // per)
    x = np.zeros((n_blocks, 128), np.float32)
    for b in range(n_blocks):
        chunk = pts[b * per:(b + 1) * per]
        x[b, :chunk.size] = chunk
        x[b, 127] = 448.0                     # amax 448 -> s = 1 exactly
    flat = np.concatenate([x.ravel(), np.zeros(-x.size % 1024, np.float32)])
    xb = wl.f32_to_bf16_bits(flat.reshape(-1, 1024))     # zero padding = whole zero blocks
    T = xb.shape[0]
    rng = np.random.default_rng(26)
    idx = wl.draw_topk(rng, T, 4, 1, "uniform")
    wts = np.ones((T, 1), np.float32)
    c_in = wl.f32_to_bf16_bits(rng.standard_normal((T, 1024)).astype(np.float32))
    run_case(xb, wts, idx, 4, 2, quant="fp8_e4m3_b128", combine_input=c_in)


def test_mxfp4_exhaustive_code_points():
    """Every E2M1 value and midpoint at a range of block exponents."""
    log("mxfp4 code points")
    pos = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    pts = np.concatenate([pos, (pos[:-1] + pos[1:]) / 2, [5.5, 6.5, 7, 7.5]])
    blocks = []
    for e in range(-20, 21, 4):
        for sign in (1, -1):
            v = np.zeros(32)
            v[:pts.size] = sign * pts * 2.0 ** e
            v[31] = 4 * 2.0 ** e              # amax in [4, 8) * 2^e: scale exponent e
            blocks.append(v)
    x = np.concatenate(blocks).astype(np.float32)
    x = np.concatenate([x, np.zeros(-x.size % 256, np.float32)]).reshape(-1, 256)
    xb = wl.f32_to_bf16_bits(x)
    T = xb.shape[0]
    rng = np.random.default_rng(27)
    idx = wl.draw_topk(rng, T, 4, 2, "uniform")
    wts = wl.softmax_weights(rng, T, 2)
    c_in = wl.f32_to_bf16_bits(rng.standard_normal((T * 2, 256)).astype(np.float32))
    run_case(xb, wts, idx, 4, 2, quant="mxfp4_b32", combine_input=c_in)


# ---- determinism, state and reuse ---------------------------------------------------------

def test_deterministic_and_reusable():
    log("determinism and reuse")
    w = wl.WORKLOADS["deepseek_v3_bf16"]
    inp = inputs_for("deepseek_v3_bf16", 1024)
    cfg = EpDispatchCombineConfig(w.tokens, w.hidden, w.topk, w.experts, w.ranks)
    op = EpDispatchCombineOp(cfg, DEV)
    x = bf16_dev(inp["x"])
    idx = torch.from_numpy(inp["indices"]).to(DEV)
    wt = torch.from_numpy(inp["weights"]).to(DEV)
    snaps = []
    for rep in range(3):
        if rep == 1:   # a differently sized call in between must not disturb the next
            op.dispatch(x[:100], wt[:100], None, idx[:100])
        out, out_w, _, out_idx, recv = op.dispatch(x, wt, None, idx)
        y, y_w = op.combine(out, out_w, out_idx)
        n = int(recv.sum())
        snaps.append((bits16(out[:n]), bits16(y), op.get_dispatch_src_token_pos()[:n].cpu().numpy()))
    for s in snaps[1:]:
        for a, b in zip(snaps[0], s):
            np.testing.assert_array_equal(a, b)


def test_combine_needs_dispatch():
    log("state errors")
    op = EpDispatchCombineOp(EpDispatchCombineConfig(16, 64, 2, 4, 2), DEV)
    buf = torch.zeros((32, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(B.EpdcError) as ei:
        op.combine(buf)
    assert ei.value.status == B.EPDC_ERR_BAD_STATE
    idx = torch.zeros((4, 2), dtype=torch.int32, device=DEV)
    op.dispatch(torch.zeros((4, 64), dtype=torch.bfloat16, device=DEV), None, None, idx)
    op.combine(buf)
    op.reset()
    with pytest.raises(B.EpdcError) as ei:
        op.combine(buf)
    assert ei.value.status == B.EPDC_ERR_BAD_STATE
    with pytest.raises(B.EpdcError) as ei:
        op.get_dispatch_src_token_pos()
    assert ei.value.status == B.EPDC_ERR_BAD_STATE


def test_single_tile_dispatch_is_one_launch():
    """At most 1024 pairs: routing happens inside the scatter launch."""
    log("single-tile launch count")
    w = wl.WORKLOADS["decode_bf16"]
    inp = inputs_for("decode_bf16")
    op = EpDispatchCombineOp(EpDispatchCombineConfig(w.tokens, w.hidden, w.topk, w.experts,
                                                     w.ranks), DEV)
    op.profile_begin(8)
    out, out_w, _, out_idx, _ = op.dispatch(bf16_dev(inp["x"]), torch.from_numpy(
        inp["weights"]).to(DEV), None, torch.from_numpy(inp["indices"]).to(DEV))
    op.combine(out, out_w, out_idx)
    prof = op.profile_end()
    assert set(prof) == {"k_scatter_copy", "k_combine"}


# tiles x experts <= 8192: the scatter blocks scan the tile table themselves;
# larger tables are scanned by the last rank block: no scan launch either way
@pytest.mark.parametrize("name,tokens,kernels", [
    ("deepseek_v3_bf16", 1024, {"k_route_rank", "k_scatter_copy", "k_combine"}),
    ("qwen3_moe_mxfp4", 9000, {"k_route_rank", "k_scatter_mxfp4", "k_combine"}),
])
def test_profile_events_time_every_kernel(name, tokens, kernels):
    log(f"profile events {name}")
    w = wl.WORKLOADS[name]
    inp = inputs_for(name, tokens)
    op = EpDispatchCombineOp(EpDispatchCombineConfig(tokens, w.hidden, w.topk, w.experts,
                                                     w.ranks, quant=w.quant), DEV)
    x = bf16_dev(inp["x"])
    idx = torch.from_numpy(inp["indices"]).to(DEV)
    wt = torch.from_numpy(inp["weights"]).to(DEV)
    c_in = bf16_dev(inp["combine_input"])
    op.profile_begin(16)
    for _ in range(3):
        out, out_w, _, out_idx, _ = op.dispatch(x, wt, None, idx)
        op.combine(out if w.quant == "none" else c_in, out_w, out_idx)
    prof = op.profile_end()
    assert set(prof) == kernels
    for k, (ms, n) in prof.items():
        assert n == 3 and ms > 0, k


def test_scatter_blocks_straddling_two_tiles():
    """4 tokens x 6 pairs per block: blocks cross tile boundaries, so the
    blocks' own scan must give the second tile's bases too."""
    log("straddling blocks")
    rng = np.random.default_rng(25)
    T, H, K, E, R = 4096, 256, 6, 96, 3
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    idx = wl.draw_topk(rng, T, E, K, "zipf", 1.1)
    run_case(x, wl.softmax_weights(rng, T, K), idx, E, R)


@pytest.mark.parametrize("T,H,K", [
    (1024, 7168, 1),   # 7168 waves: 16 copying waves per routing block, 4-wave combine blocks
    (100, 7168, 10),   # 700 waves: 3 per routing block
    (73, 1000, 14),    # 73 waves, one per row: a partial round of blocks
    (341, 4104, 3),    # 1705 waves, 5 segments with a ragged last one: 7 per block
    (512, 2056, 2),    # 1536 waves: 6 per block
])
def test_one_tile_xcd_order(T, H, K):
    """Batches of one routing tile number their (token, segment) items in XCD
    order in the scatter, its replay and the combine; the grids are whole
    rounds of 8 blocks, so the last round holds items past the end."""
    log(f"xcd order T={T} H={H} K={K}")
    rng = np.random.default_rng(T * 31 + K)
    E, R = 64, 4
    idx = wl.draw_topk(rng, T, E, K, "uniform")
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    w = wl.softmax_weights(rng, T, K)
    op, ref = run_case(x, w, idx, E, R)
    x2 = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    out2 = op.dispatch_replay(bf16_dev(x2), torch.from_numpy(w).to(DEV), None)[0]
    torch.cuda.synchronize()
    n = ref["n_valid"]
    ref2 = oracle.dispatch(x2, w, idx, E, R)
    np.testing.assert_array_equal(bits16(out2[:n]), ref2["out"], err_msg="replay payload")


@pytest.mark.parametrize("T,H,K", [
    (2100, 1152, 4),   # 144 vectors per row: one wave per row, the second pass 16 vectors
    (2048, 4224, 8),   # 528 vectors: five passes, the last one partial
    (2300, 928, 2),    # hidden % 128 != 0: scale bytes stored one by one
])
def test_mxfp4_one_wave_per_row(T, H, K):
    """Many tokens: the MXFP4 scatter runs one wave per row and stores the
    row's scale bytes from its LDS stage as words; widths that are not a
    multiple of 128 keep byte stores."""
    log(f"mxfp4 rows T={T} H={H} K={K}")
    rng = np.random.default_rng(T + H + K)
    E, R = 64, 4
    idx = wl.draw_topk(rng, T, E, K, "zipf", 1.3)
    x = wl.f32_to_bf16_bits((rng.standard_normal((T, H)) *
                             np.where(rng.random((T, H)) < 0.01, 20.0, 1.0)).astype(np.float32))
    c_in = wl.f32_to_bf16_bits(rng.standard_normal((T * K, H)).astype(np.float32))
    run_case(x, wl.softmax_weights(rng, T, K), idx, E, R, quant="mxfp4_b32", combine_input=c_in)


@pytest.mark.parametrize("T", [100, 700])   # 400 pairs: routed inline; 2800: three tiles
def test_every_expert_id_invalid(T):
    """No pair has a row: every rank receives 0, nothing is written, combine
    gives +0 with weight 0 everywhere, and the device flag is raised."""
    log(f"all ids invalid T={T}")
    rng = np.random.default_rng(T + 5)
    H, K, E, R = 128, 4, 16, 4
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    idx = np.where(rng.random((T, K)) < 0.5, -1, E + 3).astype(np.int32)
    wts = rng.random((T, K)).astype(np.float32)
    op, ref = run_case(x, wts, idx, E, R)
    assert ref["n_valid"] == 0 and ref["recv_count"].tolist() == [0] * R
    # the deduplicated path sees no unit either
    op.dispatch_dedup(bf16_dev(x), torch.from_numpy(wts).to(DEV), None,
                      torch.from_numpy(idx).to(DEV))
    uo, _, _ = op.get_unit_routing()
    assert uo.cpu().tolist() == [0] * (R + 1)
    y, y_w = op.combine_units(None, None)
    torch.cuda.synchronize()
    assert not bits16(y).any() and not y_w.cpu().numpy().any()
    assert op.device_error() == 1
