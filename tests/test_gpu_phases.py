"""Routing replay and split-phase dispatch/combine against the CPU oracle.

Routing replay ("Choosing an EP API and backend" page, "EP paths" table):
a new payload for the same tokens lands where a fresh dispatch with the same
expert ids would put it, so the oracle's dispatch of the new payload is the
expected result, bit-exact.  Split phases ("Communication APIs" page, methods
table): the results equal those of the one-call methods, with unrelated work
enqueued on the caller's stream between send and receive.
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


def check_dispatch(views, ref, weighted=True):
    out, out_w, out_sc, out_idx, recv = views
    n = ref["n_valid"]
    np.testing.assert_array_equal(recv.cpu().numpy(), ref["recv_count"], err_msg="recv_count")
    np.testing.assert_array_equal(bytes_of(out[:n]), ref["out"].view(np.uint8).reshape(n, -1),
                                  err_msg="payload")
    np.testing.assert_array_equal(out_idx[:n].cpu().numpy(), ref["out_indices"],
                                  err_msg="out_indices")
    if weighted:
        np.testing.assert_array_equal(out_w[:n].cpu().numpy().view(np.uint32),
                                      ref["out_weights"].view(np.uint32), err_msg="out_weights")
    if ref["out_scales"] is not None:
        np.testing.assert_array_equal(bytes_of(out_sc[:n]),
                                      ref["out_scales"].view(np.uint8).reshape(n, -1),
                                      err_msg="out_scales")


def check_combine(y, y_w, c_in_host, ref, T, K):
    ry, ry_w = oracle.combine(c_in_host, ref["out_weights"], ref["slot_of"], T, K)
    np.testing.assert_array_equal(y.contiguous().view(torch.int16).cpu().numpy().view(np.uint16),
                                  ry, err_msg="combine")
    np.testing.assert_array_equal(y_w.cpu().numpy().view(np.uint32), ry_w.view(np.uint32),
                                  err_msg="combine weights")


# T*K <= 1024 takes the fused single-launch dispatch; larger T the routing kernels.
@pytest.mark.parametrize("T,quant", [(100, "none"), (2000, "none"), (4096, "none"),
                                     (300, "fp8_e4m3_b128"), (100, "fp8_e4m3_b128"),
                                     (700, "mxfp4_b32")])
def test_dispatch_replay_matches_fresh_dispatch(T, quant):
    log(f"replay T={T} quant={quant}")
    rng = np.random.default_rng(T + 31)
    H, K, E, R = 7168, 8, 256, 8
    if quant == "mxfp4_b32":
        H = 4096
    idx = wl.draw_topk(rng, T, E, K, "zipf", 1.1)
    x1 = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    w1 = wl.softmax_weights(rng, T, K)
    x2 = wl.f32_to_bf16_bits((3.0 * rng.standard_normal((T, H))).astype(np.float32))
    w2 = wl.softmax_weights(rng, T, K)
    op = EpDispatchCombineOp(EpDispatchCombineConfig(T, H, K, E, R, quant=quant), DEV)
    idx_d = torch.from_numpy(idx).to(DEV)
    op.dispatch(bf16_dev(x1), torch.from_numpy(w1).to(DEV), None, idx_d)
    # the routing inputs may change after the dispatch: replay must not read them
    idx_d.fill_(-1)
    views = op.dispatch_replay(bf16_dev(x2), torch.from_numpy(w2).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.dispatch(x2, w2, idx, E, R, quant=quant)
    check_dispatch(views, ref)
    np.testing.assert_array_equal(op.get_dispatch_src_token_pos()[:ref["n_valid"]].cpu().numpy(),
                                  ref["src_token_pos"], err_msg="src_token_pos")
    assert op.device_error() == 0
    c_in_host = (ref["out"] if quant == "none" else
                 wl.f32_to_bf16_bits(rng.standard_normal((T * K, H)).astype(np.float32)))
    c_in = views[0] if quant == "none" else bf16_dev(c_in_host)
    y, y_w = op.combine(c_in, views[1], views[3])
    torch.cuda.synchronize()
    check_combine(y, y_w, c_in_host, ref, T, K)


@pytest.mark.parametrize("T", [513, 100])
def test_replay_raw_rows_scales_and_no_weights(T):
    log(f"replay raw rows T={T}")
    rng = np.random.default_rng(41)
    K, E, R, RB = 8, 256, 8, 7168
    idx = wl.draw_topk(rng, T, E, K, "uniform")
    raw1 = rng.integers(0, 256, (T, RB), dtype=np.uint8)
    raw2 = rng.integers(0, 256, (T, RB), dtype=np.uint8)
    sc1 = rng.standard_normal((T, 56)).astype(np.float32)
    sc2 = rng.standard_normal((T, 56)).astype(np.float32)
    op = EpDispatchCombineOp(EpDispatchCombineConfig(T, 256, K, E, R, raw_row_bytes=RB,
                                                     scale_row_bytes=sc1[0].nbytes), DEV)
    w = wl.softmax_weights(rng, T, K)
    op.dispatch(torch.from_numpy(raw1).to(DEV), torch.from_numpy(w).to(DEV),
                torch.from_numpy(sc1).to(DEV), torch.from_numpy(idx).to(DEV))
    views = op.dispatch_replay(torch.from_numpy(raw2).to(DEV), None, torch.from_numpy(sc2).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.dispatch(raw2, w, idx, E, R, scales=sc2)
    check_dispatch(views, ref, weighted=False)
    assert views[1] is None
    # the replay without weights left the recorded dispatch's weights in place
    np.testing.assert_array_equal(op._out_weights[:ref["n_valid"]].cpu().numpy().view(np.uint32),
                                  ref["out_weights"].view(np.uint32))


def test_replay_needs_a_dispatch_and_zero_tokens_is_empty():
    log("replay state")
    T, H, K, E, R = 64, 256, 4, 16, 4
    op = EpDispatchCombineOp(EpDispatchCombineConfig(T, H, K, E, R), DEV)
    x = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(B.EpdcError) as ei:
        op.dispatch_replay(x)
    assert ei.value.status == B.EPDC_ERR_BAD_STATE
    idx = torch.zeros((T, K), dtype=torch.int32, device=DEV)
    op.dispatch(x, None, None, idx)
    op.reset()
    with pytest.raises(B.EpdcError) as ei:
        op.dispatch_replay(x)
    assert ei.value.status == B.EPDC_ERR_BAD_STATE
    op.dispatch(x[:0], None, None, idx[:0])
    out = op.dispatch_replay(x[:0])[0]
    torch.cuda.synchronize()
    assert out.shape[0] == T * K     # capacity view; nothing was written


@pytest.mark.parametrize("name,tokens", [("deepseek_v3_bf16", None), ("decode_bf16", None),
                                         ("deepseek_v3_fp8", 1000)])
def test_split_phase_matches_oracle(name, tokens):
    w = wl.WORKLOADS[name]
    log(f"split phase {name} tokens={tokens}")
    inp = wl.make_inputs(w, tokens=tokens, with_combine_input=True)
    T = inp["x"].shape[0]
    op = EpDispatchCombineOp(EpDispatchCombineConfig(T, w.hidden, w.topk, w.experts, w.ranks,
                                                     quant=w.quant), DEV)
    x = bf16_dev(inp["x"])
    idx = torch.from_numpy(inp["indices"]).to(DEV)
    wts = torch.from_numpy(inp["weights"]).to(DEV)
    busy = torch.randn((2048, 2048), device=DEV)

    op.dispatch_send(x, wts, None, idx)
    del x, wts, idx                      # recorded on the side stream: memory stays valid
    z = busy @ busy                      # compute on the caller's stream meanwhile
    views = op.dispatch_recv()
    ref = oracle.dispatch(inp["x"], inp["weights"], inp["indices"], w.experts, w.ranks,
                          quant=w.quant)
    if w.combine_input == "independent":
        c_in_host = inp["combine_input"]
        c_in = bf16_dev(c_in_host)
    else:
        c_in_host = ref["out"]
        c_in = views[0]
    op.combine_send(c_in, views[1], views[3])
    z = z @ busy
    y, y_w = op.combine_recv()
    # read on the caller's stream only: recv ordered it after the side stream
    y_h, y_w_h = y.cpu(), y_w.cpu()
    check_dispatch([v.cpu() if v is not None else None for v in views], ref)
    check_combine(y_h, y_w_h, c_in_host, ref, T, w.topk)
    assert torch.isfinite(z).all()


def test_recv_without_send_is_an_error():
    log("recv without send")
    op = EpDispatchCombineOp(EpDispatchCombineConfig(8, 64, 2, 4, 2), DEV)
    for stage in (op.dispatch_recv, op.combine_recv):
        with pytest.raises(B.EpdcError) as ei:
            stage()
        assert ei.value.status == B.EPDC_ERR_BAD_STATE
    # the C entry points check the same state themselves
    for fn in (B.epdc_dispatch_recv, B.epdc_combine_recv):
        with pytest.raises(B.EpdcError) as ei:
            fn(op._op, torch.cuda.current_stream(DEV).cuda_stream)
        assert ei.value.status == B.EPDC_ERR_BAD_STATE


# ---- registered combine-input buffer ------------------------------------------------

@pytest.mark.parametrize("name,tokens", [("deepseek_v3_bf16", 1500), ("decode_bf16", None)])
def test_registered_combine_input_buffer(name, tokens):
    """Expert outputs written into the op's registered buffer ("Communication
    APIs" page, methods table: get_registered_combine_input_buffer) are
    combined from it, bit-exact against the oracle's combine of the same rows."""
    w = wl.WORKLOADS[name]
    log(f"registered combine buffer {name} tokens={tokens}")
    inp = wl.make_inputs(w, tokens=tokens, with_combine_input=True)
    T, K = inp["indices"].shape
    op = EpDispatchCombineOp(EpDispatchCombineConfig(T, w.hidden, K, w.experts, w.ranks), DEV)
    _, out_w, _, out_idx, recv = op.dispatch(bf16_dev(inp["x"]),
                                             torch.from_numpy(inp["weights"]).to(DEV), None,
                                             torch.from_numpy(inp["indices"]).to(DEV))
    buf = op.get_registered_combine_input_buffer()
    assert buf.dtype == torch.bfloat16 and buf.shape == (T * K, w.hidden)
    assert buf.data_ptr() == op.get_registered_combine_input_buffer().data_ptr()  # one buffer
    with pytest.raises(ValueError):
        op.get_registered_combine_input_buffer(torch.float32)
    buf.copy_(bf16_dev(inp["combine_input"]))      # the "expert output"
    y, y_w = op.combine(buf, out_w, out_idx)
    torch.cuda.synchronize()
    ref = oracle.dispatch(inp["x"], inp["weights"], inp["indices"], w.experts, w.ranks)
    assert int(recv.sum()) == ref["n_valid"]
    check_combine(y, y_w, inp["combine_input"], ref, T, K)


# ---- debug check of combine's indices ------------------------------------------------

@pytest.mark.parametrize("T", [700, 100])   # 5600 pairs: routing launches; 800: one launch
def test_combine_indices_debug_check(T):
    """With the debug check on, combine compares the given indices with the
    recorded routing and raises bit 4 of the device error flag on a
    mismatch; the combine itself still runs.  Off (the default), the indices
    are not read."""
    log(f"indices debug check T={T}")
    rng = np.random.default_rng(T + 77)
    H, K, E, R = 512, 8, 64, 8
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    idx = wl.draw_topk(rng, T, E, K, "zipf", 1.1)
    wts = wl.softmax_weights(rng, T, K)
    op = EpDispatchCombineOp(EpDispatchCombineConfig(T, H, K, E, R), DEV)
    out, out_w, _, out_idx, _ = op.dispatch(bf16_dev(x), torch.from_numpy(wts).to(DEV), None,
                                            torch.from_numpy(idx).to(DEV))
    ref = oracle.dispatch(x, wts, idx, E, R)
    eo, ro = op.get_offsets()
    np.testing.assert_array_equal(eo.cpu().numpy(), ref["expert_off"], err_msg="expert_off")
    np.testing.assert_array_equal(ro.cpu().numpy(), ref["rank_off"], err_msg="rank_off")
    n = ref["n_valid"]
    bad = out_idx.clone()
    s = n // 2
    k = int(ref["src_token_pos"][s]) % K
    bad[s, k] = (bad[s, k] + 1) % E      # row s no longer names its own expert in entry k
    other = out_idx.clone()
    other[s, (k + 1) % K] = (other[s, (k + 1) % K] + 1) % E   # an entry the check does not own

    assert op.device_error() == 0
    op.combine(out, out_w, bad)           # debug off: indices are not read
    assert op.device_error() == 0
    op.set_debug(True)
    for given, flag in ((out_idx, 0), (None, 0), (other, 0), (bad, 4)):
        y, y_w = op.combine(out, out_w, given)
        assert op.device_error() == flag
        check_combine(y, y_w, ref["out"], ref, T, K)
    y, y_w = op.combine_scatter(out, out_w, bad)
    assert op.device_error() == 4
    check_combine(y, y_w, ref["out"], ref, T, K)
    op.set_debug(False)
    op.combine(out, out_w, bad)
    assert op.device_error() == 0
    with pytest.raises(B.EpdcError) as ei:
        B.epdc_set_debug(op._op, 2)
    assert ei.value.status == B.EPDC_ERR_INVALID_ARGS


def test_indices_check_after_deduplicated_dispatch():
    """The pair routing recorded by the rank-deduplicated dispatch is what the
    check compares with: the expert-layout indices from the conversion pass,
    a corrupted entry is flagged."""
    log("indices check after dedup")
    rng = np.random.default_rng(91)
    T, H, K, E, R = 600, 256, 8, 64, 8
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    idx = wl.draw_topk(rng, T, E, K, "zipf", 1.1)
    wts = wl.softmax_weights(rng, T, K)
    op = EpDispatchCombineOp(EpDispatchCombineConfig(T, H, K, E, R), DEV)
    op.set_debug(True)
    op.dispatch_dedup(bf16_dev(x), torch.from_numpy(wts).to(DEV), None,
                      torch.from_numpy(idx).to(DEV))
    e_out, e_w, _, e_i, _ = op.units_to_experts()
    ref = oracle.dispatch(x, wts, idx, E, R)
    y, y_w = op.combine(e_out, e_w, e_i)
    assert op.device_error() == 0
    check_combine(y, y_w, ref["out"], ref, T, K)
    bad = e_i.clone()
    s = 17
    k = int(ref["src_token_pos"][s]) % K
    bad[s, k] = (bad[s, k] + 1) % E
    op.combine(e_out, e_w, bad)
    assert op.device_error() == 4


@pytest.mark.parametrize("name,recent", [("deepseek_v3_bf16", True), ("deepseek_v3_fp8", True),
                                         ("deepseek_v3_bf16", False)])
def test_combine_hint_changes_no_result(name, recent):
    """The combine-input hint only picks the output stores' cache policy: at
    full size the combine stays bit-identical to the oracle either way."""
    w = wl.WORKLOADS[name]
    log(f"combine hint {name} recent={recent}")
    inp = wl.make_inputs(w, with_combine_input=True)
    op = EpDispatchCombineOp(EpDispatchCombineConfig(w.tokens, w.hidden, w.topk, w.experts,
                                                     w.ranks, quant=w.quant), DEV)
    op.set_combine_hint(recent)
    out, out_w, _, out_idx, _ = op.dispatch(bf16_dev(inp["x"]),
                                            torch.from_numpy(inp["weights"]).to(DEV), None,
                                            torch.from_numpy(inp["indices"]).to(DEV))
    ref = oracle.dispatch(inp["x"], inp["weights"], inp["indices"], w.experts, w.ranks,
                          quant=w.quant)
    identity = w.quant == "none"
    c_in_host = ref["out"] if identity else inp["combine_input"]
    y, y_w = op.combine(out if identity else bf16_dev(c_in_host), out_w, out_idx)
    check_combine(y, y_w, c_in_host, ref, w.tokens, w.topk)
    with pytest.raises(B.EpdcError) as ei:
        B.epdc_set_combine_hint(op._op, 7)
    assert ei.value.status == B.EPDC_ERR_INVALID_ARGS
