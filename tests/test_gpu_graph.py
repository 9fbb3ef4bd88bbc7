"""Graph capture and replay of dispatch + combine (MORI "Choosing an EP API and
backend" page, "Validation before tuning": graph replay is one of the checks).

The launches record no memset node (the kernels write every count and offset
themselves), so a captured step can be replayed.  Each replay is checked
against the eager result, with eager work that overwrites the outputs between
replays.
"""
import numpy as np
import pytest
import torch

from combine_routing_histogram_amd import workloads as wl
from combine_routing_histogram_amd.op import EpDispatchCombineConfig, EpDispatchCombineOp

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)


@pytest.mark.parametrize("name,tokens", [("decode_bf16", None), ("deepseek_v3_bf16", 1024),
                                         ("deepseek_v3_fp8", 300)])
def test_graph_replay_matches_eager(name, tokens):
    w = wl.WORKLOADS[name]
    print(f"graph replay {name} tokens={tokens}", flush=True)
    inp = wl.make_inputs(w, tokens=tokens, with_combine_input=True)
    T = inp["x"].shape[0]
    x = torch.from_numpy(inp["x"].view(np.int16)).view(torch.bfloat16).to(DEV)
    idx = torch.from_numpy(inp["indices"]).to(DEV)
    wts = torch.from_numpy(inp["weights"]).to(DEV)
    c_in = (torch.from_numpy(inp["combine_input"].view(np.int16)).view(torch.bfloat16).to(DEV)
            if w.combine_input == "independent" else None)
    op = EpDispatchCombineOp(EpDispatchCombineConfig(T, w.hidden, w.topk, w.experts, w.ranks,
                                                     quant=w.quant), DEV)

    def step():
        out, out_w, _, out_idx, recv = op.dispatch(x, wts, None, idx)
        y, y_w = op.combine(out if c_in is None else c_in, out_w, out_idx)
        return out, recv, y, y_w

    out, recv, y, y_w = step()
    torch.cuda.synchronize()
    n = int(recv.sum())
    ref = [out[:n].view(torch.uint8).clone(), recv.clone(), y.clone(), y_w.clone(),
           op.get_dispatch_src_token_pos()[:n].clone()]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        g_out, g_recv, g_y, g_yw = step()
    torch.cuda.synchronize()

    for rep in range(3):
        # eager work between replays: clobber everything the replay must rewrite
        g_out.view(torch.uint8).fill_(0xA5)
        g_recv.fill_(-1)
        g_y.fill_(3.0)
        g_yw.fill_(-2.0)
        op.get_dispatch_src_token_pos().fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [g_out[:n].view(torch.uint8), g_recv, g_y, g_yw, op.get_dispatch_src_token_pos()[:n]]
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"
