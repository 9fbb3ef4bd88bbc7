"""Two ops at once: independent state, any stream.

Each op owns its workspace and receive buffers, and the library keeps no
device state of its own, so two ops with different configurations can be
driven in any interleaving — on two streams that run concurrently, or
alternately on one stream — and each must give exactly what it gives alone.
Checked bit for bit against the oracle (payload, FP8 codes and scales,
routing, combine).  Streams keep the default priority.
"""
import numpy as np
import pytest
import torch

from combine_routing_histogram_amd import workloads as wl
from combine_routing_histogram_amd.op import EpDispatchCombineConfig, EpDispatchCombineOp
from oracle import oracle

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)


def bits16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


class Case:
    """One op, its device inputs and the oracle's expected outputs."""

    def __init__(self, T, H, K, E, R, quant, seed):
        rng = np.random.default_rng(seed)
        self.T, self.K = T, K
        self.x = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
        self.idx = wl.draw_topk(rng, T, E, K, "zipf", 1.1)
        self.w = wl.softmax_weights(rng, T, K)
        self.op = EpDispatchCombineOp(EpDispatchCombineConfig(T, H, K, E, R, quant=quant), DEV)
        self.x_d, self.idx_d = bf16_dev(self.x), torch.from_numpy(self.idx).to(DEV)
        self.w_d = torch.from_numpy(self.w).to(DEV)
        self.ref = oracle.dispatch(self.x, self.w, self.idx, E, R, quant=quant)
        n = self.ref["n_valid"]
        if quant == "none":
            self.c_in_host, self.c_in = self.ref["out"], None     # identity expert
        else:
            self.c_in_host = wl.f32_to_bf16_bits(rng.standard_normal((n, H)).astype(np.float32))
            self.c_in = bf16_dev(self.c_in_host)
        self.ry, self.ry_w = oracle.combine(self.c_in_host, self.ref["out_weights"],
                                            self.ref["slot_of"], T, K)

    def dispatch(self):
        self.got = self.op.dispatch(self.x_d, self.w_d, None, self.idx_d)

    def combine(self):
        out, out_w, _, out_idx, _ = self.got
        self.y = self.op.combine(out if self.c_in is None else self.c_in, out_w, out_idx)

    def check(self):
        out, out_w, out_sc, out_idx, recv = self.got
        ref, n = self.ref, self.ref["n_valid"]
        np.testing.assert_array_equal(recv.cpu().numpy(), ref["recv_count"])
        np.testing.assert_array_equal(self.op.get_routing()[2].cpu().numpy(), ref["slot_of"])
        np.testing.assert_array_equal(out[:n].contiguous().view(torch.uint8).cpu().numpy(),
                                      ref["out"].view(np.uint8).reshape(n, -1))
        if ref["out_scales"] is not None:
            np.testing.assert_array_equal(
                out_sc[:n].contiguous().view(torch.uint8).cpu().numpy(),
                ref["out_scales"].view(np.uint8).reshape(n, -1))
        np.testing.assert_array_equal(out_idx[:n].cpu().numpy(), ref["out_indices"])
        y, y_w = self.y
        np.testing.assert_array_equal(bits16(y), self.ry)
        np.testing.assert_array_equal(y_w.cpu().numpy().view(np.uint32), self.ry_w.view(np.uint32))


def cases():
    # 1500 x 8 pairs: 12 routing tiles; 150 x 6: one tile, routed in the scatter launch
    return [Case(1500, 1024, 8, 64, 8, "none", 41), Case(150, 2048, 6, 48, 4, "fp8_e4m3_b128", 42)]


def test_two_ops_on_two_streams():
    a, b = cases()
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(DEV), torch.cuda.Stream(DEV)
    for it in range(3):
        print(f"two streams, iteration {it}", flush=True)
        with torch.cuda.stream(sa):
            a.dispatch()
        with torch.cuda.stream(sb):
            b.dispatch()
        with torch.cuda.stream(sa):
            a.combine()
        with torch.cuda.stream(sb):
            b.combine()
    torch.cuda.synchronize()
    a.check()
    b.check()


def test_two_ops_interleaved_on_one_stream():
    a, b = cases()
    print("one stream, A and B alternating", flush=True)
    a.dispatch()
    b.dispatch()        # B's routing does not disturb A's recorded routing
    a.combine()
    b.combine()
    torch.cuda.synchronize()
    a.check()
    b.check()
