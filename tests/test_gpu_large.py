"""Large token counts: thousands of routing tiles, so the one-block scan
keeps only part of each expert column in registers and re-reads the rest
from the tile table (more than 16 tiles per column chunk), for the pair
routing and for the unit routing of the rank-deduplicated dispatch.  Small
rows keep the oracle fast; every output is compared bit for bit.
"""
import numpy as np
import pytest
import torch

from combine_routing_histogram_amd import workloads as wl
from combine_routing_histogram_amd.op import EpDispatchCombineConfig, EpDispatchCombineOp
from oracle import oracle
from test_gpu_parity import run_case

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)


def u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("T,H,K,E,R,skew", [
    (16384, 256, 8, 256, 8, 1.1),     # 128 tiles: 32 per column chunk for E = 256
    (131072, 64, 8, 512, 8, 1.3),     # 1024 tiles: 512 per chunk for E = 512
])
def test_many_tiles_pair_path(T, H, K, E, R, skew):
    print(f"large pair T={T} E={E}", flush=True)
    rng = np.random.default_rng(T + E)
    idx = wl.draw_topk(rng, T, E, K, "zipf", skew)
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    run_case(x, wl.softmax_weights(rng, T, K), idx, E, R)


def test_many_tiles_unit_path():
    """2,344 tiles: the unit-level scan (8 keys, 128 threads per column) also
    leaves its registers."""
    T, H, K, E, R = 300000, 32, 8, 64, 8
    print(f"large units T={T}", flush=True)
    rng = np.random.default_rng(77)
    idx = wl.draw_topk(rng, T, E, K, "zipf", 1.2)
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    w = wl.softmax_weights(rng, T, K)
    op = EpDispatchCombineOp(EpDispatchCombineConfig(T, H, K, E, R), DEV)
    out, out_w, _, _, recv = op.dispatch_dedup(bf16_dev(x), torch.from_numpy(w).to(DEV), None,
                                               torch.from_numpy(idx).to(DEV))
    torch.cuda.synchronize()
    d = oracle.dispatch_dedup(x, w, idx, E, R)
    U = d["units"]
    np.testing.assert_array_equal(recv.cpu().numpy(), d["unit_cnt"])
    uo, uof, usrc = op.get_unit_routing()
    np.testing.assert_array_equal(uo.cpu().numpy(), d["unit_off"])
    np.testing.assert_array_equal(uof.cpu().numpy(), d["unit_of"])
    np.testing.assert_array_equal(usrc[:U].cpu().numpy(), d["unit_src"])
    np.testing.assert_array_equal(u16(out[:U]), d["out"])
    eo, ro, so = op.get_routing()
    np.testing.assert_array_equal(eo.cpu().numpy(), d["expert_off"])
    np.testing.assert_array_equal(so.cpu().numpy(), d["slot_of"])
    e_out = op.units_to_experts()[0]
    part = op.experts_to_units(e_out, op._out_weights)
    y, _ = op.combine_units(None, out_w)
    torch.cuda.synchronize()
    n = d["n_valid"]
    pair = oracle.dispatch(x, w, idx, E, R)
    np.testing.assert_array_equal(u16(e_out[:n]), pair["out"])
    rpart = oracle.experts_to_units(pair["out"], pair["out_weights"], d["unit_src"], d["unit_of"],
                                    d["slot_of"], K)
    np.testing.assert_array_equal(u16(part[:U]), rpart)
    ry, _ = oracle.combine_units(rpart, d["out_weights"], d["unit_of"], T, K)
    np.testing.assert_array_equal(u16(y), ry)


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)
