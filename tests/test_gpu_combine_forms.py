"""GPU parity of the gather combine's launch forms against the oracle.

The op picks the form from the batch and from what the caller says about the
input (epdc_set_combine_hint):
- a batch of at most one routing tile: one wave per (token, segment), XCD order;
- larger, input marked as just written: the same kernel, device-scope stores;
- larger, cold input, rows whose byte size is not a power of two: the staged
  form (groups of up to four rows per block, assembled in LDS);
- larger, cold input, power-of-two rows: the plain form, with fewer waves per
  CU once the input rows span 768 MiB or more.
Every form must give the oracle's bits, including ragged groups and
segments, missing pairs (invalid expert ids) and the generic-K path.
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


def combine_both_hints(T, H, K, E, R, seed, invalid=0, independent=True, weighted=True):
    """Dispatch once, then combine with each hint; both must equal the oracle."""
    print(f"combine forms T={T} H={H} K={K} E={E} R={R} invalid={invalid} "
          f"independent={independent} weighted={weighted}", flush=True)
    rng = np.random.default_rng(seed)
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    idx = wl.draw_topk(rng, T, E, K, "zipf", 1.1)
    for i in range(invalid):
        idx[(i * 7919) % T, i % K] = -1 if i % 2 else E + i
    wts = wl.softmax_weights(rng, T, K)
    op = EpDispatchCombineOp(EpDispatchCombineConfig(T, H, K, E, R), DEV)
    out, out_w, _, out_idx, _ = op.dispatch(bf16_dev(x), torch.from_numpy(wts).to(DEV), None,
                                            torch.from_numpy(idx).to(DEV))
    ref = oracle.dispatch(x, wts, idx, E, R)
    if independent:
        c_host = wl.f32_to_bf16_bits(rng.standard_normal((T * K, H)).astype(np.float32))
        c_in = bf16_dev(c_host)
    else:
        c_host, c_in = ref["out"], out
    ry, ry_w = oracle.combine(c_host, ref["out_weights"] if weighted else None, ref["slot_of"],
                              T, K)
    for recent in (False, True):
        op.set_combine_hint(recent_input=recent)
        y, y_w = op.combine(c_in, out_w if weighted else None, out_idx)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits16(y), ry, err_msg=f"combine (recent={recent})")
        np.testing.assert_array_equal(y_w.cpu().numpy().view(np.uint32), ry_w.view(np.uint32),
                                      err_msg=f"combine weights (recent={recent})")
        y.fill_(0)
    assert op.device_error() == int(ref["invalid"] > 0)
    return ref


@pytest.mark.parametrize("T,H,K,E,R", [
    (1021, 7168, 8, 256, 8),   # staged: 4 rows of 14 KiB per block, last group of 1
    (333, 2880, 4, 64, 4),     # staged: 360 vectors, the last 1 KiB segment partial
    (190, 5000, 6, 40, 8),     # staged: 625 vectors per row, 1140 pairs (two tiles)
    (400, 1000, 3, 12, 3),     # staged, generic K (3 is not a compiled count)
    (130, 7168, 8, 256, 8),    # 1040 pairs: the smallest batch past one tile
])
def test_staged_combine_matches_oracle(T, H, K, E, R):
    combine_both_hints(T, H, K, E, R, seed=T + H)


def test_staged_combine_with_missing_pairs():
    ref = combine_both_hints(777, 7168, 8, 256, 8, seed=5, invalid=9)
    assert ref["invalid"] == 9


def test_staged_combine_unweighted():
    combine_both_hints(700, 7168, 8, 256, 8, seed=9, weighted=False)


def test_staged_combine_of_the_dispatch_output():
    combine_both_hints(513, 7168, 8, 256, 8, seed=6, independent=False)


def test_power_of_two_rows_plain_form():
    combine_both_hints(1500, 4096, 8, 128, 8, seed=7)


def test_few_waves_form_at_768_mib_of_input():
    """12288 tokens x top-8 x 4096 bf16: 768 MiB of input rows, the threshold."""
    combine_both_hints(12288, 4096, 8, 128, 8, seed=8)
