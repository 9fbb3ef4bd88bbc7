"""The widest rows the C ABI accepts, compared bit for bit with the oracle.

hidden = 2^24 (32 MiB bf16 rows, 2^21 16-byte vectors, 16,384 segments per
row) for bf16, FP8 and MXFP4 on the single-launch path (one routing tile);
hidden = 2^18 over two routing tiles (the scan folded into the scatter
blocks); raw rows of 2^25 bytes.  Row offsets stay below 2^25 bytes inside a
row and row starts are 64-bit, so these sizes exercise the same kernels as
the workloads, at the far end of every index.
"""
import numpy as np
import pytest

from combine_routing_histogram_amd import workloads as wl
from test_gpu_parity import run_case

pytestmark = pytest.mark.gpu

QUANTS = ["none", "fp8_e4m3_b128", "mxfp4_b32"]


def _case(T, H, K, E, R, quant, seed):
    print(f"max size T={T} H={H} K={K} E={E} R={R} quant={quant}", flush=True)
    rng = np.random.default_rng(seed)
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    idx = wl.draw_topk(rng, T, E, K, "uniform")
    wts = wl.softmax_weights(rng, T, K)
    c_in = None
    if quant != "none":
        c_in = wl.f32_to_bf16_bits(rng.standard_normal((T * K, H), dtype=np.float32))
    run_case(x, wts, idx, E, R, quant=quant, combine_input=c_in)


@pytest.mark.parametrize("quant", QUANTS)
def test_max_hidden_one_tile(quant):
    _case(3, 1 << 24, 2, 4, 2, quant, 91)


@pytest.mark.parametrize("quant", QUANTS)
def test_wide_rows_two_tiles(quant):
    _case(130, 1 << 18, 8, 16, 4, quant, 92)      # 1040 pairs: two routing tiles


def test_max_raw_row_bytes():
    print("max raw row bytes 2^25", flush=True)
    rng = np.random.default_rng(93)
    T, K, E, R = 3, 2, 4, 2
    raw = rng.integers(0, 256, (T, 1 << 25), dtype=np.uint8)
    sc = rng.standard_normal((T, 4)).astype(np.float32)
    idx = wl.draw_topk(rng, T, E, K, "uniform")
    wts = wl.softmax_weights(rng, T, K)
    c_in = wl.f32_to_bf16_bits(rng.standard_normal((T * K, 256)).astype(np.float32))
    run_case(raw, wts, idx, E, R, hidden=256, raw_row_bytes=1 << 25, scales=sc,
             combine_input=c_in)
