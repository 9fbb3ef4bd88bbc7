"""The OpenMP build of the oracle (the all-cores CPU baseline) gives results
identical to the plain single-thread build on the same inputs: dispatch
(routing, payload, produced FP8/MXFP4 codes and scales, carried rows) and
combine.  Only the loops over tokens are parallel, and each token's
iteration writes only its own rows."""
import numpy as np
import pytest

from combine_routing_histogram_amd import workloads as wl
from oracle import oracle


def _run(w, inp):
    d = oracle.dispatch(inp["x"], inp["weights"], inp["indices"], w.experts, w.ranks,
                        quant=w.quant)
    c_in = d["out"] if w.quant == "none" else inp["combine_input"]
    y, y_w = oracle.combine(c_in, d["out_weights"], d["slot_of"], inp["x"].shape[0], w.topk)
    return [d["recv_count"], d["slot_of"], d["src_token_pos"], d["out"], d["out_weights"],
            d["out_indices"], d["out_scales"], y, y_w]


@pytest.mark.parametrize("name,tokens", [("deepseek_v3_bf16", 300), ("deepseek_v3_fp8", 200),
                                         ("qwen3_moe_mxfp4", 500), ("tiny_bf16", None)])
def test_openmp_build_matches_plain(name, tokens):
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w, tokens=tokens, with_combine_input=w.quant != "none")
    plain = _run(w, inp)
    try:
        threads = oracle.use_openmp(True)
        assert threads >= 1
        par = _run(w, inp)
    finally:
        assert oracle.use_openmp(False) == 1
    for i, (a, b) in enumerate(zip(plain, par)):
        if a is None:
            assert b is None
            continue
        np.testing.assert_array_equal(np.ascontiguousarray(a).view(np.uint8),
                                      np.ascontiguousarray(b).view(np.uint8),
                                      err_msg=f"output {i}")
