"""Pins for the oracle's gather combine and the whole dispatch -> combine loop.

Combine is a weighted top-k sum accumulated in fp32 and rounded to bf16
(MORI "Choosing an EP API and backend" page, "EP paths" table: gather combine
in BF16/FP32; "Communication APIs" page, MORI-EP methods table: combine
returns (output, weights)).  Pins: an fp64 evaluation of the same sum within
the bf16 tolerance, exact special cases (K = 1 with unit weight is the inverse
permutation; one-hot weights are an exact gather), the identity-expert
invariant combine(dispatch(x)) = x * sum_k w (the benchmark check named under
"Validation before tuning" on the first page), and the returned weights.
"""
import numpy as np
import pytest

from combine_routing_histogram_amd import workloads as wl
from oracle import oracle


def bf16_ulp(a):
    """Spacing of bf16 at |a| (normal range)."""
    a = np.maximum(np.abs(a), np.float64(2.0) ** -126)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(np.int64) - 7)


def assert_within_tolerance(got_bits, exact, abs_sum):
    """|got - exact| <= max(1 bf16 ulp of |exact|, 8e-3 |exact|, 2^-20 sum|w x|)."""
    got = wl.bf16_bits_to_f32(got_bits).astype(np.float64)
    tol = np.maximum(np.maximum(bf16_ulp(exact), 8e-3 * np.abs(exact)), 2.0 ** -20 * abs_sum)
    err = np.abs(got - exact)
    bad = err > tol
    assert not bad.any(), f"{bad.sum()} elements out of tolerance; worst {err.max()}"


def fp64_combine(inp_bits, weights, slot_of, T, K):
    x = wl.bf16_bits_to_f32(inp_bits).astype(np.float64)
    H = x.shape[1]
    so = slot_of.reshape(T, K)
    y = np.zeros((T, H))
    s_abs = np.zeros((T, H))
    for k in range(K):
        s = so[:, k]
        ok = s >= 0
        w = np.zeros(T)
        if weights is None:
            w[ok] = 1.0
        else:
            w[ok] = weights[s[ok], k]
        rows = np.where(ok[:, None], x[np.maximum(s, 0)], 0.0)
        y += w[:, None] * rows
        s_abs += np.abs(w[:, None] * rows)
    return y, s_abs


@pytest.mark.parametrize("name,tokens", [("tiny_bf16", None), ("deepseek_v3_bf16", 48),
                                         ("qwen3_moe_mxfp4", 40)])
def test_combine_vs_fp64(name, tokens):
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w, tokens=tokens, with_combine_input=True)
    T = inp["x"].shape[0]
    d = oracle.dispatch(inp["x"], inp["weights"], inp["indices"], w.experts, w.ranks)
    c_in = inp["combine_input"]
    y, y_w = oracle.combine(c_in, d["out_weights"], d["slot_of"], T, w.topk)
    exact, s_abs = fp64_combine(c_in, d["out_weights"], d["slot_of"], T, w.topk)
    assert_within_tolerance(y, exact, s_abs)
    np.testing.assert_array_equal(y_w, inp["weights"])      # bit-exact weights back


def test_identity_expert_invariant():
    w = wl.WORKLOADS["deepseek_v3_bf16"]
    inp = wl.make_inputs(w, tokens=64)
    T = 64
    d = oracle.dispatch(inp["x"], inp["weights"], inp["indices"], w.experts, w.ranks)
    y, y_w = oracle.combine(d["out"], d["out_weights"], d["slot_of"], T, w.topk)
    x = wl.bf16_bits_to_f32(inp["x"]).astype(np.float64)
    wsum = inp["weights"].astype(np.float64).sum(axis=1, keepdims=True)
    exact = x * wsum
    s_abs = np.abs(x) * wsum
    assert_within_tolerance(y, exact, s_abs)
    np.testing.assert_array_equal(y_w, inp["weights"])


def test_k1_unit_weight_is_inverse_permutation():
    rng = np.random.default_rng(11)
    T, H, E, R = 50, 64, 8, 2
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    idx = rng.integers(0, E, (T, 1)).astype(np.int32)
    ones = np.ones((T, 1), np.float32)
    d = oracle.dispatch(x, ones, idx, E, R)
    y, _ = oracle.combine(d["out"], d["out_weights"], d["slot_of"], T, 1)
    np.testing.assert_array_equal(y, x)
    y2, _ = oracle.combine(d["out"], None, d["slot_of"], T, 1)
    np.testing.assert_array_equal(y2, x)


def test_one_hot_weights_are_exact_gather():
    rng = np.random.default_rng(12)
    T, H, K, E, R = 30, 96, 4, 16, 4
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    r = oracle.route(idx, E, R)
    N = T * K
    c_in = wl.f32_to_bf16_bits(rng.standard_normal((N, H)).astype(np.float32) + 3.0)
    hot = rng.integers(0, K, T)
    wts = np.zeros((N, K), np.float32)
    so = r["slot_of"].reshape(T, K)
    for t in range(T):
        for k in range(K):
            wts[so[t, k], k] = 1.0 if k == hot[t] else 0.0
    y, y_w = oracle.combine(c_in, wts, r["slot_of"], T, K)
    want = c_in[so[np.arange(T), hot]]
    np.testing.assert_array_equal(wl.bf16_bits_to_f32(y), wl.bf16_bits_to_f32(want))
    np.testing.assert_array_equal(y_w, np.eye(K, dtype=np.float32)[hot])


def test_unweighted_sum_and_invalid_pairs():
    rng = np.random.default_rng(13)
    T, H, K, E, R = 20, 32, 3, 8, 2
    idx = rng.integers(0, E, (T, K)).astype(np.int32)
    idx[4, 1] = -5
    idx[9, 2] = E
    r = oracle.route(idx, E, R)
    c_in = wl.f32_to_bf16_bits(rng.standard_normal((T * K, H)).astype(np.float32))
    y, y_w = oracle.combine(c_in, None, r["slot_of"], T, K)
    exact, s_abs = fp64_combine(c_in, None, r["slot_of"], T, K)
    assert_within_tolerance(y, exact, s_abs)
    assert y_w[4, 1] == 0 and y_w[9, 2] == 0 and y_w[0, 0] == 1


def test_tolerance_catches_a_dropped_term():
    """The tolerance is tight enough to see a missing k term."""
    w = wl.WORKLOADS["tiny_bf16"]
    inp = wl.make_inputs(w, with_combine_input=True)
    d = oracle.dispatch(inp["x"], inp["weights"], inp["indices"], w.experts, w.ranks)
    so = d["slot_of"].copy().reshape(-1, w.topk)
    so_drop = so.copy()
    so_drop[:, 1] = -1
    y_bad, _ = oracle.combine(inp["combine_input"], d["out_weights"], so_drop.ravel(),
                              w.tokens, w.topk)
    exact, s_abs = fp64_combine(inp["combine_input"], d["out_weights"], so.ravel(),
                                w.tokens, w.topk)
    with pytest.raises(AssertionError):
        assert_within_tolerance(y_bad, exact, s_abs)


def test_dispatch_carries_rows():
    w = wl.WORKLOADS["tiny_bf16"]
    inp = wl.make_inputs(w)
    rng = np.random.default_rng(5)
    sc = rng.standard_normal((w.tokens, 4)).astype(np.float32)
    d = oracle.dispatch(inp["x"], inp["weights"], inp["indices"], w.experts, w.ranks, scales=sc)
    tok = d["src_token_pos"] // w.topk
    np.testing.assert_array_equal(d["out"], inp["x"][tok])
    np.testing.assert_array_equal(d["out_weights"], inp["weights"][tok])
    np.testing.assert_array_equal(d["out_indices"], inp["indices"][tok])
    np.testing.assert_array_equal(d["out_scales"], sc[tok])


def test_push_combine_is_the_gather_combine():
    """Scatter combine (push weighted rows to per-pair staging rows, then add
    them in k order) forms the same fp32 products and adds them in the same
    order as the gather combine, so the two agree bit for bit; the staging
    rows hold w * x exactly."""
    rng = np.random.default_rng(31)
    T, H, K, E, R = 150, 96, 6, 24, 4
    idx = wl.draw_topk(rng, T, E, K, "zipf", 1.2)
    idx[4, 1], idx[9, 5] = -1, E          # pairs without a row
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wts = wl.softmax_weights(rng, T, K)
    d = oracle.dispatch(x, wts, idx, E, R)
    c_in = wl.f32_to_bf16_bits(rng.standard_normal((d["n_valid"], H)).astype(np.float32))
    for w in (d["out_weights"], None):
        y1, yw1 = oracle.combine(c_in, w, d["slot_of"], T, K)
        y2, yw2, st = oracle.combine_push(c_in, w, d["src_token_pos"], d["slot_of"], T, K)
        np.testing.assert_array_equal(y2, y1)
        np.testing.assert_array_equal(yw2.view(np.uint32), yw1.view(np.uint32))
        # staging row of pair p = its weight times its received row, in fp32
        xin = wl.bf16_bits_to_f32(c_in)
        for p in (0, 7, 100, T * K - 1):
            s = d["slot_of"][p]
            if s < 0:
                assert not st[p].any()
                continue
            wk = np.float32(1.0) if w is None else w[s, p % K]
            np.testing.assert_array_equal(st[p], (wk * xin[s]).astype(np.float32))
