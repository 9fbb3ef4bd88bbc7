"""Randomized CPU check of the configuration rules of include/epdc.h: for
configurations drawn around every boundary, epdc_workspace_bytes accepts
exactly those the header's rules allow (a model of them written here from
the header's field comments), and for accepted ones the workspace size and
row sizes follow their definitions.  No GPU work."""
import pytest
from hypothesis import given, settings, strategies as st

from combine_routing_histogram_amd import binding as B
from combine_routing_histogram_amd import build as hip_build


@pytest.fixture(scope="module", autouse=True)
def lib():
    if hip_build.is_stale():
        hip_build.build()
    return B.lib()


def allowed(c) -> bool:
    """The rules the header states for epdc_config."""
    if c["max_tokens"] < 0:
        return False
    if not (0 < c["hidden"] <= 1 << 24 and c["hidden"] % 8 == 0):
        return False
    if not 1 <= c["topk"] <= 16 or not 1 <= c["num_experts"] <= 512:
        return False
    if c["num_ranks"] < 1 or c["num_experts"] % c["num_ranks"]:
        return False
    if c["max_tokens"] * c["topk"] > 1 << 30:
        return False
    if c["input_kind"] not in (0, 1) or c["quant"] not in (0, 1, 2):
        return False
    if c["scale_row_bytes"] < 0 or c["scale_row_bytes"] % 4:
        return False
    if c["quant"] == 1 and c["hidden"] % 128:
        return False
    if c["quant"] == 2 and c["hidden"] % 32:
        return False
    if c["quant"] and (c["input_kind"] != 0 or c["scale_row_bytes"] != 0):
        return False
    if c["input_kind"] == 1 and not (0 < c["raw_row_bytes"] <= 1 << 25
                                     and c["raw_row_bytes"] % 16 == 0):
        return False
    return True


def near(*values):
    """Integers at and around the given boundaries."""
    return st.sampled_from(sorted({v + d for v in values for d in (-1, 0, 1)}))


configs = st.fixed_dictionaries({
    "max_tokens": st.one_of(near(0, 4096, 1 << 26, 1 << 27), st.integers(0, 70000)),
    "hidden": st.one_of(near(8, 32, 128, 7168, 1 << 24), st.integers(-16, 9000)),
    "topk": near(1, 8, 16),
    "num_experts": st.one_of(near(1, 64, 256, 512), st.integers(1, 600)),
    "num_ranks": st.one_of(near(1, 8, 16), st.integers(1, 40)),
    "input_kind": near(0, 1),
    "quant": near(0, 1, 2),
    "raw_row_bytes": st.one_of(st.just(0), near(16, 7168, 1 << 25)),
    "scale_row_bytes": st.one_of(st.just(0), near(4, 224)),
})


@settings(max_examples=600, deadline=None)
@given(configs)
def test_config_rules(c):
    cfg = B.make_config(**c)
    ok = allowed(c)
    if not ok:
        with pytest.raises(B.EpdcError) as e:
            B.epdc_workspace_bytes(cfg)
        assert e.value.status == B.EPDC_ERR_INVALID_ARGS
        return
    n = B.epdc_workspace_bytes(cfg)
    pairs = c["max_tokens"] * c["topk"]
    assert n % 256 == 0 and n >= 4 * 3 * pairs + 4 * (c["num_experts"] + 1)
    p, s = B.epdc_row_bytes(cfg)
    H = c["hidden"]
    if c["quant"] == 1:
        assert (p, s) == (H, 4 * (H // 128))
    elif c["quant"] == 2:
        assert (p, s) == (H // 2, H // 32)
    elif c["input_kind"] == 1:
        assert (p, s) == (c["raw_row_bytes"], c["scale_row_bytes"])
    else:
        assert (p, s) == (2 * H, c["scale_row_bytes"])


@settings(max_examples=200, deadline=None)
@given(st.integers(0, 1 << 20), st.integers(0, 1 << 20), st.sampled_from([1, 2, 8, 16]),
       st.sampled_from([(8, 2), (64, 8), (256, 8), (512, 16)]))
def test_workspace_grows_with_max_tokens(t1, t2, k, er):
    e, r = er
    a = B.epdc_workspace_bytes(B.make_config(min(t1, t2), 256, k, e, r))
    b = B.epdc_workspace_bytes(B.make_config(max(t1, t2), 256, k, e, r))
    assert a <= b
