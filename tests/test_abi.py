"""CPU checks of the C-ABI boundary: the library loads, exports every entry
point include/epdc.h declares, and its host-only calls (sizes, config
validation, argument checks) behave as documented.  No GPU work is launched.
"""
import ctypes
import os
import re

import pytest

from combine_routing_histogram_amd import binding as B
from combine_routing_histogram_amd import build as hip_build
from combine_routing_histogram_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if hip_build.is_stale():
        hip_build.build()
    return B.lib()


def test_exports_every_declared_entry_point(lib):
    names = B.header_entry_points()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/epdc.h but not exported"
    assert set(names) == set(B._SIGNATURES), "binding and header disagree"


def test_enum_values_match_header():
    text = open(B.HEADER).read()
    for name, val in re.findall(r"\b(EPDC_[A-Z0-9_]+)\s*=\s*(-?\d+)", text):
        assert getattr(B, name) == int(val), name


def _cfg(w, **kw):
    q = {"none": 0, "fp8_e4m3_b128": 1, "mxfp4_b32": 2}[w.quant]
    args = dict(max_tokens=w.tokens, hidden=w.hidden, topk=w.topk, num_experts=w.experts,
                num_ranks=w.ranks, quant=q)
    if w.raw_row_bytes:
        args.update(input_kind=B.EPDC_IN_RAW, raw_row_bytes=w.raw_row_bytes,
                    scale_row_bytes=w.scale_row_bytes)
    args.update(kw)
    return B.make_config(**args)


@pytest.mark.parametrize("name", sorted(wl.WORKLOADS))
def test_workspace_and_row_bytes(lib, name):
    w = wl.WORKLOADS[name]
    c = _cfg(w)
    n = B.epdc_workspace_bytes(c)
    N = w.tokens * w.topk
    # control words + tile table + 3 per-pair int arrays + offsets, 256-aligned
    assert n >= 4 * 3 * N + 4 * (w.experts + 1)
    assert n % 256 == 0
    p, s = B.epdc_row_bytes(c)
    want = {"none": (2 * w.hidden, 0), "fp8_e4m3_b128": (w.hidden, 4 * w.hidden // 128),
            "mxfp4_b32": (w.hidden // 2, w.hidden // 32)}[w.quant]
    if w.raw_row_bytes:
        want = (w.raw_row_bytes, w.scale_row_bytes)
    assert (p, s) == want


def test_raw_carry_row_bytes(lib):
    c = B.make_config(64, 7168, 8, 256, 8, input_kind=B.EPDC_IN_RAW, raw_row_bytes=7168,
                      scale_row_bytes=224)
    assert B.epdc_row_bytes(c) == (7168, 224)


@pytest.mark.parametrize("kw,msg", [
    (dict(hidden=100), "hidden"),
    (dict(topk=0), "topk"),
    (dict(topk=17), "topk"),
    (dict(num_experts=513), "num_experts"),
    (dict(num_ranks=3), "num_ranks"),
    (dict(max_tokens=-1), "max_tokens"),
    (dict(quant=1, hidden=64), "128"),
    (dict(quant=2, hidden=48), "32"),
    (dict(quant=7), "quant"),
    (dict(input_kind=1, raw_row_bytes=10), "raw_row_bytes"),
    (dict(input_kind=1, quant=1, raw_row_bytes=16), "bf16"),
    (dict(scale_row_bytes=6), "scale_row_bytes"),
    (dict(quant=1, scale_row_bytes=8), "scale_row_bytes"),
    (dict(max_tokens=1 << 28, topk=8), "2^30"),
    (dict(hidden=(1 << 24) + 8), "2^24"),
    (dict(input_kind=1, raw_row_bytes=(1 << 25) + 16), "2^25"),
])
def test_invalid_configs_rejected(lib, kw, msg):
    args = dict(max_tokens=128, hidden=256, topk=2, num_experts=8, num_ranks=2)
    args.update(kw)
    with pytest.raises(B.EpdcError) as ei:
        B.epdc_workspace_bytes(B.make_config(**args))
    assert ei.value.status == B.EPDC_ERR_INVALID_ARGS
    assert msg in str(ei.value)


def test_null_op_and_state_errors(lib):
    with pytest.raises(B.EpdcError) as ei:
        B.epdc_dispatch(0, 0, 1, 1, 0, 0, 1, 1, 0, 0, 0, 1)
    assert ei.value.status == B.EPDC_ERR_INVALID_ARGS
    with pytest.raises(B.EpdcError) as ei:
        B.epdc_combine(0, 0, 1, 0, 0, 1, 0)
    assert ei.value.status == B.EPDC_ERR_INVALID_ARGS
    with pytest.raises(B.EpdcError):
        B.epdc_reset(0)
    assert lib.epdc_destroy(None) == B.EPDC_SUCCESS
    assert B.epdc_last_error() == ""


def test_kernel_names(lib):
    names = [B.epdc_kernel_name(k) for k in range(B.EPDC_NUM_KERNELS)]
    assert names == ["k_route_rank", "k_route_scan", "k_scatter_copy", "k_scatter_fp8",
                     "k_scatter_mxfp4", "k_combine", "k_units_to_experts",
                     "k_experts_to_units", "k_combine_units", "k_combine_push",
                     "k_combine_reduce", "k_check_indices"]
    assert B.epdc_kernel_name(B.EPDC_NUM_KERNELS) is None


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libepdc.so"))
    with pytest.raises(RuntimeError, match="not built"):
        B.lib()


def test_product_code_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "combine_routing_histogram_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle|liboracle|epdc_oracle", text,
                                     flags=re.M), f
    hdr = open(os.path.join(ROOT, "include", "epdc.h")).read()
    assert "oracle" not in hdr


def test_every_entry_point_rejects_a_null_op(lib):
    calls = [
        lambda: B.epdc_dispatch_replay(0, 0, 1, 0, 0, 1, 0, 0),
        lambda: B.epdc_dispatch_send(0, 0, 1, 1, 0, 0, 1, 1, 0, 0, 0, 1),
        lambda: B.epdc_dispatch_recv(0, 0),
        lambda: B.epdc_combine_send(0, 0, 1, 0, 0, 1, 0),
        lambda: B.epdc_combine_recv(0, 0),
        lambda: B.epdc_combine_scatter(0, 0, 1, 0, 0, 1, 1, 0),
        lambda: B.epdc_dispatch_dedup(0, 0, 1, 1, 0, 0, 1, 1, 0, 0, 0, 1),
        lambda: B.epdc_get_unit_routing(0),
        lambda: B.epdc_units_to_experts(0, 0, 1, 0, 0, 0, 1, 0, 0, 0),
        lambda: B.epdc_experts_to_units(0, 0, 1, 0, 1),
        lambda: B.epdc_combine_units(0, 0, 1, 0, 1, 0),
        lambda: B.epdc_get_routing(0),
        lambda: B.epdc_get_offsets(0),
        lambda: B.epdc_set_debug(0, 1),
        lambda: B.epdc_set_combine_hint(0, 1),
        lambda: B.epdc_get_dispatch_src_token_pos(0),
    ]
    for call in calls:
        with pytest.raises(B.EpdcError) as ei:
            call()
        assert ei.value.status == B.EPDC_ERR_INVALID_ARGS


def test_header_is_plain_c(tmp_path):
    """include/epdc.h compiles as C99 with warnings as errors, and every
    declared entry point can be named from C."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    names = B.header_entry_points()
    src = tmp_path / "use_header.c"
    src.write_text('#include "epdc.h"\n'
                   + "typedef void (*any_fn)(void);\n"
                   + "".join(f"any_fn p_{n} = (any_fn)&{n};\n" for n in names)
                   + "int main(void) { return 0; }\n")
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only",
                    "-I", os.path.join(ROOT, "include"), str(src)], check=True)


def test_static_create_rejects_configs_beyond_its_workspace(lib):
    """epdc_create_static checks the workspace a config needs against the
    library's static array before it touches any device."""
    big = B.make_config(1 << 17, 7168, 8, 256, 8)      # 1M pairs: about 26 MiB
    assert B.epdc_workspace_bytes(big) > B.EPDC_STATIC_WORKSPACE_BYTES
    with pytest.raises(B.EpdcError) as ei:
        B.epdc_create_static(big)
    assert ei.value.status == B.EPDC_ERR_INVALID_ARGS
    assert "static workspace" in str(ei.value)
    with pytest.raises(B.EpdcError) as ei:
        B.epdc_create_static(B.make_config(128, 100, 2, 8, 2))   # invalid config first
    assert ei.value.status == B.EPDC_ERR_INVALID_ARGS
    # every configuration the benchmarks use fits the static workspace
    for name, w in wl.WORKLOADS.items():
        assert B.epdc_workspace_bytes(_cfg(w)) <= B.EPDC_STATIC_WORKSPACE_BYTES, name


def test_unit_conversion_rejects_undersized_tensors():
    """units_to_experts checks rows, widths and dtypes of caller tensors on the
    host: the kernel reads up to T * min(K, R) rows of each."""
    import torch

    from combine_routing_histogram_amd.op import EpDispatchCombineConfig, EpDispatchCombineOp

    op = EpDispatchCombineOp.__new__(EpDispatchCombineOp)   # host state only, no device
    op.config = EpDispatchCombineConfig(16, 256, 4, 8, 2)
    op.device = torch.device("cpu")
    op._dev_index = -1
    op._tokens = 10
    op.payload_row_bytes, op.scale_row_bytes = 512, 0
    rows = 10 * 2                                            # T * min(K, R)
    good = dict(input=torch.zeros(rows, 256, dtype=torch.bfloat16),
                weights=torch.zeros(rows, 4), scales=None,
                indices=torch.zeros(rows, 4, dtype=torch.int32))
    op._check_unit_rows(**good)
    bad = [dict(good, input=torch.zeros(rows - 1, 256, dtype=torch.bfloat16)),
           dict(good, input=torch.zeros(rows, 128, dtype=torch.bfloat16)),
           dict(good, weights=torch.zeros(rows - 1, 4)),
           dict(good, weights=torch.zeros(rows, 4, dtype=torch.float64)),
           dict(good, indices=torch.zeros(rows, 3, dtype=torch.int32)),
           dict(good, indices=torch.zeros(rows, 4, dtype=torch.int64))]
    for kw in bad:
        with pytest.raises(ValueError):
            op._check_unit_rows(**kw)


def test_kernel_type_enum_and_config_checks():
    """The pages' kernel-type enum imports with its values; only the
    intra-node type exists on one GPU, and the config says so on creation."""
    from combine_routing_histogram_amd.op import (EpDispatchCombineConfig,
                                                  EpDispatchCombineKernelType)
    assert [(k.name, int(k)) for k in EpDispatchCombineKernelType] == [
        ("IntraNode", 0), ("InterNode", 1), ("InterNodeV1", 2), ("InterNodeV1LL", 3),
        ("AsyncLL", 4)]
    cfg = EpDispatchCombineConfig(16, 256, 2, 8, 2)
    assert cfg.kernel_type == EpDispatchCombineKernelType.IntraNode
    for kt in (1, 2, 3, 4):
        with pytest.raises(ValueError, match="IntraNode"):
            EpDispatchCombineConfig(16, 256, 2, 8, 2, kernel_type=kt)
    with pytest.raises(ValueError):
        EpDispatchCombineConfig(16, 256, 2, 8, 2, kernel_type=7)
    with pytest.raises(ValueError, match="quant"):
        EpDispatchCombineConfig(16, 256, 2, 8, 2, quant="fp8")
