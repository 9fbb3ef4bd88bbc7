"""The oracle's pins catch plausible mistakes in the oracle (CPU only).

Each mutant below is a copy of ``oracle/epdc_oracle.c`` with one planted
mistake of the kind a reader could make when writing the oracle from the
pages: an off-by-one or a wrong index, a rounding rule taken the wrong way
(ties away from zero, truncation), a dropped term, a wrong constant, a
swapped nibble order.  The copy is built with the oracle's own gcc flags and
the committed pin tests (``tests/test_oracle_*.py``) run against it in a
child process; every mutant must make at least one pin fail, and the
unmodified source must pass them all.  Every mutant stays in bounds (no
index it produces can leave its buffer), so a failure is a wrong value, never
a crash.

Mistakes the pins cannot see by design are not listed: the order of the
fp32 additions of a combine and a fused multiply-add both stay inside the
combine tolerance, and the GPU parity tests compare those bit for bit.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from oracle import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_TESTS = ["tests/test_oracle_route.py", "tests/test_oracle_quant.py",
             "tests/test_oracle_combine.py", "tests/test_oracle_dedup.py"]

# name -> (text in the oracle, replacement, replace every occurrence)
MUTANTS = {
    # routing: scan, offsets, order, source positions
    "rank_off_indexed_by_rank": (
        "rank_off[r] = expert_off[r * per_rank];", "rank_off[r] = expert_off[r];", False),
    "recv_count_is_expert_count": (
        "recv_count[r] = rank_off[r + 1] - rank_off[r];", "recv_count[r] = cnt[r];", False),
    "slots_in_descending_pair_order": (
        "    for (long p = 0; p < n; ++p) {\n        int32_t e = indices[p];\n"
        "        if (e < 0 || e >= E) {\n            slot_of[p] = -1;",
        "    for (long p = n - 1; p >= 0; --p) {\n        int32_t e = indices[p];\n"
        "        if (e < 0 || e >= E) {\n            slot_of[p] = -1;", False),
    "src_token_pos_is_token": (
        "src_token_pos[s] = (int32_t)p;", "src_token_pos[s] = (int32_t)(p / K);", False),
    # row copies
    "copy_reads_wrong_token_row": (
        "memcpy(dst + (long)s * row_bytes, src + (long)t * row_bytes,",
        "memcpy(dst + (long)s * row_bytes, src + (long)(T - 1 - t) * row_bytes,", False),
    # FP8 E4M3
    "fp8_max_240": ("s = amax / 448.0f;", "s = amax / 240.0f;", False),
    "fp8_multiplies_by_reciprocal": (
        "float y = bf16_to_f32(xb[i]) / s;", "float y = bf16_to_f32(xb[i]) * (1.0f / s);", False),
    "fp8_stores_amax_as_scale": (
        "scales[(long)t * (H / B) + j] = s;", "scales[(long)t * (H / B) + j] = amax;", False),
    "e4m3_ties_away": (
        "double r = nearbyint(a / q) * q;             /* default mode: ties-to-even */",
        "double r = round(a / q) * q;", False),
    "e4m3_no_saturation": ("    if (r > 448.0)\n        r = 448.0;\n", "", False),
    "e4m3_drops_sign_of_zero": ("    if (r == 0.0)\n        return sign;",
                                "    if (r == 0.0)\n        return 0;", False),
    # MXFP4
    "mxfp4_emax_1": ("e = (ex - 1) - 2;", "e = (ex - 1) - 1;", False),
    "mxfp4_scale_sign": (
        "uint8_t lo = oracle_e2m1_encode(ldexp((double)bf16_to_f32(xb[i]), -e));",
        "uint8_t lo = oracle_e2m1_encode(ldexp((double)bf16_to_f32(xb[i]), e));", False),
    "mxfp4_nibbles_swapped": ("qb[i / 2] = (uint8_t)(lo | (hi << 4));",
                              "qb[i / 2] = (uint8_t)(hi | (lo << 4));", False),
    "e2m1_ties_away": ("    double r = nearbyint(a / q) * q;\n    if (r > 6.0)",
                       "    double r = round(a / q) * q;\n    if (r > 6.0)", False),
    "e2m1_no_saturation": ("    if (r > 6.0)\n        r = 6.0;\n", "", False),
    # bf16 rounding
    "bf16_ties_away": ("    return (lo & 1u) ? hi : lo;\n}", "    return hi;\n}", False),
    # gather combine
    "combine_weight_column_0": (
        "w[k] = (s < 0) ? 0.0f : (weights ? weights[(long)s * K + k] : 1.0f);",
        "w[k] = (s < 0) ? 0.0f : (weights ? weights[(long)s * K] : 1.0f);", False),
    "combine_drops_last_term": (
        "            for (int k = 0; k < K; ++k) {\n"
        "                int32_t s = slot_of[(long)t * K + k];\n"
        "                if (s < 0)\n                    continue;\n                float prod",
        "            for (int k = 0; k < K - 1; ++k) {\n"
        "                int32_t s = slot_of[(long)t * K + k];\n"
        "                if (s < 0)\n                    continue;\n                float prod", False),
    "combine_truncates_to_bf16": (
        "                acc = acc + prod;\n            }\n"
        "            out[(long)t * H + h] = f32_to_bf16_rne(acc);",
        "                acc = acc + prod;\n            }\n"
        "            { uint32_t u_; memcpy(&u_, &acc, 4); out[(long)t * H + h] = (uint16_t)(u_ >> 16); }",
        False),
    # scatter (push) combine
    "push_weight_column_0": (
        "int k = (int)(p % K);\n        float w = weights ? weights[(long)s * K + k] : 1.0f;",
        "int k = (int)(p % K);\n        float w = weights ? weights[(long)s * K] : 1.0f;", False),
    # rank-deduplicated dispatch and the standard-MoE conversion
    "units_round_robin_ranks": ("int r = e / per_rank;", "int r = e % R;", True),
    "experts_to_units_weight_column_0": (
        "continue;\n                float w = weights ? weights[(long)s * K + k] : 1.0f;",
        "continue;\n                float w = weights ? weights[(long)s * K] : 1.0f;", False),
    "combine_units_adds_a_unit_twice": (
        "            if (seen)\n                continue;\n", "", False),
    "combine_units_weight_column_0": (
        "unit_weights[(long)u * K + k]", "unit_weights[(long)u * K]", False),
    "units_placed_in_descending_token_order": (
        "    for (int t = 0; t < T; ++t) {\n        for (int r = 0; r < R; ++r)\n"
        "            open[r] = -1;",
        "    for (int t = T - 1; t >= 0; --t) {\n        for (int r = 0; r < R; ++r)\n"
        "            open[r] = -1;", False),
    "units_to_experts_skips_pair_0": (
        "for (long p = 0; p < n_pairs; ++p) {\n        if (slot_of[p] < 0 || unit_of[p] < 0)",
        "for (long p = 1; p < n_pairs; ++p) {\n        if (slot_of[p] < 0 || unit_of[p] < 0)",
        False),
    # more routing, quantization and format mistakes
    "rank_off_end_short_by_last_expert": (
        "rank_off[R] = expert_off[E];", "rank_off[R] = expert_off[E - 1];", False),
    "fp8_amax_without_abs": (
        "float a = fabsf(bf16_to_f32(xb[i]));\n                if (a > amax)\n"
        "                    amax = a;\n            }\n            float s = 0.0f;",
        "float a = bf16_to_f32(xb[i]);\n                if (a > amax)\n"
        "                    amax = a;\n            }\n            float s = 0.0f;", False),
    "mxfp4_amax_without_abs": (
        "float a = fabsf(bf16_to_f32(xb[i]));\n                if (a > amax)\n"
        "                    amax = a;\n            }\n            int e;",
        "float a = bf16_to_f32(xb[i]);\n                if (a > amax)\n"
        "                    amax = a;\n            }\n            int e;", False),
    "e8m0_bias_128": ("(uint8_t)(e + 127)", "(uint8_t)(e + 128)", False),
    "mxfp4_zero_block_exponent_0": ("if (amax == 0.0f) {\n                e = -127;",
                                    "if (amax == 0.0f) {\n                e = 0;", False),
    "e4m3_bias_8_as_in_fnuz": ("int e_field = (ex - 1) + 7;", "int e_field = (ex - 1) + 8;",
                               False),
    "e4m3_subnormal_spacing_halved": (
        "q = ldexp(1.0, -9);                      /* subnormal spacing */",
        "q = ldexp(1.0, -10);                     /* subnormal spacing */", False),
    "e2m1_top_binade_spacing_1": ("(a < 4.0 ? 1.0 : 2.0)", "(a < 4.0 ? 1.0 : 1.0)", False),
}


def _mutate(src: str, name: str) -> str:
    old, new, every = MUTANTS[name]
    n = src.count(old)
    assert n >= 1, f"mutant {name}: its text is no longer in the oracle"
    assert every or n == 1, f"mutant {name}: its text occurs {n} times"
    return src.replace(old, new)


def _run_pins(src_text: str, workdir: str, tag: str) -> subprocess.CompletedProcess:
    c_path = os.path.join(workdir, f"{tag}.c")
    so_path = os.path.join(workdir, f"{tag}.so")
    with open(c_path, "w") as f:
        f.write(src_text)
    cmd = [a for a in oracle.GCC_CMD if a != oracle._SRC] + [c_path, "-o", so_path, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True)
    env = dict(os.environ, EPDC_ORACLE_LIB=so_path)
    return subprocess.run(
        [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
         *PIN_TESTS], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def test_every_mutant_fails_a_pin(tmp_path):
    src = open(oracle._SRC).read()
    jobs = {"unmodified": src}
    jobs.update({name: _mutate(src, name) for name in MUTANTS})
    with ThreadPoolExecutor(max_workers=4) as pool:
        res = dict(zip(jobs, pool.map(lambda kv: _run_pins(kv[1], str(tmp_path), kv[0]),
                                      jobs.items())))
    ctl = res.pop("unmodified")
    assert ctl.returncode == 0, f"the pins fail on the unmodified oracle:\n{ctl.stdout[-2000:]}"
    # exit status 1: tests ran and at least one failed (not a crash or a usage error)
    survivors = [n for n, r in res.items() if r.returncode != 1]
    detail = {n: (res[n].returncode, res[n].stdout[-300:]) for n in survivors}
    assert not survivors, f"mutants no pin catches: {detail}"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_text_present_once(name):
    """Each planted mistake still applies to the current oracle source."""
    _mutate(open(oracle._SRC).read(), name)
