"""bench.py end to end on the GPU with few steps: the one JSON line carries
the measured fields, every timed step of every workload is bit-exact against
the oracle, and the other paths and graph mode run and check parity too."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args, timeout=300):
    print("bench.py " + " ".join(args), flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=timeout, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


def test_default_line():
    d = run_bench("--steps", "4", "--warmup", "1", "--warm-steps", "3", "--clean-steps", "3",
                  "--kernel-steps", "3", "--extra-steps", "3", "--cpu-reps", "1", "--layers", "2")
    assert d["metric"].startswith("dispatch+combine tokens/s and achieved HBM GB/s")
    assert d["unit"] == "tokens/s" and d["value"] > 0 and d["ms_per_step"] > 0
    assert d["n_gpus"] == 1 and d["higher_is_better"] is True and d["dtype"] == "bf16"
    assert d["config"]["workload"] == "deepseek_v3_bf16" and "512 MiB" in d["config"]["protocol"]
    assert d["config"]["gpu_arch"].startswith("gfx950")
    assert d["parity"] == "bit-exact on all 4 timed steps"
    assert d["warm"]["parity"].startswith("bit-exact") and d["clean_flush"]["parity"].startswith(
        "bit-exact")
    assert d["layers"]["layers"] == 2 and d["layers"]["parity"] == (
        "bit-exact on the last step of each of 2 layers")
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["peak"] == 8000.0 and roof["unit"] == "GB/s"
    assert 0 < roof["frac"] < 1 and abs(roof["achieved"] / roof["peak"] - roof["frac"]) < 1e-9
    vs = roof["vs_measured_hbm"]
    assert vs["bound_us"] > 0 and vs["frac_mix_headline"] > roof["frac"]
    assert set(d["kernels"]) >= {"k_route_rank", "k_scatter_copy", "k_combine"}
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["openmp_result_identical"]
    assert [leg["cores"] for leg in cpu["legs"]][0] == 1
    assert set(d["workloads"]) == {"deepseek_v3_fp8", "qwen3_moe_mxfp4", "decode_bf16",
                                   "deepseek_v3_raw_fp8"}
    ce = d["ceilings"]
    assert min(ce["read_gbps"], ce["write_gbps"], ce["copy_gbps"]) > 1000
    assert max(ce["read_gbps"], ce["write_gbps"], ce["copy_gbps"]) < 8000
    assert set(ce["kernels"]) >= {"k_scatter_copy", "k_combine"}
    for k, v in ce["kernels"].items():
        assert v["bound_us"] > 0 and v["frac_headline"] > 0 and v["frac_warm"] > 0, k
        assert v["mix_bound_us"] > 0 and v["frac_mix_headline"] > 0, k
    for name, r in d["workloads"].items():
        assert r["parity"] == "bit-exact on all 3 timed steps", name
        assert r["ms_per_step"] > 0 and r["kernels"], name
        assert r["ceilings"]["k_combine"]["bound_us"] > 0, name
        assert r["clean_flush"]["parity"] == "bit-exact on all 3 timed steps", name
        assert r["warm"]["parity"].startswith("bit-exact"), name


@pytest.mark.parametrize("args", [("--path", "dedup"), ("--combine", "scatter"),
                                  ("--workload", "decode_bf16", "--graph")])
def test_other_paths(args):
    d = run_bench(*args, "--steps", "3", "--warmup", "1", "--warm-steps", "2", "--clean-steps",
                  "0", "--kernel-steps", "2", "--cpu-reps", "0", "--device-copy", "0")
    assert d["parity"] == "bit-exact on all 3 timed steps"
    assert d["warm"]["parity"].startswith("bit-exact")
    assert d["value"] > 0
