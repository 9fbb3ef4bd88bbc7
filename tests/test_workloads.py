"""The seeded input recipe: reproducible draws, and the .npy save/load path.

input_fingerprints.json is written by tests/golden/make_input_fingerprints.py
(which calls only the input generators); a change to the recipe or to numpy's
generators changes what every benchmark and parity test runs on, so it must
show up here first.
"""
import json
import os

import numpy as np
import pytest

from combine_routing_histogram_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "input_fingerprints.json")


def golden():
    with open(GOLDEN) as fh:
        return json.load(fh)


@pytest.mark.parametrize("name", sorted(wl.WORKLOADS))
def test_inputs_match_recorded_fingerprints(name):
    rec = golden()[name]
    inp = wl.make_inputs(wl.WORKLOADS[name], tokens=rec["tokens"], with_combine_input=True)
    assert wl.fingerprint(inp) == rec["arrays"]


def test_every_workload_has_a_fingerprint():
    assert sorted(golden()) == sorted(wl.WORKLOADS)


def test_save_load_roundtrip(tmp_path):
    w = wl.WORKLOADS["tiny_bf16"]
    m = wl.save_inputs(w, str(tmp_path))
    assert m["tokens"] == w.tokens and m["workload"]["name"] == "tiny_bf16"
    got = wl.load_inputs(str(tmp_path))
    ref = wl.make_inputs(w)
    assert sorted(got) == sorted(ref)
    for k in ref:
        assert got[k].dtype == ref[k].dtype
        np.testing.assert_array_equal(got[k], ref[k])


def test_load_rejects_a_changed_array(tmp_path):
    wl.save_inputs(wl.WORKLOADS["tiny_bf16"], str(tmp_path))
    p = tmp_path / "indices.npy"
    a = np.load(p, allow_pickle=False)
    a[0, 0] ^= 1
    np.save(p, a, allow_pickle=False)
    with pytest.raises(ValueError, match="indices"):
        wl.load_inputs(str(tmp_path))


def test_cli_fingerprint(capsys):
    assert wl.main(["fingerprint", "tiny_bf16"]) == 0
    out = json.loads(capsys.readouterr().out)
    rec = golden()["tiny_bf16"]["arrays"]
    # the CLI draws what the workload uses: no combine input for identity experts
    assert sorted(out) == ["indices", "weights", "x"]
    assert all(out[k] == rec[k] for k in out)
