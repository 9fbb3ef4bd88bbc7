"""Write input_fingerprints.json: SHA-256 of the seeded inputs of each
workload (whole for the small ones, a 64-token draw of the large ones), so a
change to the input recipe, or to numpy's generators, shows up as a test
failure instead of silently changing what the benchmarks measure.

    python tests/golden/make_input_fingerprints.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
from combine_routing_histogram_amd import workloads as wl  # noqa: E402

SMALL = 1 << 20   # workloads with fewer input elements than this are drawn whole


def cases():
    for name in sorted(wl.WORKLOADS):
        w = wl.WORKLOADS[name]
        whole = w.tokens * max(w.hidden, w.raw_row_bytes) < SMALL
        yield name, None if whole else 64


def main():
    out = {}
    for name, tokens in cases():
        inp = wl.make_inputs(wl.WORKLOADS[name], tokens=tokens, with_combine_input=True)
        out[name] = {"tokens": tokens, "arrays": wl.fingerprint(inp)}
    with open(os.path.join(HERE, "input_fingerprints.json"), "w") as fh:
        json.dump(out, fh, indent=1, sort_keys=True)
        fh.write("\n")


if __name__ == "__main__":
    main()
