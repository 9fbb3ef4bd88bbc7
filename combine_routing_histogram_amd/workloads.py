"""Seeded synthetic inputs for MoE expert-parallel dispatch/combine.

This module only draws inputs: token rows, top-k expert choices, routing
weights and (for the quantized workloads) an independent expert output.  It
holds none of the dispatch/combine arithmetic, so both the CPU oracle and the
HIP path can be fed from it without sharing any of the method's code.

The shapes follow the workloads the MORI EP pages are written for (MORI
"Communication APIs" page, MORI-EP section: dispatch takes input, weights,
scales and indices; "Choosing an EP API and backend" page, the FP8/FP4
restrictions list): DeepSeek-V3-like (hidden 7168, 256 experts, top-8) and
Qwen3-MoE-like (hidden 4096, 128 experts, top-8) layers, plus a tiny case and
decode-sized cases.  No dataset or trained weights are involved.

Recipe (all numpy PCG64, one SeedSequence per workload spawned into six
independent streams: x, routing, logits, outliers, combine input, carried
scales):
  * x: N(0,1) float32 -> bfloat16 with round-to-nearest-even (torch CPU cast);
    for the Qwen-like case 1% of elements (Bernoulli mask) are multiplied by 20
    before the cast.
  * routing: K distinct experts per token, sampled without replacement by the
    Gumbel-top-k trick from either a uniform distribution or a Zipf(s) law
    p_j ~ (j+1)^-s over popularity ranks j, where rank j is expert perm[j] for a
    seeded permutation perm.  Row order = draw order.
  * weights: float32 softmax over K N(0,1) logits per token.
  * combine input (quantized and pre-quantized workloads): independent N(0,1)
    bfloat16 rows in the received layout [T*K, H].
  * pre-quantized rows (raw workloads, payloads quantized before dispatch and
    carried unchanged): uniform random bytes [T, raw_row_bytes] drawn from
    the x stream (dispatch treats them as opaque), and per-token fp32 scale
    rows |N(0,1)|/448 [T, scale_row_bytes/4].
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    tokens: int          # T
    hidden: int          # H
    topk: int            # K
    experts: int         # E
    ranks: int           # R virtual ranks, E/R experts each
    routing: str         # "uniform" or "zipf"
    zipf_s: float = 0.0
    quant: str = "none"  # "none", "fp8_e4m3_b128", "mxfp4_b32"
    outlier_frac: float = 0.0
    outlier_mult: float = 1.0
    combine_input: str = "identity"  # "identity" (dispatch output) or "independent"
    seed: int = 0
    raw_row_bytes: int = 0    # > 0: pre-quantized byte rows carried unchanged
    scale_row_bytes: int = 0  # bytes of the fp32 scale row carried with each raw row

    @property
    def pairs(self) -> int:
        return self.tokens * self.topk


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_bf16", 128, 256, 2, 8, 2, "uniform", seed=1001),
        Workload("deepseek_v3_bf16", 4096, 7168, 8, 256, 8, "zipf", zipf_s=1.1, seed=1002),
        Workload("deepseek_v3_fp8", 4096, 7168, 8, 256, 8, "zipf", zipf_s=1.1,
                 quant="fp8_e4m3_b128", combine_input="independent", seed=1002),
        Workload("decode_bf16", 128, 7168, 8, 256, 8, "uniform", seed=1004),
        Workload("decode_sparse_bf16", 16, 7168, 8, 256, 8, "uniform", seed=1014),
        Workload("qwen3_moe_mxfp4", 16384, 4096, 8, 128, 8, "zipf", zipf_s=1.3,
                 quant="mxfp4_b32", outlier_frac=0.01, outlier_mult=20.0,
                 combine_input="independent", seed=1005),
        # DeepSeek-V3 shape and routing with FP8 payloads quantized before
        # dispatch: 7168-byte rows and 56 fp32 block scales carried as is
        Workload("deepseek_v3_raw_fp8", 4096, 7168, 8, 256, 8, "zipf", zipf_s=1.1,
                 combine_input="independent", seed=1002, raw_row_bytes=7168,
                 scale_row_bytes=224),
    ]
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> bfloat16 bit patterns (uint16), round to nearest even."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def draw_topk(rng: np.random.Generator, tokens: int, experts: int, topk: int,
              routing: str, zipf_s: float = 0.0) -> np.ndarray:
    """K distinct experts per token by Gumbel-top-k; returns int32 [T, K]."""
    if topk > experts:
        raise ValueError("topk > experts")
    logp = np.zeros(experts, dtype=np.float64)
    if routing == "zipf":
        perm = rng.permutation(experts)
        logp[perm] = -zipf_s * np.log(np.arange(1, experts + 1, dtype=np.float64))
    elif routing != "uniform":
        raise ValueError(routing)
    keys = logp[None, :] + rng.gumbel(size=(tokens, experts))
    order = np.argsort(-keys, axis=1, kind="stable")[:, :topk]
    return np.ascontiguousarray(order.astype(np.int32))


def softmax_weights(rng: np.random.Generator, tokens: int, topk: int) -> np.ndarray:
    logits = rng.standard_normal((tokens, topk), dtype=np.float32)
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    return np.ascontiguousarray((z / z.sum(axis=1, keepdims=True)).astype(np.float32))


def make_inputs(w: Workload, tokens: Optional[int] = None,
                with_combine_input: Optional[bool] = None) -> Dict[str, np.ndarray]:
    """Draw the inputs of workload ``w``.

    Returns numpy arrays: ``x`` uint16 [T,H] (bf16 bits) — uint8
    [T,raw_row_bytes] for a raw workload, which also returns ``scales``
    float32 [T,scale_row_bytes/4] — ``indices`` int32 [T,K], ``weights``
    float32 [T,K] and, when requested (default: when the workload's combine
    input is independent), ``combine_input`` uint16 [T*K,H] (bf16 bits).
    ``tokens`` overrides T (a prefix-sized draw with the same recipe; it is a
    different draw, not a slice).
    """
    T = w.tokens if tokens is None else int(tokens)
    ss = np.random.SeedSequence(w.seed)
    # children depend only on their index: the sixth stream leaves the
    # first five, and so every other workload's inputs, unchanged
    s_x, s_route, s_logit, s_out, s_comb, s_scale = ss.spawn(6)
    out = {}
    if w.raw_row_bytes > 0:
        out["x"] = np.random.default_rng(s_x).integers(0, 256, (T, w.raw_row_bytes),
                                                      dtype=np.uint8)
        sc = np.abs(np.random.default_rng(s_scale).standard_normal(
            (T, w.scale_row_bytes // 4), dtype=np.float32)) / np.float32(448.0)
        out["scales"] = np.ascontiguousarray(sc, dtype=np.float32)
    else:
        x = np.random.default_rng(s_x).standard_normal((T, w.hidden), dtype=np.float32)
        if w.outlier_frac > 0.0:
            mask = np.random.default_rng(s_out).random((T, w.hidden)) < w.outlier_frac
            x[mask] *= np.float32(w.outlier_mult)
        out["x"] = f32_to_bf16_bits(x)
        del x
    out["indices"] = draw_topk(np.random.default_rng(s_route), T, w.experts, w.topk,
                               w.routing, w.zipf_s)
    out["weights"] = softmax_weights(np.random.default_rng(s_logit), T, w.topk)
    if with_combine_input is None:
        with_combine_input = w.combine_input == "independent"
    if with_combine_input:
        c = np.random.default_rng(s_comb).standard_normal((T * w.topk, w.hidden),
                                                          dtype=np.float32)
        out["combine_input"] = f32_to_bf16_bits(c)
    return out


def fingerprint(inputs: Dict[str, np.ndarray]) -> Dict[str, dict]:
    """Shape, dtype and SHA-256 of each drawn array (of its bytes, C order)."""
    import hashlib
    return {k: {"shape": list(v.shape), "dtype": str(v.dtype),
                "sha256": hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest()}
            for k, v in sorted(inputs.items())}


def save_inputs(w: Workload, out_dir: str, tokens: Optional[int] = None) -> Dict[str, dict]:
    """Write the inputs of ``w`` as .npy files (plain arrays, no pickles) and
    a manifest.json with the workload and each array's fingerprint, so a run
    can be repeated on exactly these inputs elsewhere.  Returns the manifest."""
    import json
    import os
    os.makedirs(out_dir, exist_ok=True)
    inputs = make_inputs(w, tokens=tokens)
    for k, v in inputs.items():
        np.save(os.path.join(out_dir, f"{k}.npy"), v, allow_pickle=False)
    manifest = {"workload": dataclasses.asdict(w),
                "tokens": w.tokens if tokens is None else int(tokens),
                "arrays": fingerprint(inputs)}
    with open(os.path.join(out_dir, "manifest.json"), "w") as fh:
        json.dump(manifest, fh, indent=1)
    return manifest


def load_inputs(in_dir: str) -> Dict[str, np.ndarray]:
    """Read arrays written by save_inputs, checking them against the manifest."""
    import json
    import os
    with open(os.path.join(in_dir, "manifest.json")) as fh:
        manifest = json.load(fh)
    out = {k: np.load(os.path.join(in_dir, f"{k}.npy"), allow_pickle=False)
           for k in manifest["arrays"]}
    got = fingerprint(out)
    if got != manifest["arrays"]:
        bad = [k for k in got if got[k] != manifest["arrays"].get(k)]
        raise ValueError(f"arrays do not match the manifest: {bad}")
    return out


def main(argv=None) -> int:
    import argparse
    import json
    ap = argparse.ArgumentParser(description="Draw a workload's inputs and save them as .npy")
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("save")
    s.add_argument("workload", choices=sorted(WORKLOADS))
    s.add_argument("out_dir")
    s.add_argument("--tokens", type=int, default=None)
    f = sub.add_parser("fingerprint")
    f.add_argument("workload", choices=sorted(WORKLOADS))
    f.add_argument("--tokens", type=int, default=None)
    a = ap.parse_args(argv)
    w = WORKLOADS[a.workload]
    if a.cmd == "save":
        m = save_inputs(w, a.out_dir, a.tokens)
    else:
        m = fingerprint(make_inputs(w, tokens=a.tokens))
    print(json.dumps(m, indent=1))
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
