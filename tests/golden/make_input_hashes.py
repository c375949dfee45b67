"""Writes tests/golden/input_hashes.json: sha256 digests of small seeded input
sets drawn on the CPU by kda_inputs (the generator only; no method arithmetic).
A change of torch's generators, or of the recipe, changes them.

usage: python tests/golden/make_input_hashes.py
"""
from __future__ import annotations

import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import kda_inputs  # noqa: E402

CASES = {
    "prefill_bf16_b2_t40_h3_d16_h0_seed9": dict(B=2, T=40, H=3, D=16, dtype="bf16", h0=True, seed=9),
    "prefill_f32_b1_t64_h1_d16_seed20261201": dict(B=1, T=64, H=1, D=16, dtype="f32", h0=False, seed=20261201),
    "prefill_bf16_logits_b1_t33_h2_d128_seed5": dict(B=1, T=33, H=2, D=128, dtype="bf16", h0=True, seed=5,
                                                      gate_logits="bf16"),
}


def digests(case: dict) -> dict:
    args = dict(case)
    x = kda_inputs.prefill_inputs(args.pop("B"), args.pop("T"), args.pop("H"), args.pop("D"), args.pop("dtype"),
                                  device="cpu", **args)
    out = {}
    for name in sorted(x):
        t = x[name]
        if t is None:
            continue
        raw = t.contiguous().view(-1).view(torch_uint8()).numpy().tobytes()
        out[name] = hashlib.sha256(raw).hexdigest()
    return out


def torch_uint8():
    import torch
    return torch.uint8


def main():
    res = {k: digests(v) for k, v in CASES.items()}
    with open(os.path.join(HERE, "input_hashes.json"), "w") as f:
        json.dump(res, f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main()
