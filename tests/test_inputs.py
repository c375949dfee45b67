"""Seeded input generator: determinism, segment regeneration, distributions,
and the gate range the pages fix (tests/golden/gate_range.json)."""
from __future__ import annotations

import json
import math
import os

import torch

import kda_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "gate_range.json")


def test_deterministic():
    a = kda_inputs.prefill_inputs(2, 40, 3, 16, "bf16", h0=True, seed=9)
    b = kda_inputs.prefill_inputs(2, 40, 3, 16, "bf16", h0=True, seed=9)
    for n in ("q", "k", "v", "g", "beta", "h0"):
        assert torch.equal(a[n], b[n]), n
    c = kda_inputs.prefill_inputs(2, 40, 3, 16, "bf16", h0=True, seed=10)
    assert not torch.equal(a["q"], c["q"])


def test_segment_regenerates_alone():
    T = kda_inputs.SEGMENT + 37
    full = kda_inputs.prefill_inputs(1, T, 1, 4, "bf16", seed=3)
    bufs = {n: torch.empty_like(full[n][:, kda_inputs.SEGMENT:]) for n in ("q", "k", "v", "g", "beta")}
    kda_inputs.fill_prefill_segment(bufs, 0, 37, seed=3, seg=1)
    for n in bufs:
        assert torch.equal(bufs[n], full[n][:, kda_inputs.SEGMENT:]), n


def test_distributions():
    x = kda_inputs.prefill_inputs(1, 2048, 4, 128, "bf16", h0=True, seed=1)
    qn = x["q"].float().norm(dim=-1)
    assert (qn - 1).abs().max() < 2e-2            # unit norm up to bf16 rounding
    assert x["q"].dtype == torch.bfloat16 and x["g"].dtype == torch.float32
    assert abs(x["v"].float().std().item() - 1) < 0.02
    assert 0 < x["beta"].min() and x["beta"].max() < 1
    assert abs(x["h0"].std().item() - 0.1) < 0.005
    assert abs(x["g"].mean().item() + 2.5) < 0.05


def test_raw_qk_keeps_the_direction():
    # raw q, k are the same N(0, 1) draws as the normalised ones, times a
    # per-token length factor e^z: same directions, spread-out lengths
    a = kda_inputs.prefill_inputs(1, 256, 3, 128, "f32", seed=3)
    b = kda_inputs.prefill_inputs(1, 256, 3, 128, "f32", seed=3, raw_qk=True)
    for n in ("q", "k"):
        ln = b[n].norm(dim=-1, keepdim=True)
        assert (b[n] / ln - a[n]).abs().max() < 1e-5
        z = torch.log(ln / 128 ** 0.5)  # about N(0, 1), with the chi spread of the N(0, 1) length on top
        assert abs(z.mean().item()) < 0.2 and 0.8 < z.std().item() < 1.2
    for n in ("v", "beta", "g"):
        assert torch.equal(a[n], b[n])
    d = kda_inputs.decode_inputs(4, 2, 16, "bf16", seed=4, raw_qk=True)
    assert (d["k"].float().norm(dim=-1) - 1).abs().max() > 0.1


def test_gate_range_from_pages():
    fx = json.load(open(GOLDEN))
    g_min, C = fx["g_min"], fx["chunk"]
    x = kda_inputs.prefill_inputs(1, 512, 2, 64, "f32", seed=2)
    assert x["g"].min() >= g_min and x["g"].max() <= 0.0
    assert kda_inputs.G_MIN == g_min and kda_inputs.CHUNK == C
    # the claim: reciprocal factors exp(+-C*g_min) inside one chunk stay in bf16 normal range
    assert math.exp(-g_min * C) < fx["bf16_max"]
    assert math.exp(g_min * C) > fx["bf16_min_normal"]
    # and a 17th token would already leave it on the small side of fp32/bf16 normals
    assert math.exp(g_min * 2 * C) < fx["bf16_min_normal"]


def test_decode_inputs_shapes():
    x = kda_inputs.decode_inputs(5, 3, 16, "bf16", seed=4)
    assert x["q"].shape == (5, 3, 16) and x["beta"].shape == (5, 3)
    assert x["state"].shape == (5, 3, 16, 16) and x["state"].dtype == torch.float32


def test_rel_err():
    ref = torch.tensor([3.0, -4.0])
    assert abs(kda_inputs.rel_err(ref + torch.tensor([0.0, 0.5]), ref) - 0.5 / math.sqrt(12.5)) < 1e-12


def test_generator_digests_are_recorded():
    """The seeded CPU inputs hash to the digests recorded by
    tests/golden/make_input_hashes.py: a change of torch's generators or of
    the input recipe shows up here rather than as a shift in parity errors."""
    import importlib.util

    here = os.path.join(os.path.dirname(__file__), "golden")
    spec = importlib.util.spec_from_file_location("make_input_hashes", os.path.join(here, "make_input_hashes.py"))
    mk = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mk)
    with open(os.path.join(here, "input_hashes.json")) as f:
        want = json.load(f)
    assert sorted(want) == sorted(mk.CASES)
    for name, case in mk.CASES.items():
        assert mk.digests(case) == want[name], name
