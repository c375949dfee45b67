"""The MFMA prefill's pacing of the four value slices of a head.

Every 8 steps the slices report their step in a small device array tagged with
the launch's epoch, and a slice far ahead of a started slice of its head waits
(boundedly) for it.  The pacing only delays work, so results must not depend
on it:

* a grid with more work-groups than the device runs at once (slices of a head
  may then not all be resident) matches the oracle;
* two launches running at the same time on two streams (their epochs interleave
  in the same report slots) give bitwise the results of separate launches;
* with enough heads to fill the report array's range, the results are right;
* past that range (more than 16384 heads) the launch runs unpaced and the
  results are right.
"""
from __future__ import annotations

import sys

import pytest
import torch

import kda_inputs
import linear_attention_recurrence_10_amd as kda
from gpu_helpers import oracle_sampled, pick, rel_err, tol_for

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def fwd(x, stream=None):
    return kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x.get("h0"), stream=stream)


def test_more_work_groups_than_the_device_holds():
    # 6 x 24 = 144 heads, 576 work-groups of 12 waves: more than one per CU
    x = kda_inputs.prefill_inputs(6, 1024, 24, 128, "bf16", h0=True, seed=91, device=DEV, gate_mean=-6.0)
    o, hT = fwd(x)
    torch.cuda.synchronize()
    heads, cols = [0, 13, 23], [0, 64, 127]
    o_ref, s_ref = oracle_sampled(x, heads, cols)
    eo = rel_err(pick(o, heads, cols), o_ref)
    eh = rel_err(pick(hT, heads, cols, head_dim=1, col_dim=3), s_ref)
    say("  576 work-groups: o %.3e hT %.3e" % (eo, eh))
    assert eo <= tol_for("bf16") and eh <= tol_for("bf16")


def test_concurrent_launches_on_two_streams():
    xa = kda_inputs.prefill_inputs(1, 4096, 28, 128, "bf16", h0=True, seed=92, device=DEV)
    xb = kda_inputs.prefill_inputs(1, 4096, 28, 128, "bf16", h0=True, seed=93, device=DEV)
    oa, ha = fwd(xa)
    ob, hb = fwd(xb)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    results = []
    for _ in range(3):
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            ra = fwd(xa, stream=s1)
        with torch.cuda.stream(s2):
            rb = fwd(xb, stream=s2)
        torch.cuda.synchronize()
        results.append((ra, rb))
    for ra, rb in results:
        assert torch.equal(ra[0], oa) and torch.equal(ra[1], ha)
        assert torch.equal(rb[0], ob) and torch.equal(rb[1], hb)


def test_many_heads_across_the_report_range():
    # B H = 4096 heads: 16384 report slots, a quarter of the array, used by one launch
    x = kda_inputs.prefill_inputs(64, 64, 64, 128, "bf16", h0=False, seed=94, device=DEV)
    o, hT = fwd(x)
    torch.cuda.synchronize()
    heads, cols = [0, 31, 63], [5, 100]
    o_ref, s_ref = oracle_sampled(x, heads, cols)
    assert rel_err(pick(o, heads, cols), o_ref) <= tol_for("bf16")
    assert rel_err(pick(hT, heads, cols, head_dim=1, col_dim=3), s_ref) <= tol_for("bf16")


def test_more_heads_than_report_slots_runs_unpaced():
    # B H = 16400 heads (past the 16384 the report array serves): no slice
    # reports or waits, and the results are right; a ragged 20-token sequence
    say("case unpaced: B=2 H=8200 T=20")
    x = kda_inputs.prefill_inputs(2, 20, 8200, 128, "bf16", h0=True, seed=95, device=DEV)
    o, hT = fwd(x)
    torch.cuda.synchronize()
    heads, cols = [0, 4099, 8199], [0, 77, 127]
    o_ref, s_ref = oracle_sampled(x, heads, cols)
    eo = rel_err(pick(o, heads, cols), o_ref)
    eh = rel_err(pick(hT, heads, cols, head_dim=1, col_dim=3), s_ref)
    say("  16400 heads: o %.3e hT %.3e" % (eo, eh))
    assert eo <= tol_for("bf16") and eh <= tol_for("bf16")
