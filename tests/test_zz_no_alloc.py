"""kda_chunk_fwd_kcp_noalloc: the segmented prefill with the library's fixed
per-device workspace, for callers that cannot allocate device memory.  Its
results must equal those of kda_chunk_fwd_kcp (same kernels, caller
workspace) on the same inputs, call after call, also when a second call is
smaller than the first (the array keeps the last call's contents)."""
from __future__ import annotations

import sys

import pytest
import torch

import kda_inputs
import linear_attention_recurrence_10_amd as kda

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def both(x, n_seg):
    ref_o, ref_h = kda.chunk_fwd_kcp(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], n_seg=n_seg)
    o, h = kda.chunk_fwd_kcp_noalloc(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], n_seg=n_seg)
    torch.cuda.synchronize()
    return (o, h), (ref_o, ref_h)


def test_noalloc_matches_workspace_entry_twice_second_smaller():
    # first call: 7 heads x 2 batch rows x 8 segments of 128 tokens (B * n_seg * H = 112 state sets)
    x1 = kda_inputs.prefill_inputs(2, 1024, 7, 128, "bf16", h0=True, seed=71, device=DEV, gate_mean=-6.0)
    say("case noalloc call 1: B=2 T=1024 H=7 n_seg=8")
    (o1, h1), (r1, rh1) = both(x1, 8)
    assert torch.equal(o1, r1) and torch.equal(h1, rh1)
    # second call, smaller, with a ragged segment length: fewer state sets than the first left behind
    x2 = kda_inputs.prefill_inputs(1, 150, 3, 128, "bf16", h0=True, seed=72, device=DEV, gate_mean=-6.0)
    say("case noalloc call 2: B=1 T=150 H=3 n_seg=5")
    (o2, h2), (r2, rh2) = both(x2, 5)
    assert torch.equal(o2, r2) and torch.equal(h2, rh2)
    # and the plain prefill agrees within the rounding of the split summation
    o3, h3 = kda.chunk_fwd(x2["q"], x2["k"], x2["v"], x2["g"], x2["beta"], x2["h0"])
    torch.cuda.synchronize()
    assert kda_inputs.rel_err(o2.cpu(), o3.cpu()) < 1e-3 and kda_inputs.rel_err(h2.cpu(), h3.cpu()) < 1e-3


def test_noalloc_d16_fp32_and_no_initial_state():
    x = kda_inputs.prefill_inputs(3, 96, 4, 16, "f32", h0=False, seed=73, device=DEV, gate_mean=-6.0)
    say("case noalloc d16 fp32")
    (o, h), (r, rh) = both(x, 4)
    assert torch.equal(o, r) and torch.equal(h, rh)


def test_noalloc_rejects_a_workspace_larger_than_the_array():
    lib = kda.library()
    cap = int(lib.kda_chunk_fwd_kcp_noalloc_max_bytes())
    assert cap == 32 << 20
    # B * n_seg * H = 171 state sets of 128 x 128 need 3 * 171 * 64 KiB > 32 MiB
    x = kda_inputs.prefill_inputs(1, 171 * 16, 1, 128, "bf16", seed=74, device=DEV)
    assert kda.kcp_ws_bytes(1, 171 * 16, 1, 128, 128, 171) > cap
    with pytest.raises(kda.KdaError) as ei:
        kda.chunk_fwd_kcp_noalloc(x["q"], x["k"], x["v"], x["g"], x["beta"], None, n_seg=171)
    assert ei.value.status == 2  # KDA_ERR_UNSUPPORTED
    # 170 sets fit
    x = kda_inputs.prefill_inputs(1, 170 * 16, 1, 128, "bf16", seed=75, device=DEV)
    (o, h), (r, rh) = both(x, 170)
    assert torch.equal(o, r) and torch.equal(h, rh)
