"""The fused gate prologue (kda_chunk_fwd_gate) against the fp64 oracle.

The kernel takes the gate logits x and forms g = g_min * sigmoid(x) itself;
the oracle forms the same g in fp64 from the stored logits
(``oracle.gate_from_logit``) and runs the token recurrence.  Tolerance as for
the plain prefill: max|gpu - oracle| / rms(oracle) <= 2e-2 for bf16 q/k/v and
<= 1e-4 for fp32 q/k/v, for o and the final state.
"""
from __future__ import annotations

import sys

import pytest
import torch

import kda_inputs
import linear_attention_recurrence_10_amd as kda
import oracle
from gpu_helpers import ErrAcc, head_groups, host64, oracle_heads, pick, rel_err, tol_for

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_with_gate(x, g_min, heads=None, cols=None):
    """Oracle on (a sample of) the inputs, with g formed from the stored logits."""
    xs = x["x"] if heads is None else x["x"].index_select(2, torch.as_tensor(heads, device=x["x"].device))
    g = oracle.gate_from_logit(xs, g_min)
    if heads is None:
        args = [host64(x[n]) for n in ("q", "k", "v")]
        beta = host64(x["beta"])
        h0 = None if x.get("h0") is None else host64(x["h0"])
        return oracle.kda_fwd(args[0], args[1], args[2], g, beta, h0=h0)
    hi = torch.as_tensor(heads, device=x["q"].device)
    ci = torch.as_tensor(cols, device=x["q"].device)
    q, k = (host64(x[n].index_select(2, hi)) for n in ("q", "k"))
    v = host64(x["v"].index_select(2, hi).index_select(3, ci))
    beta = host64(x["beta"].index_select(2, hi))
    h0 = None if x.get("h0") is None else host64(x["h0"].index_select(1, hi).index_select(3, ci))
    return oracle.kda_fwd(q, k, v, g, beta, h0=h0)


@pytest.mark.parametrize("gate_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [16, 128])
@pytest.mark.parametrize("T", [1, 17, 50, 130])
def test_gate_parity(gate_dtype, dtype, D, T):
    x = kda_inputs.prefill_inputs(2, T, 3, D, dtype, h0=True, seed=300 + T + D, device=DEV,
                                  gate_logits=gate_dtype)
    label = "gate x=%s D=%d T=%d %s" % (gate_dtype, D, T, dtype)
    say("case " + label)
    o, hT = kda.chunk_fwd_gate(x["q"], x["k"], x["v"], x["x"], x["beta"], x["h0"])
    torch.cuda.synchronize()
    o_ref, h_ref = oracle_with_gate(x, -5.0)
    eo, eh = rel_err(o.cpu(), o_ref), rel_err(hT.cpu(), h_ref)
    say("%s: err_o=%.3e err_hT=%.3e" % (label, eo, eh))
    tol = tol_for(dtype)
    assert eo <= tol and eh <= tol, (label, eo, eh)


@pytest.mark.parametrize("g_min", [-5.0, -1.0, -0.1])
def test_gate_floor(g_min):
    """Other floors (weaker decay), bf16 inputs and logits, several chunks."""
    x = kda_inputs.prefill_inputs(1, 200, 4, 128, "bf16", h0=True, seed=41, device=DEV, gate_logits="bf16")
    say("case gate floor %g" % g_min)
    o, hT = kda.chunk_fwd_gate(x["q"], x["k"], x["v"], x["x"], x["beta"], x["h0"], g_min=g_min)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle_with_gate(x, g_min)
    eo, eh = rel_err(o.cpu(), o_ref), rel_err(hT.cpu(), h_ref)
    say("gate floor %g: err_o=%.3e err_hT=%.3e" % (g_min, eo, eh))
    assert eo <= 2e-2 and eh <= 2e-2


def test_gate_matches_log_decay_entry():
    """The same gate handed over as fp32 logits or as the fp32 log-decay that
    torch forms from them: the two launches agree far inside the tolerance
    (they differ only in how sigmoid is rounded)."""
    x = kda_inputs.prefill_inputs(2, 300, 3, 128, "bf16", h0=True, seed=8, device=DEV, gate_logits="f32")
    g = kda_inputs.G_MIN * torch.sigmoid(x["x"])
    o1, h1 = kda.chunk_fwd_gate(x["q"], x["k"], x["v"], x["x"], x["beta"], x["h0"])
    o2, h2 = kda.chunk_fwd(x["q"], x["k"], x["v"], g, x["beta"], x["h0"])
    torch.cuda.synchronize()
    eo, eh = rel_err(o1.cpu(), o2.cpu()), rel_err(h1.cpu(), h2.cpu())
    say("gate vs log-decay entry: %.3e %.3e" % (eo, eh))
    assert eo < 1e-4 and eh < 1e-4


def test_gate_extreme_logits():
    """Logits at +-1e4 and +-inf give the gate's limits (g_min and 0) with no
    nan; a sequence whose gate is 0 everywhere keeps its whole history."""
    x = kda_inputs.prefill_inputs(1, 40, 2, 128, "bf16", h0=True, seed=9, device=DEV, gate_logits="f32")
    xs = x["x"]
    xs[:, 0::4] = 1e4
    xs[:, 1::4] = -1e4
    xs[:, 2::4] = float("inf")
    xs[:, 3::4] = float("-inf")
    o, hT = kda.chunk_fwd_gate(x["q"], x["k"], x["v"], xs, x["beta"], x["h0"])
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(hT).all()
    o_ref, h_ref = oracle_with_gate(x, -5.0)
    assert rel_err(o.cpu(), o_ref) <= 2e-2 and rel_err(hT.cpu(), h_ref) <= 2e-2


def test_gate_64k_whole():
    """The 64K-token, 56-head workload with bf16 logits, in the launch
    configuration of the benchmark.  Every element of o and hT is compared
    with the oracle (g formed in fp64 from the stored logits), 28 heads at a
    time; one max|err| / rms per tensor."""
    cfg = kda_inputs.PREFILL_64K
    say("case gate " + cfg.name)
    x = kda_inputs.prefill_inputs(cfg.B, cfg.T, cfg.H, cfg.D, cfg.dtype, h0=cfg.h0, seed=cfg.seed, device=DEV,
                                  gate_logits="bf16")
    o, hT = kda.chunk_fwd_gate(x["q"], x["k"], x["v"], x["x"], x["beta"], None)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(hT).all()
    acc_o, acc_h = ErrAcc(), ErrAcc()
    for heads in head_groups(cfg.H, 28):
        hi = torch.as_tensor(heads, device=DEV)
        g = oracle.gate_from_logit(x["x"].index_select(2, hi), -5.0)
        o_ref, h_ref = oracle_heads(x, heads, g=g)
        acc_o.add(o.index_select(2, hi), o_ref)
        acc_h.add(hT.index_select(1, hi), h_ref)
        say("  heads %d..%d done" % (heads[0], heads[-1]))
        del g, o_ref, h_ref
    eo, eh = acc_o.value(), acc_h.value()
    say("gate 64k whole tensors: err_o=%.3e err_hT=%.3e" % (eo, eh))
    assert eo <= 2e-2 and eh <= 2e-2


def test_gate_repeat_runs_are_bitwise_identical():
    """The gate variants run with two k-side waves per SIMD and eight partial
    Grams; their sum has a fixed order, so repeated launches agree bit for bit."""
    x = kda_inputs.prefill_inputs(2, 300, 8, 128, "bf16", h0=True, seed=44, device=DEV, gate_logits="bf16")
    say("case gate repeat")
    o1, h1 = kda.chunk_fwd_gate(x["q"], x["k"], x["v"], x["x"], x["beta"], x["h0"])
    o2, h2 = kda.chunk_fwd_gate(x["q"], x["k"], x["v"], x["x"], x["beta"], x["h0"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


@pytest.mark.parametrize("T1", [16, 45])
def test_gate_split_run_matches_single_run(T1):
    """Resuming from a prefix's final state (prefix-cache reuse) gives the same
    o and final state as one run over the whole sequence."""
    T = 160
    x = kda_inputs.prefill_inputs(1, T, 4, 128, "bf16", h0=True, seed=45, device=DEV, gate_logits="bf16")
    say("case gate split %d" % T1)
    o, hT = kda.chunk_fwd_gate(x["q"], x["k"], x["v"], x["x"], x["beta"], x["h0"])
    part = {n: x[n][:, :T1].contiguous() for n in ("q", "k", "v", "x", "beta")}
    rest = {n: x[n][:, T1:].contiguous() for n in ("q", "k", "v", "x", "beta")}
    o1, h1 = kda.chunk_fwd_gate(part["q"], part["k"], part["v"], part["x"], part["beta"], x["h0"])
    o2, h2 = kda.chunk_fwd_gate(rest["q"], rest["k"], rest["v"], rest["x"], rest["beta"], h1)
    torch.cuda.synchronize()
    assert rel_err(o1.cpu(), o[:, :T1].cpu()) < 1e-3
    assert rel_err(o2.cpu(), o[:, T1:].cpu()) < 1e-3
    assert rel_err(h2.cpu(), hT.cpu()) < 1e-3


def test_gate_value_columns_are_independent():
    """Changing value column j (and h0's column j) changes nothing in any other
    column of o or the final state: the four 32-column slices and their two
    column tiles each see only their own columns."""
    x = kda_inputs.prefill_inputs(1, 70, 2, 128, "bf16", h0=True, seed=46, device=DEV, gate_logits="bf16")
    say("case gate columns")
    o1, h1 = kda.chunk_fwd_gate(x["q"], x["k"], x["v"], x["x"], x["beta"], x["h0"])
    j = 77
    v2, h02 = x["v"].clone(), x["h0"].clone()
    v2[..., j] = -v2[..., j] + 0.5
    h02[..., j] = 0.0
    o2, h2 = kda.chunk_fwd_gate(x["q"], x["k"], v2, x["x"], x["beta"], h02)
    torch.cuda.synchronize()
    keep = [c for c in range(128) if c != j]
    assert torch.equal(o1[..., keep], o2[..., keep]) and torch.equal(h1[..., keep], h2[..., keep])
    assert not torch.equal(o1[..., j], o2[..., j])
