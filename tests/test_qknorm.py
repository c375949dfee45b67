"""The prefill and the decode step with the q/k normalisation fused in, against
the fp64 oracle applied to the normalised vectors: ``oracle.l2_normalize``
(x / max(||x||, eps)) of the stored q and k, then the token recurrence.

Inputs are the raw vectors of the generator's ``raw_qk`` recipe (N(0, 1) per
channel times a per-token length factor e^z, z ~ N(0, 1)).  Tolerance as for
the plain prefill: max|gpu - oracle| / rms(oracle) <= 2e-2 for bf16 q/k/v and
<= 1e-4 for fp32 q/k/v, per tensor.
"""
from __future__ import annotations

import sys

import pytest
import torch

import kda_inputs
import linear_attention_recurrence_10_amd as kda
import oracle
from gpu_helpers import ErrAcc, head_groups, host64, rel_err, tol_for

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_qknorm(x, eps, gate_logits=False, heads=None):
    sel = (lambda t: t) if heads is None else (lambda t: t.index_select(2, torch.as_tensor(heads, device=t.device)))
    q = oracle.l2_normalize(host64(sel(x["q"])), eps)
    k = oracle.l2_normalize(host64(sel(x["k"])), eps)
    g = oracle.gate_from_logit(host64(sel(x["x"])), kda_inputs.G_MIN) if gate_logits else host64(sel(x["g"]))
    h0 = x.get("h0")
    if h0 is not None and heads is not None:
        h0 = h0.index_select(1, torch.as_tensor(heads, device=h0.device))
    return oracle.kda_fwd(q, k, host64(sel(x["v"])), g, host64(sel(x["beta"])),
                          h0=None if h0 is None else host64(h0))


def run_qknorm(x, eps, gate_logits=False, **kw):
    g = x["x"] if gate_logits else x["g"]
    o, hT = kda.chunk_fwd_qknorm(x["q"], x["k"], x["v"], g, x["beta"], x.get("h0"), eps=eps,
                                 gate_logits=gate_logits, **kw)
    torch.cuda.synchronize()
    return o, hT


@pytest.mark.parametrize("gate", ["log_decay", "logit_f32", "logit_bf16"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [16, 128])
@pytest.mark.parametrize("T", [1, 17, 50, 130])
def test_qknorm_parity(gate, dtype, D, T):
    logits = {"log_decay": None, "logit_f32": "f32", "logit_bf16": "bf16"}[gate]
    x = kda_inputs.prefill_inputs(2, T, 3, D, dtype, h0=True, seed=700 + T + D, device=DEV, raw_qk=True,
                                  gate_logits=logits)
    label = "qknorm %s D=%d T=%d %s" % (gate, D, T, dtype)
    say("case " + label)
    o, hT = run_qknorm(x, 1e-6, gate_logits=logits is not None)
    o_ref, h_ref = oracle_qknorm(x, 1e-6, gate_logits=logits is not None)
    eo, eh = rel_err(o.cpu(), o_ref), rel_err(hT.cpu(), h_ref)
    say("%s: err_o=%.3e err_hT=%.3e" % (label, eo, eh))
    tol = tol_for(dtype)
    assert eo <= tol and eh <= tol, (label, eo, eh)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_qknorm_zero_vectors_and_floor(dtype):
    """Zero q and k vectors stay zero (their factor is 1/eps), and with a large
    eps most tokens take the floor branch: x / eps instead of x / ||x||."""
    x = kda_inputs.prefill_inputs(1, 70, 2, 128, dtype, h0=True, seed=31, device=DEV, raw_qk=True)
    for t in (0, 5, 16, 31, 69):   # whole vectors set to zero, in and across chunks
        x["k"][:, t] = 0
        x["q"][:, t + (1 if t < 69 else -1)] = 0
    for eps in (1e-12, 12.0):
        say("case zero vectors %s eps=%g" % (dtype, eps))
        o, hT = run_qknorm(x, eps)
        assert torch.isfinite(o).all() and torch.isfinite(hT).all()
        o_ref, h_ref = oracle_qknorm(x, eps)
        eo, eh = rel_err(o.cpu(), o_ref), rel_err(hT.cpu(), h_ref)
        say("  err_o=%.3e err_hT=%.3e" % (eo, eh))
        assert eo <= tol_for(dtype) and eh <= tol_for(dtype)


def test_qknorm_of_unit_inputs_is_the_plain_prefill():
    """fp32 unit-length q and k: the normalisation changes them only by
    rounding, so the result equals the plain prefill's to fp32 accuracy."""
    x = kda_inputs.prefill_inputs(1, 64, 2, 128, "f32", h0=True, seed=32, device=DEV)
    o1, h1 = kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
    o2, h2 = run_qknorm(x, 1e-12)
    assert rel_err(o2.cpu(), o1.cpu()) < 1e-5 and rel_err(h2.cpu(), h1.cpu()) < 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_qknorm_length_invariance(dtype):
    """Scaling q and k by powers of two (exact in bf16 and fp32) leaves the
    result unchanged: only the directions of q and k count."""
    x = kda_inputs.prefill_inputs(1, 50, 2, 128, dtype, h0=True, seed=33, device=DEV, raw_qk=True)
    o1, h1 = run_qknorm(x, 1e-12)
    y = dict(x)
    y["q"] = x["q"] * 8.0
    y["k"] = x["k"] * 0.25
    o2, h2 = run_qknorm(y, 1e-12)
    assert rel_err(o2.cpu(), o1.cpu()) < 1e-5 and rel_err(h2.cpu(), h1.cpu()) < 1e-5


def test_qknorm_64k_whole():
    """Full size (B=1, H=56, T=65536, bf16) with raw q and k, every element of
    o and hT against the oracle (28 heads at a time)."""
    cfg = kda_inputs.PREFILL_64K
    say("case qknorm " + cfg.name)
    x = kda_inputs.prefill_inputs(cfg.B, cfg.T, cfg.H, cfg.D, cfg.dtype, seed=cfg.seed, device=DEV, raw_qk=True)
    o, hT = run_qknorm(x, 1e-6)
    assert torch.isfinite(o).all() and torch.isfinite(hT).all()
    acc_o, acc_h = ErrAcc(), ErrAcc()
    for heads in head_groups(cfg.H, 28):
        o_ref, h_ref = oracle_qknorm(x, 1e-6, heads=heads)
        hi = torch.as_tensor(heads, device=DEV)
        acc_o.add(o.index_select(2, hi), o_ref)
        acc_h.add(hT.index_select(1, hi), h_ref)
        say("  heads %d..%d done" % (heads[0], heads[-1]))
        del o_ref, h_ref
    eo, eh = acc_o.value(), acc_h.value()
    say("qknorm %s whole tensors: err_o=%.3e err_hT=%.3e" % (cfg.name, eo, eh))
    assert eo <= 2e-2 and eh <= 2e-2


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [16, 128])
def test_decode_qknorm_parity(dtype, D):
    d = kda_inputs.decode_inputs(5, 3, D, dtype, seed=40 + D, device=DEV, raw_qk=True)
    d["k"][1, 2] = 0   # a zero key stays zero
    s0 = host64(d["state"])
    say("case decode qknorm D=%d %s" % (D, dtype))
    o = kda.decode_step_qknorm(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], eps=1e-6)
    torch.cuda.synchronize()
    q = oracle.l2_normalize(host64(d["q"]), 1e-6)
    k = oracle.l2_normalize(host64(d["k"]), 1e-6)
    o_ref, s_ref = oracle.kda_decode(q, k, host64(d["v"]), host64(d["g"]), host64(d["beta"]), s0)
    eo, es = rel_err(o.cpu(), o_ref), rel_err(d["state"].cpu(), s_ref)
    say("  err_o=%.3e err_state=%.3e" % (eo, es))
    assert eo <= tol_for(dtype) and es <= tol_for(dtype)


def test_decode_qknorm_b256_h56_whole():
    cfg = kda_inputs.DECODE_B256
    say("case decode qknorm " + cfg.name)
    d = kda_inputs.decode_inputs(cfg.B, cfg.H, cfg.D, cfg.dtype, seed=cfg.seed, device=DEV, raw_qk=True)
    s0 = d["state"].clone()
    o = kda.decode_step_qknorm(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], eps=1e-6)
    torch.cuda.synchronize()
    acc_o, acc_s = ErrAcc(), ErrAcc()
    for b0 in range(0, cfg.B, 64):
        rows = torch.arange(b0, min(cfg.B, b0 + 64), device=DEV)
        q = oracle.l2_normalize(host64(d["q"].index_select(0, rows)), 1e-6)
        k = oracle.l2_normalize(host64(d["k"].index_select(0, rows)), 1e-6)
        sub = [host64(d[n].index_select(0, rows)) for n in ("v", "g", "beta")]
        o_ref, s_ref = oracle.kda_decode(q, k, *sub, host64(s0.index_select(0, rows)))
        acc_o.add(o.index_select(0, rows), o_ref)
        acc_s.add(d["state"].index_select(0, rows), s_ref)
    eo, es = acc_o.value(), acc_s.value()
    say("decode qknorm whole tensors: err_o=%.3e err_state=%.3e" % (eo, es))
    assert eo <= 2e-2 and es <= 2e-2
