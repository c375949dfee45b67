"""HIP path vs the fp64 oracle, element by element, through the C ABI.

Tolerance: max|gpu - oracle| / rms(oracle) <= 2e-2 for bf16 q/k/v and <= 1e-4
for fp32 q/k/v, for both o and the final state, per tensor.
"""
from __future__ import annotations

import sys

import pytest
import torch

import kda_inputs
import linear_attention_recurrence_10_amd as kda
from gpu_helpers import ErrAcc, head_groups, oracle_full, oracle_heads, oracle_sampled, pick, rel_err, tol_for, host64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_and_check(x, dtype, label, h0=None):
    h0 = x.get("h0") if h0 is None else h0
    o, hT = kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], h0)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle_full(x, h0=h0)
    eo, eh = rel_err(o.cpu(), o_ref), rel_err(hT.cpu(), h_ref)
    say("%s: err_o=%.3e err_hT=%.3e" % (label, eo, eh))
    tol = tol_for(dtype)
    assert eo <= tol and eh <= tol, (label, eo, eh)
    return eo, eh


# --- the named workloads ----------------------------------------------------

def test_tiny_f32_d16():
    cfg = kda_inputs.TINY
    say("case tiny " + cfg.name)
    x = kda_inputs.config_inputs(cfg, device=DEV)
    run_and_check(x, cfg.dtype, cfg.name)


def test_prefill_b4_h16_t4096_full():
    cfg = kda_inputs.PREFILL_B4
    say("case " + cfg.name)
    x = kda_inputs.config_inputs(cfg, device=DEV)
    run_and_check(x, cfg.dtype, cfg.name)


def test_prefill_64k_whole():
    """Full size (B=1, H=56, T=65536), in the launch configuration of the
    benchmark.  Every element of o and hT is compared with the oracle, which
    runs over 28 heads at a time; one max|err| / rms per tensor."""
    cfg = kda_inputs.PREFILL_64K
    say("case " + cfg.name)
    x = kda_inputs.config_inputs(cfg, device=DEV)
    o, hT = kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], None)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(hT).all()
    acc_o, acc_h = ErrAcc(), ErrAcc()
    for heads in head_groups(cfg.H, 28):
        o_ref, h_ref = oracle_heads(x, heads)
        hi = torch.as_tensor(heads, device=DEV)
        acc_o.add(o.index_select(2, hi), o_ref)
        acc_h.add(hT.index_select(1, hi), h_ref)
        say("  heads %d..%d done" % (heads[0], heads[-1]))
        del o_ref, h_ref
    eo, eh = acc_o.value(), acc_h.value()
    say("%s whole tensors: err_o=%.3e err_hT=%.3e" % (cfg.name, eo, eh))
    assert eo <= 2e-2 and eh <= 2e-2


def test_prefill_64k_sampled():
    """Full size; oracle on 3 heads x 8 columns over the whole sequence (a fast
    check beside the whole-tensor comparison)."""
    cfg = kda_inputs.PREFILL_64K
    say("case sampled " + cfg.name)
    x = kda_inputs.config_inputs(cfg, device=DEV)
    o, hT = kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], None)
    torch.cuda.synchronize()
    heads, cols = [0, 29, 55], [0, 5, 31, 32, 63, 64, 100, 127]
    o_ref, h_ref = oracle_sampled(x, heads, cols)
    eo = rel_err(pick(o, heads, cols), o_ref)
    eh = rel_err(pick(hT, heads, cols, 1, 3), h_ref)
    say("%s sampled: err_o=%.3e err_hT=%.3e" % (cfg.name, eo, eh))
    assert eo <= 2e-2 and eh <= 2e-2


def test_decode_b256_h56_whole():
    """All 256 x 56 states and outputs of one decode step against the oracle
    (the state is cloned before the in-place update)."""
    cfg = kda_inputs.DECODE_B256
    say("case " + cfg.name)
    d = kda_inputs.decode_inputs(cfg.B, cfg.H, cfg.D, cfg.dtype, seed=cfg.seed, device=DEV)
    s0 = d["state"].clone()
    o = kda.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"])
    torch.cuda.synchronize()
    import oracle
    acc_o, acc_s = ErrAcc(), ErrAcc()
    for b0 in range(0, cfg.B, 64):
        rows = torch.arange(b0, min(cfg.B, b0 + 64), device=DEV)
        sub = [host64(d[n].index_select(0, rows)) for n in ("q", "k", "v", "g", "beta")]
        o_ref, s_ref = oracle.kda_decode(*sub, host64(s0.index_select(0, rows)))
        acc_o.add(o.index_select(0, rows), o_ref)
        acc_s.add(d["state"].index_select(0, rows), s_ref)
    eo, es = acc_o.value(), acc_s.value()
    say("%s whole tensors: err_o=%.3e err_state=%.3e" % (cfg.name, eo, es))
    assert eo <= 2e-2 and es <= 2e-2


@pytest.mark.timeout(900)
def test_prefill_1m_whole():
    """Full size (B=1, H=56, T=2^20, random h0).  o is compared on the first
    65,536 tokens of every head, and the final state of every head by
    replaying the oracle segment by segment (65,536 tokens each, the fp64
    state carried across segments)."""
    cfg = kda_inputs.PREFILL_1M
    say("case " + cfg.name)
    x = kda_inputs.config_inputs(cfg, device=DEV)
    o, hT = kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
    torch.cuda.synchronize()
    say("gpu done")
    assert torch.isfinite(hT).all()
    seg = kda_inputs.SEGMENT
    acc_o, acc_h = ErrAcc(), ErrAcc()
    for heads in head_groups(cfg.H, 28):
        hi = torch.as_tensor(heads, device=DEV)
        S = None
        for s, t0 in enumerate(range(0, cfg.T, seg)):
            o_ref, S = oracle_heads(x, heads, t0=t0, t1=t0 + seg, S0=S)
            if s == 0:
                acc_o.add(o[:, :seg].index_select(2, hi), o_ref)
            del o_ref
            say("  heads %d..%d segment %d done" % (heads[0], heads[-1], s))
        acc_h.add(hT.index_select(1, hi), S)
    eo, eh = acc_o.value(), acc_h.value()
    say("%s whole tensors: err_o=%.3e (first segment) err_hT=%.3e (segment replay)" % (cfg.name, eo, eh))
    assert eo <= 2e-2 and eh <= 2e-2
    del x, o, hT
    torch.cuda.empty_cache()


# --- shapes, dtypes and edge cases -----------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [16, 128])
@pytest.mark.parametrize("T", [1, 15, 16, 17, 50])
def test_ragged_lengths(dtype, D, T):
    x = kda_inputs.prefill_inputs(2, T, 3, D, dtype, h0=True, seed=100 + T + D, device=DEV)
    run_and_check(x, dtype, "ragged D=%d T=%d %s" % (D, T, dtype))


@pytest.mark.parametrize("D", [16, 128])
def test_f32_longer(D):
    x = kda_inputs.prefill_inputs(1, 300, 2, D, "f32", h0=True, seed=7, device=DEV)
    run_and_check(x, "f32", "f32 D=%d T=300" % D)


def test_zero_initial_state_is_default():
    x = kda_inputs.prefill_inputs(1, 40, 2, 128, "bf16", h0=False, seed=3, device=DEV)
    o1, h1 = kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], None)
    z = torch.zeros(1, 2, 128, 128, device=DEV)
    o2, h2 = kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], z)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


def test_empty_sequence():
    x = kda_inputs.prefill_inputs(2, 0, 3, 128, "bf16", h0=True, seed=4, device=DEV)
    o, hT = kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 3, 128)
    assert torch.equal(hT, x["h0"])
    _, hz = kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], None)
    assert torch.equal(hz, torch.zeros_like(hz))


def test_state_in_place_alias():
    x = kda_inputs.prefill_inputs(1, 33, 2, 128, "bf16", h0=True, seed=5, device=DEV)
    o_ref, h_ref = kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
    st = x["h0"].clone()
    o, hT = kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], st, hT=st)
    torch.cuda.synchronize()
    assert hT.data_ptr() == st.data_ptr()
    assert torch.equal(o, o_ref) and torch.equal(st, h_ref)


def test_no_final_state():
    x = kda_inputs.prefill_inputs(1, 20, 1, 128, "bf16", seed=6, device=DEV)
    o, hT = kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], output_final_state=False)
    o2, _ = kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"])
    assert hT is None and torch.equal(o, o2)


def test_explicit_scale():
    x = kda_inputs.prefill_inputs(1, 20, 2, 128, "f32", h0=True, seed=8, device=DEV)
    o, hT = kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], scale=0.3)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle_full(x, scale=0.3)
    assert rel_err(o.cpu(), o_ref) <= 1e-4 and rel_err(hT.cpu(), h_ref) <= 1e-4


# --- numerical stress cases ------------------------------------------------

def _stress(kind, dtype="bf16", T=160, H=2):
    x = kda_inputs.prefill_inputs(1, T, H, 128, dtype, h0=True, seed=21, device=DEV,
                                  gate_mean=(-4.0 if kind == "weak_decay" else 0.0))
    if kind == "floor_gate":        # every gate at the floor: gamma reaches -80 in a chunk
        x["g"].fill_(-5.0)
    elif kind == "no_decay":        # g = 0: plain DeltaNet
        x["g"].zero_()
    elif kind == "beta_one":
        x["beta"].fill_(1.0)
    elif kind == "beta_zero":
        x["beta"].zero_()
    elif kind == "mixed_extremes":  # alternate floor and zero gates per channel
        x["g"][..., ::2] = -5.0
        x["g"][..., 1::2] = 0.0
    return x


@pytest.mark.parametrize("kind", ["floor_gate", "no_decay", "beta_one", "beta_zero", "weak_decay", "mixed_extremes"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_stress(kind, dtype):
    x = _stress(kind, dtype)
    run_and_check(x, dtype, "stress %s %s" % (kind, dtype))


def test_weak_decay_long():
    x = kda_inputs.prefill_inputs(2, 4096, 4, 128, "bf16", h0=True, seed=31, device=DEV, gate_mean=-4.0)
    run_and_check(x, "bf16", "weak decay T=4096")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [16, 128])
def test_decode_small(dtype, D):
    d = kda_inputs.decode_inputs(7, 5, D, dtype, seed=D, device=DEV)
    s0 = host64(d["state"])
    o = kda.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"])
    torch.cuda.synchronize()
    import oracle
    o_ref, s_ref = oracle.kda_decode(*[host64(d[n]) for n in ("q", "k", "v", "g", "beta")], s0)
    tol = tol_for(dtype)
    assert rel_err(o.cpu(), o_ref) <= tol and rel_err(d["state"].cpu(), s_ref) <= tol
