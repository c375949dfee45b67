"""The fp64 oracle against its pins (CPU only).

* Every pin in ``oracle_pins`` runs against the C oracle and the numpy oracle.
* The two oracles agree to 1e-12 on random inputs and the tiny workload.
* Mistakes planted in copies of the numpy oracle (swapped order, read before
  write, gate on the wrong axis, dropped beta, sign and transpose errors, ...)
  each fail at least one pin, which shows the pins can tell a wrong recurrence
  from the right one.
"""
from __future__ import annotations

import numpy as np
import pytest

import kda_inputs
import oracle
from oracle.ref_numpy import kda_fwd_numpy

from oracle_pins import ALL_PINS


def c_fwd(q, k, v, g, beta, h0, scale):
    return oracle.kda_fwd(q, k, v, g, beta, h0=h0, scale=scale)


def np_fwd(q, k, v, g, beta, h0, scale):
    return kda_fwd_numpy(q, k, v, g, beta, h0=h0, scale=scale)


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
@pytest.mark.parametrize("impl", [c_fwd, np_fwd], ids=["c", "numpy"])
def test_pin(pin, impl):
    pin(impl)


def test_two_oracles_agree_random():
    rng = np.random.default_rng(123)
    B, T, H, Dk, Dv = 2, 40, 3, 16, 12
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk)) / 4
    v = rng.standard_normal((B, T, H, Dv))
    g = -5 / (1 + np.exp(-rng.standard_normal((B, T, H, Dk))))
    beta = rng.uniform(0, 1, (B, T, H))
    h0 = rng.standard_normal((B, H, Dk, Dv))
    o1, S1 = oracle.kda_fwd(q, k, v, g, beta, h0=h0)
    o2, S2 = kda_fwd_numpy(q, k, v, g, beta, h0=h0)
    assert np.abs(o1 - o2).max() <= 1e-12 * np.abs(o2).max()
    assert np.abs(S1 - S2).max() <= 1e-12 * np.abs(S2).max()


def test_two_oracles_agree_tiny_workload():
    x = kda_inputs.config_inputs(kda_inputs.TINY)
    args = [x[n].double().numpy() for n in ("q", "k", "v", "g", "beta")]
    o1, S1 = oracle.kda_fwd(*args, h0=None)
    o2, S2 = kda_fwd_numpy(*args, h0=None)
    assert np.abs(o1 - o2).max() <= 1e-12 * np.abs(o2).max()
    assert np.abs(S1 - S2).max() <= 1e-12 * np.abs(S2).max()


def test_decode_is_one_token_prefill():
    x = kda_inputs.decode_inputs(3, 2, 8, "f32", seed=5)
    args = [x[n].double().numpy() for n in ("q", "k", "v", "g", "beta")]
    o, S = oracle.kda_decode(*args, x["state"].double().numpy())
    o2, S2 = kda_fwd_numpy(*[a[:, None] for a in args], h0=x["state"].double().numpy())
    assert np.abs(o - o2[:, 0]).max() < 1e-13
    assert np.abs(S - S2).max() < 1e-13


def test_oracle_rejects_bad_dims():
    with pytest.raises(AssertionError):
        oracle.kda_fwd(np.zeros((1, 2, 1, 4)), np.zeros((1, 2, 1, 3)), np.zeros((1, 2, 1, 4)),
                       np.zeros((1, 2, 1, 4)), np.zeros((1, 2, 1)))


def test_oracle_empty_sequence_returns_h0():
    h0 = np.arange(12.0).reshape(1, 1, 3, 4)
    z = np.zeros((1, 0, 1, 3))
    o, S = oracle.kda_fwd(z, z, np.zeros((1, 0, 1, 4)), z, np.zeros((1, 0, 1)), h0=h0)
    assert o.shape == (1, 0, 1, 4)
    assert np.array_equal(S, h0)


# ---------------------------------------------------------------------------
# Planted mistakes: each mutant is the numpy oracle with one plausible error.
# ---------------------------------------------------------------------------

def _mutant(kind):
    def fwd(q, k, v, g, beta, h0, scale):
        q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
        B, T, H, Dk = q.shape
        Dv = v.shape[-1]
        S = np.zeros((B, H, Dk, Dv)) if h0 is None else np.array(h0, dtype=np.float64)
        o = np.zeros((B, T, H, Dv))
        for t in range(T):
            a = np.exp(g[:, t])
            if kind == "erase_before_decay":
                r = np.einsum("bhij,bhi->bhj", S, k[:, t])
                S = a[..., None] * S
            else:
                if kind == "decay_value_axis":
                    S = S * a[..., None, :]
                elif kind == "no_decay":
                    pass
                elif kind == "decay_sign":
                    S = np.exp(-g[:, t])[..., None] * S
                else:
                    S = a[..., None] * S
                if kind == "recall_transposed":
                    r = np.einsum("bhji,bhi->bhj", S, k[:, t])
                else:
                    r = np.einsum("bhij,bhi->bhj", S, k[:, t])
            o_before = scale * np.einsum("bhij,bhi->bhj", S, q[:, t])
            if kind == "no_beta":
                e = v[:, t] - r
            elif kind == "erase_sign":
                e = beta[:, t][..., None] * (v[:, t] + r)
            elif kind == "beta_on_value_only":
                e = beta[:, t][..., None] * v[:, t] - r
            elif kind == "no_erase":
                e = beta[:, t][..., None] * v[:, t]
            else:
                e = beta[:, t][..., None] * (v[:, t] - r)
            S = S + k[:, t][..., :, None] * e[..., None, :]
            if kind == "read_before_write":
                o[:, t] = o_before
            elif kind == "read_transposed":
                o[:, t] = scale * np.einsum("bhji,bhi->bhj", S, q[:, t])
            elif kind == "no_scale":
                o[:, t] = np.einsum("bhij,bhi->bhj", S, q[:, t])
            else:
                o[:, t] = scale * np.einsum("bhij,bhi->bhj", S, q[:, t])
        return o, S
    return fwd


MUTANTS = ["erase_before_decay", "decay_value_axis", "no_decay", "decay_sign", "recall_transposed",
           "no_beta", "erase_sign", "beta_on_value_only", "no_erase", "read_before_write",
           "read_transposed", "no_scale"]


def test_unmutated_copy_passes_all_pins():
    fwd = _mutant("none")
    for pin in ALL_PINS:
        pin(fwd)


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistake_is_caught(kind):
    fwd = _mutant(kind)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(fwd)
        except Exception:  # AssertionError or a shape error from the broken code
            failed.append(pin.__name__)
    assert failed, "mutant %s passed every pin" % kind


# ---- the gate prologue: g = g_min * sigmoid(x) (Kimi K3 paper digest, section 2.1 (1)) ----

def test_gate_closed_forms():
    gm = -5.0
    g = oracle.gate_from_logit(np.array([0.0, 800.0, -800.0, np.log(3.0)]), gm)
    assert g[0] == gm / 2                       # sigmoid(0) = 1/2
    assert g[1] == gm and g[2] == 0.0           # the two limits, with no overflow to nan
    assert abs(g[3] - gm * 0.75) < 1e-15        # sigmoid(ln 3) = 3/4


def test_gate_symmetry_and_monotone():
    x = np.linspace(-30.0, 30.0, 2001)
    for gm in (-5.0, -1.0, -0.25):
        g = oracle.gate_from_logit(x, gm)
        # sigmoid(x) + sigmoid(-x) = 1
        assert np.max(np.abs(g + oracle.gate_from_logit(-x, gm) - gm)) < 1e-14
        assert np.all(np.diff(g) < 0) or np.all(np.diff(g) <= 0)  # decreasing (g_min < 0)
        assert np.all((g <= 0) & (g >= gm))


def test_gate_matches_library_sigmoid():
    from scipy.special import expit

    x = np.random.default_rng(5).normal(0.0, 3.0, size=10000)
    for gm in (-5.0, -2.5):
        # a few ulp of |g| <= 5 (the two routines round in a different order)
        assert np.max(np.abs(oracle.gate_from_logit(x, gm) - gm * expit(x))) < 8 * np.finfo(float).eps * abs(gm)


def test_gate_slope_at_zero():
    # d/dx [g_min sigmoid(x)] at 0 is g_min / 4
    h = 1e-6
    d = (oracle.gate_from_logit(np.array([h]), -5.0) - oracle.gate_from_logit(np.array([-h]), -5.0)) / (2 * h)
    assert abs(d[0] - (-5.0 / 4)) < 1e-8


def test_gate_takes_bf16_logits_as_stored():
    import torch

    x = torch.tensor([0.1, -1.7, 3.3], dtype=torch.bfloat16)
    xs = x.float().double().numpy()  # the stored bf16 values, exactly
    assert np.array_equal(oracle.gate_from_logit(x, -5.0), -5.0 / (1.0 + np.exp(-xs)))


# ---- the q/k normalisation prologue: x / max(||x||, eps) along the last axis ----

def _l2_pin_closed_forms(f):
    y = f(np.array([[3.0, 4.0], [0.0, -2.0], [0.0, 0.0]]), 1e-12)
    assert np.array_equal(y, np.array([[0.6, 0.8], [0.0, -1.0], [0.0, 0.0]]))  # 3-4-5 triangle; zero stays zero


def _l2_pin_eps_floor(f):
    # a vector shorter than eps is divided by eps, not by its length
    y = f(np.array([3e-13, 4e-13]), 1e-12)
    assert np.allclose(y, [0.3, 0.4], rtol=1e-14, atol=0)
    y = f(np.array([3.0, 4.0]), 10.0)
    assert np.allclose(y, [0.3, 0.4], rtol=1e-15, atol=0)


def _l2_pin_unit_length_and_direction(f):
    x = np.random.default_rng(9).normal(size=(5, 7, 33)) * np.exp(np.random.default_rng(10).uniform(-3, 3, (5, 7, 1)))
    y = f(x, 1e-12)
    assert np.max(np.abs(np.sqrt((y * y).sum(-1)) - 1.0)) < 1e-14
    # parallel to x with a positive factor: y . x = ||x||
    assert np.max(np.abs((y * x).sum(-1) - np.sqrt((x * x).sum(-1)))) < 1e-12 * np.max(np.abs(x))


def _l2_pin_last_axis_only(f):
    # rows are independent, and the length is taken over the last axis
    x = np.array([[1.0, 0.0, 0.0, 0.0], [0.0, 2.0, 0.0, 0.0], [1.0, 1.0, 1.0, 1.0]])
    y = f(x, 1e-12)
    assert np.array_equal(y, np.array([[1.0, 0, 0, 0], [0, 1.0, 0, 0], [0.5, 0.5, 0.5, 0.5]]))


def _l2_pin_invariances(f):
    x = np.random.default_rng(11).normal(size=(4, 16))
    y = f(x, 1e-12)
    assert np.max(np.abs(f(7.5 * x, 1e-12) - y)) < 1e-15   # positive scaling
    assert np.array_equal(f(-x, 1e-12), -y)                 # odd
    assert np.max(np.abs(f(y, 1e-12) - y)) < 1e-15          # idempotent


L2_PINS = [_l2_pin_closed_forms, _l2_pin_eps_floor, _l2_pin_unit_length_and_direction, _l2_pin_last_axis_only,
           _l2_pin_invariances]


@pytest.mark.parametrize("pin", L2_PINS, ids=lambda p: p.__name__)
def test_l2_normalize_pin(pin):
    pin(oracle.l2_normalize)


_L2_MUTANTS = {
    "squared_length": lambda x, eps: x / np.maximum((x * x).sum(-1, keepdims=True), eps),
    "l1_length": lambda x, eps: x / np.maximum(np.abs(x).sum(-1, keepdims=True), eps),
    "eps_added": lambda x, eps: x / (np.sqrt((x * x).sum(-1, keepdims=True)) + 1e-3 * (eps > 0)),
    "first_axis": lambda x, eps: x / np.maximum(np.sqrt((x * x).sum(0, keepdims=True)), eps),
    "no_floor": lambda x, eps: x / np.sqrt((x * x).sum(-1, keepdims=True) + 1e-300),
    "eps_floor_squared": lambda x, eps: x / np.maximum(np.sqrt((x * x).sum(-1, keepdims=True)), eps * eps),
}


@pytest.mark.parametrize("kind", sorted(_L2_MUTANTS))
def test_l2_planted_mistake_is_caught(kind):
    f = _L2_MUTANTS[kind]
    failed = []
    for pin in L2_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(f)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "mutant %s passed every pin" % kind


def test_l2_normalize_takes_bf16_as_stored():
    import torch

    x = torch.tensor([[0.1, -1.7, 3.3]], dtype=torch.bfloat16)
    xs = x.float().double().numpy()
    y = oracle.l2_normalize(x)
    assert y.dtype == np.float64
    assert np.max(np.abs(y * np.sqrt((xs * xs).sum()) - xs)) < 1e-15
