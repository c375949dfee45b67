"""The segment-parallel oracle (``oracle.kcp``) against what the recurrence fixes (CPU only).

* Reassembled by the state scan, the segments give the whole-sequence
  recurrence's o and hT for every segment count (the affine split is exact).
* The transition matrix has closed forms: without writes it is the product
  of the decays; one token without decay is the erase I - beta k k^T, a
  projector when beta |k|^2 = 1.
* Built from explicit per-token matrices, it equals the recurrence's final
  state from the identity with zero values (a second route).
* Planted mistakes in the scan (transposed transition, write before the
  transition, scan not started from h0, segments out of order) are caught.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle.kcp import kcp_fwd, kcp_transition


def _inputs(B, T, H, Dk, Dv, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, Dv))
    g = -5 / (1 + np.exp(-rng.standard_normal((B, T, H, Dk))))
    beta = rng.uniform(0, 1, (B, T, H))
    h0 = rng.standard_normal((B, H, Dk, Dv))
    return q, k, v, g, beta, h0


def _rel(a, b):
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


@pytest.mark.parametrize("n_seg", [1, 2, 3, 4, 6, 12])
@pytest.mark.parametrize("with_h0", [False, True])
def test_scan_reassembles_the_whole_sequence(n_seg, with_h0):
    q, k, v, g, beta, h0 = _inputs(2, 12, 3, 5, 4, seed=10 + n_seg)
    h0 = h0 if with_h0 else None
    o_ref, s_ref = oracle.kda_fwd(q, k, v, g, beta, h0=h0)
    o, s, parts = kcp_fwd(q, k, v, g, beta, h0=h0, n_seg=n_seg)
    assert _rel(o, o_ref) < 1e-12 and _rel(s, s_ref) < 1e-12
    assert parts["M"].shape == (2, n_seg, 3, 5, 5) and parts["S_in"].shape == (2, n_seg, 3, 5, 4)
    # segment 0 starts from h0; every later one from the state after the tokens before it
    np.testing.assert_array_equal(parts["S_in"][:, 0], np.zeros_like(s) if h0 is None else h0)
    L = 12 // n_seg
    for p in range(1, n_seg):
        _, s_p = oracle.kda_fwd(q[:, :p * L], k[:, :p * L], v[:, :p * L], g[:, :p * L], beta[:, :p * L], h0=h0)
        assert _rel(parts["S_in"][:, p], s_p) < 1e-12


def test_segment_count_must_divide_length():
    q, k, v, g, beta, _ = _inputs(1, 10, 1, 3, 3, seed=1)
    with pytest.raises(ValueError):
        kcp_fwd(q, k, v, g, beta, n_seg=4)


def test_transition_without_writes_is_the_decay_product():
    _, k, _, g, _, _ = _inputs(2, 7, 2, 6, 6, seed=2)
    M = kcp_transition(k, g, np.zeros((2, 7, 2)))
    expect = np.zeros_like(M)
    idx = np.arange(6)
    expect[..., idx, idx] = np.exp(g.sum(axis=1))
    assert _rel(M, expect) < 1e-14


def test_one_token_without_decay_is_the_erase():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((1, 1, 1, 8))
    beta = np.full((1, 1, 1), 0.37)
    M = kcp_transition(k, np.zeros_like(k), beta)[0, 0]
    kk = k[0, 0, 0]
    assert _rel(M, np.eye(8) - 0.37 * np.outer(kk, kk)) < 1e-15
    # beta |k|^2 = 1: a projector that removes k
    P = kcp_transition(k, np.zeros_like(k), np.full((1, 1, 1), 1 / (kk @ kk)))[0, 0]
    assert np.abs(P @ kk).max() < 1e-14 and np.abs(P @ P - P).max() < 1e-14


def test_empty_span_is_the_identity():
    z = np.zeros((1, 0, 2, 4))
    M = kcp_transition(z, z, np.zeros((1, 0, 2)))
    np.testing.assert_array_equal(M, np.broadcast_to(np.eye(4), (1, 2, 4, 4)))


def test_transition_is_the_state_from_the_identity_with_zero_values():
    q, k, _, g, beta, _ = _inputs(2, 9, 3, 6, 6, seed=4)
    eye = np.broadcast_to(np.eye(6), (2, 3, 6, 6)).copy()
    _, s = oracle.kda_fwd(q, k, np.zeros((2, 9, 3, 6)), g, beta, h0=eye)
    assert _rel(kcp_transition(k, g, beta), s) < 1e-13


def test_segment_map_is_affine_in_the_incoming_state():
    q, k, v, g, beta, h0 = _inputs(1, 8, 2, 5, 3, seed=5)
    M = kcp_transition(k, g, beta)
    _, b = oracle.kda_fwd(q, k, v, g, beta, h0=None)
    _, s = oracle.kda_fwd(q, k, v, g, beta, h0=h0)
    assert _rel(s, M @ h0 + b) < 1e-13


# ---- planted mistakes in the reassembly ----

def _mutant_scan(kind, q, k, v, g, beta, h0, n_seg):
    B, T, H, Dk = q.shape
    L = T // n_seg
    spans = [slice(p * L, (p + 1) * L) for p in range(n_seg)]
    Ms = [kcp_transition(k[:, sp], g[:, sp], beta[:, sp]) for sp in spans]
    Bs = [oracle.kda_fwd(q[:, sp], k[:, sp], v[:, sp], g[:, sp], beta[:, sp])[1] for sp in spans]
    S = np.zeros_like(Bs[0]) if (h0 is None or kind == "scan_from_zero") else h0.copy()
    order = list(range(n_seg))[::-1] if kind == "reversed" else list(range(n_seg))
    S_in = [None] * n_seg
    for p in order:
        S_in[p] = S
        if kind == "transposed":
            S = np.swapaxes(Ms[p], -1, -2) @ S + Bs[p]
        elif kind == "write_first":
            S = Ms[p] @ (S + Bs[p])
        else:
            S = Ms[p] @ S + Bs[p]
    o = np.concatenate([oracle.kda_fwd(q[:, sp], k[:, sp], v[:, sp], g[:, sp], beta[:, sp], h0=S_in[p])[0]
                        for p, sp in enumerate(spans)], axis=1)
    return o, S


@pytest.mark.parametrize("kind", ["none", "transposed", "write_first", "scan_from_zero", "reversed"])
def test_planted_scan_mistake_is_caught(kind):
    q, k, v, g, beta, h0 = _inputs(1, 12, 2, 5, 5, seed=6)
    o_ref, s_ref = oracle.kda_fwd(q, k, v, g, beta, h0=h0)
    o, s = _mutant_scan(kind, q, k, v, g, beta, h0, n_seg=3)
    good = _rel(o, o_ref) < 1e-12 and _rel(s, s_ref) < 1e-12
    assert good == (kind == "none"), kind
