"""Pins of the fp64 backward oracle (oracle.kda_bwd, oracle.kda_bwd_numpy).

The gradient of the KDA forward pass is fixed by the forward recurrence
itself; these tests tie the oracle's adjoint to things other than itself:

* central finite differences of the (separately pinned) forward oracle, for
  every element of every input, on tiny cases, and along random directions on
  a larger one that spans two of the oracle's recompute blocks;
* closed forms: one token from a zero state; beta = 0 (pure decay of h0);
* linearity in (dO, dhT);
* agreement of the C and numpy implementations;
* planted mistakes in copies of the numpy adjoint are caught by the
  finite-difference check.
The loss is L = sum(o * dO) + sum(hT * dhT), so dO and dhT are the upstream
gradients.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle


def inputs(B, T, H, D, seed, h0=True, gate=0.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, D))
    k = rng.standard_normal((B, T, H, D))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, D))
    g = -5.0 / (1.0 + np.exp(-(rng.standard_normal((B, T, H, D)) + gate)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    hh = 0.3 * rng.standard_normal((B, H, D, D)) if h0 else None
    dO = rng.standard_normal((B, T, H, D))
    dhT = rng.standard_normal((B, H, D, D))
    return dict(q=q, k=k, v=v, g=g, beta=beta, h0=hh), dO, dhT


def loss(x, dO, dhT):
    o, hT = oracle.kda_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], h0=x["h0"])
    return float(np.sum(o * dO) + np.sum(hT * dhT))


def grads(x, dO, dhT, fn=None):
    fn = fn or oracle.kda_bwd
    dq, dk, dv, dg, db, dh0 = fn(x["q"], x["k"], x["v"], x["g"], x["beta"], dO, h0=x["h0"], dhT=dhT)
    return dict(q=dq, k=dk, v=dv, g=dg, beta=db, h0=dh0)


def fd_grad(x, dO, dhT, name, eps=1e-6):
    base = x[name]
    out = np.zeros_like(base)
    for idx in np.ndindex(base.shape):
        xp = dict(x)
        a = base.copy()
        a[idx] += eps
        xp[name] = a
        lp = loss(xp, dO, dhT)
        a = base.copy()
        a[idx] -= eps
        xp[name] = a
        lm = loss(xp, dO, dhT)
        out[idx] = (lp - lm) / (2 * eps)
    return out


@pytest.mark.parametrize("T,D,h0", [(1, 4, True), (5, 4, True), (6, 3, False), (17, 2, True)])
def test_every_gradient_element_matches_finite_differences(T, D, h0):
    x, dO, dhT = inputs(1, T, 2, D, seed=T * 10 + D, h0=h0)
    gr = grads(x, dO, dhT)
    names = ["q", "k", "v", "g", "beta"] + (["h0"] if h0 else [])
    for n in names:
        fd = fd_grad(x, dO, dhT, n)
        scale = max(1.0, float(np.abs(fd).max()))
        assert np.abs(gr[n] - fd).max() <= 2e-7 * scale, (n, np.abs(gr[n] - fd).max())


def test_directional_derivatives_across_recompute_blocks():
    """T = 150 spans three of the oracle's 64-token recompute blocks."""
    x, dO, dhT = inputs(2, 150, 2, 6, seed=3)
    gr = grads(x, dO, dhT)
    rng = np.random.default_rng(9)
    for trial in range(3):
        u = {n: rng.standard_normal(x[n].shape) for n in x}
        eps = 1e-6
        xp = {n: x[n] + eps * u[n] for n in x}
        xm = {n: x[n] - eps * u[n] for n in x}
        fd = (loss(xp, dO, dhT) - loss(xm, dO, dhT)) / (2 * eps)
        an = sum(float(np.sum(gr[n] * u[n])) for n in x)
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (trial, fd, an)


def test_single_token_from_zero_state_closed_form():
    """o = scale beta (q.k) v and hT = beta k v^T, so with s = scale:
    dq = s beta (dO.v) k, dk = s beta (dO.v) q + beta dhT v, dv = s beta (q.k) dO + beta dhT^T k,
    dbeta = s (q.k)(dO.v) + k^T dhT v, dg = 0, dh0 = Diag(e^g)(dS_1 + k dr^T) with
    dS_1 = dhT + s q dO^T and dr = -beta dS_1^T k."""
    x, dO, dhT = inputs(1, 1, 1, 5, seed=4, h0=False)
    gr = grads(x, dO, dhT)
    q, k, v, g = (x[n][0, 0, 0] for n in ("q", "k", "v", "g"))
    b = x["beta"][0, 0, 0]
    do, dh = dO[0, 0, 0], dhT[0, 0]
    s = 5 ** -0.5
    np.testing.assert_allclose(gr["q"][0, 0, 0], s * b * (do @ v) * k, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(gr["k"][0, 0, 0], s * b * (do @ v) * q + b * dh @ v, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(gr["v"][0, 0, 0], s * b * (q @ k) * do + b * dh.T @ k, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(gr["beta"][0, 0, 0], s * (q @ k) * (do @ v) + k @ dh @ v, rtol=1e-12)
    np.testing.assert_allclose(gr["g"], 0.0, atol=1e-15)
    dS1 = dh + s * np.outer(q, do)
    dr = -b * dS1.T @ k
    np.testing.assert_allclose(gr["h0"][0, 0], np.exp(g)[:, None] * (dS1 + np.outer(k, dr)), rtol=1e-12, atol=1e-14)


def test_no_writes_closed_form():
    """beta = 0: o_t = s (e^{G_t} * q_t)^T h0 and hT = Diag(e^{G_T}) h0 with
    G_t = g_1 + ... + g_t, hence dq_t = s e^{G_t} * (h0 do_t),
    dh0 = s sum_t (e^{G_t} * q_t) do_t^T + Diag(e^{G_T}) dhT, dv = dk = 0,
    and dg_u = sum_{t >= u} s e^{G_t} * q_t * (h0 do_t) + e^{G_T} * rowsum(h0 * dhT)."""
    x, dO, dhT = inputs(1, 9, 1, 4, seed=5)
    x["beta"][:] = 0.0
    gr = grads(x, dO, dhT)
    s = 4 ** -0.5
    q, g, h0 = x["q"][0, :, 0], x["g"][0, :, 0], x["h0"][0, 0]
    do, dh = dO[0, :, 0], dhT[0, 0]
    G = np.cumsum(g, axis=0)
    term = s * np.exp(G) * q * (do @ h0.T)          # [T, D]: s e^{G_t} q_t (h0 do_t)
    np.testing.assert_allclose(gr["q"][0, :, 0], s * np.exp(G) * (do @ h0.T), rtol=1e-12)
    np.testing.assert_allclose(gr["v"], 0.0, atol=1e-15)
    np.testing.assert_allclose(gr["k"], 0.0, atol=1e-15)
    final = np.exp(G[-1]) * np.sum(h0 * dh, axis=1)
    dg_ref = np.cumsum(term[::-1], axis=0)[::-1] + final
    np.testing.assert_allclose(gr["g"][0, :, 0], dg_ref, rtol=1e-11)
    dh0_ref = s * (np.exp(G) * q).T @ do + np.exp(G[-1])[:, None] * dh
    np.testing.assert_allclose(gr["h0"][0, 0], dh0_ref, rtol=1e-11)


def test_linear_in_upstream_gradients():
    x, dO, dhT = inputs(2, 40, 2, 6, seed=6)
    _, dO2, dhT2 = inputs(2, 40, 2, 6, seed=7)
    g1, g2 = grads(x, dO, dhT), grads(x, dO2, dhT2)
    g3 = grads(x, 2.0 * dO - 0.5 * dO2, 2.0 * dhT - 0.5 * dhT2)
    for n in g1:
        np.testing.assert_allclose(g3[n], 2.0 * g1[n] - 0.5 * g2[n], rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("B,T,H,D,h0,dh", [(2, 70, 3, 8, True, True), (1, 130, 2, 5, False, False),
                                           (3, 1, 2, 4, True, False), (1, 64, 1, 16, False, True)])
def test_c_and_numpy_adjoints_agree(B, T, H, D, h0, dh):
    x, dO, dhT = inputs(B, T, H, D, seed=B + T + D, h0=h0)
    dhT = dhT if dh else None
    a = grads(x, dO, dhT)
    b = grads(x, dO, dhT, fn=oracle.kda_bwd_numpy)
    for n in a:
        if n == "h0" and not h0:
            continue
        np.testing.assert_allclose(a[n], b[n], rtol=1e-12, atol=1e-12)


def _mutant(kind):
    """A copy of the numpy adjoint with one plausible mistake."""
    def bwd(q, k, v, g, beta, dO, h0=None, dhT=None, scale=None):
        B, T, H, Dk = q.shape
        scale = Dk ** -0.5 if scale is None else scale
        S = np.zeros((B, H, Dk, Dk)) if h0 is None else np.array(h0)
        prev = []
        for t in range(T):
            prev.append(S)
            Sd = np.exp(g[:, t])[..., None] * S
            rec = np.einsum("bhij,bhi->bhj", Sd, k[:, t])
            S = Sd + k[:, t][..., :, None] * (beta[:, t][..., None] * (v[:, t] - rec))[..., None, :]
        dS = np.zeros_like(S) if dhT is None else np.array(dhT)
        dq, dk, dv, dg = (np.zeros_like(x) for x in (q, k, v, g))
        db = np.zeros_like(beta)
        for t in reversed(range(T)):
            a = np.exp(g[:, t])
            Sd = a[..., None] * prev[t]
            rec = np.einsum("bhij,bhi->bhj", Sd, k[:, t])
            diff = v[:, t] - rec
            e = beta[:, t][..., None] * diff
            St = Sd + k[:, t][..., :, None] * e[..., None, :]
            if kind != "no_read_term":
                dS = dS + scale * q[:, t][..., :, None] * dO[:, t][..., None, :]
            dq[:, t] = scale * np.einsum("bhij,bhj->bhi", (Sd if kind == "read_before_write" else St), dO[:, t])
            de = np.einsum("bhij,bhi->bhj", dS, k[:, t])
            dk[:, t] = np.einsum("bhij,bhj->bhi", dS, e)
            db[:, t] = np.sum(de * (v[:, t] if kind == "dbeta_no_recall" else diff), axis=-1)
            dv[:, t] = beta[:, t][..., None] * de
            drec = (1.0 if kind == "recall_sign" else -1.0) * beta[:, t][..., None] * de
            dSd = dS + k[:, t][..., :, None] * drec[..., None, :]
            if kind != "no_recall_dk":
                dk[:, t] = dk[:, t] + np.einsum("bhij,bhj->bhi", Sd, drec)
            dg[:, t] = np.sum(dSd * (prev[t] if kind == "dg_undecayed" else Sd), axis=-1)
            dS = dSd if kind == "no_decay_in_dS" else a[..., None] * dSd
        return dq, dk, dv, dg, db, dS
    return bwd


@pytest.mark.parametrize("kind", ["no_read_term", "read_before_write", "dbeta_no_recall", "recall_sign",
                                  "no_recall_dk", "dg_undecayed", "no_decay_in_dS"])
def test_planted_mistakes_fail_finite_differences(kind):
    x, dO, dhT = inputs(1, 4, 1, 3, seed=8)
    wrong = grads(x, dO, dhT, fn=_mutant(kind))
    caught = False
    for n in ("q", "k", "v", "g", "beta", "h0"):
        fd = fd_grad(x, dO, dhT, n)
        if np.abs(wrong[n] - fd).max() > 1e-5 * max(1.0, float(np.abs(fd).max())):
            caught = True
            break
    assert caught, kind
