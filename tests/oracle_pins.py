"""Checks that pin the KDA oracle to facts other than itself.

Each ``pin_*`` takes a forward function ``fwd(q, k, v, g, beta, h0, scale) ->
(o, hT)`` (fp64 numpy arrays, layouts [B, T, H, D] / [B, H, Dk, Dv]) and raises
AssertionError if the function disagrees with a closed form, a special case or
an invariant that the pages and the mathematics fix.  The same pins run against
the C oracle, the numpy oracle and deliberately broken copies of the numpy
oracle (which must fail at least one pin).

Facts used, by source:
* "Kimi K3 Architecture Explained", section 3 "Kimi Delta Attention (KDA)":
  DeltaNet recalls with the incoming key and writes only the difference
  (exact recall of a unit key written with beta = 1); Gated DeltaNet adds a
  forget gate; KDA decays first, then erases, then writes.
* Kimi K3 paper digest (devpress.csdn.net), section 2.1 (1): per-channel
  forget gate on a fixed-size state; section 2.4 (1) KCP: the state splits into
  a transition part and a zero-initial-state part (linearity in h0); section
  2.4 (4): state checkpoints allow resuming a prefix (split-run equality).
* Special cases with textbook closed forms: single token; g = 0 with
  orthonormal keys (plain linear attention); beta = 2, v = 0 (a product of
  Householder reflections); beta = 0 and one-hot keys (decayed linear attention
  as a sum of decay products); d_k = d_v = 1 (a first-order scalar filter).
"""
from __future__ import annotations

import numpy as np

TOL = 1e-11


def _rng(seed):
    return np.random.default_rng(seed)


def _unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand_inputs(rng, B=2, T=12, H=3, Dk=6, Dv=5, h0=True):
    q = _unit_rows(rng.standard_normal((B, T, H, Dk)))
    k = _unit_rows(rng.standard_normal((B, T, H, Dk)))
    v = rng.standard_normal((B, T, H, Dv))
    g = -5.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H, Dk))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    S0 = 0.1 * rng.standard_normal((B, H, Dk, Dv)) if h0 else None
    return q, k, v, g, beta, S0


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a)
    b = np.asarray(b)
    scale = max(1.0, float(np.abs(b).max()) if b.size else 1.0)
    err = float(np.abs(a - b).max()) if a.size else 0.0
    assert err <= tol * scale, "%s: max abs err %.3e (scale %.3e)" % (what, err, scale)


def pin_single_token_zero_state(fwd):
    """T = 1, h0 = 0: o = scale * beta (q.k) v and hT = beta k v^T."""
    rng = _rng(1)
    q, k, v, g, beta, _ = _rand_inputs(rng, B=2, T=1, H=3, Dk=5, Dv=4, h0=False)
    scale = 0.37
    o, S = fwd(q, k, v, g, beta, None, scale)
    qk = np.sum(q[:, 0] * k[:, 0], axis=-1)                      # [B, H]
    o_ref = scale * (beta[:, 0] * qk)[..., None] * v[:, 0]
    S_ref = beta[:, 0][..., None, None] * k[:, 0][..., :, None] * v[:, 0][..., None, :]
    _close(o[:, 0], o_ref, what="single-token o")
    _close(S, S_ref, what="single-token hT")


def pin_single_token_with_state(fwd):
    """T = 1, h0 != 0: with D = Diag(exp g) h0 (decayed state),
    o = scale * (D^T q + beta (k.q) (v - D^T k)), hT = D + beta k (v - D^T k)^T."""
    rng = _rng(2)
    q, k, v, g, beta, S0 = _rand_inputs(rng, B=1, T=1, H=2, Dk=4, Dv=6)
    scale = 0.5
    o, S = fwd(q, k, v, g, beta, S0, scale)
    for h in range(2):
        D = np.diag(np.exp(g[0, 0, h])) @ S0[0, h]
        err = v[0, 0, h] - D.T @ k[0, 0, h]
        o_ref = scale * (D.T @ q[0, 0, h] + beta[0, 0, h] * np.dot(k[0, 0, h], q[0, 0, h]) * err)
        S_ref = D + beta[0, 0, h] * np.outer(k[0, 0, h], err)
        _close(o[0, 0, h], o_ref, what="single-token-with-state o")
        _close(S[0, h], S_ref, what="single-token-with-state hT")


def pin_exact_recall(fwd):
    """After any history, writing a unit key with beta = 1 makes the state
    return exactly the written value for that key: S_t^T k_t = v_t, so a query
    equal to the key reads scale * v_t."""
    rng = _rng(3)
    B, T, H, Dk, Dv = 1, 20, 2, 8, 5
    q, k, v, g, beta, S0 = _rand_inputs(rng, B=B, T=T, H=H, Dk=Dk, Dv=Dv)
    probe = [5, 11, 19]
    for t in probe:
        beta[:, t] = 1.0
        q[:, t] = k[:, t]
    scale = 0.25
    o, S = fwd(q, k, v, g, beta, S0, scale)
    for t in probe:
        _close(o[:, t], scale * v[:, t], what="exact recall at t=%d" % t)
    _close(np.einsum("bhij,bhi->bhj", S, k[:, T - 1]), v[:, T - 1], what="final-state recall")


def pin_deltanet_orthonormal(fwd):
    """g = 0 (no decay), beta = 1, h0 = 0, orthonormal keys: every erase term
    vanishes, so the result is plain (unnormalised) linear attention,
    o_t = scale * sum_{s<=t} (q_t . k_s) v_s and hT = sum_s k_s v_s^T."""
    rng = _rng(4)
    B, T, H, Dk, Dv = 1, 7, 2, 9, 4
    k = np.zeros((B, T, H, Dk))
    for h in range(H):
        Qm, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
        k[0, :, h] = Qm[:, :T].T
    q = rng.standard_normal((B, T, H, Dk))
    v = rng.standard_normal((B, T, H, Dv))
    g = np.zeros((B, T, H, Dk))
    beta = np.ones((B, T, H))
    scale = 0.3
    o, S = fwd(q, k, v, g, beta, None, scale)
    scores = np.einsum("bthi,bshi->bhts", q, k)
    causal = np.tril(np.ones((T, T)))
    o_ref = scale * np.einsum("bhts,bshj->bthj", scores * causal, v)
    _close(o, o_ref, what="DeltaNet orthonormal o")
    _close(S, np.einsum("bshi,bshj->bhij", k, v), what="DeltaNet orthonormal hT")


def pin_householder(fwd):
    """g = 0, beta = 2, v = 0, unit keys: each step maps S to (I - 2 k k^T) S,
    a reflection, so hT = H_T ... H_1 h0 and the Frobenius norm is preserved."""
    rng = _rng(5)
    B, T, H, Dk, Dv = 1, 9, 1, 5, 3
    q, k, v, g, beta, S0 = _rand_inputs(rng, B=B, T=T, H=H, Dk=Dk, Dv=Dv)
    g[:] = 0.0
    beta[:] = 2.0
    v[:] = 0.0
    _, S = fwd(q, k, v, g, beta, S0, 1.0)
    M = S0[0, 0].copy()
    for t in range(T):
        kk = k[0, t, 0]
        M = (np.eye(Dk) - 2.0 * np.outer(kk, kk)) @ M
    _close(S[0, 0], M, what="Householder product")
    assert abs(np.linalg.norm(S[0, 0]) - np.linalg.norm(S0[0, 0])) < 1e-12


def pin_beta_zero(fwd):
    """beta = 0: nothing is written; with G_t = sum_{s<=t} g_s,
    o_t = scale * (exp(G_t) * q_t)^T h0 and hT = Diag(exp(G_T)) h0."""
    rng = _rng(6)
    q, k, v, g, beta, S0 = _rand_inputs(rng, B=2, T=10, H=2, Dk=6, Dv=3)
    beta[:] = 0.0
    scale = 0.2
    o, S = fwd(q, k, v, g, beta, S0, scale)
    G = np.cumsum(g, axis=1)
    o_ref = scale * np.einsum("bthi,bhij->bthj", np.exp(G) * q, S0)
    _close(o, o_ref, what="beta=0 o")
    _close(S, np.exp(G[:, -1])[..., None] * S0, what="beta=0 hT")


def pin_one_hot_decayed_linear_attention(fwd):
    """Distinct one-hot keys, h0 = 0, any beta: the recalled value is always 0,
    so the method is decayed linear attention,
    o_t = scale * sum_{s<=t} beta_s ((q_t * exp(G_t - G_s)) . k_s) v_s and
    hT = sum_s beta_s exp(G_T - G_s) * k_s v_s^T, with G_t = sum_{u<=t} g_u."""
    rng = _rng(7)
    B, T, H, Dk, Dv = 1, 6, 2, 8, 3
    q, _, v, g, beta, _ = _rand_inputs(rng, B=B, T=T, H=H, Dk=Dk, Dv=Dv, h0=False)
    k = np.zeros((B, T, H, Dk))
    for h in range(H):
        idx = rng.permutation(Dk)[:T]
        k[0, np.arange(T), h, idx] = 1.0
    scale = 0.6
    o, S = fwd(q, k, v, g, beta, None, scale)
    G = np.cumsum(g, axis=1)
    o_ref = np.zeros_like(o)
    S_ref = np.zeros_like(S)
    for h in range(H):
        for t in range(T):
            for s in range(t + 1):
                w = np.dot(q[0, t, h] * np.exp(G[0, t, h] - G[0, s, h]), k[0, s, h])
                o_ref[0, t, h] += scale * beta[0, s, h] * w * v[0, s, h]
        for s in range(T):
            S_ref[0, h] += beta[0, s, h] * np.outer(np.exp(G[0, -1, h] - G[0, s, h]) * k[0, s, h], v[0, s, h])
    _close(o, o_ref, what="one-hot decayed LA o")
    _close(S, S_ref, what="one-hot decayed LA hT")


def pin_small_beta_limit(fwd):
    """beta = eps * b, h0 = 0, general unit keys: the erase term is O(eps^2),
    so o / eps tends to decayed linear attention with weights b."""
    rng = _rng(8)
    B, T, H, Dk, Dv = 1, 8, 1, 5, 4
    q, k, v, g, b, _ = _rand_inputs(rng, B=B, T=T, H=H, Dk=Dk, Dv=Dv, h0=False)
    G = np.cumsum(g, axis=1)
    ref = np.zeros((B, T, H, Dv))
    for t in range(T):
        for s in range(t + 1):
            w = np.dot(q[0, t, 0] * np.exp(G[0, t, 0] - G[0, s, 0]), k[0, s, 0])
            ref[0, t, 0] += b[0, s, 0] * w * v[0, s, 0]
    errs = []
    for eps in (1e-3, 1e-4):
        o, _ = fwd(q, k, v, g, eps * b, None, 1.0)
        errs.append(float(np.abs(o / eps - ref).max()))
    scale_ref = float(np.abs(ref).max())
    assert errs[1] < 1e-3 * scale_ref, errs
    assert errs[1] < 0.2 * errs[0], errs      # the gap shrinks linearly in eps


def pin_scalar_filter(fwd):
    """d_k = d_v = 1: S_t = a_t S_{t-1} + c_t with a_t = exp(g_t)(1 - beta_t k_t^2)
    and c_t = beta_t k_t v_t, so S_t = P_t S_0 + sum_{s<=t} (P_t / P_s) c_s with
    P_t = prod_{u<=t} a_u, and o_t = scale * S_t q_t."""
    rng = _rng(9)
    T = 30
    q = rng.standard_normal((1, T, 1, 1))
    k = rng.uniform(-1.2, 1.2, (1, T, 1, 1))
    v = rng.standard_normal((1, T, 1, 1))
    g = -rng.uniform(0.0, 1.0, (1, T, 1, 1))
    beta = rng.uniform(0.0, 1.0, (1, T, 1))
    S0 = np.array([[[[0.7]]]])
    o, S = fwd(q, k, v, g, beta, S0, 0.9)
    a = np.exp(g[0, :, 0, 0]) * (1.0 - beta[0, :, 0] * k[0, :, 0, 0] ** 2)
    c = beta[0, :, 0] * k[0, :, 0, 0] * v[0, :, 0, 0]
    P = np.cumprod(a)
    St = np.array([P[t] * 0.7 + sum(np.prod(a[s + 1:t + 1]) * c[s] for s in range(t + 1)) for t in range(T)])
    _close(o[0, :, 0, 0], 0.9 * St * q[0, :, 0, 0], what="scalar filter o")
    _close(S[0, 0, 0, 0], St[-1], what="scalar filter hT")


def pin_linearity(fwd):
    """(o, hT) is jointly linear in (v, h0), and o is linear in q; in
    particular hT(h0) = M h0 + hT(0) (the transition / zero-initial-state split
    used by KDA context parallelism)."""
    rng = _rng(10)
    q, k, v1, g, beta, h1 = _rand_inputs(rng, B=1, T=9, H=2, Dk=4, Dv=3)
    _, _, v2, _, _, h2 = _rand_inputs(rng, B=1, T=9, H=2, Dk=4, Dv=3)
    a, b = 0.7, -1.3
    o1, S1 = fwd(q, k, v1, g, beta, h1, 0.5)
    o2, S2 = fwd(q, k, v2, g, beta, h2, 0.5)
    o12, S12 = fwd(q, k, a * v1 + b * v2, g, beta, a * h1 + b * h2, 0.5)
    _close(o12, a * o1 + b * o2, what="linearity o")
    _close(S12, a * S1 + b * S2, what="linearity hT")
    q2 = rng.standard_normal(q.shape)
    oq, _ = fwd(a * q + b * q2, k, v1, g, beta, h1, 0.5)
    oq2, _ = fwd(q2, k, v1, g, beta, h1, 0.5)
    _close(oq, a * o1 + b * oq2, what="linearity in q")
    # transition matrix from the basis, applied to a random h0
    Dk = q.shape[-1]
    zero_v = np.zeros_like(v1)
    _, S0 = fwd(q, k, v1, g, beta, None, 0.5)
    M = np.zeros((2, Dk, Dk))
    for i in range(Dk):
        e = np.zeros((1, 2, Dk, Dk))
        e[0, :, i, i] = 1.0
        _, Se = fwd(q, k, np.zeros(v1.shape[:-1] + (Dk,)), g, beta, e, 0.5)
        M[:, :, i] = Se[0, :, :, i]
    _close(S1, np.einsum("hij,bhjk->bhik", M, h1) + S0, what="transition + zero-state split")
    del zero_v


def pin_state_passing(fwd):
    """Running a prefix, then resuming from its final state, equals one run:
    fwd(x[:T], h0) == fwd(x[T1:], h0 = hT(x[:T1], h0)) on o[T1:] and hT."""
    rng = _rng(11)
    q, k, v, g, beta, S0 = _rand_inputs(rng, B=2, T=15, H=2, Dk=5, Dv=4)
    o, S = fwd(q, k, v, g, beta, S0, 0.4)
    T1 = 6
    oa, Sa = fwd(q[:, :T1], k[:, :T1], v[:, :T1], g[:, :T1], beta[:, :T1], S0, 0.4)
    ob, Sb = fwd(q[:, T1:], k[:, T1:], v[:, T1:], g[:, T1:], beta[:, T1:], Sa, 0.4)
    _close(np.concatenate([oa, ob], axis=1), o, what="split-run o")
    _close(Sb, S, what="split-run hT")


def pin_column_and_head_independence(fwd):
    """Value column j of (o, S) depends only on v[..., j] and h0[..., j]; heads
    and batch rows are independent of each other."""
    rng = _rng(12)
    q, k, v, g, beta, S0 = _rand_inputs(rng, B=2, T=8, H=3, Dk=4, Dv=6)
    o, S = fwd(q, k, v, g, beta, S0, 0.5)
    cols = [1, 4]
    oc, Sc = fwd(q, k, v[..., cols], g, beta, S0[..., cols], 0.5)
    _close(oc, o[..., cols], what="column subset o")
    _close(Sc, S[..., cols], what="column subset hT")
    perm = [2, 0, 1]
    op, Sp = fwd(q[:, :, perm], k[:, :, perm], v[:, :, perm], g[:, :, perm], beta[:, :, perm], S0[:, perm], 0.5)
    _close(op, o[:, :, perm], what="head permutation o")
    _close(Sp, S[:, perm], what="head permutation hT")
    ob, Sb = fwd(q[1:], k[1:], v[1:], g[1:], beta[1:], S0[1:], 0.5)
    _close(ob, o[1:], what="batch row o")
    _close(Sb, S[1:], what="batch row hT")


ALL_PINS = [
    pin_single_token_zero_state,
    pin_single_token_with_state,
    pin_exact_recall,
    pin_deltanet_orthonormal,
    pin_householder,
    pin_beta_zero,
    pin_one_hot_decayed_linear_attention,
    pin_small_beta_limit,
    pin_scalar_filter,
    pin_linearity,
    pin_state_passing,
    pin_column_and_head_independence,
]
