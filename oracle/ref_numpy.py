"""Second, independent writing of the KDA recurrence in numpy (fp64).

TEST INFRASTRUCTURE ONLY; used to cross-check the C oracle on small inputs.
Vectorised over (b, h); sequential over tokens.  Same source passages and
readings as ``kda_oracle.c``: decay the key channels, recall with the incoming
key, write beta times the difference, then read the updated state with the
query ("Kimi K3 Architecture Explained", section 3; Kimi K3 paper digest,
section 2.1 (1)).
"""
from __future__ import annotations

import numpy as np


def kda_fwd_numpy(q, k, v, g, beta, h0=None, scale=None):
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    S = np.zeros((B, H, Dk, Dv)) if h0 is None else np.array(h0, dtype=np.float64)
    if scale is None:
        scale = Dk ** -0.5
    o = np.zeros((B, T, H, Dv))
    for t in range(T):
        S = np.exp(g[:, t])[..., None] * S                       # decay key channels
        recalled = np.einsum("bhij,bhi->bhj", S, k[:, t])        # S^T k
        delta = beta[:, t][..., None] * (v[:, t] - recalled)     # beta (v - S^T k)
        S = S + k[:, t][..., :, None] * delta[..., None, :]      # S + k delta^T
        o[:, t] = scale * np.einsum("bhij,bhi->bhj", S, q[:, t])  # S^T q
    return o, S


def kda_bwd_numpy(q, k, v, g, beta, dO, h0=None, dhT=None, scale=None):
    """Gradients of the recurrence above by its reverse-mode adjoint (fp64),
    keeping every state of the forward pass (small inputs only).

    Returns (dq, dk, dv, dg, dbeta, dh0) shaped like (q, k, v, g, beta, h0).
    """
    q, k, v, g, beta, dO = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta, dO))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if scale is None:
        scale = Dk ** -0.5
    S = np.zeros((B, H, Dk, Dv)) if h0 is None else np.array(h0, dtype=np.float64)
    prev = []                     # S_{t-1} for every token
    for t in range(T):
        prev.append(S)
        Sd = np.exp(g[:, t])[..., None] * S
        rec = np.einsum("bhij,bhi->bhj", Sd, k[:, t])
        S = Sd + k[:, t][..., :, None] * (beta[:, t][..., None] * (v[:, t] - rec))[..., None, :]
    dS = np.zeros((B, H, Dk, Dv)) if dhT is None else np.array(dhT, dtype=np.float64)
    dq, dk, dv, dg = (np.zeros_like(x) for x in (q, k, v, g))
    dbeta = np.zeros_like(beta)
    for t in reversed(range(T)):
        a = np.exp(g[:, t])
        Sd = a[..., None] * prev[t]                               # decayed state
        rec = np.einsum("bhij,bhi->bhj", Sd, k[:, t])
        diff = v[:, t] - rec
        e = beta[:, t][..., None] * diff
        St = Sd + k[:, t][..., :, None] * e[..., None, :]
        dS = dS + scale * q[:, t][..., :, None] * dO[:, t][..., None, :]
        dq[:, t] = scale * np.einsum("bhij,bhj->bhi", St, dO[:, t])
        de = np.einsum("bhij,bhi->bhj", dS, k[:, t])
        dk[:, t] = np.einsum("bhij,bhj->bhi", dS, e)
        dbeta[:, t] = np.sum(de * diff, axis=-1)
        dv[:, t] = beta[:, t][..., None] * de
        drec = -beta[:, t][..., None] * de
        dSd = dS + k[:, t][..., :, None] * drec[..., None, :]
        dk[:, t] = dk[:, t] + np.einsum("bhij,bhj->bhi", Sd, drec)
        dg[:, t] = np.sum(dSd * Sd, axis=-1)
        dS = a[..., None] * dSd
    return dq, dk, dv, dg, dbeta, dS
