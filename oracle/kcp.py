"""Segment-parallel KDA forward (state-transition split), fp64.  TEST INFRASTRUCTURE ONLY.

The Kimi K3 paper digest (devpress.csdn.net), section 2.4 (1), splits the
recurrent state of a sequence segment into a transition-matrix part and a
zero-initial-state part, and reassembles the states across segments with a
prefix scan.  Written out for the recurrence of ``kda_oracle.c``: one token
maps the state affinely,

    S <- (I - beta k k^T) Diag(exp g) S + beta k v^T,

so a segment of tokens maps it as S_out = M S_in + B, where

    M = prod over the segment's tokens, latest on the left, of
        (I - beta_t k_t k_t^T) Diag(exp g_t)                    (d_k x d_k)
    B = the segment's final state from S_in = 0.

Here M is built from those explicit per-token matrices (not by running the
recurrence on the identity), B with the token recurrence of ``kda_fwd``; the
scan S_{p+1} = M_p S_p + B_p runs in segment order, and each segment's
outputs are the token recurrence started from its S_p.  The pins in
``tests/test_oracle.py`` tie the result to the whole-sequence recurrence.
"""
from __future__ import annotations

import numpy as np

from . import kda_fwd


def kcp_transition(k, g, beta) -> np.ndarray:
    """Transition matrix of a token span: k, g [B, L, H, Dk], beta [B, L, H] -> [B, H, Dk, Dk].

    The product of the per-token maps (I - beta k k^T) Diag(exp g), the first
    token's rightmost; the identity for an empty span.
    """
    k, g, beta = (np.asarray(x, dtype=np.float64) for x in (k, g, beta))
    B, L, H, Dk = k.shape
    M = np.broadcast_to(np.eye(Dk), (B, H, Dk, Dk)).copy()
    eye = np.eye(Dk)
    for t in range(L):
        kt = k[:, t]                                            # [B, H, Dk]
        erase = eye - beta[:, t, :, None, None] * kt[..., :, None] * kt[..., None, :]
        decay = np.exp(g[:, t])[..., :, None]                   # scales rows (key channels)
        M = erase @ (decay * M)
    return M


def kcp_fwd(q, k, v, g, beta, h0=None, n_seg: int = 1, scale=None):
    """KDA forward over ``n_seg`` equal segments, reassembled by the state scan.

    Shapes as ``kda_fwd``; T must be a multiple of n_seg and Dk == Dv is not
    required.  Returns (o, hT, parts) with parts = dict(M [B, P, H, Dk, Dk],
    Bs [B, P, H, Dk, Dv], S_in [B, P, H, Dk, Dv]) in fp64.
    """
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if n_seg < 1 or T % n_seg != 0:
        raise ValueError("T=%d is not a multiple of n_seg=%d" % (T, n_seg))
    L = T // n_seg
    M = np.zeros((B, n_seg, H, Dk, Dk))
    Bs = np.zeros((B, n_seg, H, Dk, Dv))
    S_in = np.zeros((B, n_seg, H, Dk, Dv))
    spans = [slice(p * L, (p + 1) * L) for p in range(n_seg)]
    for p, sp in enumerate(spans):
        M[:, p] = kcp_transition(k[:, sp], g[:, sp], beta[:, sp])
        _, Bs[:, p] = kda_fwd(q[:, sp], k[:, sp], v[:, sp], g[:, sp], beta[:, sp], h0=None, scale=scale)
    S = np.zeros((B, H, Dk, Dv)) if h0 is None else np.asarray(h0, dtype=np.float64).copy()
    for p in range(n_seg):
        S_in[:, p] = S
        S = M[:, p] @ S + Bs[:, p]
    o = np.zeros((B, T, H, Dv))
    for p, sp in enumerate(spans):
        o[:, sp], _ = kda_fwd(q[:, sp], k[:, sp], v[:, sp], g[:, sp], beta[:, sp], h0=S_in[:, p], scale=scale)
    return o, S, {"M": M, "Bs": Bs, "S_in": S_in}
