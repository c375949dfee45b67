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
