"""Helpers for GPU tests: run the fp64 oracle on (a sample of) device inputs."""
from __future__ import annotations

import numpy as np
import torch

import kda_inputs
import oracle

TOL_BF16 = 2e-2
TOL_F32 = 1e-4

_NAMES = ("q", "k", "v", "g", "beta")


def tol_for(dtype: str) -> float:
    return TOL_BF16 if dtype == "bf16" else TOL_F32


def host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").double().numpy()


def oracle_full(x: dict, h0=None, scale=None):
    """Oracle on every (b, h, column) of a device input dict."""
    args = [host64(x[n]) for n in _NAMES]
    h = x.get("h0") if h0 is None else h0
    return oracle.kda_fwd(*args, h0=None if h is None else host64(h), scale=scale)


def oracle_sampled(x: dict, heads, cols, t0=0, t1=None, S0=None, h0_from_inputs=True):
    """Oracle on heads ``heads`` and value columns ``cols`` over tokens [t0, t1).

    Column j of the result depends only on v[..., j] and the initial state's
    column j, so a column subset is exact.  S0 ([B, len(heads), Dk, len(cols)]
    fp64) overrides the initial state; otherwise x["h0"] is sampled (or zero).
    Returns (o [B, t1-t0, len(heads), len(cols)], S) in fp64.
    """
    T = x["q"].shape[1]
    t1 = T if t1 is None else t1
    hi = torch.as_tensor(heads, device=x["q"].device)
    ci = torch.as_tensor(cols, device=x["q"].device)
    sl = lambda t: t[:, t0:t1].index_select(2, hi)
    q, k, g = (host64(sl(x[n])) for n in ("q", "k", "g"))
    v = host64(sl(x["v"]).index_select(3, ci))
    beta = host64(x["beta"][:, t0:t1].index_select(2, hi))
    if S0 is None and h0_from_inputs and x.get("h0") is not None:
        S0 = host64(x["h0"].index_select(1, hi).index_select(3, ci))
    return oracle.kda_fwd(q, k, v, g, beta, h0=S0)


def pick(t: torch.Tensor, heads, cols, head_dim=2, col_dim=3) -> torch.Tensor:
    hi = torch.as_tensor(heads, device=t.device)
    ci = torch.as_tensor(cols, device=t.device)
    return t.index_select(head_dim, hi).index_select(col_dim, ci).cpu()


rel_err = kda_inputs.rel_err
