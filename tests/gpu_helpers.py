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


class ErrAcc:
    """One ``max|x - ref| / rms(ref)`` over a tensor that is compared in pieces.

    ``add`` takes one piece (any shape) and keeps the running maximum of the
    absolute error and the running sum of squares of the reference, so the
    result equals ``rel_err`` of the whole tensor while only one piece is held
    on the host at a time.
    """

    def __init__(self):
        self.max_err = 0.0
        self.sumsq = 0.0
        self.n = 0

    def add(self, x, ref) -> None:
        x = torch.as_tensor(x).double().cpu()
        ref = torch.as_tensor(ref).double().cpu()
        assert x.shape == ref.shape, (x.shape, ref.shape)
        if ref.numel() == 0:
            return
        self.max_err = max(self.max_err, float((x - ref).abs().max().item()))
        self.sumsq += float(ref.pow(2).sum().item())
        self.n += ref.numel()

    def value(self) -> float:
        rms = (self.sumsq / self.n) ** 0.5 if self.n else 0.0
        return self.max_err / rms if rms > 0.0 else self.max_err


def head_groups(H: int, per: int):
    """Consecutive head index lists of at most ``per`` heads covering 0 .. H-1."""
    return [list(range(h, min(H, h + per))) for h in range(0, H, per)]


def oracle_heads(x: dict, heads, t0=0, t1=None, S0=None, g=None):
    """Oracle over every value column of heads ``heads``, tokens [t0, t1).

    S0 ([B, len(heads), Dk, Dv] fp64) is the initial state; when None,
    x["h0"] of those heads is used (or zeros).  ``g`` overrides x["g"] (for the
    gate-logit entry, whose log-decay the oracle forms itself).
    Returns (o [B, t1-t0, len(heads), Dv], S [B, len(heads), Dk, Dv]) in fp64.
    """
    T = x["q"].shape[1]
    t1 = T if t1 is None else t1
    hi = torch.as_tensor(heads, device=x["q"].device)
    sl = lambda t: t[:, t0:t1].index_select(2, hi)
    q, k, v = (host64(sl(x[n])) for n in ("q", "k", "v"))
    gg = host64(sl(x["g"])) if g is None else np.ascontiguousarray(g)
    beta = host64(x["beta"][:, t0:t1].index_select(2, hi))
    if S0 is None and x.get("h0") is not None:
        S0 = host64(x["h0"].index_select(1, hi))
    return oracle.kda_fwd(q, k, v, gg, beta, h0=S0)
