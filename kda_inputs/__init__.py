"""Seeded synthetic inputs for the KDA forward pass.

This module only draws random tensors; it holds none of the recurrence's
arithmetic.  It serves both the HIP path's tests/benchmark and the CPU oracle,
which is why it lives in a package of its own.

Distributions (the workloads the path is measured on):

* q, k ~ N(0, 1), L2-normalised per (batch, token, head) in fp32 with
  ``x / max(||x||, 1e-12)``, then stored in the input dtype (bf16 by
  round-to-nearest-even, or fp32).  With ``raw_qk`` (inputs of the fused q/k
  normalisation) they are left unnormalised instead: N(0, 1) per channel
  times a length factor e^z per (batch, token, head), z ~ N(0, 1), drawn
  separately for q and k.
* v ~ N(0, 1), stored in the input dtype.
* beta = sigmoid(N(0, 1)) per (batch, token, head), fp32.
* g = g_min * sigmoid(x) per channel with x ~ N(mu, 1), g_min = -5 and mu = 0
  (mu = -4 gives the weak-decay stress case), fp32.  The bounded scaled-sigmoid
  gate with floor -5 is the parametrisation named in the Kimi K3 paper digest
  (devpress.csdn.net), section 2.1 (1), "数值稳定优化".
* initial / decode state ~ N(0, 0.01) (variance 0.01, std 0.1), fp32.

Every tensor is drawn from its own torch Philox/MT stream, seeded from
(seed, tensor id, segment), where a segment is SEGMENT tokens.  Any segment of
a long sequence can therefore be regenerated on its own, and a sequence is
generated segment by segment straight into a preallocated (device) tensor.
Streams differ between devices: tensors drawn on the GPU are copied to the host
when the oracle needs them.
"""
from __future__ import annotations

import dataclasses

import torch

SEGMENT = 65536
G_MIN = -5.0
CHUNK = 16

_TID = {"q": 0, "k": 1, "v": 2, "beta": 3, "gate": 4, "h0": 5, "q_len": 6, "k_len": 7}


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    name: str
    B: int
    H: int
    T: int
    D: int
    dtype: str          # "bf16" or "f32" (q, k, v storage)
    h0: bool            # random initial state (else zero)
    seed: int


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    B: int
    H: int
    D: int
    dtype: str
    seed: int


# The five measured workloads.
TINY = PrefillConfig("kda_tiny_f32_b1_h1_t64_d16", 1, 1, 64, 16, "f32", False, 20261201)
PREFILL_B4 = PrefillConfig("kda_prefill_bf16_b4_h16_t4096_d128_h0", 4, 16, 4096, 128, "bf16", True, 20261202)
PREFILL_64K = PrefillConfig("kda_prefill_bf16_b1_h56_t65536_d128", 1, 56, 65536, 128, "bf16", False, 20261203)
DECODE_B256 = DecodeConfig("kda_decode_bf16_b256_h56_d128", 256, 56, 128, "bf16", 20261204)
PREFILL_1M = PrefillConfig("kda_prefill_bf16_b1_h56_t1048576_d128_h0", 1, 56, 1 << 20, 128, "bf16", True, 20261205)

# One long sequence on a 7-head share of the 56 heads (the 56 heads split over
# 8 devices): too few (b, h) pairs to fill the device, the case of the
# segmented prefill.
PREFILL_256K_H7 = PrefillConfig("kda_prefill_bf16_b1_h7_t262144_d128", 1, 7, 1 << 18, 128, "bf16", False, 20261206)
PREFILL_CONFIGS = {c.name: c for c in (TINY, PREFILL_B4, PREFILL_64K, PREFILL_1M, PREFILL_256K_H7)}


def torch_dtype(name: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def _gen(seed: int, tid: int, seg: int, device) -> torch.Generator:
    gen = torch.Generator(device=device)
    gen.manual_seed((seed * 1_000_003 + tid * 65_537 + seg * 7_919) % (1 << 62))
    return gen


def _normal(shape, seed, tid, seg, device, mean=0.0, std=1.0):
    x = torch.empty(shape, dtype=torch.float32, device=device)
    x.normal_(mean, std, generator=_gen(seed, tid, seg, device))
    return x


def _unit(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)


def _raw(x: torch.Tensor, seed, tid, seg, device) -> torch.Tensor:
    return x * torch.exp(_normal(x.shape[:-1] + (1,), seed, tid, seg, device))


def fill_prefill_segment(bufs: dict, t0: int, t1: int, *, seed: int, seg: int,
                         gate_mean: float = 0.0, raw_qk: bool = False) -> None:
    """Draw tokens [t0, t1) of every per-token tensor into ``bufs`` (in place)."""
    q = bufs["q"]
    B, _, H, D = q.shape
    Dv = bufs["v"].shape[-1]
    dev = q.device
    n = t1 - t0
    for name in ("q", "k"):
        x = _normal((B, n, H, D), seed, _TID[name], seg, dev)
        x = _raw(x, seed, _TID[name + "_len"], seg, dev) if raw_qk else _unit(x)
        bufs[name][:, t0:t1] = x.to(q.dtype)
    bufs["v"][:, t0:t1] = _normal((B, n, H, Dv), seed, _TID["v"], seg, dev).to(q.dtype)
    bufs["beta"][:, t0:t1] = torch.sigmoid(_normal((B, n, H), seed, _TID["beta"], seg, dev))
    x = _normal((B, n, H, D), seed, _TID["gate"], seg, dev, mean=gate_mean)
    bufs["g"][:, t0:t1] = G_MIN * torch.sigmoid(x)
    if "x" in bufs:  # the gate logits themselves, in their storage dtype
        bufs["x"][:, t0:t1] = x.to(bufs["x"].dtype)


def prefill_inputs(B: int, T: int, H: int, D: int, dtype: str = "bf16", *,
                   h0: bool = False, seed: int = 0, device="cpu",
                   gate_mean: float = 0.0, Dv: int | None = None,
                   gate_logits: str | None = None, raw_qk: bool = False) -> dict:
    """Allocate and draw a full prefill input set.

    Returns a dict with q, k, v ([B, T, H, D], dtype), g ([B, T, H, D], fp32),
    beta ([B, T, H], fp32) and h0 ([B, H, D, Dv] fp32, or None).  With
    ``gate_logits`` ("f32" or "bf16") it also holds x, the gate logits g is
    drawn from, stored in that dtype.  ``raw_qk`` leaves q and k unnormalised
    (see the module docstring).
    """
    Dv = D if Dv is None else Dv
    td = torch_dtype(dtype)
    bufs = {
        "q": torch.empty((B, T, H, D), dtype=td, device=device),
        "k": torch.empty((B, T, H, D), dtype=td, device=device),
        "v": torch.empty((B, T, H, Dv), dtype=td, device=device),
        "g": torch.empty((B, T, H, D), dtype=torch.float32, device=device),
        "beta": torch.empty((B, T, H), dtype=torch.float32, device=device),
    }
    if gate_logits is not None:
        bufs["x"] = torch.empty((B, T, H, D), dtype=torch_dtype(gate_logits), device=device)
    for seg, t0 in enumerate(range(0, T, SEGMENT)):
        fill_prefill_segment(bufs, t0, min(T, t0 + SEGMENT), seed=seed, seg=seg, gate_mean=gate_mean,
                             raw_qk=raw_qk)
    bufs["h0"] = _normal((B, H, D, Dv), seed, _TID["h0"], 0, device, std=0.1) if h0 else None
    return bufs


def config_inputs(cfg: PrefillConfig, device="cpu", T: int | None = None) -> dict:
    """Inputs of a named prefill workload (optionally only its first T tokens)."""
    T = cfg.T if T is None else T
    return prefill_inputs(cfg.B, T, cfg.H, cfg.D, cfg.dtype, h0=cfg.h0, seed=cfg.seed, device=device)


def decode_inputs(B: int, H: int, D: int, dtype: str = "bf16", *, seed: int = 0,
                  device="cpu", gate_mean: float = 0.0, Dv: int | None = None, raw_qk: bool = False) -> dict:
    """One new token per sequence: q, k, v [B, H, D]; g [B, H, D]; beta [B, H];
    state [B, H, D, Dv] ~ N(0, 0.01), all drawn as for prefill."""
    Dv = D if Dv is None else Dv
    td = torch_dtype(dtype)

    def qk(name):
        x = _normal((B, H, D), seed, _TID[name], 0, device)
        return (_raw(x, seed, _TID[name + "_len"], 0, device) if raw_qk else _unit(x)).to(td)

    return {
        "q": qk("q"),
        "k": qk("k"),
        "v": _normal((B, H, Dv), seed, _TID["v"], 0, device).to(td),
        "beta": torch.sigmoid(_normal((B, H), seed, _TID["beta"], 0, device)),
        "g": G_MIN * torch.sigmoid(_normal((B, H, D), seed, _TID["gate"], 0, device, mean=gate_mean)),
        "state": _normal((B, H, D, Dv), seed, _TID["h0"], 0, device, std=0.1),
    }


def rel_err(x, ref) -> float:
    """max|x - ref| / rms(ref), over the whole tensor, in fp64."""
    x = torch.as_tensor(x).double().cpu()
    ref = torch.as_tensor(ref).double().cpu()
    rms = ref.pow(2).mean().sqrt().item()
    if rms == 0.0:
        return float((x - ref).abs().max().item()) if ref.numel() else 0.0
    return float((x - ref).abs().max().item() / rms)
