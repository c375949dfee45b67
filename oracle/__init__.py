"""Independent fp64 CPU oracle for the Kimi Delta Attention (KDA) forward pass.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  It shares no
code with the HIP library or its binding and imports neither.

Two implementations of the same token-by-token recurrence live here:

* ``kda_oracle.c`` (loaded with ctypes): plain C, fp64, OpenMP over (b, h).
  It is the oracle the GPU path is compared with.
* ``ref_numpy.py``: the same recurrence in numpy, vectorised over (b, h), used
  to cross-check the C code on small inputs.

``kcp.py`` adds the segment-parallel form of the same forward pass (per-segment
transition matrices and zero-start states, reassembled by a scan).

The recurrence follows the prose of "Kimi K3 Architecture Explained", section 3
"Kimi Delta Attention (KDA)" (decay stale context first, then erase, then
write; DeltaNet's eraser recalls with the incoming key and writes only the
difference) and the Kimi K3 paper digest (devpress.csdn.net), section 2.1 (1)
(delta-rule recursion with a per-channel forget gate on a fixed-size state).
The readings taken where the pages are silent are listed in the C file's
header.  Every function here is pinned by closed forms and invariants in
``tests/test_oracle.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

from .ref_numpy import kda_bwd_numpy, kda_fwd_numpy  # noqa: F401  (re-export)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_SRC_BWD = os.path.join(_HERE, "kda_oracle_bwd.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile ``kda_oracle.c`` and ``kda_oracle_bwd.c`` with gcc into ``libkda_oracle.so`` (fp64, OpenMP)."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", _SRC, _SRC_BWD, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build()
            lib = ctypes.CDLL(_LIB)
            dp = ctypes.POINTER(ctypes.c_double)
            L = ctypes.c_long
            lib.kda_oracle_fwd.argtypes = [dp] * 7 + [L] * 5 + [ctypes.c_double]
            lib.kda_oracle_fwd.restype = ctypes.c_int
            lib.kda_oracle_bwd.argtypes = [dp] * 14 + [L] * 5 + [ctypes.c_double]
            lib.kda_oracle_bwd.restype = ctypes.c_int
            lib.kda_oracle_num_threads.argtypes = []
            lib.kda_oracle_num_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def num_threads() -> int:
    """Threads the C oracle's OpenMP loop uses (OMP_NUM_THREADS or all cores)."""
    return int(_load().kda_oracle_num_threads())


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def gate_from_logit(x, g_min: float = -5.0) -> np.ndarray:
    """Per-channel log-decay from the gate logit, in fp64:
    ``g = g_min * sigmoid(x) = g_min / (1 + exp(-x))``.

    The bounded scaled-sigmoid gate with floor ``g_min`` of the Kimi K3 paper
    digest (devpress.csdn.net), section 2.1 (1) ("数值稳定优化"): the gate is
    kept in (g_min, 0) so that the in-chunk reciprocal factors stay in range.
    ``x`` is taken exactly as stored (bf16 or fp32 converted to fp64).
    """
    x = _f64(x.float().cpu().numpy() if hasattr(x, "float") else x)
    # exp(-x) overflows to inf for x < -709: the quotient is then 0, the limit
    with np.errstate(over="ignore"):
        return g_min / (1.0 + np.exp(-x))


def l2_normalize(x, eps: float = 1e-12) -> np.ndarray:
    """Every vector along the last axis divided by its Euclidean length, in
    fp64: ``x / max(||x||_2, eps)``.  A zero vector stays zero; a vector
    shorter than ``eps`` is divided by ``eps``.

    The q/k normalisation in front of the recurrence.  The pages do not write
    it out.  Reading: the erase-then-write step with the incoming key
    ("Kimi K3 Architecture Explained", section 3, the DeltaNet eraser) removes
    exactly the recalled value only for a unit key, and the bound on the
    state that the bounded gate of the Kimi K3 paper digest (devpress.csdn.net,
    section 2.1 (1)) protects assumes keys of bounded length; so keys (and,
    as is usual for delta-rule attention, queries) are unit vectors, with the
    floor ``eps`` keeping a zero vector finite.  ``x`` is taken exactly as
    stored (bf16 or fp32 converted to fp64).
    """
    x = _f64(x.float().cpu().numpy() if hasattr(x, "float") else x)
    length = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(length, eps)


def kda_fwd(q, k, v, g, beta, h0=None, scale=None):
    """Token-sequential KDA forward in fp64 (C implementation).

    q, k, g: [B, T, H, Dk]; v: [B, T, H, Dv]; beta: [B, T, H]; h0: [B, H, Dk, Dv]
    or None (zero state).  Any real dtype; values are converted exactly to fp64.
    scale defaults to Dk ** -0.5.  Returns (o [B, T, H, Dv], hT [B, H, Dk, Dv]),
    both fp64.
    """
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == (B, T, H, Dk) and g.shape == (B, T, H, Dk)
    assert v.shape == (B, T, H, Dv) and beta.shape == (B, T, H)
    S = np.zeros((B, H, Dk, Dv)) if h0 is None else _f64(h0).copy()
    assert S.shape == (B, H, Dk, Dv)
    o = np.zeros((B, T, H, Dv))
    if scale is None:
        scale = Dk ** -0.5
    rc = _load().kda_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                _ptr(S), _ptr(o), B, T, H, Dk, Dv, float(scale))
    if rc != 0:
        raise RuntimeError("kda_oracle_fwd failed with code %d" % rc)
    return o, S


def kda_bwd(q, k, v, g, beta, dO, h0=None, dhT=None, scale=None):
    """Gradients of the token-sequential KDA forward pass in fp64 (C implementation).

    Inputs as in :func:`kda_fwd`; dO [B, T, H, Dv] is dL/do and dhT
    [B, H, Dk, Dv] (or None for zero) is dL/dhT.  Returns
    (dq, dk, dv, dg, dbeta, dh0) shaped like (q, k, v, g, beta, states), fp64:
    the plain reverse-mode adjoint of the recurrence, token by token
    (kda_oracle_bwd.c).
    """
    q, k, v, g, beta, dO = (_f64(x) for x in (q, k, v, g, beta, dO))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == (B, T, H, Dk) and g.shape == (B, T, H, Dk)
    assert v.shape == (B, T, H, Dv) and beta.shape == (B, T, H) and dO.shape == (B, T, H, Dv)
    h0 = None if h0 is None else _f64(h0)
    dhT = None if dhT is None else _f64(dhT)
    for s_ in (h0, dhT):
        assert s_ is None or s_.shape == (B, H, Dk, Dv)
    dq, dk, dg = (np.zeros((B, T, H, Dk)) for _ in range(3))
    dv = np.zeros((B, T, H, Dv))
    dbeta = np.zeros((B, T, H))
    dh0 = np.zeros((B, H, Dk, Dv))
    if scale is None:
        scale = Dk ** -0.5
    null = ctypes.POINTER(ctypes.c_double)()
    rc = _load().kda_oracle_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                null if h0 is None else _ptr(h0), _ptr(dO), null if dhT is None else _ptr(dhT),
                                _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(dh0),
                                B, T, H, Dk, Dv, float(scale))
    if rc != 0:
        raise RuntimeError("kda_oracle_bwd failed with code %d" % rc)
    return dq, dk, dv, dg, dbeta, dh0


def kda_decode(q, k, v, g, beta, state, scale=None):
    """One-token KDA update: inputs [B, H, D] (beta [B, H]), state [B, H, Dk, Dv].

    Returns (o [B, H, Dv], new_state), fp64; the input state is not modified.
    This is ``kda_fwd`` with T = 1.
    """
    q, k, v, g = (_f64(x)[:, None] for x in (q, k, v, g))
    beta = _f64(beta)[:, None]
    o, S = kda_fwd(q, k, v, g, beta, h0=state, scale=scale)
    return o[:, 0], S
