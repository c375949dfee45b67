"""Python binding of the MI355X KDA forward library (``libkda.so``, include/kda.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  PyTorch provides device memory and the current
stream.  If the library has not been built this module raises on first use;
there is no CPU fallback.

    o, hT = chunk_fwd(q, k, v, g, beta, h0)      # prefill, optional initial state
    o = decode_step(q, k, v, g, beta, state)     # one token, state updated in place
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = ["chunk_bwd", "bwd_ws_bytes", "chunk_fwd", "chunk_fwd_ckpt", "chunk_fwd_gate", "chunk_fwd_kcp", "chunk_kda",
           "chunk_fwd_kcp_noalloc", "chunk_fwd_qknorm", "kcp_ws_bytes", "decode_step", "decode_step_qknorm",
           "KdaError", "library", "library_path", "version"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libkda.so")
_lock = threading.Lock()
_lib = None

KDA_OK = 0
KDA_F32 = 0
KDA_BF16 = 1
KDA_GATE_LOG_DECAY = 0
KDA_GATE_LOGIT_F32 = 1
KDA_GATE_LOGIT_BF16 = 2


class KdaError(RuntimeError):
    """A non-OK status from the C ABI; ``status`` holds the code."""

    def __init__(self, status: int, name: str, detail: str):
        super().__init__("%s: %s" % (name, detail))
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def library() -> ctypes.CDLL:
    """The loaded ``libkda.so`` with argument types set (raises if not built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise RuntimeError("libkda.so is not built (run `python -m linear_attention_recurrence_10_amd.build`)")
            lib = ctypes.CDLL(_LIB_PATH)
            vp, fp, i64 = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64
            lib.kda_chunk_fwd.argtypes = [vp, vp, vp, fp, fp, fp, fp, fp, i64, i64, i64, i64, i64,
                                          ctypes.c_int, ctypes.c_float, vp]
            lib.kda_chunk_fwd.restype = ctypes.c_int
            lib.kda_chunk_fwd_ckpt.argtypes = [vp, vp, vp, fp, fp, fp, fp, fp, fp, i64, i64, i64, i64, i64, i64,
                                               ctypes.c_int, ctypes.c_float, vp]
            lib.kda_chunk_fwd_ckpt.restype = ctypes.c_int
            lib.kda_chunk_fwd_gate.argtypes = [vp, vp, vp, vp, ctypes.c_int, ctypes.c_float, fp, fp, fp, fp,
                                               i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_float, vp]
            lib.kda_chunk_fwd_gate.restype = ctypes.c_int
            lib.kda_chunk_fwd_qknorm.argtypes = [vp, vp, vp, vp, ctypes.c_int, ctypes.c_float, ctypes.c_float, fp,
                                                 fp, fp, fp, i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_float,
                                                 vp]
            lib.kda_chunk_fwd_qknorm.restype = ctypes.c_int
            lib.kda_chunk_fwd_kcp.argtypes = [vp, vp, vp, fp, fp, fp, fp, fp, i64, vp, ctypes.c_uint64,
                                              i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_float, vp]
            lib.kda_chunk_fwd_kcp.restype = ctypes.c_int
            lib.kda_chunk_fwd_kcp_noalloc.argtypes = [vp, vp, vp, fp, fp, fp, fp, fp, i64, i64, i64, i64, i64, i64,
                                                      ctypes.c_int, ctypes.c_float, vp]
            lib.kda_chunk_fwd_kcp_noalloc.restype = ctypes.c_int
            lib.kda_chunk_fwd_kcp_noalloc_max_bytes.argtypes = []
            lib.kda_chunk_fwd_kcp_noalloc_max_bytes.restype = ctypes.c_uint64
            lib.kda_chunk_fwd_kcp_ws_bytes.argtypes = [i64, i64, i64, i64, i64, i64]
            lib.kda_chunk_fwd_kcp_ws_bytes.restype = ctypes.c_uint64
            lib.kda_chunk_bwd.argtypes = [vp, vp, vp, fp, fp, fp, fp, fp, fp, fp, fp, fp, fp, fp, vp,
                                          ctypes.c_uint64, i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_float, vp]
            lib.kda_chunk_bwd.restype = ctypes.c_int
            lib.kda_chunk_bwd_ws_bytes.argtypes = [i64, i64, i64, i64, i64]
            lib.kda_chunk_bwd_ws_bytes.restype = ctypes.c_uint64
            lib.kda_decode_step.argtypes = [vp, vp, vp, fp, fp, fp, fp, i64, i64, i64, i64,
                                            ctypes.c_int, ctypes.c_float, vp]
            lib.kda_decode_step.restype = ctypes.c_int
            lib.kda_decode_step_qknorm.argtypes = [vp, vp, vp, fp, fp, fp, fp, i64, i64, i64, i64,
                                                   ctypes.c_int, ctypes.c_float, ctypes.c_float, vp]
            lib.kda_decode_step_qknorm.restype = ctypes.c_int
            lib.kda_status_string.argtypes = [ctypes.c_int]
            lib.kda_status_string.restype = ctypes.c_char_p
            lib.kda_last_error.argtypes = []
            lib.kda_last_error.restype = ctypes.c_char_p
            lib.kda_version.argtypes = []
            lib.kda_version.restype = ctypes.c_int
            _lib = lib
    return _lib


def version() -> int:
    return int(library().kda_version())


def _check(status: int) -> None:
    if status != KDA_OK:
        lib = library()
        raise KdaError(status, lib.kda_status_string(status).decode(), lib.kda_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError("q, k, v and gate logits must be bfloat16 or float32, got %s" % t.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def chunk_fwd(q, k, v, g, beta, h0=None, *, scale: float | None = None, o=None, hT=None,
              output_final_state: bool = True, stream=None):
    """Chunked KDA prefill (``kda_chunk_fwd``).

    q, k: [B, T, H, Dk] and v: [B, T, H, Dv] (bf16 or fp32, same dtype); g:
    [B, T, H, Dk] fp32; beta: [B, T, H] fp32; h0: [B, H, Dk, Dv] fp32 or None.
    Returns (o [B, T, H, Dv] fp32, hT [B, H, Dk, Dv] fp32 or None).  ``o`` and
    ``hT`` may be given to write into (``hT`` may be ``h0`` itself).
    """
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    _need(g, "g", torch.float32)
    _need(beta, "beta", torch.float32)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if h0 is not None:
        _need(h0, "h0", torch.float32)
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=torch.float32, device=q.device)
    _need(o, "o", torch.float32)
    if hT is None and output_final_state:
        hT = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device)
    if hT is not None:
        _need(hT, "hT", torch.float32)
    shapes_ok = (k.shape == q.shape and g.shape == q.shape and v.shape[:3] == (B, T, H)
                 and beta.shape == (B, T, H) and o.shape == (B, T, H, Dv)
                 and (h0 is None or h0.shape == (B, H, Dk, Dv))
                 and (hT is None or hT.shape == (B, H, Dk, Dv)))
    if not shapes_ok:
        raise ValueError("inconsistent shapes")
    lib = library()
    _check(lib.kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o), _ptr(hT),
                             B, T, H, Dk, Dv, _dtype_code(q), float(scale or 0.0), _stream(stream)))
    return o, hT


def chunk_fwd_gate(q, k, v, x, beta, h0=None, *, g_min: float = -5.0, scale: float | None = None, o=None,
                   hT=None, output_final_state: bool = True, stream=None):
    """Chunked KDA prefill with the gate given as its logit (``kda_chunk_fwd_gate``).

    x: [B, T, H, Dk] gate logits, fp32 or bf16; the kernel uses the log-decay
    g = g_min * sigmoid(x), with -5 <= g_min < 0.  Everything else as
    :func:`chunk_fwd`.
    """
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    _need(x, "x")
    _need(beta, "beta", torch.float32)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if h0 is not None:
        _need(h0, "h0", torch.float32)
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=torch.float32, device=q.device)
    _need(o, "o", torch.float32)
    if hT is None and output_final_state:
        hT = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device)
    if hT is not None:
        _need(hT, "hT", torch.float32)
    shapes_ok = (k.shape == q.shape and x.shape == q.shape and v.shape[:3] == (B, T, H)
                 and beta.shape == (B, T, H) and o.shape == (B, T, H, Dv)
                 and (h0 is None or h0.shape == (B, H, Dk, Dv))
                 and (hT is None or hT.shape == (B, H, Dk, Dv)))
    if not shapes_ok:
        raise ValueError("inconsistent shapes")
    lib = library()
    _check(lib.kda_chunk_fwd_gate(_ptr(q), _ptr(k), _ptr(v), _ptr(x), _dtype_code(x), float(g_min), _ptr(beta),
                                  _ptr(h0), _ptr(o), _ptr(hT), B, T, H, Dk, Dv, _dtype_code(q),
                                  float(scale or 0.0), _stream(stream)))
    return o, hT


def chunk_fwd_qknorm(q, k, v, g, beta, h0=None, *, eps: float = 1e-12, gate_logits: bool = False,
                     g_min: float = -5.0, scale: float | None = None, o=None, hT=None,
                     output_final_state: bool = True, stream=None):
    """Chunked KDA prefill with q and k normalised in the kernel (``kda_chunk_fwd_qknorm``).

    q and k are the raw (unnormalised) vectors; each is used as
    x / max(||x||, eps).  g is the fp32 log-decay, or with ``gate_logits`` the
    gate logits (fp32 or bf16) with g = g_min * sigmoid(x).  Everything else
    as :func:`chunk_fwd`.
    """
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    if gate_logits:
        _need(g, "g")
        gate = KDA_GATE_LOGIT_BF16 if _dtype_code(g) == KDA_BF16 else KDA_GATE_LOGIT_F32
    else:
        _need(g, "g", torch.float32)
        gate = KDA_GATE_LOG_DECAY
    _need(beta, "beta", torch.float32)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if h0 is not None:
        _need(h0, "h0", torch.float32)
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=torch.float32, device=q.device)
    _need(o, "o", torch.float32)
    if hT is None and output_final_state:
        hT = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device)
    if hT is not None:
        _need(hT, "hT", torch.float32)
    shapes_ok = (k.shape == q.shape and g.shape == q.shape and v.shape[:3] == (B, T, H)
                 and beta.shape == (B, T, H) and o.shape == (B, T, H, Dv)
                 and (h0 is None or h0.shape == (B, H, Dk, Dv))
                 and (hT is None or hT.shape == (B, H, Dk, Dv)))
    if not shapes_ok:
        raise ValueError("inconsistent shapes")
    lib = library()
    _check(lib.kda_chunk_fwd_qknorm(_ptr(q), _ptr(k), _ptr(v), _ptr(g), gate, float(g_min), float(eps), _ptr(beta),
                                    _ptr(h0), _ptr(o), _ptr(hT), B, T, H, Dk, Dv, _dtype_code(q),
                                    float(scale or 0.0), _stream(stream)))
    return o, hT


def kcp_ws_bytes(B: int, T: int, H: int, Dk: int, Dv: int, n_seg: int) -> int:
    """Workspace bytes of :func:`chunk_fwd_kcp` (``kda_chunk_fwd_kcp_ws_bytes``); 0 if none is needed."""
    return int(library().kda_chunk_fwd_kcp_ws_bytes(B, T, H, Dk, Dv, n_seg))


def chunk_fwd_kcp(q, k, v, g, beta, h0=None, *, n_seg: int, ws=None, scale: float | None = None, o=None,
                  hT=None, output_final_state: bool = True, stream=None):
    """Chunked KDA prefill over ``n_seg`` parallel segments (``kda_chunk_fwd_kcp``).

    Arguments and results as in :func:`chunk_fwd`; T must be a multiple of
    ``n_seg``.  ``ws`` is an optional device byte tensor of at least
    :func:`kcp_ws_bytes` bytes (allocated here when omitted).
    """
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    _need(g, "g", torch.float32)
    _need(beta, "beta", torch.float32)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if h0 is not None:
        _need(h0, "h0", torch.float32)
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=torch.float32, device=q.device)
    _need(o, "o", torch.float32)
    if hT is None and output_final_state:
        hT = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device)
    if hT is not None:
        _need(hT, "hT", torch.float32)
    shapes_ok = (k.shape == q.shape and g.shape == q.shape and v.shape[:3] == (B, T, H)
                 and beta.shape == (B, T, H) and o.shape == (B, T, H, Dv)
                 and (h0 is None or h0.shape == (B, H, Dk, Dv))
                 and (hT is None or hT.shape == (B, H, Dk, Dv)))
    if not shapes_ok:
        raise ValueError("inconsistent shapes")
    lib = library()
    need = int(lib.kda_chunk_fwd_kcp_ws_bytes(B, T, H, Dk, Dv, n_seg))
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    if ws is not None:
        _need(ws, "ws")
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(lib.kda_chunk_fwd_kcp(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o), _ptr(hT),
                                 int(n_seg), _ptr(ws), ws_bytes, B, T, H, Dk, Dv, _dtype_code(q),
                                 float(scale or 0.0), _stream(stream)))
    return o, hT


def chunk_fwd_kcp_noalloc(q, k, v, g, beta, h0=None, *, n_seg: int, scale: float | None = None, o=None, hT=None,
                          output_final_state: bool = True, stream=None):
    """:func:`chunk_fwd_kcp` with the library's fixed per-device workspace
    (``kda_chunk_fwd_kcp_noalloc``): the C call allocates nothing.  Pass ``o``
    (and ``hT``) to keep this function allocation-free as well.  Calls that
    overlap in time on one device race on that workspace."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    _need(g, "g", torch.float32)
    _need(beta, "beta", torch.float32)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if h0 is not None:
        _need(h0, "h0", torch.float32)
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=torch.float32, device=q.device)
    _need(o, "o", torch.float32)
    if hT is None and output_final_state:
        hT = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device)
    if hT is not None:
        _need(hT, "hT", torch.float32)
    shapes_ok = (k.shape == q.shape and g.shape == q.shape and v.shape[:3] == (B, T, H)
                 and beta.shape == (B, T, H) and o.shape == (B, T, H, Dv)
                 and (h0 is None or h0.shape == (B, H, Dk, Dv))
                 and (hT is None or hT.shape == (B, H, Dk, Dv)))
    if not shapes_ok:
        raise ValueError("inconsistent shapes")
    lib = library()
    _check(lib.kda_chunk_fwd_kcp_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o),
                                         _ptr(hT), int(n_seg), B, T, H, Dk, Dv, _dtype_code(q),
                                         float(scale or 0.0), _stream(stream)))
    return o, hT


def chunk_fwd_ckpt(q, k, v, g, beta, h0=None, *, ckpt_every: int, scale: float | None = None, o=None,
                   hT=None, ckpt=None, output_final_state: bool = True, write_o: bool = True, stream=None):
    """Chunked KDA prefill that also returns state checkpoints (``kda_chunk_fwd_ckpt``).

    Arguments as in :func:`chunk_fwd`; ``ckpt_every`` is the number of tokens
    between checkpoints (a positive multiple of 16).  Returns (o, hT, ckpt)
    with ckpt [T // ckpt_every, B, H, Dk, Dv] fp32: ckpt[i] is the state
    after the first (i + 1) * ckpt_every tokens, usable as ``h0``.  With
    ``write_o=False`` no output is formed (o is None; pass no ``o``): only the
    states are written, by a cheaper pass.
    """
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    _need(g, "g", torch.float32)
    _need(beta, "beta", torch.float32)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if h0 is not None:
        _need(h0, "h0", torch.float32)
    if not write_o:
        if o is not None:
            raise ValueError("write_o=False takes no o")
    else:
        if o is None:
            o = torch.empty((B, T, H, Dv), dtype=torch.float32, device=q.device)
        _need(o, "o", torch.float32)
    if hT is None and output_final_state:
        hT = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device)
    if hT is not None:
        _need(hT, "hT", torch.float32)
    n_ckpt = T // ckpt_every if ckpt_every > 0 else 0
    if ckpt is None:
        ckpt = torch.empty((n_ckpt, B, H, Dk, Dv), dtype=torch.float32, device=q.device)
    _need(ckpt, "ckpt", torch.float32)
    shapes_ok = (k.shape == q.shape and g.shape == q.shape and v.shape[:3] == (B, T, H)
                 and beta.shape == (B, T, H) and (o is None or o.shape == (B, T, H, Dv))
                 and (h0 is None or h0.shape == (B, H, Dk, Dv))
                 and (hT is None or hT.shape == (B, H, Dk, Dv))
                 and ckpt.shape == (n_ckpt, B, H, Dk, Dv))
    if not shapes_ok:
        raise ValueError("inconsistent shapes")
    lib = library()
    # with no checkpoint to write (T < ckpt_every) the tensor is empty and may have no storage; a
    # non-null placeholder keeps ckpt_every validated by the library, which never touches ckpt then
    ck = _ptr(ckpt) if ckpt.numel() > 0 else ctypes.c_void_p(16)
    _check(lib.kda_chunk_fwd_ckpt(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o), _ptr(hT),
                                  ck, int(ckpt_every), B, T, H, Dk, Dv, _dtype_code(q), float(scale or 0.0),
                                  _stream(stream)))
    return o, hT, ckpt


def bwd_ws_bytes(B: int, T: int, H: int, Dk: int, Dv: int) -> int:
    """Workspace bytes of :func:`chunk_bwd` (``kda_chunk_bwd_ws_bytes``)."""
    return int(library().kda_chunk_bwd_ws_bytes(B, T, H, Dk, Dv))


def chunk_bwd(q, k, v, g, beta, dO, h0=None, dhT=None, *, scale: float | None = None, need_dh0: bool = True,
              ws=None, out=None, stream=None):
    """Gradients of :func:`chunk_fwd` (``kda_chunk_bwd``).

    Inputs as in :func:`chunk_fwd`; dO [B, T, H, Dv] fp32 is dL/do and dhT
    [B, H, Dk, Dv] fp32 (or None for zero) is dL/dhT.  Returns
    (dq, dk, dv, dg, dbeta, dh0), fp32, shaped like (q, k, v, g, beta, h0);
    dh0 is None unless ``need_dh0``.  ``ws`` is an optional device byte
    tensor of at least :func:`bwd_ws_bytes` bytes (allocated here when
    omitted); ``out`` an optional tuple of the six output tensors.
    """
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    _need(g, "g", torch.float32)
    _need(beta, "beta", torch.float32)
    _need(dO, "dO", torch.float32)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    for t, n in ((h0, "h0"), (dhT, "dhT")):
        if t is not None:
            _need(t, n, torch.float32)
    if out is None:
        f32 = dict(dtype=torch.float32, device=q.device)
        out = (torch.empty((B, T, H, Dk), **f32), torch.empty((B, T, H, Dk), **f32),
               torch.empty((B, T, H, Dv), **f32), torch.empty((B, T, H, Dk), **f32),
               torch.empty((B, T, H), **f32), torch.empty((B, H, Dk, Dv), **f32) if need_dh0 else None)
    dq, dk, dv, dg, dbeta, dh0 = out
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv"), (dg, "dg"), (dbeta, "dbeta")):
        _need(t, n, torch.float32)
    if dh0 is not None:
        _need(dh0, "dh0", torch.float32)
    shapes_ok = (k.shape == q.shape and g.shape == q.shape and v.shape[:3] == (B, T, H)
                 and beta.shape == (B, T, H) and dO.shape == (B, T, H, Dv)
                 and all(t is None or t.shape == (B, H, Dk, Dv) for t in (h0, dhT, dh0))
                 and dq.shape == q.shape and dk.shape == q.shape and dg.shape == q.shape
                 and dv.shape == v.shape and dbeta.shape == beta.shape)
    if not shapes_ok:
        raise ValueError("inconsistent shapes")
    lib = library()
    need = int(lib.kda_chunk_bwd_ws_bytes(B, T, H, Dk, Dv))
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _need(ws, "ws")
    ws_bytes = ws.numel() * ws.element_size()
    _check(lib.kda_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(dO), _ptr(dhT),
                             _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(dh0), _ptr(ws), ws_bytes,
                             B, T, H, Dk, Dv, _dtype_code(q), float(scale or 0.0), _stream(stream)))
    return dq, dk, dv, dg, dbeta, dh0


class _ChunkKDA(torch.autograd.Function):
    """The prefill as an autograd function: forward is kda_chunk_fwd, backward kda_chunk_bwd."""

    @staticmethod
    def forward(ctx, q, k, v, g, beta, h0, scale):
        o, hT = chunk_fwd(q, k, v, g, beta, h0, scale=scale)
        ctx.save_for_backward(q, k, v, g, beta, h0)
        ctx.scale = scale
        return o, hT

    @staticmethod
    def backward(ctx, dO, dhT):
        q, k, v, g, beta, h0 = ctx.saved_tensors
        need_dh0 = h0 is not None and ctx.needs_input_grad[5]
        dq, dk, dv, dg, dbeta, dh0 = chunk_bwd(q, k, v, g, beta, dO.float().contiguous(), h0,
                                               dhT.float().contiguous(), scale=ctx.scale, need_dh0=need_dh0)
        # the gradients of q, k and v take their inputs' dtype (rounded from fp32 for bf16 inputs)
        return dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), dg, dbeta, dh0, None


def chunk_kda(q, k, v, g, beta, h0=None, *, scale: float | None = None):
    """Differentiable chunked KDA prefill: returns (o, hT) as :func:`chunk_fwd`,
    with gradients for q, k, v, g, beta and h0 from :func:`chunk_bwd`."""
    return _ChunkKDA.apply(q, k, v, g, beta, h0, scale)


def decode_step(q, k, v, g, beta, state, *, scale: float | None = None, o=None, stream=None):
    """One-token KDA update (``kda_decode_step``); ``state`` is updated in place.

    q, k: [B, H, Dk], v: [B, H, Dv] (bf16 or fp32); g: [B, H, Dk] fp32; beta:
    [B, H] fp32; state: [B, H, Dk, Dv] fp32.  Returns o [B, H, Dv] fp32.
    """
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    _need(g, "g", torch.float32)
    _need(beta, "beta", torch.float32)
    _need(state, "state", torch.float32)
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    if o is None:
        o = torch.empty((B, H, Dv), dtype=torch.float32, device=q.device)
    _need(o, "o", torch.float32)
    if not (k.shape == q.shape and g.shape == q.shape and v.shape[:2] == (B, H) and beta.shape == (B, H)
            and state.shape == (B, H, Dk, Dv) and o.shape == (B, H, Dv)):
        raise ValueError("inconsistent shapes")
    lib = library()
    _check(lib.kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(o),
                               B, H, Dk, Dv, _dtype_code(q), float(scale or 0.0), _stream(stream)))
    return o


def decode_step_qknorm(q, k, v, g, beta, state, *, eps: float = 1e-12, scale: float | None = None, o=None,
                       stream=None):
    """:func:`decode_step` with q and k normalised in the kernel (``kda_decode_step_qknorm``):
    each is used as x / max(||x||, eps)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    _need(g, "g", torch.float32)
    _need(beta, "beta", torch.float32)
    _need(state, "state", torch.float32)
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    if o is None:
        o = torch.empty((B, H, Dv), dtype=torch.float32, device=q.device)
    _need(o, "o", torch.float32)
    if not (k.shape == q.shape and g.shape == q.shape and v.shape[:2] == (B, H) and beta.shape == (B, H)
            and state.shape == (B, H, Dk, Dv) and o.shape == (B, H, Dv)):
        raise ValueError("inconsistent shapes")
    lib = library()
    _check(lib.kda_decode_step_qknorm(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(o),
                                      B, H, Dk, Dv, _dtype_code(q), float(scale or 0.0), float(eps),
                                      _stream(stream)))
    return o
