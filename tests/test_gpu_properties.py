"""Properties of the HIP path that hold at any size, and C-ABI error handling
on a real device (all rejected before any launch)."""
from __future__ import annotations

import ctypes
import os
import sys

import pytest
import torch

import kda_inputs
import linear_attention_recurrence_10_amd as kda
from gpu_helpers import rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def fwd(x, h0=None, sl=slice(None)):
    return kda.chunk_fwd(x["q"][:, sl].contiguous(), x["k"][:, sl].contiguous(), x["v"][:, sl].contiguous(),
                         x["g"][:, sl].contiguous(), x["beta"][:, sl].contiguous(), h0)


@pytest.mark.parametrize("T1", [16, 37, 512])
def test_split_run_matches_single_run(T1):
    """Resuming from a prefix's final state equals one pass (state checkpoints)."""
    x = kda_inputs.prefill_inputs(2, 1024, 4, 128, "bf16", h0=True, seed=41, device=DEV)
    o, hT = fwd(x, x["h0"])
    oa, ha = fwd(x, x["h0"], slice(0, T1))
    ob, hb = fwd(x, ha, slice(T1, None))
    torch.cuda.synchronize()
    assert rel_err(torch.cat([oa, ob], 1).cpu(), o.cpu()) < 1e-3
    assert rel_err(hb.cpu(), hT.cpu()) < 1e-3


def test_prefill_then_decode_equals_longer_prefill():
    x = kda_inputs.prefill_inputs(3, 101, 4, 128, "bf16", h0=True, seed=42, device=DEV)
    o_full, h_full = fwd(x, x["h0"])
    _, h_pre = fwd(x, x["h0"], slice(0, 100))
    st = h_pre.clone()
    od = kda.decode_step(*(x[n][:, 100].contiguous() for n in ("q", "k", "v", "g", "beta")), st)
    torch.cuda.synchronize()
    assert rel_err(od.cpu(), o_full[:, 100].cpu()) < 1e-3
    assert rel_err(st.cpu(), h_full.cpu()) < 1e-3


def test_repeat_runs_are_bitwise_identical():
    x = kda_inputs.prefill_inputs(2, 300, 8, 128, "bf16", h0=True, seed=43, device=DEV)
    o1, h1 = fwd(x, x["h0"])
    o2, h2 = fwd(x, x["h0"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


def test_value_columns_are_independent():
    """Changing value column j changes nothing in any other column."""
    x = kda_inputs.prefill_inputs(1, 200, 2, 128, "bf16", h0=True, seed=44, device=DEV)
    o1, h1 = fwd(x, x["h0"])
    x["v"][..., 70] = -x["v"][..., 70] * 3
    o2, h2 = fwd(x, x["h0"])
    torch.cuda.synchronize()
    keep = [j for j in range(128) if j != 70]
    assert torch.equal(o1[..., keep], o2[..., keep]) and torch.equal(h1[..., keep], h2[..., keep])
    assert not torch.equal(o1[..., 70], o2[..., 70])


def test_heads_and_batches_are_independent():
    x = kda_inputs.prefill_inputs(2, 64, 5, 128, "bf16", h0=True, seed=45, device=DEV)
    o1, h1 = fwd(x, x["h0"])
    perm = torch.tensor([3, 0, 4, 1, 2], device=DEV)
    xp = {n: x[n].index_select(2, perm).contiguous() for n in ("q", "k", "v", "g", "beta")}
    o2, h2 = fwd(xp, x["h0"].index_select(1, perm).contiguous())
    torch.cuda.synchronize()
    assert torch.equal(o2, o1.index_select(2, perm)) and torch.equal(h2, h1.index_select(1, perm))


def test_linearity_in_values_and_state():
    x = kda_inputs.prefill_inputs(1, 96, 2, 128, "f32", h0=True, seed=46, device=DEV)
    o1, h1 = fwd(x, x["h0"])
    y = dict(x)
    y["v"] = 2.0 * x["v"]
    o2, h2 = fwd(y, 2.0 * x["h0"])
    torch.cuda.synchronize()
    assert rel_err(o2.cpu(), 2.0 * o1.cpu()) < 1e-5 and rel_err(h2.cpu(), 2.0 * h1.cpu()) < 1e-5


def test_decode_repeated_steps_track_prefill():
    """Eight decode steps in a row equal an 8-token prefill from the same state."""
    x = kda_inputs.prefill_inputs(4, 8, 3, 128, "bf16", h0=True, seed=47, device=DEV)
    o_ref, h_ref = fwd(x, x["h0"])
    st = x["h0"].clone()
    outs = []
    for t in range(8):
        outs.append(kda.decode_step(*(x[n][:, t].contiguous() for n in ("q", "k", "v", "g", "beta")), st))
    torch.cuda.synchronize()
    assert rel_err(torch.stack(outs, 1).cpu(), o_ref.cpu()) < 1e-3
    assert rel_err(st.cpu(), h_ref.cpu()) < 1e-3


# --- C-ABI errors on a device (nothing is launched) ------------------------

def _call(q, k, v, g, beta, h0, o, hT, B, T, H, D, dtype=1, ptr_override=None):
    lib = kda.library()
    ptrs = [None if t is None else t.data_ptr() for t in (q, k, v, g, beta, h0, o, hT)]
    if ptr_override:
        for i, p in ptr_override.items():
            ptrs[i] = p
    ptrs = [None if p is None else ctypes.c_void_p(p) for p in ptrs]
    return lib.kda_chunk_fwd(*ptrs, B, T, H, D, D, dtype, 0.0, None), lib.kda_last_error().decode()


def _small():
    x = kda_inputs.prefill_inputs(1, 32, 2, 128, "bf16", h0=True, seed=48, device=DEV)
    o = torch.empty(1, 32, 2, 128, device=DEV)
    hT = torch.empty(1, 2, 128, 128, device=DEV)
    return x, o, hT


def test_abi_rejects_host_pointer():
    x, o, hT = _small()
    host = torch.zeros(1, 32, 2, 128, dtype=torch.bfloat16)
    st, msg = _call(host, x["k"], x["v"], x["g"], x["beta"], x["h0"], o, hT, 1, 32, 2, 128)
    assert st == 1 and "not a device allocation" in msg


def test_abi_rejects_misaligned_pointer():
    x, o, hT = _small()
    st, msg = _call(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], o, hT, 1, 32, 2, 128,
                    ptr_override={0: x["q"].data_ptr() + 2})
    assert st == 1 and "aligned" in msg


def test_abi_rejects_buffer_too_small():
    x, o, hT = _small()
    # claim 1,000,000 tokens for 32-token buffers in a fresh, separately allocated pool
    big_T = 1 << 26
    st, msg = _call(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], o, hT, 1, big_T, 2, 128)
    assert st == 1 and ("past the end" in msg or "overlaps" in msg)


def test_binding_raises_kda_error():
    x, o, hT = _small()
    with pytest.raises(kda.KdaError):
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], o=x["g"].view(1, 32, 2, 128))


@pytest.mark.parametrize("dtype,tol", [("bf16", 2e-3), ("f32", 2e-5)])
def test_mfma_and_valu_kernels_agree(tmp_path, dtype, tol):
    """The matrix-core kernels (bf16 pairs for bf16 inputs, fp32 products for
    fp32 inputs, d=128) and the fp32 vector kernel compute the same chunk
    form; all are checked against the oracle elsewhere.  The library reads
    KDA_DISABLE_MFMA once per process, so the vector kernel runs in a child
    process on the same seeded inputs."""
    import subprocess

    x = kda_inputs.prefill_inputs(2, 200, 3, 128, dtype, h0=True, seed=49, device=DEV)
    o1, h1 = fwd(x, x["h0"])
    torch.cuda.synchronize()
    out = str(tmp_path / "valu.pt")
    script = (
        "import sys, torch; sys.path[:0] = %r\n"
        "import kda_inputs, linear_attention_recurrence_10_amd as kda\n"
        "x = kda_inputs.prefill_inputs(2, 200, 3, 128, %r, h0=True, seed=49, device='cuda:0')\n"
        "o, h = kda.chunk_fwd(x['q'], x['k'], x['v'], x['g'], x['beta'], x['h0'])\n"
        "torch.cuda.synchronize()\n"
        "torch.save({'o': o.cpu(), 'h': h.cpu()}, %r)\n" % ([ROOT, HERE], dtype, out))
    env = dict(os.environ, KDA_DISABLE_MFMA="1")
    r = subprocess.run([sys.executable, "-c", script], env=env, timeout=300, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    ref = torch.load(out, weights_only=True)
    assert rel_err(o1.cpu(), ref["o"]) < tol and rel_err(h1.cpu(), ref["h"]) < tol
    assert not torch.equal(o1.cpu(), ref["o"])  # the child really ran the other kernel
