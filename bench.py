"""Benchmark of the KDA forward hot path on one MI355X.

One step = one chunked prefill over the 64K-token full-width workload
(B=1, H=56, T=65536, d=128, bf16 q/k/v, fp32 g/beta/o/state) and one
decode step over 256 sequences x 56 heads (fp32 state updated in place).
The K prefills run first, then the K decode steps (a decode loop); each
launch is timed with events on its stream.  Inputs are resident in HBM
before timing starts.

Prints ONE JSON line on stdout:
  value          prefill tokens/s (B*T / mean prefill kernel time)
  roofline       the prefill kernel against the HBM roofline (algorithmic bytes)
  decode         the decode kernel's algorithmic GB/s against the HBM peak
  segmented      the segmented prefill (kda_chunk_fwd_kcp) beside the single
                 pass on one long sequence with 7 heads (B=1, T=262144)
  backward       the backward pass (kda_chunk_bwd) at B=4 H=16 T=4096
  configs        the other prefill workloads (tiny fp32, B=4 H=16 T=4096, T=2^20)
  copy           a plain 1 GiB device copy (the streaming rate this part reaches)
  cpu_baseline   the fp64 oracle on the host cores, on a bounded token sample
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s (H=56,d=128,T=64K); decode-step HBM GB/s vs peak"
HBM_PEAK_GBPS = 8000.0
COPY_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kda_prefill_64k_traffic.json")
_CSRC = os.path.join(ROOT, "linear_attention_recurrence_10_amd", "csrc")
KERNEL_SOURCES = [os.path.join(_CSRC, f) for f in ("kda_prefill_mfma.h", "kda_prefill_mfma.hip", "kda_prefill_mfma_gate.hip",
                                                     "kda_internal.h")]
DECODE_SOURCES = [os.path.join(_CSRC, f) for f in ("kda_decode.hip", "kda_internal.h")]


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def prefill_bytes(B, T, H, D, in_bytes=2, h0=False, hT=True, gate_bytes=4):
    """Algorithmic HBM bytes of one prefill: q, k, v (in dtype), the gate (fp32
    log-decay, or logits of gate_bytes each) and beta (fp32) read once, o (fp32)
    written once, states read/written once."""
    per_tok_head = 3 * D * in_bytes + gate_bytes * D + 4 + 4 * D
    state = 4 * D * D
    return B * T * H * per_tok_head + B * H * state * (int(h0) + int(hT))


def backward_bytes(B, T, H, D, in_bytes=2, h0=True, dhT=True, dh0=True):
    """Algorithmic HBM bytes of one backward pass: q, k, v (in dtype), g, beta
    and dO (fp32) read once; dq, dk, dg, dv, dbeta (fp32) written once; the
    states h0 and dhT read and dh0 written once."""
    per_tok_head = 3 * D * in_bytes + 4 * D + 4 + 4 * D + 4 * (3 * D + D) + 4
    return B * T * H * per_tok_head + B * H * 4 * D * D * (int(h0) + int(dhT) + int(dh0))


def decode_bytes(B, H, D, in_bytes=2):
    """State read + written once, q, k, v in dtype, g fp32, beta fp32, o fp32."""
    return B * H * (2 * 4 * D * D + 3 * D * in_bytes + 4 * D + 4 + 4 * D)


def source_hash(files=None):
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES if files is None else files):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel="prefill"):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None
    when they are missing or were taken on different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    pre = kernel in ("prefill", "gate", "qknorm")  # the prefill variants share their sources
    sha = t.get("kernel_src_sha") if pre else t.get("decode_src_sha")
    if sha != source_hash(KERNEL_SOURCES if pre else DECODE_SOURCES):
        return None
    return (t.get(kernel) or {}).get("hbm_bytes_per_launch")


def cpu_baseline(target_s: float):
    """Time the fp64 oracle on a prefix of the same workload (all 56 heads)."""
    import numpy as np
    import kda_inputs
    import oracle

    cfg = kda_inputs.PREFILL_64K
    threads = oracle.num_threads()

    def run(T):
        x = kda_inputs.prefill_inputs(cfg.B, T, cfg.H, cfg.D, cfg.dtype, seed=cfg.seed, device="cpu")
        args = [np.ascontiguousarray(x[n].double().numpy()) for n in ("q", "k", "v", "g", "beta")]
        t0 = time.perf_counter()
        oracle.kda_fwd(*args)
        return time.perf_counter() - t0

    probe_T = 64
    dt = run(probe_T)
    T = int(min(cfg.T, max(probe_T, probe_T * target_s / max(dt, 1e-6))))
    T = max(16, T // 16 * 16)
    dt = run(T)
    return {
        "value": cfg.B * T / dt,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": "first %d of %d tokens of the B=1 H=56 d=128 workload, all heads, fp64 token-sequential C "
                  "(OpenMP over heads), %.1f s wall" % (T, cfg.T, dt),
    }


def time_segmented(kda, torch, stream, n_seg, steps, single=True):
    """The segmented prefill against the single pass (unless not `single`) on
    one long sequence with few heads (its own inputs, freed before returning)."""
    import kda_inputs

    cfg = kda_inputs.PREFILL_256K_H7
    dev = torch.device("cuda:0")
    log("segmented prefill: %s, %d segments" % (cfg.name, n_seg))
    x = kda_inputs.prefill_inputs(cfg.B, cfg.T, cfg.H, cfg.D, cfg.dtype, h0=cfg.h0, seed=cfg.seed, device=dev)
    o = torch.empty((cfg.B, cfg.T, cfg.H, cfg.D), dtype=torch.float32, device=dev)
    hT = torch.empty((cfg.B, cfg.H, cfg.D, cfg.D), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, kda.kcp_ws_bytes(cfg.B, cfg.T, cfg.H, cfg.D, cfg.D, n_seg)), dtype=torch.uint8,
                     device=dev)

    def single_pass():
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], None, o=o, hT=hT, stream=stream)

    def split():
        kda.chunk_fwd_kcp(x["q"], x["k"], x["v"], x["g"], x["beta"], None, n_seg=n_seg, ws=ws, o=o, hT=hT,
                          stream=stream)

    out = {"single_pass": None}
    runs = (("single_pass", single_pass), ("segmented", split)) if single else (("segmented", split),)
    for name, fn in runs:
        fn()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for e in ev:
            e[0].record(stream)
            fn()
            e[1].record(stream)
        torch.cuda.synchronize()
        ms = [e[0].elapsed_time(e[1]) for e in ev]
        out[name] = sum(ms) / len(ms)
    del x, o, hT, ws
    torch.cuda.empty_cache()
    tokens = cfg.B * cfg.T
    sp = out["single_pass"]
    return {"workload": cfg.name, "n_seg": n_seg, "ms": out["segmented"], "single_pass_ms": sp,
            "tokens_per_s": tokens / (out["segmented"] * 1e-3), "speedup": sp / out["segmented"] if sp else None,
            "unit": "tokens/s"}


def time_launches(torch, stream, fn, steps):
    """Mean and min of `steps` event-timed launches of fn() on `stream` (after one untimed call)."""
    fn()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in ev:
        e[0].record(stream)
        fn()
        e[1].record(stream)
    torch.cuda.synchronize()
    ms = [e[0].elapsed_time(e[1]) for e in ev]
    return sum(ms) / len(ms), min(ms)


def time_configs(kda, torch, stream, names, steps):
    """The other prefill workloads (parity cases of the same entry point), each
    timed on its own inputs with its algorithmic bytes and roofline fraction.
    Inputs are generated on the device and freed before the next workload."""
    import kda_inputs

    out = {}
    for name in names:
        cfg = kda_inputs.PREFILL_CONFIGS[name]
        log("config %s" % name)
        x = kda_inputs.config_inputs(cfg, device=torch.device("cuda:0"))
        o = torch.empty((cfg.B, cfg.T, cfg.H, cfg.D), dtype=torch.float32, device="cuda:0")
        hT = torch.empty((cfg.B, cfg.H, cfg.D, cfg.D), dtype=torch.float32, device="cuda:0")
        torch.cuda.synchronize()

        def fn():
            kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], o=o, hT=hT, stream=stream)

        n = steps if cfg.B * cfg.T * cfg.H <= (1 << 22) else max(3, steps // 5)
        avg, mn = time_launches(torch, stream, fn, n)
        esz = 2 if cfg.dtype == "bf16" else 4
        nbytes = prefill_bytes(cfg.B, cfg.T, cfg.H, cfg.D, esz, h0=cfg.h0, hT=True)
        gbps = nbytes / (avg * 1e-3) / 1e9
        out[name] = {"B": cfg.B, "H": cfg.H, "T": cfg.T, "d": cfg.D, "dtype": cfg.dtype, "h0": cfg.h0,
                     "launches": n, "ms": avg, "min_ms": mn, "tokens_per_s": cfg.B * cfg.T / (avg * 1e-3),
                     "alg_bytes_per_launch": nbytes, "achieved": gbps, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS}
        del x, o, hT
        torch.cuda.empty_cache()
    return out


def time_backward(kda, torch, stream, steps, calibrate=False):
    """The backward pass (kda_chunk_bwd: forward checkpoints, the adjoint, the
    slice sums) on the B=4 H=16 T=4096 workload with random dO and dhT.
    ``calibrate``: run the plain copy of COPY_BYTES right before the first
    backward launch (the reference of the traffic counters)."""
    import kda_inputs

    cfg = kda_inputs.PREFILL_B4
    dev = torch.device("cuda:0")
    log("backward: %s" % cfg.name)
    x = kda_inputs.config_inputs(cfg, device=dev)
    gen = torch.Generator(device=dev).manual_seed(2)
    dO = torch.randn((cfg.B, cfg.T, cfg.H, cfg.D), generator=gen, device=dev)
    dhT = torch.randn((cfg.B, cfg.H, cfg.D, cfg.D), generator=gen, device=dev)
    ws = torch.empty(kda.bwd_ws_bytes(cfg.B, cfg.T, cfg.H, cfg.D, cfg.D), dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = (torch.empty_like(dO), torch.empty_like(dO), torch.empty_like(dO), torch.empty_like(dO),
           torch.empty((cfg.B, cfg.T, cfg.H), **f32), torch.empty((cfg.B, cfg.H, cfg.D, cfg.D), **f32))

    def fn():
        kda.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], dO, x["h0"], dhT, ws=ws, out=out, stream=stream)

    if calibrate:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    avg, mn = time_launches(torch, stream, fn, max(3, steps // 4))
    nbytes = backward_bytes(cfg.B, cfg.T, cfg.H, cfg.D)
    gbps = nbytes / (avg * 1e-3) / 1e9
    del x, dO, dhT, ws, out
    torch.cuda.empty_cache()
    return {"workload": cfg.name, "ms": avg, "min_ms": mn, "tokens_per_s": cfg.B * cfg.T / (avg * 1e-3),
            "alg_bytes_per_launch": nbytes, "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": gbps / HBM_PEAK_GBPS,
            "note": "forward checkpoint pass + chunk-form adjoint (fp32 MFMA) + slice sums; latency bound"}


def copy_bandwidth(torch, stream, nbytes=1 << 30, steps=10):
    """A plain device-to-device copy of nbytes: the streaming rate this part
    reaches (read + write bytes over time), context for the HBM fractions."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    avg, mn = time_launches(torch, stream, lambda: dst.copy_(src), steps)
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_moved": 2 * nbytes, "ms": avg, "achieved": 2 * nbytes / (avg * 1e-3) / 1e9, "unit": "GB/s",
            "frac_of_peak": 2 * nbytes / (avg * 1e-3) / 1e9 / HBM_PEAK_GBPS}


def decode_host_cost(kda, torch, calls=200):
    """Host microseconds per kda_decode_step call (argument checks and the
    launch, no synchronisation) at a small batch, through the C ABI."""
    import ctypes
    import kda_inputs

    d = kda_inputs.decode_inputs(1, 8, 128, "bf16", seed=3, device=torch.device("cuda:0"))
    o = torch.empty((1, 8, 128), dtype=torch.float32, device="cuda:0")
    lib = kda.library()
    p = [ctypes.c_void_p(d[n].data_ptr()) for n in ("q", "k", "v", "g", "beta", "state")]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = p + [ctypes.c_void_p(o.data_ptr()), 1, 8, 128, 128, 1, ctypes.c_float(0.0), stream]
    for _ in range(10):
        lib.kda_decode_step(*args)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(calls):
        st = lib.kda_decode_step(*args)
    t1 = time.perf_counter()
    torch.cuda.synchronize()
    assert st == 0
    out = {"batch": "B=1 H=8 d=128 bf16", "calls": calls, "host_us_per_call": 1e6 * (t1 - t0) / calls}
    # wall time per step to completion: an eager loop of calls, and the same
    # steps replayed from a captured HIP graph of 32 steps (no host work per step)
    t0 = time.perf_counter()
    for _ in range(calls):
        lib.kda_decode_step(*args)
    torch.cuda.synchronize()
    out["eager_us_per_step"] = 1e6 * (time.perf_counter() - t0) / calls
    steps = 32
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            gargs = args[:-1] + [cs]
            for _ in range(steps):
                lib.kda_decode_step(*gargs)
        g.replay()
        torch.cuda.synchronize()
        reps = max(1, calls // steps)
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        out["graph_us_per_step"] = 1e6 * (time.perf_counter() - t0) / (reps * steps)
    except RuntimeError as e:  # reported, not fatal: the figure is context for serving loops
        out["graph_us_per_step"] = None
        out["graph_error"] = str(e)[:200]
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--ckpt-every", type=int, default=0,
                    help="also time the prefill that writes state checkpoints every N tokens (N a multiple of 16)")
    ap.add_argument("--gate-logits", choices=["none", "f32", "bf16"], default="bf16",
                    help="also time the fused gate prologue (kda_chunk_fwd_gate) with logits of this dtype")
    ap.add_argument("--segments", type=int, default=8,
                    help="also time the segmented prefill (kda_chunk_fwd_kcp) with this many segments on one "
                         "long 7-head sequence, beside the single pass (0 = skip)")
    ap.add_argument("--segmented-only", action="store_true",
                    help="time only the segmented prefill (for a kernel trace of its launches alone)")
    ap.add_argument("--no-backward", action="store_true", help="skip timing the backward pass")
    ap.add_argument("--no-qknorm", action="store_true",
                    help="skip timing the prefill and decode step with the fused q/k normalisation")
    ap.add_argument("--no-f32", action="store_true",
                    help="skip timing the same prefill workload with fp32 q, k and v (the fp32 matrix-core kernel)")
    ap.add_argument("--no-host-cost", action="store_true",
                    help="skip the host cost per decode call (its small launches would mix into a kernel trace)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip timing the other prefill workloads (tiny, B=4 H=16 T=4096, T=2^20)")
    ap.add_argument("--backward-only", action="store_true",
                    help="time only the backward pass (for a kernel trace of its launches alone)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one plain device copy of %d bytes first (for the traffic counters)" % (1 << 30))
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the KDA forward path here runs on a single MI355X and has no "
              "multi-GPU mode (asked for --gpus %d, WORLD_SIZE=%d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch
    import kda_inputs
    import linear_attention_recurrence_10_amd as kda

    if not os.path.exists(kda.library_path()):
        log("libkda.so missing: building")
        from linear_attention_recurrence_10_amd import build
        build.build()
    kda.library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.backward_only:
        bw = time_backward(kda, torch, torch.cuda.current_stream(), args.steps, calibrate=args.copy_calibration)
        print(json.dumps({"metric": "KDA backward tokens/s", "value": bw["tokens_per_s"], "unit": "tokens/s",
                          "n_gpus": 1, "steps": max(3, args.steps // 4), "warmup": 1, "ms_per_step": bw["ms"],
                          "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
                          "config": {"workload": bw["workload"]}, "backward": bw}), flush=True)
        return

    if args.segmented_only:
        n_seg = args.segments if args.segments > 0 else 8
        seg = time_segmented(kda, torch, torch.cuda.current_stream(), n_seg, args.steps, single=False)
        print(json.dumps({"metric": "KDA segmented prefill tokens/s", "value": seg["tokens_per_s"],
                          "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": 1,
                          "ms_per_step": seg["ms"], "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
                          "config": {"workload": seg["workload"], "n_seg": n_seg}, "segmented": seg}), flush=True)
        return

    cfg = kda_inputs.PREFILL_64K
    log("generating %s on the device" % cfg.name)
    gate_dt = None if args.gate_logits == "none" else args.gate_logits
    x = kda_inputs.prefill_inputs(cfg.B, cfg.T, cfg.H, cfg.D, cfg.dtype, h0=cfg.h0, seed=cfg.seed, device=dev,
                                  gate_logits=gate_dt)
    o = torch.empty((cfg.B, cfg.T, cfg.H, cfg.D), dtype=torch.float32, device=dev)
    hT = torch.empty((cfg.B, cfg.H, cfg.D, cfg.D), dtype=torch.float32, device=dev)
    dcfg = kda_inputs.DECODE_B256
    d = None
    if not args.no_decode:
        d = kda_inputs.decode_inputs(dcfg.B, dcfg.H, dcfg.D, dcfg.dtype, seed=dcfg.seed, device=dev)
        od = torch.empty((dcfg.B, dcfg.H, dcfg.D), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def prefill(ev=None):
        if ev:
            ev[0].record(stream)
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], None, o=o, hT=hT, stream=stream)
        if ev:
            ev[1].record(stream)

    def decode(ev=None):
        if ev:
            ev[0].record(stream)
        kda.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], o=od, stream=stream)
        if ev:
            ev[1].record(stream)

    if args.copy_calibration:
        # a plain device copy of known size: the reference that scales the
        # FETCH_SIZE / WRITE_SIZE counters to bytes
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    log("warmup %d" % args.warmup)
    for _ in range(args.warmup):
        prefill()
        if d is not None:
            decode()
    torch.cuda.synchronize()

    # prefill steps, then decode steps (a decode loop), each timed per launch
    # with events on the stream the kernels run on
    pre_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    dec_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    log("timing %d steps" % args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        prefill(pre_ev[i])
    torch.cuda.synchronize()
    wall_pre = time.perf_counter() - t0
    t0 = time.perf_counter()
    if d is not None:
        for i in range(args.steps):
            decode(dec_ev[i])
    torch.cuda.synchronize()
    wall_dec = time.perf_counter() - t0
    ck_ms = []
    if args.ckpt_every > 0:
        n_ck = cfg.T // args.ckpt_every
        ck = torch.empty((n_ck, cfg.B, cfg.H, cfg.D, cfg.D), dtype=torch.float32, device=dev)
        ck_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        kda.chunk_fwd_ckpt(x["q"], x["k"], x["v"], x["g"], x["beta"], None, ckpt_every=args.ckpt_every, o=o,
                           hT=hT, ckpt=ck, stream=stream)
        for i in range(args.steps):
            ck_ev[i][0].record(stream)
            kda.chunk_fwd_ckpt(x["q"], x["k"], x["v"], x["g"], x["beta"], None, ckpt_every=args.ckpt_every, o=o,
                               hT=hT, ckpt=ck, stream=stream)
            ck_ev[i][1].record(stream)
        torch.cuda.synchronize()
        ck_ms = [e[0].elapsed_time(e[1]) for e in ck_ev]
        del ck
    gate_ms = []
    if gate_dt is not None:
        # the fused gate prologue: the same workload with the gate given as logits
        gate_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        kda.chunk_fwd_gate(x["q"], x["k"], x["v"], x["x"], x["beta"], None, o=o, hT=hT, stream=stream)
        for i in range(args.steps):
            gate_ev[i][0].record(stream)
            kda.chunk_fwd_gate(x["q"], x["k"], x["v"], x["x"], x["beta"], None, o=o, hT=hT, stream=stream)
            gate_ev[i][1].record(stream)
        torch.cuda.synchronize()
        gate_ms = [e[0].elapsed_time(e[1]) for e in gate_ev]
    qkn = None
    if not args.no_qknorm:
        # the fused q/k normalisation: the same workloads and the same bytes
        # (q and k are read once either way); the generator's q and k are unit
        # vectors, which changes nothing in the work done
        log("q/k normalisation")
        qkn = {"prefill": time_launches(torch, stream, lambda: kda.chunk_fwd_qknorm(
            x["q"], x["k"], x["v"], x["g"], x["beta"], None, eps=1e-6, o=o, hT=hT, stream=stream), args.steps)}
        if d is not None:
            qkn["decode"] = time_launches(torch, stream, lambda: kda.decode_step_qknorm(
                d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], eps=1e-6, o=od, stream=stream), args.steps)
    f32 = None
    if not args.no_f32:
        # the same workload with fp32 q, k and v: the fp32 matrix-core kernel
        # (a few launches: each reads 7.5 GB)
        log("fp32 inputs")
        xf = kda_inputs.prefill_inputs(cfg.B, cfg.T, cfg.H, cfg.D, "f32", seed=cfg.seed, device=dev)
        f32 = time_launches(torch, stream, lambda: kda.chunk_fwd(
            xf["q"], xf["k"], xf["v"], xf["g"], xf["beta"], None, o=o, hT=hT, stream=stream), min(args.steps, 5))
        del xf
        torch.cuda.empty_cache()
    seg = None
    if args.segments > 0:
        seg = time_segmented(kda, torch, stream, args.segments, args.steps)
    pre_ms = [e[0].elapsed_time(e[1]) for e in pre_ev]
    dec_ms = [e[0].elapsed_time(e[1]) for e in dec_ev] if d is not None else []
    pre_avg = sum(pre_ms) / len(pre_ms)
    ms_per_step = 1e3 * (wall_pre + wall_dec) / args.steps
    log("prefill avg %.3f ms (min %.3f), decode avg %s ms, wall/step %.3f ms" % (
        pre_avg, min(pre_ms), ("%.3f" % (sum(dec_ms) / len(dec_ms))) if dec_ms else "-", ms_per_step))

    tokens = cfg.B * cfg.T
    pbytes = prefill_bytes(cfg.B, cfg.T, cfg.H, cfg.D, 2, h0=False, hT=True)
    achieved = pbytes / (pre_avg * 1e-3) / 1e9
    traffic = load_traffic()
    result = {
        "metric": METRIC,
        "value": tokens / (pre_avg * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "H": cfg.H, "T": cfg.T, "d_k": cfg.D, "d_v": cfg.D,
                   "chunk": kda_inputs.CHUNK, "inputs": "q,k,v bf16; g,beta fp32; o,state fp32",
                   "decode_workload": None if d is None else dcfg.name},
        "prefill_ms": pre_avg,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel": "kda prefill", "alg_bytes_per_launch": pbytes},
    }
    if d is not None:
        dbytes = decode_bytes(dcfg.B, dcfg.H, dcfg.D, 2)
        dec_avg = sum(dec_ms) / len(dec_ms)
        dg = dbytes / (dec_avg * 1e-3) / 1e9
        result["decode"] = {"workload": dcfg.name, "ms": dec_avg, "achieved": dg, "peak": HBM_PEAK_GBPS,
                            "unit": "GB/s", "frac": dg / HBM_PEAK_GBPS, "alg_bytes_per_launch": dbytes,
                            "traffic": load_traffic("decode")}
    if ck_ms:
        ck_avg = sum(ck_ms) / len(ck_ms)
        n_ck = cfg.T // args.ckpt_every
        ck_bytes = pbytes + n_ck * cfg.B * cfg.H * 4 * cfg.D * cfg.D
        result["checkpoints"] = {"every_tokens": args.ckpt_every, "count": n_ck, "ms": ck_avg,
                                 "overhead": ck_avg / pre_avg - 1.0, "alg_bytes_per_launch": ck_bytes,
                                 "achieved_GBps": ck_bytes / (ck_avg * 1e-3) / 1e9}
    if gate_ms:
        g_avg = sum(gate_ms) / len(gate_ms)
        g_bytes = prefill_bytes(cfg.B, cfg.T, cfg.H, cfg.D, 2, h0=False, hT=True,
                                gate_bytes=2 if gate_dt == "bf16" else 4)
        g_ach = g_bytes / (g_avg * 1e-3) / 1e9
        result["gate_fused"] = {"workload": cfg.name + "_gate_logits_" + gate_dt, "ms": g_avg,
                                "vs_log_decay_entry": g_avg / pre_avg, "achieved": g_ach, "peak": HBM_PEAK_GBPS,
                                "unit": "GB/s", "frac": g_ach / HBM_PEAK_GBPS, "alg_bytes_per_launch": g_bytes,
                                "traffic": load_traffic("gate") if gate_dt == "bf16" else None}
    if qkn is not None:
        q_avg, q_min = qkn["prefill"]
        q_ach = pbytes / (q_avg * 1e-3) / 1e9
        result["qknorm"] = {"workload": cfg.name + "_qknorm", "ms": q_avg, "min_ms": q_min,
                            "vs_plain_entry": q_avg / pre_avg, "achieved": q_ach, "peak": HBM_PEAK_GBPS,
                            "unit": "GB/s", "frac": q_ach / HBM_PEAK_GBPS, "alg_bytes_per_launch": pbytes,
                            "traffic": load_traffic("qknorm")}
        if "decode" in qkn:
            dq_avg, dq_min = qkn["decode"]
            dq_bytes = decode_bytes(dcfg.B, dcfg.H, dcfg.D, 2)
            dq_ach = dq_bytes / (dq_avg * 1e-3) / 1e9
            result["qknorm"]["decode"] = {"workload": dcfg.name + "_qknorm", "ms": dq_avg, "min_ms": dq_min,
                                          "achieved": dq_ach, "frac": dq_ach / HBM_PEAK_GBPS,
                                          "alg_bytes_per_launch": dq_bytes, "traffic": load_traffic("decode_qknorm")}
    if f32 is not None:
        f_avg, f_min = f32
        f_bytes = prefill_bytes(cfg.B, cfg.T, cfg.H, cfg.D, 4, h0=False, hT=True)
        f_ach = f_bytes / (f_avg * 1e-3) / 1e9
        result["prefill_f32"] = {"workload": cfg.name.replace("bf16", "f32"), "ms": f_avg, "min_ms": f_min,
                                 "tokens_per_s": tokens / (f_avg * 1e-3), "achieved": f_ach,
                                 "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": f_ach / HBM_PEAK_GBPS,
                                 "alg_bytes_per_launch": f_bytes,
                                 "note": "fp32 q, k, v on the fp32 matrix cores (16x16x4); latency bound"}
    if seg is not None:
        result["segmented"] = seg
    result["copy"] = copy_bandwidth(torch, stream)
    if not args.no_backward:
        result["backward"] = time_backward(kda, torch, stream, args.steps)
    if d is not None and not args.no_host_cost:
        result["decode"]["host"] = decode_host_cost(kda, torch)
    if not args.no_configs:
        import kda_inputs
        del d
        torch.cuda.empty_cache()
        result["configs"] = time_configs(kda, torch, stream, [kda_inputs.TINY.name, kda_inputs.PREFILL_B4.name,
                                                                kda_inputs.PREFILL_1M.name], args.steps)
    if not args.no_cpu_baseline:
        del x, o, hT
        log("cpu baseline (oracle), ~%.0f s" % args.cpu_seconds)
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
        result["cpu_baseline"]["gpu_over_cpu"] = result["value"] / result["cpu_baseline"]["value"]
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
