"""Turn rocprofv3 runs of bench.py into the per-launch HBM traffic figures.

Inputs are three rocprofv3 output directories made with the commands below
(each one a separate run; counters never share a run with other tracing):

  rocprofv3 --kernel-trace --stats --output-format csv -d DIR_T -o trace -- \\
      python3 bench.py --steps 20 --warmup 1 --no-cpu-baseline --segments 0 --no-configs --no-backward --no-host-cost
  rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR_F -o fetch -- \\
      python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --segments 0 --no-configs --no-backward --no-host-cost --copy-calibration
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR_W -o write -- \\
      python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --segments 0 --no-configs --no-backward --no-host-cost --copy-calibration

FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what the same
counter reads for the runtime's plain copy of COPY_BYTES bytes, so that a
copy counts exactly COPY_BYTES read and COPY_BYTES written.  Writes
OUT/kda_prefill_64k_traffic.json (read by bench.py while the kernel sources
are unchanged) and OUT/kda_prefill_64k_decode_b256_rocprof.md.

usage: python3 bench_traffic.py DIR_T DIR_F DIR_W OUT
       python3 bench_traffic.py --segmented N_SEG DIR_T OUT   (trace summary of
           bench.py --segmented-only: OUT/kda_prefill_256k_h7_segmented_rocprof.md)
       python3 bench_traffic.py --util DIR_U OUT   (issue and pipe utilisation of the
           prefill from one counter run: OUT/kda_prefill_64k_util.md)
       python3 bench_traffic.py --backward-util DIR_U OUT   (the same for the
           backward's chunk kernel: OUT/kda_bwd_b4_h16_t4096_util.md)
       python3 bench_traffic.py --backward DIR_T DIR_F DIR_W OUT   (trace and traffic of
           bench.py --backward-only: OUT/kda_bwd_b4_h16_t4096_rocprof.md)
       python3 bench_traffic.py --waits prefill|backward DIR_S OUT   (where the waves' cycles
           go, from one counter run: OUT/kda_prefill_64k_waits.md or
           OUT/kda_bwd_b4_h16_t4096_waits.md)
"""
from __future__ import annotations

import csv
import glob
import json
import os
import statistics
import sys

import bench

PREFILL = "prefill_mfma_kernel<false, 0, 0>" # plain prefill (fp32 log-decay gate)
GATE = "prefill_mfma_kernel<false, 2, 0>"    # fused gate prologue, bf16 logits
DECODE = "decode_kernel"
QKNORM = "prefill_mfma_qknorm_kernel<0>"  # the prefill with the fused q/k normalisation
DECODE_QKNORM = "decode_qknorm_kernel"
COPY = "copyBuffer"
# the backward's chunk kernel and the helpers it includes
BWD_SOURCES = [os.path.join(bench._CSRC, f) for f in ("kda_bwd.hip", "kda_internal.h", "kda_f32mfma.h")]


def _csv(d, suffix):
    files = glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)
    if not files:
        raise SystemExit("no *%s under %s" % (suffix, d))
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def per_dispatch(d, counter):
    """{dispatch id: (kernel name, summed counter value)} for one counter run."""
    out = {}
    for r in _csv(d, "counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        k = int(r["Dispatch_Id"])
        name, v = out.get(k, (r["Kernel_Name"], 0.0))
        out[k] = (name, v + float(r["Counter_Value"]))
    return out


def calibration_copy(disp):
    """The copy bench.py --copy-calibration runs right before the first KDA
    kernel (earlier copies belong to input generation)."""
    first_kda = min(k for k, (name, _) in disp.items() if PREFILL in name or DECODE in name)
    copies = [k for k, (name, _) in disp.items() if COPY in name and k < first_kda]
    if not copies:
        raise SystemExit("copy calibration dispatch not found")
    return disp[max(copies)][1]


TIMED_STEPS = 20  # --steps of the trace command


def timed_means(dt, names):
    """{kernel name (as in the stats): (mean ns, n)} over each kernel's last
    TIMED_STEPS dispatches in the kernel trace."""
    durs = {}
    for r in _csv(dt, "kernel_trace.csv"):
        name = r["Kernel_Name"][:90]
        if name in names:
            durs.setdefault(name, []).append((int(r["Dispatch_Id"]),
                                              int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    out = {}
    for name, v in durs.items():
        v.sort()
        last = [d for _, d in v[-TIMED_STEPS:]]
        out[name] = (statistics.mean(last), len(last))
    return out


def mean_for(disp, key):
    vals = [v for name, v in disp.values() if key in name]
    return statistics.mean(vals) if vals else None, len(vals)


def main(dt, df, dw, out):
    fetch = per_dispatch(df, "FETCH_SIZE")
    write = per_dispatch(dw, "WRITE_SIZE")
    copy_f = calibration_copy(fetch)
    copy_w = calibration_copy(write)
    kib = bench.COPY_BYTES / 1024.0
    sf, sw = kib / copy_f, kib / copy_w
    res = {"copy_bytes": bench.COPY_BYTES, "fetch_scale": sf, "write_scale": sw,
           "kernel_src_sha": bench.source_hash(), "decode_src_sha": bench.source_hash(bench.DECODE_SOURCES)}
    for key, tag in ((PREFILL, "prefill"), (GATE, "gate"), (DECODE, "decode"), (QKNORM, "qknorm"),
                     (DECODE_QKNORM, "decode_qknorm")):
        f, nf = mean_for(fetch, key)
        w, nw = mean_for(write, key)
        if f is None or w is None:
            continue
        res[tag] = {"fetch_kib_raw": f, "write_kib_raw": w, "dispatches": [nf, nw],
                    "fetch_bytes": f * 1024 * sf, "write_bytes": w * 1024 * sw,
                    "hbm_bytes_per_launch": f * 1024 * sf + w * 1024 * sw}
    res["hbm_bytes_per_launch"] = res["prefill"]["hbm_bytes_per_launch"]
    stats = _csv(dt, "kernel_stats.csv")
    res["kernel_stats"] = [{"name": r["Name"][:90], "calls": int(r["Calls"]), "avg_ns": float(r["AverageNs"]),
                            "min_ns": float(r["MinNs"]), "max_ns": float(r["MaxNs"])}
                           for r in stats if "prefill_mfma_kernel" in r["Name"] or DECODE in r["Name"]
                           or "qknorm_kernel" in r["Name"] or COPY in r["Name"]]
    # the launches bench.py times with events (the last TIMED_STEPS of each
    # kernel; the first is the warmup, whose cold start the --stats average
    # includes): their mean is the figure comparable with the bench line
    timed = timed_means(dt, [r["name"] for r in res["kernel_stats"]])
    for r in res["kernel_stats"]:
        r["timed_avg_ns"], r["timed_calls"] = timed.get(r["name"], (None, 0))
    os.makedirs(out, exist_ok=True)
    with open(os.path.join(out, "kda_prefill_64k_traffic.json"), "w") as f:
        json.dump(res, f, indent=1)
    alg_p = bench.prefill_bytes(1, 65536, 56, 128)
    alg_d = bench.decode_bytes(256, 56, 128)
    lines = ["# rocprofv3: KDA prefill (B=1 H=56 T=65536 d=128; fp32 log-decay gate, bf16 gate logits with "
             "the fused gate prologue, and the fused q/k normalisation) and decode (B=256 H=56 d=128, without "
             "and with the q/k normalisation)", "",
             "Commands (from the repository root):", "",
             "    rocprofv3 --kernel-trace --stats --output-format csv -d DIR_T -o trace -- "
             "python3 bench.py --steps 20 --warmup 1 --no-cpu-baseline --segments 0 --no-configs --no-backward --no-host-cost",
             "    rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR_F -o fetch -- "
             "python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --segments 0 --no-configs --no-backward --no-host-cost --copy-calibration",
             "    rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR_W -o write -- "
             "python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --segments 0 --no-configs --no-backward --no-host-cost --copy-calibration",
             "    python3 bench_traffic.py DIR_T DIR_F DIR_W profiles", "",
             "Kernel source hash: prefill %s, decode %s" % (res["kernel_src_sha"], res["decode_src_sha"]), "",
             "## Kernel trace (--stats)", "",
             "The last column is the mean over the last %d launches of each kernel (the ones bench.py times; "
             "the first launch is its warmup)." % TIMED_STEPS, "",
             "| kernel | calls | avg us | min us | max us | timed avg us |", "|---|---|---|---|---|---|"]
    for r in res["kernel_stats"]:
        t = r["timed_avg_ns"]
        lines.append("| %s | %d | %.1f | %.1f | %.1f | %s |" % (r["name"], r["calls"], r["avg_ns"] / 1e3,
                                                               r["min_ns"] / 1e3, r["max_ns"] / 1e3,
                                                               "%.1f" % (t / 1e3) if t else "-"))
    lines += ["", "## HBM traffic (FETCH_SIZE, WRITE_SIZE)", "",
              "Copy calibration: %d bytes copied; raw FETCH_SIZE %.1f KiB, WRITE_SIZE %.1f KiB; "
              "scale factors %.4f (fetch), %.4f (write)." % (bench.COPY_BYTES, copy_f, copy_w, sf, sw), "",
              "| kernel | raw fetch KiB | raw write KiB | scaled bytes | algorithmic bytes | ratio |",
              "|---|---|---|---|---|---|"]
    alg_g = bench.prefill_bytes(1, 65536, 56, 128, gate_bytes=2)
    for tag, alg in (("prefill", alg_p), ("gate", alg_g), ("decode", alg_d), ("qknorm", alg_p),
                     ("decode_qknorm", alg_d)):
        if tag not in res:
            continue
        r = res[tag]
        lines.append("| %s | %.0f | %.0f | %.4g | %.4g | %.3f |" % (tag, r["fetch_kib_raw"], r["write_kib_raw"],
                                                                  r["hbm_bytes_per_launch"], alg,
                                                                  r["hbm_bytes_per_launch"] / alg))
    with open(os.path.join(out, "kda_prefill_64k_decode_b256_rocprof.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps({k: res[k] for k in ("fetch_scale", "write_scale", "hbm_bytes_per_launch")}))


SEG_KERNELS = (("prefill_mfma_kernel<false, 0, 1>", "pass 1: zero start, no o (segment writes B_p)"),
               ("prefill_mfma_kernel<false, 0, 2>", "pass 1: identity start, zero values (transition M_p)"),
               ("fill_identity_kernel", "identity states"),
               ("combine_kernel", "scan over the segments (incoming states, hT)"),
               ("prefill_mfma_kernel<false, 0, 0>", "pass 2: from the incoming states, writes o"))


def segmented(dt, out, n_seg):
    """Kernel-trace summary of ``bench.py --segmented-only`` (the segmented prefill alone)."""
    stats = _csv(dt, "kernel_stats.csv")
    cmd = ("rocprofv3 --kernel-trace --stats --output-format csv -d DIR_T -o trace -- "
           "python3 bench.py --segmented-only --segments %d --steps 10" % n_seg)
    lines = ["# rocprofv3: segmented KDA prefill (B=1 H=7 T=262144 d=128, %d segments)" % n_seg, "",
             "Commands (from the repository root):", "", "    " + cmd,
             "    python3 bench_traffic.py --segmented %d DIR_T profiles" % n_seg, "",
             "Kernel source hash: prefill %s, segment combine %s" % (
                 bench.source_hash(), bench.source_hash([os.path.join(bench._CSRC, "kda_kcp.hip")])), "",
             "| kernel | role | calls | avg us | min us | max us |", "|---|---|---|---|---|---|"]
    total = 0.0
    for key, role in SEG_KERNELS:
        for r in stats:
            if key in r["Name"]:
                avg = float(r["AverageNs"]) / 1e3
                total += avg
                lines.append("| %s | %s | %d | %.1f | %.1f | %.1f |" % (key, role, int(r["Calls"]), avg,
                                                                       float(r["MinNs"]) / 1e3,
                                                                       float(r["MaxNs"]) / 1e3))
    lines += ["", "Sum of the per-launch averages (one segmented prefill): %.1f us" % total]
    os.makedirs(out, exist_ok=True)
    with open(os.path.join(out, "kda_prefill_256k_h7_segmented_rocprof.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


BWD_KERNELS = (("prefill_mfma_kernel<true, 0, 1>", "forward with a state checkpoint every 16 tokens, no o"),
               ("bwd_chunk_kernel", "chunk-form adjoint on fp32 matrix cores, 32-column slices"),
               ("bwd_sum_kernel", "sum of the slices' partial sums (dq, dk, dg, dbeta)"))


def backward(dt, df, dw, out):
    """Kernel trace and HBM traffic of ``bench.py --backward-only`` (B=4 H=16 T=4096)."""
    stats = _csv(dt, "kernel_stats.csv")
    fetch = per_dispatch(df, "FETCH_SIZE")
    write = per_dispatch(dw, "WRITE_SIZE")

    def calib(disp):
        first = min(k for k, (name, _) in disp.items() if "kda::" in name)
        copies = [k for k, (name, _) in disp.items() if COPY in name and k < first]
        if not copies:
            raise SystemExit("copy calibration dispatch not found")
        return disp[max(copies)][1]

    kib = bench.COPY_BYTES / 1024.0
    sf, sw = kib / calib(fetch), kib / calib(write)
    cmds = ["rocprofv3 --kernel-trace --stats --output-format csv -d DIR_T -o trace -- "
            "python3 bench.py --backward-only --steps 20",
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR_F -o fetch -- "
            "python3 bench.py --backward-only --steps 4 --copy-calibration",
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR_W -o write -- "
            "python3 bench.py --backward-only --steps 4 --copy-calibration",
            "python3 bench_traffic.py --backward DIR_T DIR_F DIR_W profiles"]
    alg = bench.backward_bytes(4, 4096, 16, 128)
    lines = ["# rocprofv3: KDA backward pass (B=4 H=16 T=4096 d=128, bf16 q/k/v, random h0, dO and dhT)", "",
             "Commands (from the repository root):", ""] + ["    " + c for c in cmds] + [
             "", "Kernel source hash: backward %s, prefill %s" % (
                 bench.source_hash(BWD_SOURCES),
                 bench.source_hash()),
             "", "Copy calibration scale factors %.4f (fetch), %.4f (write)." % (sf, sw), "",
             "| kernel | role | calls | avg us | min us | scaled HBM bytes per launch |", "|---|---|---|---|---|---|"]
    total_t, total_b = 0.0, 0.0
    for key, role in BWD_KERNELS:
        if not any(key in r["Name"] for r in stats):
            raise SystemExit("kernel %s not in the trace under %s" % (key, dt))
        f, _ = mean_for(fetch, key)
        w, _ = mean_for(write, key)
        hb = (f or 0.0) * 1024 * sf + (w or 0.0) * 1024 * sw
        for r in stats:
            if key in r["Name"]:
                avg = float(r["AverageNs"]) / 1e3
                total_t += avg
                total_b += hb
                lines.append("| %s | %s | %d | %.1f | %.1f | %.4g |" % (key, role, int(r["Calls"]), avg,
                                                                      float(r["MinNs"]) / 1e3, hb))
    lines += ["", "One backward pass: %.1f us, %.4g HBM bytes (counters) against %.4g algorithmic bytes "
              "(%.2fx)." % (total_t, total_b, alg, total_b / alg)]
    os.makedirs(out, exist_ok=True)
    with open(os.path.join(out, "kda_bwd_b4_h16_t4096_rocprof.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


UTIL_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_INSTS_VALU SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_MFMA "
                 "SQ_INSTS_SALU SQ_INSTS_LDS GRBM_GUI_ACTIVE")


def utilisation(du, out, cus=256, simds_per_cu=4, xcds=8):
    """Issue and pipe-busy summary of the plain prefill from one counter run:

    rocprofv3 --pmc <UTIL_COUNTERS> --output-format csv -d DIR_U -o util -- \
        python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --segments 0 --no-configs --no-backward --no-host-cost --no-decode --gate-logits none --no-qknorm
    """
    import collections
    rows = _csv(du, "counter_collection.csv")
    per = collections.defaultdict(list)
    for r in rows:
        if PREFILL in r["Kernel_Name"]:
            per[r["Counter_Name"]].append(float(r["Counter_Value"]))
    m = {k: statistics.mean(v) for k, v in per.items()}
    # GRBM_GUI_ACTIVE comes summed over the XCDs' instances; the busy ratios
    # take one XCD's active cycles (the vendor's derived metrics use the max)
    active = m["GRBM_GUI_ACTIVE"] / xcds
    steps = 65536 // 16
    wgs = 56 * 4
    per_chunk_simd = lambda c: m[c] / (wgs * simds_per_cu * steps)
    cmd = ("rocprofv3 --pmc %s --output-format csv -d DIR_U -o util -- python3 bench.py --steps 2 --warmup 1 "
           "--no-cpu-baseline --segments 0 --no-configs --no-backward --no-host-cost --no-decode --gate-logits none --no-qknorm" % UTIL_COUNTERS)
    lines = ["# rocprofv3: KDA prefill (B=1 H=56 T=65536 d=128) issue and pipe utilisation", "",
             "Commands (from the repository root):", "", "    " + cmd,
             "    python3 bench_traffic.py --util DIR_U profiles", "",
             "Kernel source hash: prefill %s" % bench.source_hash(), "",
             "| figure | value |", "|---|---|",
             "| GPU active cycles per launch (GRBM_GUI_ACTIVE / %d XCDs) | %.4g |" % (xcds, active),
             "| MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / (active x %d SIMDs)) | %.1f%% |" % (
                 cus * simds_per_cu, 100.0 * m["SQ_VALU_MFMA_BUSY_CYCLES"] / (active * cus * simds_per_cu)),
             "| VALU busy (SQ_ACTIVE_INST_VALU / (active x %d CUs)) | %.1f%% |" % (
                 cus, 100.0 * m["SQ_ACTIVE_INST_VALU"] / (active * cus)),
             "| vector instructions per chunk and SIMD (SQ_INSTS_VALU, MFMA included) | %.0f |" % per_chunk_simd("SQ_INSTS_VALU"),
             "| of which MFMA (SQ_INSTS_MFMA) | %.0f |" % per_chunk_simd("SQ_INSTS_MFMA"),
             "| of which fp32 transcendental (SQ_INSTS_VALU_TRANS_F32) | %.0f |" % per_chunk_simd("SQ_INSTS_VALU_TRANS_F32"),
             "| scalar instructions per chunk and SIMD (SQ_INSTS_SALU) | %.0f |" % per_chunk_simd("SQ_INSTS_SALU"),
             "| LDS instructions per chunk and SIMD (SQ_INSTS_LDS) | %.0f |" % per_chunk_simd("SQ_INSTS_LDS"),
             "", "Per chunk and SIMD: counts divided by 224 work-groups x 4 SIMDs x 4096 chunks (launch "
             "prologue and epilogue included)."]
    os.makedirs(out, exist_ok=True)
    with open(os.path.join(out, "kda_prefill_64k_util.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def backward_utilisation(du, out, cus=256, simds_per_cu=4, xcds=8):
    """The same counters for the backward's chunk kernel (B=4 H=16 T=4096:
    256 work-groups of four waves, one wave per SIMD, 256 chunks each):

    rocprofv3 --pmc <UTIL_COUNTERS> --output-format csv -d DIR_U -o util -- \
        python3 bench.py --backward-only --steps 2
    """
    import collections
    rows = _csv(du, "counter_collection.csv")
    per = collections.defaultdict(list)
    for r in rows:
        if "bwd_chunk_kernel" in r["Kernel_Name"]:
            per[r["Counter_Name"]].append(float(r["Counter_Value"]))
    m = {k: statistics.mean(v) for k, v in per.items()}
    active = m["GRBM_GUI_ACTIVE"] / xcds
    chunks, wgs = 4096 // 16, 4 * 16 * 4
    per_chunk_simd = lambda c: m[c] / (wgs * simds_per_cu * chunks)
    cmd = ("rocprofv3 --pmc %s --output-format csv -d DIR_U -o util -- python3 bench.py --backward-only --steps 2"
           % UTIL_COUNTERS)
    mfma = per_chunk_simd("SQ_INSTS_MFMA")
    lines = ["# rocprofv3: KDA backward chunk kernel (B=4 H=16 T=4096 d=128) issue and pipe utilisation", "",
             "Commands (from the repository root):", "", "    " + cmd,
             "    python3 bench_traffic.py --backward-util DIR_U profiles", "",
             "Kernel source hash: backward %s" % bench.source_hash(BWD_SOURCES), "",
             "| figure | value |", "|---|---|",
             "| GPU active cycles per launch (GRBM_GUI_ACTIVE / %d XCDs) | %.4g |" % (xcds, active),
             "| active cycles per chunk | %.0f |" % (active / chunks),
             "| MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / (active x %d SIMDs)) | %.1f%% |" % (
                 cus * simds_per_cu, 100.0 * m["SQ_VALU_MFMA_BUSY_CYCLES"] / (active * cus * simds_per_cu)),
             "| VALU busy (SQ_ACTIVE_INST_VALU / (active x %d CUs)) | %.1f%% |" % (
                 cus, 100.0 * m["SQ_ACTIVE_INST_VALU"] / (active * cus)),
             "| vector instructions per chunk and SIMD (SQ_INSTS_VALU, MFMA included) | %.0f |" % per_chunk_simd("SQ_INSTS_VALU"),
             "| of which MFMA (SQ_INSTS_MFMA; fp32 16x16x4, 32 cycles each) | %.0f (%.0f cycles) |" % (mfma, 32 * mfma),
             "| of which fp32 transcendental (SQ_INSTS_VALU_TRANS_F32) | %.0f |" % per_chunk_simd("SQ_INSTS_VALU_TRANS_F32"),
             "| scalar instructions per chunk and SIMD (SQ_INSTS_SALU) | %.0f |" % per_chunk_simd("SQ_INSTS_SALU"),
             "| LDS instructions per chunk and SIMD (SQ_INSTS_LDS) | %.0f |" % per_chunk_simd("SQ_INSTS_LDS"),
             "", "Per chunk and SIMD: counts divided by 256 work-groups x 4 SIMDs x 256 chunks (launch "
             "prologue and epilogue included)."]
    os.makedirs(out, exist_ok=True)
    with open(os.path.join(out, "kda_bwd_b4_h16_t4096_util.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


WAIT_COUNTERS = ("SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_WAIT_INST_LDS "
                 "SQ_ACTIVE_INST_LDS SQ_VALU_MFMA_COEXEC_CYCLES GRBM_GUI_ACTIVE")


def waits(which, ds, out, xcds=8):
    """Where the waves' cycles go, from one counter run of WAIT_COUNTERS.

    SQ_WAVE_CYCLES (wave lifetime), SQ_WAIT_ANY (waiting on anything: a
    dependency, a memory or LDS count, a barrier), SQ_WAIT_INST_ANY (an
    instruction ready but not yet issued) and SQ_ACTIVE_INST_ANY (issuing)
    count wave-cycles in units of four cycles, summed over the waves (the
    three shares add up to the lifetime).  The shares are per wave-cycle, so
    they describe the average wave of the kernel.
    """
    import collections
    if which == "prefill":
        key, fname = PREFILL, "kda_prefill_64k_waits.md"
        title = "KDA prefill (B=1 H=56 T=65536 d=128)"
        cmd_tail = ("python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --segments 0 --no-configs --no-backward "
                    "--no-host-cost --no-decode --gate-logits none --no-qknorm")
        waves, chunks = 224 * 12, 65536 // 16
        srcs = None
    else:
        key, fname = "bwd_chunk_kernel", "kda_bwd_b4_h16_t4096_waits.md"
        title = "KDA backward chunk kernel (B=4 H=16 T=4096 d=128)"
        cmd_tail = "python3 bench.py --backward-only --steps 2"
        waves, chunks = 256 * 8, 4096 // 16
        srcs = BWD_SOURCES
    rows = _csv(ds, "counter_collection.csv")
    per = collections.defaultdict(list)
    for r in rows:
        if key in r["Kernel_Name"]:
            per[r["Counter_Name"]].append(float(r["Counter_Value"]))
    if not per:
        raise SystemExit("no %s dispatches under %s" % (key, ds))
    m = {k: statistics.mean(v) for k, v in per.items()}
    active = m["GRBM_GUI_ACTIVE"] / xcds
    wave_cyc = 4.0 * m["SQ_WAVE_CYCLES"]
    share = lambda c, scale: 100.0 * scale * m[c] / wave_cyc
    cmd = "rocprofv3 --pmc %s --output-format csv -d DIR_S -o waits -- %s" % (WAIT_COUNTERS, cmd_tail)
    lines = ["# rocprofv3: %s, where the waves' cycles go" % title, "",
             "Commands (from the repository root):", "", "    " + cmd,
             "    python3 bench_traffic.py --waits %s DIR_S profiles" % which, "",
             "Kernel source hash: %s %s" % (which, bench.source_hash(srcs) if srcs else bench.source_hash()), "",
             "| figure | value |", "|---|---|",
             "| GPU active cycles per launch (GRBM_GUI_ACTIVE / %d XCDs) | %.4g |" % (xcds, active),
             "| wave-cycles per launch (4 x SQ_WAVE_CYCLES) | %.4g |" % wave_cyc,
             "| the same per wave and chunk (%d waves, %d chunks) | %.0f |" % (waves, chunks, wave_cyc / (waves * chunks)),
             "| waiting on a dependency, count or barrier (4 x SQ_WAIT_ANY) | %.1f%% |" % share("SQ_WAIT_ANY", 4),
             "| ready, waiting for issue (4 x SQ_WAIT_INST_ANY) | %.1f%% |" % share("SQ_WAIT_INST_ANY", 4),
             "| issuing (4 x SQ_ACTIVE_INST_ANY) | %.1f%% |" % share("SQ_ACTIVE_INST_ANY", 4),
             "| of which LDS instructions (4 x SQ_ACTIVE_INST_LDS) | %.1f%% |" % share("SQ_ACTIVE_INST_LDS", 4),
             "| ready, waiting for LDS issue (4 x SQ_WAIT_INST_LDS) | %.1f%% |" % share("SQ_WAIT_INST_LDS", 4),
             "| MFMA busy while another vector instruction issued (SQ_VALU_MFMA_COEXEC_CYCLES / (active x %d SIMDs)) | %.1f%% |" % (
                 1024, 100.0 * m["SQ_VALU_MFMA_COEXEC_CYCLES"] / (active * 1024)),
             "", "Shares are of the waves' lifetime (wave-cycles), averaged over all waves of the kernel: waiting, "
             "ready and issuing add up to it. The LDS rows are parts of the issuing and ready rows."]
    os.makedirs(out, exist_ok=True)
    with open(os.path.join(out, fname), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    if len(sys.argv) == 5 and sys.argv[1] == "--waits" and sys.argv[2] in ("prefill", "backward"):
        waits(sys.argv[2], sys.argv[3], sys.argv[4])
        sys.exit(0)
    if len(sys.argv) == 4 and sys.argv[1] == "--backward-util":
        backward_utilisation(sys.argv[2], sys.argv[3])
        sys.exit(0)
    if len(sys.argv) == 4 and sys.argv[1] == "--util":
        utilisation(sys.argv[2], sys.argv[3])
        sys.exit(0)
    if len(sys.argv) == 6 and sys.argv[1] == "--backward":
        backward(*sys.argv[2:])
        sys.exit(0)
    if len(sys.argv) == 5 and sys.argv[1] == "--segmented":
        segmented(sys.argv[3], sys.argv[4], int(sys.argv[2]))
        sys.exit(0)
    if len(sys.argv) != 5:
        raise SystemExit(__doc__)
    main(*sys.argv[1:])
