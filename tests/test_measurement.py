"""Host logic of the measurement tools, on small synthetic rocprofv3 CSVs:
the per-launch HBM bytes from the two counter runs (scaled by the plain copy
that precedes the first KDA kernel), the mean over the launches bench.py
times, and the algorithmic byte counts the roofline divides by."""
from __future__ import annotations

import csv
import os

import pytest

import bench
import bench_traffic

PRE = "void kda::(anonymous namespace)::prefill_mfma_kernel<false, 0, 0>(kda::PrefillArgs)"
COPY = "__amd_rocclr_copyBuffer"


def write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def test_algorithmic_bytes():
    # 1,796 B per token-head at d = 128 (bf16 q, k, v; fp32 g, o; beta), plus the final state once per head
    assert bench.prefill_bytes(1, 65536, 56, 128) == 65536 * 56 * 1796 + 56 * 128 * 128 * 4
    # an initial state adds its read
    assert bench.prefill_bytes(1, 16, 1, 128, h0=True) - bench.prefill_bytes(1, 16, 1, 128) == 128 * 128 * 4
    # bf16 gate logits take 2 bytes a channel instead of 4
    assert bench.prefill_bytes(1, 1, 1, 128) - bench.prefill_bytes(1, 1, 1, 128, gate_bytes=2) == 2 * 128
    # decode: the state read and written, plus the token's vectors
    assert bench.decode_bytes(256, 56, 128) == 1904795648


def test_timed_means_take_the_last_launches(tmp_path):
    rows = []
    durs = [5000] + [4000 + i for i in range(bench_traffic.TIMED_STEPS)]  # a cold first launch, then the timed ones
    for i, d in enumerate(durs):
        rows.append({"Kernel_Name": PRE, "Dispatch_Id": str(10 + i), "Start_Timestamp": str(1000 * i),
                     "End_Timestamp": str(1000 * i + d)})
    rows.append({"Kernel_Name": "other", "Dispatch_Id": "99", "Start_Timestamp": "0", "End_Timestamp": "7"})
    write_csv(str(tmp_path / "t" / "trace_kernel_trace.csv"), rows)
    got = bench_traffic.timed_means(str(tmp_path / "t"), [PRE[:90]])
    mean, n = got[PRE[:90]]
    assert n == bench_traffic.TIMED_STEPS
    assert mean == pytest.approx(4000 + (bench_traffic.TIMED_STEPS - 1) / 2)


def test_counter_scaling_uses_the_copy_before_the_first_kda_kernel(tmp_path):
    kib = bench.COPY_BYTES / 1024.0

    def run(name, counter, copy_kib, kernel_kib):
        rows = [  # an input-generation copy, the calibration copy, then two prefill launches
            {"Dispatch_Id": "1", "Kernel_Name": COPY, "Counter_Name": counter, "Counter_Value": "123"},
            {"Dispatch_Id": "2", "Kernel_Name": COPY, "Counter_Name": counter, "Counter_Value": str(copy_kib)},
            {"Dispatch_Id": "3", "Kernel_Name": PRE, "Counter_Name": counter, "Counter_Value": str(kernel_kib / 2)},
            {"Dispatch_Id": "3", "Kernel_Name": PRE, "Counter_Name": counter, "Counter_Value": str(kernel_kib / 2)},
            {"Dispatch_Id": "4", "Kernel_Name": PRE, "Counter_Name": counter, "Counter_Value": str(kernel_kib)},
        ]
        write_csv(str(tmp_path / name / "x_counter_collection.csv"), rows)
        return bench_traffic.per_dispatch(str(tmp_path / name), counter)

    fetch = run("f", "FETCH_SIZE", kib / 2, 1000.0)  # the counter reads half of what a copy moves
    write = run("w", "WRITE_SIZE", kib, 500.0)
    # per-dispatch values are summed over the counter's instances
    assert fetch[3][1] == pytest.approx(1000.0)
    assert bench_traffic.calibration_copy(fetch) == pytest.approx(kib / 2)
    assert bench_traffic.calibration_copy(write) == pytest.approx(kib)
    mean_f, n = bench_traffic.mean_for(fetch, "prefill_mfma_kernel<false, 0, 0>")
    assert n == 2 and mean_f == pytest.approx(1000.0)
    # scaled so that the copy counts exactly its bytes: 1000 KiB read at scale 2, 500 KiB written at scale 1
    sf = kib / bench_traffic.calibration_copy(fetch)
    sw = kib / bench_traffic.calibration_copy(write)
    assert (sf, sw) == (pytest.approx(2.0), pytest.approx(1.0))


def test_wait_shares_are_fractions_of_the_wave_lifetime(tmp_path):
    # quad-cycle counters: 1000 wave quad-cycles, of which 400 waiting, 350 ready, 250 issuing (100 of them LDS)
    vals = {"SQ_WAVE_CYCLES": 1000, "SQ_WAIT_ANY": 400, "SQ_WAIT_INST_ANY": 350, "SQ_ACTIVE_INST_ANY": 250,
            "SQ_ACTIVE_INST_LDS": 100, "SQ_WAIT_INST_LDS": 50, "SQ_VALU_MFMA_COEXEC_CYCLES": 1024 * 10,
            "GRBM_GUI_ACTIVE": 8 * 100}
    rows = []
    for d in ("3", "4"):  # two launches with equal counts; another kernel's counts are ignored
        for c, v in vals.items():
            rows.append({"Dispatch_Id": d, "Kernel_Name": PRE, "Counter_Name": c, "Counter_Value": str(v)})
    rows.append({"Dispatch_Id": "5", "Kernel_Name": COPY, "Counter_Name": "SQ_WAIT_ANY", "Counter_Value": "9e9"})
    write_csv(str(tmp_path / "s" / "x_counter_collection.csv"), rows)
    bench_traffic.waits("prefill", str(tmp_path / "s"), str(tmp_path / "out"))
    text = (tmp_path / "out" / "kda_prefill_64k_waits.md").read_text()
    for row in ("| wave-cycles per launch (4 x SQ_WAVE_CYCLES) | 4000 |",
                "| waiting on a dependency, count or barrier (4 x SQ_WAIT_ANY) | 40.0% |",
                "| ready, waiting for issue (4 x SQ_WAIT_INST_ANY) | 35.0% |",
                "| issuing (4 x SQ_ACTIVE_INST_ANY) | 25.0% |",
                "| of which LDS instructions (4 x SQ_ACTIVE_INST_LDS) | 10.0% |",
                "| GPU active cycles per launch (GRBM_GUI_ACTIVE / 8 XCDs) | 100 |"):
        assert row in text, row
    assert "| 10.0% |" in text.split("COEXEC")[1]  # 1024 x 10 co-issue cycles over 100 active cycles x 1024 SIMDs


def test_source_hash_tracks_the_kernel_sources():
    # the traffic figures are tied to these files; every prefill source is listed
    names = sorted(os.path.basename(f) for f in bench.KERNEL_SOURCES)
    assert names == ["kda_internal.h", "kda_prefill_mfma.h", "kda_prefill_mfma.hip", "kda_prefill_mfma_gate.hip"]
    assert bench.source_hash() == bench.source_hash(bench.KERNEL_SOURCES)


def test_piecewise_error_equals_whole_tensor_error():
    """The whole-tensor parity tests compare a tensor in pieces (head groups,
    batch blocks); the accumulated max|err| / rms must equal the metric taken
    over the whole tensor at once."""
    import torch

    import kda_inputs
    from gpu_helpers import ErrAcc, head_groups

    gen = torch.Generator().manual_seed(5)
    ref = torch.randn(2, 33, 56, 8, generator=gen, dtype=torch.float64)
    x = ref + 1e-3 * torch.randn(2, 33, 56, 8, generator=gen, dtype=torch.float64)
    x[1, 7, 50, 3] += 0.5  # the worst element sits in the last group
    acc = ErrAcc()
    groups = head_groups(56, 28)
    assert [len(g) for g in groups] == [28, 28] and sum(groups, []) == list(range(56))
    for heads in head_groups(56, 20):
        acc.add(x[:, :, heads], ref[:, :, heads])
    whole = kda_inputs.rel_err(x, ref)
    assert abs(acc.value() - whole) <= 1e-12 * whole
    assert acc.n == ref.numel()
