"""Host logic of the rocprofv3 summaries (exact_scaled_dot_sdpa_amd/profiling.py)
on small synthetic CSV files whose derived figures are known by hand."""
import csv
import json

import pytest

from exact_scaled_dot_sdpa_amd import profiling as P

PREFILL = "_ZN4attn12_GLOBAL__N_119prefill_bf16_kernelILi128ELb1ELi4EEEvPKDF16bS3_S3_PDF16bPfiiiifii"
FP8 = "_ZN4attn12_GLOBAL__N_118prefill_fp8_kernelILi128ELb1EEEvPK14__hip_fp8_e4m3S4_S4_PDF16bPfiiiiffii"
CHUNK = "_ZN4attn12_GLOBAL__N_119decode_chunk_kernelILi128ELi4ELi3EEEvPKDF16bS3_S3_PKiPDF16bPfS8_S8_iiiiiifS5_iii"
MERGE = "_ZN4attn12_GLOBAL__N_119decode_merge_kernelILi128EEEvPKfS3_PKiPDF16bPfiiiiii"
COPY = "__amd_rocclr_copyBuffer"


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_short_names():
    assert P._short(PREFILL) == "prefill_bf16_kernel"
    assert P._short(FP8) == "prefill_fp8_kernel"
    assert P._short("void attn::(anonymous namespace)::decode_merge_kernel<128>(float const*)") == \
        "decode_merge_kernel"


def test_stats_last_dispatches(tmp_path):
    st = tmp_path / "stats.csv"
    _write(st, ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"],
           [[PREFILL, 4, 1500000, 1000000, 3000000, 99.5]])
    tr = tmp_path / "trace.csv"
    # two warm-up dispatches of 3 ms, then two timed ones of 1.0 and 1.2 ms
    _write(tr, ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
           [[PREFILL, 0, 3000000], [PREFILL, 4000000, 7000000], [PREFILL, 8000000, 9000000],
            [PREFILL, 10000000, 11200000]])
    out = tmp_path / "s.md"
    text = P.stats(str(st), "cmd", str(out), str(tr), last=2)
    assert "| prefill_bf16_kernel | 4 | 1500.00 | 1000.00 | 3000.00 | 99.50% |" in text
    assert "| prefill_bf16_kernel | 2 | 1100.00 | 1100.00 |" in text


def test_traffic_scaling(tmp_path, monkeypatch):
    monkeypatch.setattr("exact_scaled_dot_sdpa_amd.build.source_digest", lambda *a: "d")
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    # the 512 MiB copy reads half its bytes by FETCH_SIZE and writes all of them
    f = tmp_path / "f.csv"
    _write(f, hdr, [[COPY, "FETCH_SIZE", 512 * 1024 / 2], [PREFILL, "FETCH_SIZE", 1000.0],
                    [PREFILL, "FETCH_SIZE", 1200.0], [CHUNK, "FETCH_SIZE", 300.0], [MERGE, "FETCH_SIZE", 10.0]])
    w = tmp_path / "w.csv"
    _write(w, hdr, [[COPY, "WRITE_SIZE", 512 * 1024], [PREFILL, "WRITE_SIZE", 500.0],
                    [PREFILL, "WRITE_SIZE", 500.0], [CHUNK, "WRITE_SIZE", 2.0], [MERGE, "WRITE_SIZE", 1.0]])
    js = tmp_path / "t.json"
    P.traffic(str(f), str(w), 512, "cf", "cw", str(js), str(tmp_path / "t.md"))
    doc = json.load(open(js))
    assert doc["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert doc["calibration"]["write_factor"] == pytest.approx(1.0)
    pre = doc["kernels"]["prefill"]
    # median fetch 1100 KiB x 2, write 500 KiB x 1
    assert pre["read_bytes"] == 1100 * 2 * 1024 and pre["write_bytes"] == 500 * 1024
    dec = doc["kernels"]["decode"]  # both kernels of one launch summed
    assert dec["read_bytes"] == (300 + 10) * 2 * 1024 and dec["write_bytes"] == 3 * 1024
    assert "bwd" not in doc["kernels"]  # absent from the run: no entry


def test_counters_derived_figures(tmp_path):
    hdr = ["Kernel_Name", "Dispatch_Id", "Start_Timestamp", "End_Timestamp", "Counter_Name", "Counter_Value"]
    dur = 1000000  # 1 ms
    clock = 1.6    # GHz
    cyc = clock * dur  # cycles per shader engine over the dispatch
    mops_bf16 = 1.2e12 / P.MOP_FLOPS
    rows = []
    for name, counters in [
        (PREFILL, {"SQ_CYCLES": cyc * P.N_SE, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * cyc * P.N_SIMD,
                   "SQ_INSTS_VALU_MFMA_MOPS_BF16": mops_bf16, "SQ_WAVE_CYCLES": 1000.0, "SQ_WAIT_ANY": 250.0,
                   "SQ_WAIT_INST_ANY": 100.0}),
        # half the executed FLOPs on fp8: mixed peak 1 / (0.5/5000 + 0.5/2500) = 3333.3 at 2.4 GHz
        (FP8, {"SQ_CYCLES": cyc * P.N_SE, "SQ_INSTS_VALU_MFMA_MOPS_BF16": mops_bf16 / 2,
               "SQ_INSTS_VALU_MFMA_MOPS_F8": mops_bf16 / 2}),
    ]:
        for c, v in counters.items():
            rows.append([name, 1, 0, dur, c, v])
    path = tmp_path / "pmc.csv"
    _write(path, hdr, rows)
    js = tmp_path / "c.json"
    text = P.counters(str(path), "cmd", str(tmp_path / "c.md"),
                      {"prefill_bf16_kernel": 1.0e12, "prefill_fp8_kernel": 1.0e12}, str(js))
    doc = json.load(open(js))
    assert doc["kernels"]["prefill"]["clock_ghz"] == pytest.approx(1.6)
    assert doc["kernels"]["prefill"]["mfma_busy"] == pytest.approx(0.5)
    assert doc["kernels"]["fp8"]["clock_ghz"] == pytest.approx(1.6)
    assert "decode" not in doc["kernels"]  # absent from the run: no entry
    line = [l for l in text.splitlines() if l.startswith("| prefill_bf16_kernel | 1000.0 |")][0]
    cells = [c.strip() for c in line.strip("|").split("|")]
    assert cells[2] == "1.60"        # clock
    assert cells[3] == "50.0%"       # MFMA busy
    assert cells[4] == "1.2"         # executed TFLOP
    # 1 PFLOP/s algorithmic against 2500 x 1.6 / 2.4 = 1666.7 TFLOP/s
    assert cells[6] == "60.0% of 1667 TFLOP/s"
    assert cells[7] == "25.0%" and cells[8] == "10.0%"
    line8 = [l for l in text.splitlines() if l.startswith("| prefill_fp8_kernel | 1000.0 |")][0]
    cells8 = [c.strip() for c in line8.strip("|").split("|")]
    assert cells8[6] == "45.0% of 2222 TFLOP/s"
