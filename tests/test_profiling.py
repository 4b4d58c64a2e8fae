"""Host logic that turns rocprofv3 output into profiles/ summaries (CPU; synthetic CSVs).

The traffic summary scales each counter by what it reads for a copy of known
size and records the kernel-source hash; bench.py looks the traffic up only
while the sources still hash the same.  The matrix-core summary derives the
effective clock from GRBM_GUI_ACTIVE (summed over the 8 XCDs) and the
dispatch duration of the same run.
"""

import csv
import os

import pytest

from decode_attention_kv_03_amd import profiling as P

SPLIT = "void kvattn::(anonymous namespace)::gqa_split_bf16<1, 4, 2>(kvattn::DecodeArgs)"
MERGE = "void kvattn::(anonymous namespace)::lse_merge<128, true>(kvattn::DecodeArgs)"
COPY = "__amd_rocclr_copyBuffer"
FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _counter_run(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(FIELDS, r)))
    return d


def test_traffic_summary_scales_counters_and_round_trips_through_the_tag(tmp_path, monkeypatch):
    # The copy of 1 GiB reads back as half its bytes on FETCH_SIZE and exactly on WRITE_SIZE.
    copy = 1 << 30
    cf = _counter_run(tmp_path / "cf", [(1, COPY, "FETCH_SIZE", copy / 2048, 0, 1)])
    cw = _counter_run(tmp_path / "cw", [(1, COPY, "WRITE_SIZE", copy / 1024, 0, 1)])
    # Two dispatches of the split kernel (mean taken), and a merge that must be ignored.
    f = _counter_run(tmp_path / "f", [(1, SPLIT, "FETCH_SIZE", 1000.0, 0, 1), (2, SPLIT, "FETCH_SIZE", 3000.0, 0, 1),
                                      (3, MERGE, "FETCH_SIZE", 99999.0, 0, 1)])
    w = _counter_run(tmp_path / "w", [(1, SPLIT, "WRITE_SIZE", 10.0, 0, 1), (2, SPLIT, "WRITE_SIZE", 30.0, 0, 1)])
    out = tmp_path / "x_traffic.md"
    name = "llama3_8b_gqa_h32_g8_b16_s8192"
    P.summarize_traffic(name, str(out), str(f), str(w), str(cf), str(cw), copy, "cmd")
    text = out.read_text()
    assert "| HBM bytes read per launch (scaled) | 4096000 |" in text       # 2000 KiB x 1024 x 2
    assert "| HBM bytes written per launch (scaled) | 20480 |" in text      # 20 KiB x 1024 x 1
    sha = P.source_sha("gqa_split_bf16")
    assert P.kernel_of(name) == "gqa_split_bf16" and f"source_sha={sha}" in text
    monkeypatch.setattr(P, "PROFILES", str(tmp_path))
    got = P.lookup_traffic(name)
    assert got["fetch_bytes"] == 4096000 and got["write_bytes"] == 20480
    assert P.lookup_traffic("llama3_70b_gqa_h64_g8_b64_s8192") is None
    # A summary taken with other sources of the kernel is not reported.
    out.write_text(text.replace(sha, "0" * 16))
    assert P.lookup_traffic(name) is None


def test_kernel_source_hashes_cover_their_own_sources():
    # every listed source exists, and the kernels' hashes differ from each other and from the library's
    shas = {k: P.source_sha(k) for k in P.KERNEL_SOURCES}
    assert len(set(shas.values())) == len(shas) and P.source_sha() not in shas.values()
    assert P.kernel_of("deepseek_v2_mla_h128_b32_s8192") == "mla_split_bf16"
    assert P.kernel_of("llama3_70b_gqa_fp8_h64_g8_b64_s8192") == "gqa_split_fp8"


def test_trace_summary_keeps_the_library_kernels(tmp_path):
    stats = tmp_path / "run_kernel_stats.csv"
    with open(stats, "w", newline="") as f:
        w = csv.DictWriter(f, ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "StdDev"])
        w.writeheader()
        w.writerow({"Name": SPLIT, "Calls": 30, "AverageNs": 83280.0, "MinNs": 80000.0, "MaxNs": 90000.0,
                    "StdDev": 1500.0})
        w.writerow({"Name": "at::native::elementwise_kernel", "Calls": 5, "AverageNs": 1.0, "MinNs": 1.0,
                    "MaxNs": 1.0, "StdDev": 0.0})
    out = tmp_path / "t.md"
    P.summarize_trace(str(stats), str(out), "title", "cmd")
    text = out.read_text()
    assert f"| `{SPLIT}` | 30 | 83.28 | 80.00 | 90.00 | 1.50 |" in text
    assert "elementwise_kernel" not in text
    assert P._trace_kernel_us(str(out)) == pytest.approx(83.28)


def test_mfma_summary_clock_and_utilisation(tmp_path):
    # One dispatch of 100 us during which each of the 8 XCDs counted 200,000 busy clocks (2.0 GHz).
    us, clk, flops = 100.0, 2.0e9, 80e9
    ns = int(us * 1e3)
    run = _counter_run(tmp_path / "m", [(7, SPLIT, "MfmaFlopsBF16", flops, 0, ns),
                                        (7, SPLIT, "MfmaUtil", 40.0, 0, ns),
                                        (7, SPLIT, "GRBM_GUI_ACTIVE", 8 * clk * us * 1e-6, 0, ns)])
    trace = tmp_path / "t.md"
    trace.write_text(f"| `{SPLIT}` | 30 | {us:.2f} | 1 | 1 | 0 |\n")
    out = tmp_path / "m.md"
    P.summarize_mfma("w", str(out), str(run), str(trace), flops, "cmd")
    text = out.read_text()
    assert "| GRBM_GUI_ACTIVE / 8 / dispatch duration (GHz; the counter's clock, not the shader clock) | 2.000 |" in text
    assert "| counted / algorithmic | 1.0000 |" in text
    # 80 GFLOP in 100 us = 800 TFLOP/s: 0.32 of 2.5 PFLOP/s
    assert "| of the 2.5 PFLOP/s bf16 peak | 0.3200 |" in text


def test_lds_summary_conflict_ratio_and_busy_share(tmp_path):
    # One dispatch of 100 us at 2 GHz (8 XCDs x 200,000 busy clocks): 256 CUs x 200,000 = 51.2 M CU clocks,
    # of which the LDS was busy 25.6 M (one half) and stalled on bank conflicts 256,000 (1 % of that).
    clk = 200_000
    run = _counter_run(tmp_path / "l", [(3, SPLIT, "SQ_LDS_IDX_ACTIVE", 25_600_000, 0, 1),
                                        (3, SPLIT, "SQ_LDS_BANK_CONFLICT", 256_000, 0, 1),
                                        (3, SPLIT, "SQ_LDS_ADDR_CONFLICT", 0, 0, 1),
                                        (3, SPLIT, "SQ_INSTS_LDS", 1234, 0, 1),
                                        (3, SPLIT, "GRBM_GUI_ACTIVE", 8 * clk, 0, 1),
                                        (4, MERGE, "SQ_LDS_IDX_ACTIVE", 99, 0, 1)])
    out = tmp_path / "l.md"
    P.summarize_lds("w", str(out), str(run), "cmd")
    text = out.read_text()
    assert "| bank-conflict cycles / LDS-busy cycles | 0.0100 |" in text
    assert "| LDS busy, share of CU clocks (SQ_LDS_IDX_ACTIVE / (256 x clocks)) | 0.5000 |" in text
    assert f"`{SPLIT}`" in text and "lse_merge" not in text
