"""Turn rocprofv3 output into the short text summaries kept under profiles/.

    python -m decode_attention_kv_03_amd.profiling trace STATS_CSV OUT_MD TITLE COMMAND
    python -m decode_attention_kv_03_amd.profiling traffic WORKLOAD OUT_MD FETCH_DIR WRITE_DIR \
        COPY_FETCH_DIR COPY_WRITE_DIR COPY_BYTES COMMANDS
    python -m decode_attention_kv_03_amd.profiling mfma WORKLOAD OUT_MD RUN_DIR TRACE_MD ALGO_FLOPS COMMAND [KERNEL]
    python -m decode_attention_kv_03_amd.profiling lds WORKLOAD OUT_MD RUN_DIR COMMAND

``trace`` condenses a ``--kernel-trace --stats`` kernel_stats.csv into a table
of the library's kernels.  ``traffic`` turns two ``--pmc`` runs of a workload
(FETCH_SIZE, then WRITE_SIZE; KiB per dispatch) into HBM bytes per launch of
the split-K kernel, each scaled by what the same counter reads for a plain
device copy of known size, and records the hash of the kernel sources the
counters were taken with.  ``bench.py`` reports that traffic only while the
sources still hash the same.  ``mfma`` turns one ``--pmc MfmaUtil
MfmaFlopsBF16 GRBM_GUI_ACTIVE`` run into the split-K kernel's counted
matrix-core FLOPs, busy fraction and GRBM_GUI_ACTIVE rate, with the kernel's mean
duration taken from its kernel-trace summary.  ``lds`` turns one ``--pmc
SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT SQ_LDS_ADDR_CONFLICT SQ_INSTS_LDS
GRBM_GUI_ACTIVE`` run into the split-K kernel's LDS bank-conflict stall
cycles as a fraction of its LDS-busy cycles, and the share of all CU clocks
during the dispatch in which the LDS served indexed reads and writes.
"""

import csv
import glob
import hashlib
import os
import re
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(os.path.dirname(_HERE), "profiles")
_TAG = re.compile(r"<!-- kvattn-traffic (.*?) -->")


# The sources each split-K kernel is compiled and launched from: its own file, the headers it
# includes, and the split planning that sets its grid.
_COMMON = ["plan.h", "kvattn_internal.h", "device_common.h", "lds_copy.h", "cache_addr.h"]
KERNEL_SOURCES = {
    "gqa_split_bf16": ["gqa_bf16.hip", "gqa_split.h", "gqa_plan.hip", "merge.hip"] + _COMMON,
    "gqa_split_fp8": ["gqa_fp8.hip", "gqa_split.h", "gqa_plan.hip", "merge.hip"] + _COMMON,
    "gqa_split_f32": ["gqa_f32.hip", "merge.hip"] + _COMMON,
    "mla_split_bf16": ["mla_bf16.hip", "mla_plan.hip"] + _COMMON,
}


def kernel_of(workload):
    """The split-K kernel that streams the cache of a named workload."""
    from . import workloads as W

    w = W.WORKLOADS[workload]
    return f"gqa_split_{w.dtype}" if hasattr(w, "num_kv_heads") else "mla_split_bf16"


def source_sha(kernel=None):
    """sha256 over the sources a split-K kernel is built and launched from (file names and contents);
    with no kernel, over every library source."""
    h = hashlib.sha256()
    csrc = os.path.join(_HERE, "csrc")
    names = KERNEL_SOURCES[kernel] if kernel else [n for n in os.listdir(csrc) if n.endswith((".hip", ".h", ".cpp"))]
    for name in sorted(names):
        h.update(name.encode())
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _counter_rows(run_dir):
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _mean_counter(run_dir, counter, match):
    vals = [float(r["Counter_Value"]) for r in _counter_rows(run_dir)
            if r["Counter_Name"] == counter and match(r["Kernel_Name"])]
    if not vals:
        raise ValueError(f"{counter}: no dispatch matched in {run_dir}")
    return sum(vals) / len(vals), len(vals)


def _is_split(name):
    return "kvattn" in name and "split" in name


def _matcher(kernel):
    """Dispatch filter: the split-K kernel by default, else library kernels whose name contains `kernel`."""
    if not kernel:
        return _is_split
    return lambda name: "kvattn" in name and kernel in name


def _is_copy(name):
    # the device-to-device blit of the copy calibration (not the fill that creates its source)
    return "copybuffer" in name.lower()


def summarize_trace(stats_csv, out_md, title, command):
    with open(stats_csv) as fh:
        rows = list(csv.DictReader(fh))
    keep = [r for r in rows if "kvattn" in r["Name"]]
    with open(out_md, "w") as f:
        f.write(f"# {title}\n\n")
        f.write("Command (from the repository root, on one MI355X; rocprofv3 --stats output, kernel_stats.csv):\n\n")
        f.write("```\n" + command + "\n```\n\n")
        f.write("| kernel | calls | avg (us) | min (us) | max (us) | stddev (us) |\n|---|---|---|---|---|---|\n")
        for r in keep:
            f.write(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                    f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                    f"{float(r['StdDev']) / 1e3:.2f} |\n")
        other = len(rows) - len(keep)
        f.write(f"\nOther kernels in the trace ({other}) are input generation and copies outside the timed region.\n")
        f.write(f"\nLibrary sources hash: `{source_sha()}`\n")


def summarize_traffic(workload, out_md, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_bytes, commands):
    fetch_kib, n_f = _mean_counter(fetch_dir, "FETCH_SIZE", _is_split)
    write_kib, n_w = _mean_counter(write_dir, "WRITE_SIZE", _is_split)
    cfetch_kib, _ = _mean_counter(copy_fetch_dir, "FETCH_SIZE", _is_copy)
    cwrite_kib, _ = _mean_counter(copy_write_dir, "WRITE_SIZE", _is_copy)
    fetch_scale = copy_bytes / (cfetch_kib * 1024.0)
    write_scale = copy_bytes / (cwrite_kib * 1024.0)
    fetch_b = fetch_kib * 1024.0 * fetch_scale
    write_b = write_kib * 1024.0 * write_scale
    kernel = kernel_of(workload)
    sha = source_sha(kernel)
    with open(out_md, "w") as f:
        f.write(f"# HBM traffic of the split-K kernel: {workload}\n\n")
        f.write("rocprofv3 counter runs (one counter per pass), from the repository root on one MI355X:\n\n")
        f.write("```\n" + commands + "\n```\n\n")
        f.write("| quantity | value |\n|---|---|\n")
        f.write(f"| FETCH_SIZE per dispatch, split-K kernel (KiB, mean of {n_f}) | {fetch_kib:.1f} |\n")
        f.write(f"| WRITE_SIZE per dispatch, split-K kernel (KiB, mean of {n_w}) | {write_kib:.1f} |\n")
        f.write(f"| FETCH_SIZE of a {copy_bytes} B device copy (KiB) | {cfetch_kib:.1f} |\n")
        f.write(f"| WRITE_SIZE of the same copy (KiB) | {cwrite_kib:.1f} |\n")
        f.write(f"| fetch scale (true bytes per counted byte) | {fetch_scale:.4f} |\n")
        f.write(f"| write scale | {write_scale:.4f} |\n")
        f.write(f"| HBM bytes read per launch (scaled) | {fetch_b:.0f} |\n")
        f.write(f"| HBM bytes written per launch (scaled) | {write_b:.0f} |\n")
        f.write(f"| total traffic per launch | {fetch_b + write_b:.0f} |\n\n")
        f.write(f"Sources hash of `{kernel}` (its file, included headers and split planning): `{sha}`\n\n")
        f.write(f"<!-- kvattn-traffic workload={workload} source_sha={sha} fetch_bytes={fetch_b:.0f} "
                f"write_bytes={write_b:.0f} -->\n")


CUS = 256
XCDS = 8
BF16_PEAK_FLOPS = 2.5e15


def _trace_kernel_us(trace_md, match=_is_split):
    with open(trace_md) as fh:
        for line in fh:
            m = re.match(r"\| `(.*?)` \| \d+ \| ([\d.]+) \|", line)
            if m and match(m.group(1)):
                return float(m.group(2))
    raise ValueError(f"no matching kernel row in {trace_md}")


def _mean_dispatch_ns(run_dir, match):
    """Mean (End - Start) timestamp of the matching dispatches of a counter run."""
    seen = {}
    for r in _counter_rows(run_dir):
        if match(r["Kernel_Name"]):
            seen[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    return sum(seen.values()) / len(seen)


def summarize_mfma(workload, out_md, run_dir, trace_md, algo_flops, command, kernel=None):
    match = _matcher(kernel)
    flops, n = _mean_counter(run_dir, "MfmaFlopsBF16", match)
    util, _ = _mean_counter(run_dir, "MfmaUtil", match)
    gui, _ = _mean_counter(run_dir, "GRBM_GUI_ACTIVE", match)
    run_ns = _mean_dispatch_ns(run_dir, match)
    us = _trace_kernel_us(trace_md, match)
    # GRBM_GUI_ACTIVE is summed over the XCDs (each has its own GRBM; the MfmaUtil
    # expression takes their maximum instead), so one XCD's count is the sum / 8.  Its
    # rate is the counter's own clock, not the shader clock: it reads above 2.4 GHz for
    # the streaming kernels, while the shader clock measured inside the MLA kernel
    # (s_memtime against s_memrealtime) is about 1.8 GHz.
    rate = gui / XCDS / (run_ns * 1e-9)
    with open(out_md, "w") as f:
        what = f"`{kernel}`" if kernel else "the split-K kernel"
        f.write(f"# Matrix-core counters of {what}: {workload}\n\n")
        f.write("rocprofv3 counter run, from the repository root on one MI355X (the kernel's mean duration is\n"
                f"its row of `{os.path.relpath(trace_md, os.path.dirname(PROFILES))}`):\n\n")
        f.write("```\n" + command + "\n```\n\n")
        f.write("| quantity | value |\n|---|---|\n")
        f.write(f"| MfmaFlopsBF16 per dispatch (GFLOP, mean of {n}) | {flops / 1e9:.3f} |\n")
        f.write(f"| algorithmic FLOPs per launch (GFLOP) | {algo_flops / 1e9:.3f} |\n")
        f.write(f"| counted / algorithmic | {flops / algo_flops:.4f} |\n")
        f.write(f"| MfmaUtil (% of SIMD clocks with the matrix core busy) | {util:.1f} |\n")
        f.write(f"| GRBM_GUI_ACTIVE per dispatch (clocks, summed over the 8 XCDs) | {gui:.0f} |\n")
        f.write(f"| dispatch duration in the counter run (us) | {run_ns / 1e3:.2f} |\n")
        f.write(f"| GRBM_GUI_ACTIVE / 8 / dispatch duration (GHz; the counter's clock, not the shader clock) | {rate / 1e9:.3f} |\n")
        f.write(f"| kernel mean duration, kernel-trace run (us) | {us:.2f} |\n")
        f.write(f"| algorithmic FLOP rate (TFLOP/s) | {algo_flops / (us * 1e-6) / 1e12:.1f} |\n")
        f.write(f"| of the 2.5 PFLOP/s bf16 peak | {algo_flops / (us * 1e-6) / BF16_PEAK_FLOPS:.4f} |\n")


def summarize_lds(workload, out_md, run_dir, command):
    active, n = _mean_counter(run_dir, "SQ_LDS_IDX_ACTIVE", _is_split)
    bank, _ = _mean_counter(run_dir, "SQ_LDS_BANK_CONFLICT", _is_split)
    addr, _ = _mean_counter(run_dir, "SQ_LDS_ADDR_CONFLICT", _is_split)
    insts, _ = _mean_counter(run_dir, "SQ_INSTS_LDS", _is_split)
    gui, _ = _mean_counter(run_dir, "GRBM_GUI_ACTIVE", _is_split)
    names = sorted({r["Kernel_Name"] for r in _counter_rows(run_dir) if _is_split(r["Kernel_Name"])})
    # The SQ counters are summed over all compute units; GRBM_GUI_ACTIVE is summed over the
    # 8 XCDs, so one XCD's busy clocks (the dispatch's clocks) are the sum / 8.
    cu_clocks = gui / XCDS * CUS
    with open(out_md, "w") as f:
        f.write(f"# LDS counters of the split-K kernel: {workload}\n\n")
        f.write("rocprofv3 counter run, from the repository root on one MI355X:\n\n")
        f.write("```\n" + command + "\n```\n\n")
        f.write("Kernel: " + ", ".join(f"`{k}`" for k in names) + "\n\n")
        f.write("| quantity | value |\n|---|---|\n")
        f.write(f"| SQ_LDS_IDX_ACTIVE per dispatch (LDS-busy cycles, all CUs; mean of {n}) | {active:.0f} |\n")
        f.write(f"| SQ_LDS_BANK_CONFLICT per dispatch (stall cycles) | {bank:.0f} |\n")
        f.write(f"| bank-conflict cycles / LDS-busy cycles | {bank / active:.4f} |\n")
        f.write(f"| SQ_LDS_ADDR_CONFLICT per dispatch (stall cycles) | {addr:.0f} |\n")
        f.write(f"| SQ_INSTS_LDS per dispatch (instructions) | {insts:.0f} |\n")
        f.write(f"| GRBM_GUI_ACTIVE per dispatch (clocks, summed over the 8 XCDs) | {gui:.0f} |\n")
        f.write(f"| LDS busy, share of CU clocks (SQ_LDS_IDX_ACTIVE / (256 x clocks)) | {active / cu_clocks:.4f} |\n")


def lookup_traffic(workload):
    """Traffic per split-K launch recorded for `workload` with the current sources of its kernel, or None."""
    sha = source_sha(kernel_of(workload))
    for path in sorted(glob.glob(os.path.join(PROFILES, "*.md"))):
        with open(path) as fh:
            for m in _TAG.finditer(fh.read()):
                kv = dict(item.split("=", 1) for item in m.group(1).split())
                if kv.get("workload") == workload and kv.get("source_sha") == sha:
                    return {"fetch_bytes": int(kv["fetch_bytes"]), "write_bytes": int(kv["write_bytes"]),
                            "source": os.path.relpath(path, os.path.dirname(PROFILES))}
    return None


def main(argv):
    if len(argv) >= 5 and argv[0] == "trace":
        summarize_trace(argv[1], argv[2], argv[3], argv[4])
        print(open(argv[2]).read())
        return 0
    if len(argv) >= 9 and argv[0] == "traffic":
        summarize_traffic(argv[1], argv[2], argv[3], argv[4], argv[5], argv[6], int(argv[7]), argv[8])
        print(open(argv[2]).read())
        return 0
    if len(argv) >= 5 and argv[0] == "lds":
        summarize_lds(argv[1], argv[2], argv[3], argv[4])
        print(open(argv[2]).read())
        return 0
    if len(argv) >= 7 and argv[0] == "mfma":
        summarize_mfma(argv[1], argv[2], argv[3], argv[4], float(argv[5]), argv[6], argv[7] if len(argv) > 7 else None)
        print(open(argv[2]).read())
        return 0
    print(__doc__, file=sys.stderr)
    return 2


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
