"""Decode-attention benchmark: one decode step of one layer per timed step.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one full library call (split-K kernel plus, when the call splits,
the log-sum-exp merge; for MLA and for the persistent GQA form of paged
batches also the device-side work-plan kernel) over the
workload's synthetic inputs, already resident in HBM.  The default workload
is the largest single-GPU configuration, the paged GQA layer (h=64, g=8,
d=128, bf16, batch 128, 16-token blocks, lengths uniform on 1..32768).
Prints one JSON line: throughput in sequence-steps per second per layer,
the roofline of the split-K kernel that streams the cache (algorithmic HBM
bytes / its measured duration, timed with HIP events around that kernel
alone, against the 8 TB/s HBM3E peak; for MLA also its matrix-core rate
against 2.5 PFLOP/s) and of the whole call, the fp64 CPU reference timed on
a bounded sample of the same workload, and under ``all_configs`` the same
kernel and call figures for every named workload, measured in the same run.
"""

import os

# BLAS/OpenMP threads of the CPU reference: the cores this process may run on
# (capped by an OMP_NUM_THREADS the environment already sets), fixed before
# NumPy is imported.
CPU_CORES = len(os.sched_getaffinity(0))
if os.environ.get("OMP_NUM_THREADS", "").isdigit():
    CPU_CORES = max(1, min(CPU_CORES, int(os.environ["OMP_NUM_THREADS"])))
for _var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_var, str(CPU_CORES))

import argparse
import json
import math
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn achieved HBM GB/s (% peak) + MFMA util (MLA); seq-steps/s per layer"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
CUS = 256
BF16_FLOP_PER_CLK_PER_CU = 4096  # 4 SIMDs x 1024 bf16 FLOP per clock
DEFAULT_WORKLOAD = "paged_gqa_h64_g8_b128_bs16_len1_32768"
ROTATE_BYTES = 1 << 30  # rotate input copies until at least this many distinct bytes are cycled


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--split-tokens", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--no-all-configs", action="store_true", help="skip the all_configs sweep")
    p.add_argument("--mla-forms", choices=["both", "explicit", "absorbed"], default=None,
                   help="only time the absorbed and/or the reconstruct-then-attend MLA layer (one JSON line)")
    p.add_argument("--sweep-steps", type=int, default=20, help="timed calls per workload in the all_configs sweep")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                   help="instead of the workload, run a plain device copy of BYTES bytes --steps times "
                        "(reference kernel for scaling HBM traffic counters)")
    return p.parse_args()


def algorithmic(w, lens):
    """Algorithmic HBM bytes and FLOPs of one decode call (per launch).

    Bytes: every valid cached token's K and V rows (MLA: its 576-wide latent
    row, read once for all heads), the queries, the outputs, and the block
    table rows of a paged cache.  Split-K partials are implementation
    overhead and are not counted.  FLOPs: 2 per multiply-add of the score and
    attention-times-value products.
    """
    import numpy as np

    if getattr(w, "window", 0):
        lens = np.minimum(lens, w.window)  # a sliding window reads only its last `window` tokens
    ntok = int(np.sum(lens))
    if hasattr(w, "num_kv_heads"):
        eb = {"f32": 4, "bf16": 2, "fp8": 1}[w.dtype]  # cache bytes per element
        qb = 4 if w.dtype == "f32" else 2  # query/output bytes per element (bf16 beside an fp8 cache)
        kv = 2 * w.num_kv_heads * w.head_dim * eb * ntok
        qo = 2 * w.batch * w.num_q_heads * w.head_dim * qb
        scales = 2 * 4 * w.num_kv_heads if w.dtype == "fp8" else 0
        table = 4 * int(np.sum((lens + w.block_size - 1) // w.block_size)) if w.paged else 0
        flops = 4 * w.num_q_heads * w.head_dim * ntok
        return kv + qo + scales + table, flops
    width = w.d_latent + w.d_rope
    kv = width * 2 * ntok
    qo = w.batch * w.num_heads * (width + w.d_latent) * 2
    table = 4 * int(np.sum((lens + w.block_size - 1) // w.block_size)) if w.paged else 0
    flops = 2 * w.num_heads * (width + w.d_latent) * ntok
    return kv + qo + table, flops


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, x, seconds):
    """Time the fp64 oracle on whole sequences of the same inputs, cycling over them until `seconds` have passed."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    from decode_attention_kv_03_amd import workloads as W

    lens = W.host_view(x["seq_lens"])
    bf16 = w.dtype == "bf16"
    fp8 = w.dtype == "fp8"
    q = W.host_view(x["q"])
    if fp8:
        k_scale, v_scale = W.host_view(x["k_scale"]), W.host_view(x["v_scale"])
    order = [int(b) for b in np.random.default_rng(0).permutation(w.batch)]
    host = {}  # host copies of the sampled sequences' inputs, made once (not timed)

    def inputs(b):
        if b in host:
            return host[b]
        if hasattr(w, "num_kv_heads"):
            if w.paged:
                bt = W.host_view(x["block_table"][b:b + 1])
                nblk = (int(lens[b]) + w.block_size - 1) // w.block_size
                ids = bt[0, :nblk]
                k = W.host_view(x["k"][torch_index(ids, x["k"].device)])
                v = W.host_view(x["v"][torch_index(ids, x["v"].device)])
                host[b] = (k, v, np.arange(nblk, dtype=np.int64)[None])
            else:
                host[b] = (W.host_view(x["k"][b])[None], W.host_view(x["v"][b])[None], None)
        elif w.paged:
            bt = W.host_view(x["block_table"][b:b + 1])
            nblk = (int(lens[b]) + w.block_size - 1) // w.block_size
            ids = bt[0, :nblk]
            host[b] = (W.host_view(x["cache"][torch_index(ids, x["cache"].device)]),
                       np.arange(nblk, dtype=np.int64)[None])
        else:
            host[b] = (W.host_view(x["cache"][b])[None],)
        return host[b]

    done, t_total, i = 0, 0.0, 0
    while t_total < seconds:
        b = order[i % len(order)]
        i += 1
        args = inputs(b)
        t0 = time.perf_counter()
        if fp8:
            if w.paged:
                oracle.paged_gqa_decode_fp8(q[b:b + 1], args[0], args[1], k_scale, v_scale, args[2], lens[b:b + 1],
                                            w.block_size, w.scale, window=w.window)
            else:
                oracle.gqa_decode_fp8(q[b:b + 1], args[0], args[1], k_scale, v_scale, lens[b:b + 1], w.scale,
                                      window=w.window)
        elif hasattr(w, "num_kv_heads"):
            if w.paged:
                oracle.paged_gqa_decode(q[b:b + 1], args[0], args[1], args[2], lens[b:b + 1], w.block_size, w.scale,
                                        bf16=bf16, window=w.window)
            else:
                oracle.gqa_decode(q[b:b + 1], args[0], args[1], lens[b:b + 1], w.scale, bf16=bf16, window=w.window)
        elif w.paged:
            oracle.paged_mla_absorbed_decode(q[b:b + 1], args[0], args[1], lens[b:b + 1], w.block_size, w.scale,
                                             d_c=w.d_latent, bf16=bf16)
        else:
            oracle.mla_absorbed_decode(q[b:b + 1], args[0], lens[b:b + 1], w.scale, d_c=w.d_latent, bf16=bf16)
        t_total += time.perf_counter() - t0
        done += 1
    blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    distinct = min(done, len(order))
    return {
        "value": done / t_total,
        "unit": "seq-steps/s per layer",
        "cores": CPU_CORES,
        "blas_threads": int(blas_threads),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{done} single-sequence oracle calls ({distinct} distinct of the {w.batch} sequences of {w.name}, "
                  f"cycled), fp64 NumPy, {'E4M3 decoding' if fp8 else 'bf16->fp64 widening'} included, "
                  f"{t_total:.1f} s of CPU time",
    }


PROBE_TILE = 16384  # bytes per tile of the streaming-read probe


def probe_bytes(nbytes, workgroups):
    """Bytes one probe launch reads for about `nbytes`: whole 16 KiB tiles, the same count per workgroup."""
    return int(nbytes) // (PROBE_TILE * workgroups) * (PROBE_TILE * workgroups)


def probe_pitch(nbytes):
    """Distance between the probe's rotated buffers: `nbytes` rounded up to 4 KiB."""
    return (int(nbytes) + 4095) // 4096 * 4096


def hbm_probe(torch, stream, nbytes=2 << 30, copies=1, workgroups=(1024, 2048, 4096)):
    """Measured read ceiling: the library's streaming-read probe, each launch reading about `nbytes` once.

    By default one launch reads 2 GiB (beyond the 256 MB MALL).  With `copies` > 1 the launches
    cycle through that many separate buffers, as the timed decode calls cycle through their input
    copies, so a launch of a smaller size finds nothing in the last-level cache either.  For each
    workgroup count the launch reads the largest multiple of 16 KiB per workgroup that fits in
    `nbytes` (the probe splits its buffer evenly in 16 KiB tiles and reads an uneven rest with plain
    loads), and the rate is taken over the bytes actually read.
    """
    from decode_attention_kv_03_amd import hbm_read_probe

    pitch = probe_pitch(nbytes)
    buf = torch.empty(copies * pitch, dtype=torch.uint8, device="cuda:0")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    reps = max(10, copies)
    best = (0.0, 0, 0)
    for wgs in workgroups:
        nb = probe_bytes(nbytes, wgs)
        if nb == 0:
            continue
        views = [buf[c * pitch: c * pitch + nb] for c in range(copies)]
        for i in range(max(3, copies)):
            hbm_read_probe(views[i % copies], wgs, sink, stream)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for i in range(reps):
            hbm_read_probe(views[i % copies], wgs, sink, stream)
        ev[1].record(stream)
        torch.cuda.synchronize()
        gbs = reps * nb / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e9
        best = max(best, (gbs, wgs, nb))
        del views
    del buf
    return {"gbs": round(best[0], 1), "workgroups": best[1], "bytes": best[2], "copies": copies,
            "frac_of_peak": round(best[0] / HBM_PEAK_GBS, 4)}


def torch_index(ids, device):
    import torch

    return torch.from_numpy(ids.astype("int64")).to(device)


# The named workloads timed in the all_configs sweep, in this order (the headline's own
# workload is reported from its headline measurement).
SWEEP = [
    "gqa_h8_g2_d128_s512_b1_f32",
    "llama3_8b_gqa_h32_g8_b16_s8192",
    "llama3_70b_mha_h64_g64_b8_s8192",
    "llama3_70b_gqa_h64_g8_b64_s8192",
    "llama3_70b_mqa_h64_g1_b64_s8192",
    "paged_gqa_h64_g8_b128_bs16_len1_32768",
    "deepseek_v2_mla_h128_b32_s8192",
    "llama3_70b_gqa_fp8_h64_g8_b64_s8192",
    "mistral7b_swa_h32_g8_b16_s32768_w4096",
    "deepseek_v2_mla_paged_h128_b32_bs64_len1_16384",
    "llama3_70b_gqa_h64_g8_b1_s131072",
    "llama3_70b_mqa_h64_g1_b1_s131072",
    "deepseek_v2_mla_h128_b1_s131072",
]


class Prepared:
    """A workload's inputs (rotated copies), preallocated output and workspace, and one decode call."""

    def __init__(self, w, split_tokens, stream):
        import torch

        from decode_attention_kv_03_amd import gqa_workspace_bytes, mla_workspace_bytes
        from decode_attention_kv_03_amd import workloads as W

        self.w = w
        self.is_gqa = hasattr(w, "num_kv_heads")
        dev = "cuda:0"
        make = W.make_gqa_inputs if self.is_gqa else W.make_mla_inputs
        x0 = make(w, dev)
        self.x0 = x0
        self.lens = W.host_view(x0["seq_lens"])
        self.nbytes, self.flops = algorithmic(w, self.lens)
        # Enough copies of the cache that the bytes one step reads cycle through at least 1 GiB (no
        # step finds its data in the 256 MB last-level cache); a sliding window reads part of its cache.
        self.copies = max(1, min(8, math.ceil(ROTATE_BYTES / max(self.nbytes, 1))))
        self.xs = [x0]
        for _ in range(1, self.copies):
            xc = dict(x0)
            for k in ("k", "v", "cache"):
                if k in x0:
                    xc[k] = x0[k].clone()
            self.xs.append(xc)
        self.max_len = w.seq_len
        if self.is_gqa:
            self.out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=x0["q"].dtype, device=dev)
            ws_n = gqa_workspace_bytes(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, self.max_len,
                                       w.block_size, split_tokens, x0["q"].dtype)
        else:
            self.out = torch.empty((w.batch, w.num_heads, w.d_latent), dtype=x0["q"].dtype, device=dev)
            ws_n = mla_workspace_bytes(w.batch, w.num_heads, self.max_len, w.d_latent, w.d_rope, w.block_size,
                                       split_tokens)
        # The workspace needs no initialisation; it is allocated once, outside the timed calls.
        self.ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)
        self.split_tokens = split_tokens
        self.stream = stream

    def step(self, i):
        from decode_attention_kv_03_amd import gqa_decode, gqa_decode_fp8, mla_decode

        w, x = self.w, self.xs[i % self.copies]
        kw = dict(block_table=x["block_table"], max_seq_len=self.max_len, out=self.out,
                  split_tokens=self.split_tokens, workspace=self.ws, stream=self.stream)
        if self.is_gqa and w.dtype == "fp8":
            gqa_decode_fp8(x["q"], x["k"], x["v"], x["k_scale"], x["v_scale"], x["seq_lens"], w.scale,
                           window=w.window, **kw)
        elif self.is_gqa:
            gqa_decode(x["q"], x["k"], x["v"], x["seq_lens"], w.scale, window=w.window, **kw)
        else:
            mla_decode(x["q"], x["cache"], x["seq_lens"], w.scale, **kw)

    def kernel_name(self):
        return f"gqa_split_{self.w.dtype}" if self.is_gqa else "mla_split_bf16"


def timed_events(torch, prep, steps, wall=False):
    """Time `steps` calls: (wall seconds of back-to-back calls or None, per-call ms, per-split-kernel ms).

    Returns also, for MLA, the median shader clock (GHz) the split kernel's own stamps saw in region 3.
    Region 1 (only with `wall`): the calls back to back, wall time between two synchronisations,
    nothing else on the stream.  Region 2: HIP events around each whole call on the stream the
    kernels run on.  Region 3: HIP events around each call's split-K kernel alone
    (kvattn_time_next_kernel).  They are kept apart because event packets between the calls cost a
    few microseconds each.
    """
    import numpy as np

    from decode_attention_kv_03_amd import clock_next_mla, shader_clock_ghz, time_next_kernel

    stream = prep.stream

    def events(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evs:
            e.record(stream)  # creates the underlying HIP event
        return evs

    starts, ends, kstarts, kends = (events(steps) for _ in range(4))
    torch.cuda.synchronize()
    wall_s = None
    if wall:
        t0 = time.perf_counter()
        for i in range(steps):
            prep.step(i)
        torch.cuda.synchronize()
        wall_s = time.perf_counter() - t0
    for i in range(steps):
        starts[i].record(stream)
        prep.step(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    # MLA: the same calls also stamp the shader clock inside their split kernel
    # (kvattn_clock_next_mla), so the clock belongs to the kernel times reported.
    stamps = None if prep.is_gqa else torch.zeros(steps, 4, dtype=torch.int64, device="cuda:0")
    for i in range(steps):
        time_next_kernel(kstarts[i], kends[i])
        if stamps is not None:
            clock_next_mla(stamps[i])
        prep.step(i)
    torch.cuda.synchronize()
    call_ms = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])
    kern_ms = np.array([a.elapsed_time(b) for a, b in zip(kstarts, kends)])
    clock_ghz = None
    if stamps is not None:
        host = stamps.cpu()
        clock_ghz = float(np.median([shader_clock_ghz(host[i]) for i in range(steps)]))
    return wall_s, call_ms, kern_ms, clock_ghz


def rates(prep, call_ms, kern_ms, clock_ghz=None):
    """Kernel and whole-call figures of one workload from its per-call and per-kernel times (and, for MLA,
    the shader clock measured inside its kernel)."""
    import numpy as np

    w = prep.w
    kern_s = float(kern_ms.mean()) * 1e-3
    call_s = float(call_ms.mean()) * 1e-3
    r = {
        "kernel": prep.kernel_name(),
        "kernel_us_mean": round(kern_s * 1e6, 2),
        "kernel_us_p10_p50_p90": [round(float(np.percentile(kern_ms, p)) * 1e3, 2) for p in (10, 50, 90)],
        "kernel_gbs": round(prep.nbytes / kern_s / 1e9, 1),
        "frac": round(prep.nbytes / kern_s / 1e9 / HBM_PEAK_GBS, 4),
        "call_us_mean": round(call_s * 1e6, 2),
        "call_gbs": round(prep.nbytes / call_s / 1e9, 1),
        "call_frac": round(prep.nbytes / call_s / 1e9 / HBM_PEAK_GBS, 4),
        "seq_steps_per_s_from_call": round(w.batch / call_s, 1),
        "algorithmic_bytes_per_call": int(prep.nbytes),
        "algorithmic_flops_per_call": int(prep.flops),
        "intensity_flop_per_byte": round(prep.flops / prep.nbytes, 2),
    }
    if not prep.is_gqa:
        r["mfma_tflops"] = round(prep.flops / kern_s / 1e12, 1)
        r["mfma_frac_of_bf16_peak"] = round(prep.flops / kern_s / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)
        r["call_mfma_frac_of_bf16_peak"] = round(prep.flops / call_s / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)
        if clock_ghz:
            # The bf16 peak at the clock the kernel actually ran at: 256 CUs x 4096 FLOP per clock.
            peak_at_clock = CUS * BF16_FLOP_PER_CLK_PER_CU * clock_ghz * 1e9
            r["shader_clock_ghz_in_kernel"] = round(clock_ghz, 3)
            r["mfma_frac_at_measured_clock"] = round(prep.flops / kern_s / peak_at_clock, 4)
    return r


def sweep(torch, stream, names, steps, warmup, headline_name, headline_rates):
    """The all_configs record: every named workload timed as the headline is, `steps` calls each."""
    from decode_attention_kv_03_amd import workloads as W

    out = {}
    for name in names:
        if name == headline_name:
            out[name] = dict(headline_rates, note="the headline workload, from the headline measurement")
            continue
        w = W.WORKLOADS[name]
        print(f"[bench] sweep: {name}", file=sys.stderr, flush=True)
        prep = Prepared(w, 0, stream)
        # Warm up for at least `warmup` calls and 200 ms, so that short calls run at the clocks
        # long ones reach.
        t_end = time.perf_counter() + 0.2
        i = 0
        while i < warmup or time.perf_counter() < t_end:
            prep.step(i)
            i += 1
            if i % 16 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        _, call_ms, kern_ms, clk = timed_events(torch, prep, steps)
        out[name] = dict(rates(prep, call_ms, kern_ms, clk), batch=w.batch, rotated_input_copies=prep.copies)
        del prep
        torch.cuda.empty_cache()
    return out


def mla_forms(torch, stream, steps, warmup=3, forms="both"):
    """The absorbed and the naive (reconstruct-then-attend) MLA decode of the DeepSeek-V2-shaped layer, timed
    on the same inputs and weights ("MQA, GQA, and MLA" section 5 and exercise D; "One dial, four settings",
    MLA - compress instead of shrink).

    absorbed layer: query absorption (q^C W_uk^T), the latent decode, the W_uv up-projection;
    explicit: kvattn_mla_explicit_decode (rebuild k_i = c W_uk^(i), v_i = c W_uv^(i) for every head and row,
    then attend).  Both end in the same per-head outputs [B, h, 128].
    """
    import numpy as np

    from decode_attention_kv_03_amd import (mla_absorb_query, mla_decode, mla_explicit_decode,
                                            mla_explicit_workspace_bytes, mla_up_project, mla_workspace_bytes,
                                            time_next_kernel)
    from decode_attention_kv_03_amd import workloads as W

    w = W.WORKLOADS["deepseek_v2_mla_explicit_h128_b32_s8192"]
    print(f"[bench] MLA forms: {w.name}", file=sys.stderr, flush=True)
    x = W.make_mla_explicit_inputs(w, "cuda:0")
    B, h, S, d_c, d_r, d_h, d_v = w.batch, w.num_heads, w.seq_len, w.d_latent, w.d_rope, w.d_head, w.d_v
    dev = "cuda:0"
    out_e = torch.empty((B, h, d_v), dtype=torch.bfloat16, device=dev)
    ws_e = torch.empty(mla_explicit_workspace_bytes(B, h, S), dtype=torch.uint8, device=dev)
    q_abs = torch.empty((B, h, d_c + d_r), dtype=torch.bfloat16, device=dev)
    q_abs[..., d_c:] = x["q"][..., d_h:]
    q_c = x["q"][..., :d_h].contiguous()
    o_lat = torch.empty((B, h, d_c), dtype=torch.bfloat16, device=dev)
    out_a = torch.empty((B, h, d_v), dtype=torch.bfloat16, device=dev)
    ws_a = torch.empty(mla_workspace_bytes(B, h, S), dtype=torch.uint8, device=dev)

    def explicit():
        mla_explicit_decode(x["q"], x["cache"], x["w_uk"], x["w_uv"], x["seq_lens"], w.scale, out=out_e,
                            workspace=ws_e, stream=stream)

    def absorbed():
        mla_absorb_query(q_c, x["w_uk"], out=q_abs, stream=stream)
        mla_decode(q_abs, x["cache"], x["seq_lens"], w.scale, out=o_lat, workspace=ws_a, stream=stream)
        mla_up_project(o_lat, x["w_uv"], out=out_a, stream=stream)

    def time(fn, n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
        kev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
        for e in evs + kev:
            e.record(stream)
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        for i in range(n):
            evs[2 * i].record(stream)
            fn()
            evs[2 * i + 1].record(stream)
        torch.cuda.synchronize()
        for i in range(n):
            time_next_kernel(kev[2 * i], kev[2 * i + 1])
            fn()
        torch.cuda.synchronize()
        call = float(np.mean([evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(n)])) * 1e3
        kern = float(np.mean([kev[2 * i].elapsed_time(kev[2 * i + 1]) for i in range(n)])) * 1e3
        return call, kern

    n = max(3, min(steps, 10))
    nan = float("nan")  # a form not timed in this run (reported as null)
    e_call, e_attend = time(explicit, n) if forms in ("both", "explicit") else (nan, nan)
    a_call, a_decode = time(absorbed, max(n, 20)) if forms in ("both", "absorbed") else (nan, nan)
    ntok = B * S
    rec_flops = 2 * ntok * h * d_c * (d_h + d_v)            # rebuilding keys and values
    att_flops = 2 * ntok * h * (d_h + d_r + d_v)            # attention over the rebuilt rows
    rebuilt_bytes = ntok * h * (d_h + d_v) * 2              # rebuilt K and V (written once, read once)
    latent_bytes = ntok * (d_c + d_r) * 2
    weight_bytes = 2 * h * d_c * d_h * 2
    absorbed_flops = 2 * B * h * d_h * d_c + 2 * ntok * h * (2 * d_c + d_r) + 2 * B * h * d_c * d_v
    recon_us = e_call - e_attend
    att_read = rebuilt_bytes + ntok * d_r * 2 + B * h * (d_h + d_r + d_v) * 2
    del ws_e, x
    torch.cuda.empty_cache()
    out = {
        "workload": w.name,
        "explicit_call_us": round(e_call, 1),
        "explicit_attend_kernel_us": round(e_attend, 1),
        "explicit_rebuild_us": round(recon_us, 1),
        "explicit_rebuild_mfma_frac_of_bf16_peak": round(rec_flops / (recon_us * 1e-6) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                                                         4),
        "explicit_attend_hbm_frac": round(att_read / (e_attend * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "explicit_flops": int(rec_flops + att_flops),
        "explicit_hbm_bytes_min": int(latent_bytes + weight_bytes + 2 * rebuilt_bytes + ntok * d_r * 2),
        "absorbed_layer_call_us": round(a_call, 1),
        "absorbed_decode_kernel_us": round(a_decode, 1),
        "absorbed_flops": int(absorbed_flops),
        "absorbed_hbm_bytes": int(latent_bytes + weight_bytes + B * h * (d_h + d_r + d_v) * 2),
        "explicit_over_absorbed_time": round(e_call / a_call, 1),
        "explicit_over_absorbed_flops": round((rec_flops + att_flops) / absorbed_flops, 1),
        "rebuilt_bytes_per_token_over_latent": round(h * (d_h + d_v) * 2 / ((d_c + d_r) * 2), 2),
        "seq_steps_per_s": {"explicit": round(B / (e_call * 1e-6), 1), "absorbed": round(B / (a_call * 1e-6), 1)},
    }

    def clean(v):
        if isinstance(v, dict):
            return {k: clean(x) for k, x in v.items()}
        return None if isinstance(v, float) and math.isnan(v) else v

    return clean(out)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    from decode_attention_kv_03_amd.profiling import lookup_traffic
    from decode_attention_kv_03_amd import workloads as W

    if args.copy_calibration:
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4, "dispatches": args.steps}), flush=True)
        return

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    if args.mla_forms:
        print(json.dumps({"mla_absorbed_vs_explicit": mla_forms(torch, stream, args.steps, forms=args.mla_forms)}),
              flush=True)
        return
    w = W.WORKLOADS[args.workload]
    print(f"[bench] generating {w.name}", file=sys.stderr, flush=True)
    prep = Prepared(w, args.split_tokens, stream)
    nbytes, flops = prep.nbytes, prep.flops

    probe = hbm_probe(torch, stream)
    # The same probe at this call's own size: what a plain streaming read of the call's algorithmic
    # bytes reaches here, start-up and tail included (small calls lose more of their time to both).
    probe_same = hbm_probe(torch, stream, nbytes, prep.copies, workgroups=(512, 1024, 2048, 4096))

    for i in range(args.warmup):
        prep.step(i)
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps), timing {args.steps}", file=sys.stderr, flush=True)
    wall, call_ms, kern_ms, clock_ghz = timed_events(torch, prep, args.steps, wall=True)
    ms_per_step = wall * 1e3 / args.steps
    value = w.batch / (ms_per_step * 1e-3)
    head = rates(prep, call_ms, kern_ms, clock_ghz)

    # Roofline of the dominant kernel (the split-K kernel that streams the cache): the call's
    # algorithmic bytes over its mean duration.  The whole call (plus the merge, and for MLA the plan)
    # is reported beside it as call_frac: that is the figure a decode step sees.
    mean_kern_s = head["kernel_us_mean"] * 1e-6
    achieved_gbs = nbytes / mean_kern_s / 1e9
    traffic = lookup_traffic(w.name)
    roofline = {
        "bound": "hbm",
        "achieved": round(achieved_gbs, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
        "traffic": (traffic["fetch_bytes"] + traffic["write_bytes"]) if traffic else None,
        "kernel": head["kernel"],
        "kernel_us_mean": head["kernel_us_mean"],
        "kernel_us_p10_p50_p90": head["kernel_us_p10_p50_p90"],
        "algorithmic_bytes_per_launch": int(nbytes),
        "algorithmic_flops_per_launch": int(flops),
        "intensity_flop_per_byte": head["intensity_flop_per_byte"],
        "traffic_detail": traffic,
        "call_us_mean": head["call_us_mean"],
        "call_note": "whole library call: split-K kernel plus the log-sum-exp merge when the call splits, and "
                     "the device-side work-plan kernel of MLA and of the persistent GQA form (paged or ragged "
                     "batches with many splits); call_frac is the target figure, frac the kernel's own",
        "call_achieved_gbs": head["call_gbs"],
        "call_frac": head["call_frac"],
        "measured_read_ceiling_gbs": probe["gbs"],
        "frac_of_measured_ceiling": round(achieved_gbs / probe["gbs"], 4),
        "read_probe_same_bytes_gbs": probe_same["gbs"],
        "frac_of_read_probe_same_bytes": round(achieved_gbs / probe_same["gbs"], 4) if probe_same["gbs"] else None,
    }
    if not prep.is_gqa:
        roofline["mfma_tflops"] = head["mfma_tflops"]
        roofline["mfma_frac_of_bf16_peak"] = head["mfma_frac_of_bf16_peak"]
        roofline["shader_clock_ghz_in_kernel"] = head.get("shader_clock_ghz_in_kernel")
        roofline["mfma_frac_at_measured_clock"] = head.get("mfma_frac_at_measured_clock")


    cfg = {"workload": w.name, "batch": w.batch, "seq_len": w.seq_len, "dtype": w.dtype,
           "rotated_input_copies": prep.copies, "split_tokens": args.split_tokens or "auto"}
    if prep.is_gqa:
        cfg.update({"num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                    "block_size": w.block_size, "window": w.window})
        if w.paged:
            cfg["total_tokens"] = int(prep.lens.sum())
    else:
        cfg.update({"num_heads": w.num_heads, "d_latent": w.d_latent, "d_rope": w.d_rope, "block_size": w.block_size})
    all_configs = None
    if not args.no_all_configs:
        head_rates = dict(head, batch=w.batch, rotated_input_copies=prep.copies)
        all_configs = sweep(torch, stream, SWEEP, args.sweep_steps, 10, w.name, head_rates)
        all_configs["mla_absorbed_vs_explicit"] = mla_forms(torch, stream, args.sweep_steps)
    # The CPU reference last: the GPU idles meanwhile.
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU reference", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, prep.x0, args.cpu_seconds)
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "seq-steps/s per layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 cache, bf16 matrix cores, fp32 accumulation" if w.dtype == "fp8" else w.dtype,
        "data": ("synthetic (seeded iid N(0,1) over per-KV-head scales (1+U[0,1))/32, rounded to E4M3; bf16 query)"
                 if w.dtype == "fp8" else "synthetic (seeded iid N(0,1), rounded to the storage dtype)"),
        "config": cfg,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "hbm_read_probe": probe,
        "hbm_read_probe_same_bytes": probe_same,
        "all_configs": all_configs,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
