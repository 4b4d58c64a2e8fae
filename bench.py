"""Decode-attention benchmark: one decode step of one layer per timed step.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one full library call (split-K kernel plus, when the call splits,
the log-sum-exp merge) over the workload's synthetic inputs, already
resident in HBM.  The default workload is the Llama-3-8B-shaped GQA layer
(h=32, g=8, d=128, bf16, batch 16, every sequence 8192 tokens).  Prints one
JSON line: throughput in sequence-steps per second per layer, the roofline
of the split-K kernel that streams the cache (algorithmic HBM bytes / its
measured duration, timed with HIP events around that kernel alone, against the
8 TB/s HBM3E peak; for MLA also its matrix-core rate against 2.5 PFLOP/s),
and the fp64 CPU reference timed on a bounded sample of the same workload.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn achieved HBM GB/s (% peak) + MFMA util (MLA); seq-steps/s per layer"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
DEFAULT_WORKLOAD = "llama3_8b_gqa_h32_g8_b16_s8192"
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
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    distinct = min(done, len(order))
    return {
        "value": done / t_total,
        "unit": "seq-steps/s per layer",
        "cores": int(threads),
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
    `nbytes` (the probe splits its buffer evenly in 16 KiB tiles; an uneven rest would be read by a
    single workgroup), and the rate is taken over the bytes actually read.
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


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from decode_attention_kv_03_amd import (gqa_decode, gqa_decode_fp8, gqa_workspace_bytes, mla_decode,
                                            mla_workspace_bytes)
    from decode_attention_kv_03_amd import time_next_kernel
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

    w = W.WORKLOADS[args.workload]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    is_gqa = hasattr(w, "num_kv_heads")
    make = W.make_gqa_inputs if is_gqa else W.make_mla_inputs
    print(f"[bench] generating {w.name}", file=sys.stderr, flush=True)
    x0 = make(w, dev)
    lens = W.host_view(x0["seq_lens"])
    nbytes, flops = algorithmic(w, lens)
    # Enough copies of the cache that the bytes one step reads cycle through at least 1 GiB (no step
    # finds its data in the 256 MB last-level cache); a sliding window reads only part of its cache.
    copies = max(1, min(8, math.ceil(ROTATE_BYTES / max(nbytes, 1))))
    xs = [x0]
    for c in range(1, copies):
        xc = dict(x0)
        for k in ("k", "v", "cache"):
            if k in x0:
                xc[k] = x0[k].clone()
        xs.append(xc)

    stream = torch.cuda.current_stream()
    probe = hbm_probe(torch, stream)
    # The same probe at this call's own size: what a plain streaming read of the call's algorithmic
    # bytes reaches here, start-up and tail included (small calls lose more of their time to both).
    probe_same = hbm_probe(torch, stream, nbytes, copies, workgroups=(512, 1024, 2048, 4096))
    if is_gqa:
        out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=x0["q"].dtype, device=dev)
        max_len = w.seq_len
        ws_n = gqa_workspace_bytes(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, max_len, w.block_size,
                                   args.split_tokens, x0["q"].dtype)
    else:
        out = torch.empty((w.batch, w.num_heads, w.d_latent), dtype=x0["q"].dtype, device=dev)
        max_len = w.seq_len
        ws_n = mla_workspace_bytes(w.batch, w.num_heads, max_len, w.d_latent, w.d_rope, w.block_size,
                                   args.split_tokens)
    ws = torch.zeros(max(ws_n, 1), dtype=torch.uint8, device=dev)  # zero-filled once, as the ABI asks

    def step(i):
        x = xs[i % copies]
        if is_gqa and w.dtype == "fp8":
            gqa_decode_fp8(x["q"], x["k"], x["v"], x["k_scale"], x["v_scale"], x["seq_lens"], w.scale,
                           block_table=x["block_table"], max_seq_len=max_len, out=out, split_tokens=args.split_tokens,
                           workspace=ws, stream=stream, window=w.window)
        elif is_gqa:
            gqa_decode(x["q"], x["k"], x["v"], x["seq_lens"], w.scale, block_table=x["block_table"],
                       max_seq_len=max_len, out=out, split_tokens=args.split_tokens, workspace=ws, stream=stream,
                       window=w.window)
        else:
            mla_decode(x["q"], x["cache"], x["seq_lens"], w.scale, block_table=x["block_table"], max_seq_len=max_len,
                       out=out, split_tokens=args.split_tokens, workspace=ws, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps), timing {args.steps}", file=sys.stderr, flush=True)

    # Timed region 1 (the headline): the K calls back to back, wall time between two
    # synchronisations, nothing else on the stream.  Region 2: the same K calls with HIP events
    # around each whole call on the stream the kernels run on.  Region 3: HIP events around each
    # call's split-K kernel alone (kvattn_time_next_kernel), for the kernel roofline.  They are kept
    # apart because event packets between the calls cost a few microseconds each.
    def events(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evs:
            e.record(stream)  # creates the underlying HIP event
        return evs

    starts, ends, kstarts, kends = (events(args.steps) for _ in range(4))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for i in range(args.steps):
        starts[i].record(stream)
        step(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    for i in range(args.steps):
        time_next_kernel(kstarts[i], kends[i])
        step(i)
    torch.cuda.synchronize()
    call_ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    kern_ms = np.array([s.elapsed_time(e) for s, e in zip(kstarts, kends)])
    ms_per_step = wall * 1e3 / args.steps
    mean_call_s = float(call_ms.mean()) * 1e-3
    mean_kern_s = float(kern_ms.mean()) * 1e-3
    value = w.batch / (ms_per_step * 1e-3)

    # Roofline of the dominant kernel (the split-K kernel that streams the cache): the call's
    # algorithmic bytes over its mean duration.
    achieved_gbs = nbytes / mean_kern_s / 1e9
    call_gbs = nbytes / mean_call_s / 1e9
    traffic = lookup_traffic(w.name)
    roofline = {
        "bound": "hbm",
        "achieved": round(achieved_gbs, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
        "traffic": (traffic["fetch_bytes"] + traffic["write_bytes"]) if traffic else None,
        "kernel": f"gqa_split_{w.dtype}" if is_gqa else "mla_split_bf16",
        "kernel_us_mean": round(mean_kern_s * 1e6, 2),
        "kernel_us_p10_p50_p90": [round(float(np.percentile(kern_ms, p)) * 1e3, 2) for p in (10, 50, 90)],
        "algorithmic_bytes_per_launch": int(nbytes),
        "algorithmic_flops_per_launch": int(flops),
        "intensity_flop_per_byte": round(flops / nbytes, 2),
        "traffic_detail": traffic,
        "call_us_mean": round(mean_call_s * 1e6, 2),
        "call_note": "whole library call: split-K kernel plus the log-sum-exp merge when the call splits",
        "call_achieved_gbs": round(call_gbs, 1),
        "call_frac": round(call_gbs / HBM_PEAK_GBS, 4),
        "measured_read_ceiling_gbs": probe["gbs"],
        "frac_of_measured_ceiling": round(achieved_gbs / probe["gbs"], 4),
        "read_probe_same_bytes_gbs": probe_same["gbs"],
        "frac_of_read_probe_same_bytes": round(achieved_gbs / probe_same["gbs"], 4) if probe_same["gbs"] else None,
    }
    if not is_gqa:
        roofline["mfma_tflops"] = round(flops / mean_kern_s / 1e12, 1)
        roofline["mfma_frac_of_bf16_peak"] = round(flops / mean_kern_s / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU reference", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, x0, args.cpu_seconds)

    cfg = {"workload": w.name, "batch": w.batch, "seq_len": w.seq_len, "dtype": w.dtype,
           "rotated_input_copies": copies, "split_tokens": args.split_tokens or "auto"}
    if is_gqa:
        cfg.update({"num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                    "block_size": w.block_size, "window": w.window})
    else:
        cfg.update({"num_heads": w.num_heads, "d_latent": w.d_latent, "d_rope": w.d_rope, "block_size": w.block_size})
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
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
