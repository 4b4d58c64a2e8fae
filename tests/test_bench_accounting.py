"""The bench's algorithmic bytes and FLOPs per call (the numerator of its roofline), pinned (CPU).

Every expected number below is the pages' own accounting worked out for the
workload's shape, by hand: K and V bytes per token = 2 x KV heads x head
width x element size ("MQA, GQA, and MLA", section 1; "Why GQA's KV Cache
Savings Don't Fully Reduce TPOT"), (512 + 64) x 2 bytes per MLA token
("MQA, GQA, and MLA", section 5), and 2 FLOPs per multiply-add of the score
and attention-times-value products (section 4).  They are cross-checked with
the oracle's byte and intensity formulas, which are written independently
of bench.py.
"""

import importlib.util
import os

import numpy as np

import oracle.cache_bytes as cb
from decode_attention_kv_03_amd import workloads as W

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(_ROOT, "bench.py"))
bench = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(bench)


def _full(w):
    return np.full(w.batch, w.seq_len, dtype=np.int64)


def test_contiguous_gqa_family_bytes_and_flops():
    # (workload, KV bytes, query + output bytes, FLOPs), by hand at bf16 (2 bytes per element)
    cases = [
        ("llama3_8b_gqa_h32_g8_b16_s8192", 2 * 8 * 128 * 2 * 16 * 8192, 2 * 16 * 32 * 128 * 2, 4 * 32 * 128 * 16 * 8192),
        ("llama3_70b_mha_h64_g64_b8_s8192", 2 * 64 * 128 * 2 * 8 * 8192, 2 * 8 * 64 * 128 * 2, 4 * 64 * 128 * 8 * 8192),
        ("llama3_70b_gqa_h64_g8_b64_s8192", 2 * 8 * 128 * 2 * 64 * 8192, 2 * 64 * 64 * 128 * 2, 4 * 64 * 128 * 64 * 8192),
        ("llama3_70b_mqa_h64_g1_b64_s8192", 2 * 1 * 128 * 2 * 64 * 8192, 2 * 64 * 64 * 128 * 2, 4 * 64 * 128 * 64 * 8192),
    ]
    for name, kv, qo, flops in cases:
        w = W.WORKLOADS[name]
        nbytes, nflops = bench.algorithmic(w, _full(w))
        assert (nbytes, nflops) == (kv + qo, flops), name
        # the oracle's formula for the same cache (one layer) and the same FLOPs
        assert kv == cb.kv_cache_bytes(1, w.num_kv_heads, w.head_dim, w.seq_len, w.batch, 2)
        assert flops == w.batch * cb.decode_attention_flops(w.num_q_heads, w.seq_len, w.head_dim)
    # the caches of these layers: 512 MiB, 2 GiB, 2 GiB, 256 MiB of K and V
    assert [c[1] for c in cases] == [512 << 20, 2 << 30, 2 << 30, 256 << 20]


def test_intensity_rises_with_group_size():
    # FLOPs per KV byte of the one-dial sweep at bf16: 2 (h/g) / 2 = 1, 8, 64
    got = []
    for name in ("llama3_70b_mha_h64_g64_b8_s8192", "llama3_70b_gqa_h64_g8_b64_s8192", "llama3_70b_mqa_h64_g1_b64_s8192"):
        w = W.WORKLOADS[name]
        _, flops = bench.algorithmic(w, _full(w))
        kv = cb.kv_cache_bytes(1, w.num_kv_heads, w.head_dim, w.seq_len, w.batch, 2)
        got.append(flops / kv)
        assert flops / kv == cb.decode_attention_intensity(w.num_q_heads, w.num_kv_heads, 2)
    assert got == [1.0, 8.0, 64.0]


def test_fp8_cache_halves_the_kv_bytes():
    w = W.WORKLOADS["llama3_70b_gqa_fp8_h64_g8_b64_s8192"]
    nbytes, flops = bench.algorithmic(w, _full(w))
    kv = 2 * 8 * 128 * 1 * 64 * 8192  # one byte per element
    qo = 2 * 64 * 64 * 128 * 2        # bf16 queries and outputs
    scales = 2 * 4 * 8                # one fp32 K and one fp32 V scale per KV head
    assert nbytes == kv + qo + scales and kv == (1 << 30)
    assert flops == 4 * 64 * 128 * 64 * 8192


def test_mla_bytes_and_flops():
    w = W.WORKLOADS["deepseek_v2_mla_h128_b32_s8192"]
    nbytes, flops = bench.algorithmic(w, _full(w))
    cache = 32 * 8192 * 576 * 2       # one latent row per token, shared by all heads
    q = 32 * 128 * 576 * 2
    out = 32 * 128 * 512 * 2
    assert nbytes == cache + q + out == 310_902_784
    assert cache == cb.mla_cache_bytes(1, 512, 64, 8192, 32, 2)
    assert flops == 2 * 128 * (576 + 512) * 32 * 8192 == 73_014_444_032


def test_ragged_paged_and_window_accounting():
    # paged: every valid token's rows plus one 4-byte table entry per used block
    w = W.WORKLOADS["paged_gqa_h64_g8_b128_bs16_len1_32768"]
    lens = np.array([1, 16, 17, 32768] + [5] * (w.batch - 4))
    nbytes, flops = bench.algorithmic(w, lens)
    tokens = int(lens.sum())
    blocks = int(((lens + 15) // 16).sum())
    assert nbytes == 2 * 8 * 128 * 2 * tokens + 2 * w.batch * 64 * 128 * 2 + 4 * blocks
    assert flops == 4 * 64 * 128 * tokens
    # sliding window: a sequence reads only its last `window` tokens
    s = W.WORKLOADS["mistral7b_swa_h32_g8_b16_s32768_w4096"]
    lens = np.array([100, 4096, 5000, 32768] + [32768] * (s.batch - 4))
    nbytes, flops = bench.algorithmic(s, lens)
    read = 100 + 4096 * (s.batch - 1)  # 100, then 4096 for every other sequence (4096, 5000, 32768, ...)
    assert nbytes == 2 * 8 * 128 * 2 * read + 2 * s.batch * 32 * 128 * 2
    assert flops == 4 * 32 * 128 * read


def test_probe_reads_whole_tiles_per_workgroup():
    # The read probe splits its buffer evenly in 16 KiB tiles and leaves any rest to one workgroup;
    # the bench therefore hands it a whole number of tiles per workgroup, never more than asked.
    mqa = 2 * 1 * 128 * 2 * 64 * 8192 + 2 * 64 * 64 * 128 * 2  # the MQA layer's algorithmic bytes
    assert mqa == 270_532_608
    for wgs in (512, 1024, 2048, 4096):
        nb = bench.probe_bytes(mqa, wgs)
        assert nb % (16384 * wgs) == 0 and 0 < nb <= mqa and mqa - nb < 16384 * wgs
    assert bench.probe_bytes(mqa, 512) == 256 << 20
    assert bench.probe_bytes(2 << 30, 4096) == 2 << 30
    assert bench.probe_bytes(1 << 20, 512) == 0  # too small for one tile per workgroup: no probe
    assert bench.probe_pitch(4097) == 8192 and bench.probe_pitch(4096) == 4096
