"""Seeded synthetic inputs for decode attention over a KV cache.

This module holds random draws and input layout only (shapes, dtypes, the
per-sequence lengths and the block table of a paged cache); it does none of
the attention arithmetic.  The GPU tests, the bench and the CPU reference
checks all take their inputs from here, so both sides of a parity check see
the same bytes.

The named workloads are the shapes the pages discuss, made concrete:
Llama-3-8B-shaped and Llama-3-70B-shaped decode layers (the GQA dial at its
MHA, GQA-8 and MQA settings, "MQA, GQA, and MLA" sections 2-4), a paged cache
with ragged lengths ("Compressing the KV Cache ...", KV-Cache Management
Guardrails), and a DeepSeek-V2-shaped absorbed-MLA layer (128 heads, latent
512 + RoPE 64, "MQA, GQA, and MLA" section 5).  Values are iid N(0,1) drawn
in float32 and rounded to the storage dtype (round to nearest even).

An fp8 cache ("Why GQA's KV Cache Savings Don't Fully Reduce TPOT", section
"When the Serving Engineer Doesn't Get to Choose") is drawn per KV head j
with a scale s_j = (1 + u_j) / 32, u_j uniform on [0, 1) (separately for K
and V): the stored codes are torch's E4M3 rounding of N(0,1) / s_j, so the
cache holds s_j * E4M3(code) ~ N(0,1) and no draw comes near the format's
largest value (448 * s_j >= 14 standard deviations).
"""

from dataclasses import dataclass, replace
import math

import numpy as np
import torch


@dataclass(frozen=True)
class GqaWorkload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    seq_len: int  # contiguous: every sequence's length and the cache capacity; paged: maximum length
    dtype: str  # cache dtype: "f32", "bf16" or "fp8" (E4M3 codes, bf16 query and output)
    seed: int
    scale: float
    block_size: int = 0  # 0: contiguous cache [B, g, S, d]; else pool [num_blocks, g, block_size, d]
    window: int = 0  # sliding window: attend to the last `window` tokens (0: all)

    @property
    def paged(self):
        return self.block_size > 0


@dataclass(frozen=True)
class MlaWorkload:
    name: str
    batch: int
    num_heads: int
    seq_len: int
    seed: int
    scale: float
    d_latent: int = 512
    d_rope: int = 64
    dtype: str = "bf16"
    block_size: int = 0  # 0: contiguous [B, S, d_latent + d_rope]; else pool [num_blocks, block_size, 576]
    form: str = "absorbed"  # "explicit": per-head query [q^C | q^R] and weights W_uk, W_uv (reconstruct, then attend)
    d_head: int = 128  # explicit form: per-head content key width (W_uk [h, d_latent, d_head])
    d_v: int = 128  # explicit form: per-head value width (W_uv [h, d_latent, d_v])

    @property
    def paged(self):
        return self.block_size > 0


WORKLOADS = {
    w.name: w
    for w in [
        GqaWorkload("gqa_h8_g2_d128_s512_b1_f32", 1, 8, 2, 128, 512, "f32", 1, 1 / math.sqrt(128)),
        GqaWorkload("llama3_8b_gqa_h32_g8_b16_s8192", 16, 32, 8, 128, 8192, "bf16", 2, 1 / math.sqrt(128)),
        GqaWorkload("llama3_70b_mha_h64_g64_b8_s8192", 8, 64, 64, 128, 8192, "bf16", 31, 1 / math.sqrt(128)),
        GqaWorkload("llama3_70b_gqa_h64_g8_b64_s8192", 64, 64, 8, 128, 8192, "bf16", 32, 1 / math.sqrt(128)),
        GqaWorkload("llama3_70b_mqa_h64_g1_b64_s8192", 64, 64, 1, 128, 8192, "bf16", 33, 1 / math.sqrt(128)),
        # The 70B GQA-8 layer with an E4M3 cache (one K and one V scale per KV head).
        GqaWorkload("llama3_70b_gqa_fp8_h64_g8_b64_s8192", 64, 64, 8, 128, 8192, "fp8", 34, 1 / math.sqrt(128)),
        GqaWorkload("paged_gqa_h64_g8_b128_bs16_len1_32768", 128, 64, 8, 128, 32768, "bf16", 4, 1 / math.sqrt(128), 16),
        # Sliding-window decode at Mistral-7B v0.1's shape (h=32, g=8, window 4096) over 32K-token sequences.
        GqaWorkload("mistral7b_swa_h32_g8_b16_s32768_w4096", 16, 32, 8, 128, 32768, "bf16", 6, 1 / math.sqrt(128),
                    window=4096),
        MlaWorkload("deepseek_v2_mla_h128_b32_s8192", 32, 128, 8192, 5, 1 / math.sqrt(192)),
        # Paged latent cache: 64-token blocks, lengths uniform on [1, 16384], a random block permutation.
        MlaWorkload("deepseek_v2_mla_paged_h128_b32_bs64_len1_16384", 32, 128, 16384, 7, 1 / math.sqrt(192),
                    block_size=64),
        # One sequence of 128K tokens: the long-context decode of a single request, where the split
        # over tokens alone fills the chip ("MQA, GQA, and MLA" section 9 speaks of MLA at 128k context).
        GqaWorkload("llama3_70b_gqa_h64_g8_b1_s131072", 1, 64, 8, 128, 131072, "bf16", 35, 1 / math.sqrt(128)),
        GqaWorkload("llama3_70b_mqa_h64_g1_b1_s131072", 1, 64, 1, 128, 131072, "bf16", 36, 1 / math.sqrt(128)),
        MlaWorkload("deepseek_v2_mla_h128_b1_s131072", 1, 128, 131072, 9, 1 / math.sqrt(192)),
        # The same DeepSeek-V2 layer in the naive form: per-head query and synthetic up-projection weights.
        MlaWorkload("deepseek_v2_mla_explicit_h128_b32_s8192", 32, 128, 8192, 8, 1 / math.sqrt(192), form="explicit"),
    ]
}


def torch_dtype(name):
    """Query/output dtype of a workload (an fp8 cache pairs with a bfloat16 query)."""
    return {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.bfloat16}[name]


def _fp8_codes(shape, gen, device, scales, head_dim_axis, chunks=1):
    """E4M3 codes (uint8) of iid N(0,1) / scales[j], j along ``head_dim_axis``; drawn in ``chunks`` slabs."""
    out = torch.empty(shape, dtype=torch.uint8, device=device)
    view = [1] * len(shape)
    view[head_dim_axis] = -1
    inv = (1.0 / scales).reshape(view)
    n0 = shape[0]
    step = max(1, (n0 + chunks - 1) // chunks)
    for a in range(0, n0, step):
        b = min(n0, a + step)
        x = torch.randn((b - a, *shape[1:]), generator=gen, device=device, dtype=torch.float32) * inv
        out[a:b] = x.to(torch.float8_e4m3fn).view(torch.uint8)
    return out


def _randn(shape, gen, device, dtype, chunks=1, std=1.0):
    """iid N(0, std^2) drawn in float32 then rounded to ``dtype``; drawn in ``chunks`` slabs along dim 0."""
    out = torch.empty(shape, dtype=dtype, device=device)
    n0 = shape[0]
    step = max(1, (n0 + chunks - 1) // chunks)
    for a in range(0, n0, step):
        b = min(n0, a + step)
        x = torch.randn((b - a, *shape[1:]), generator=gen, device=device, dtype=torch.float32)
        out[a:b] = (x * std if std != 1.0 else x).to(dtype)
    return out


def ragged_lengths_and_table(batch, max_len, block_size, seed, lens=None):
    """Paged-cache structure: lengths uniform on {1..max_len}, then a random permutation of physical blocks.

    Logical blocks are enumerated sequence by sequence; sequence ``b``'s k-th
    block is ``perm[offset_b + k]``; unused table entries are -1.  ``lens``
    fixes the lengths instead of drawing them (the permutation is still
    drawn).  Returns (lens int32 [B], table int32 [B, ceil(max_len/block_size)],
    num_blocks).
    """
    rng = np.random.default_rng(seed)
    if lens is None:
        lens = rng.integers(1, max_len + 1, size=batch)
    else:
        lens = np.asarray(lens, dtype=np.int64)
        assert lens.shape == (batch,) and lens.min() >= 0 and lens.max() <= max_len
    nblk = (lens + block_size - 1) // block_size
    num_blocks = int(nblk.sum())
    perm = rng.permutation(num_blocks)
    max_blocks = (max_len + block_size - 1) // block_size
    table = np.full((batch, max_blocks), -1, dtype=np.int64)
    off = 0
    for b in range(batch):
        table[b, : nblk[b]] = perm[off : off + nblk[b]]
        off += int(nblk[b])
    return lens.astype(np.int32), table.astype(np.int32), num_blocks


def make_gqa_inputs(w, device="cpu", lens=None, poison_tail=False):
    """Inputs for one GQA/MHA/MQA decode step.

    Returns a dict with q [B,h,d], k, v (contiguous [B,g,S,d] or pool
    [N,g,bs,d]), seq_lens int32 [B], block_table int32 [B, max_blocks] or
    None, all on ``device``.  ``lens`` overrides the per-sequence lengths
    (default: every sequence of a contiguous cache is full; a paged cache
    draws them uniformly on {1..seq_len}).  With
    ``poison_tail`` every cache slot past a sequence's length holds NaN.
    """
    gen = torch.Generator(device=device).manual_seed(w.seed)
    dt = torch_dtype(w.dtype)
    B, h, g, d = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
    q = _randn((B, h, d), gen, device, dt)
    fp8 = w.dtype == "fp8"
    if fp8:
        k_scale = (1.0 + torch.rand(g, generator=gen, device=device, dtype=torch.float32)) / 32
        v_scale = (1.0 + torch.rand(g, generator=gen, device=device, dtype=torch.float32)) / 32

    def cache(shape, chunks, scales):
        return _fp8_codes(shape, gen, device, scales, 1, chunks) if fp8 else _randn(shape, gen, device, dt, chunks)

    if w.paged:
        lens_np, table, N = ragged_lengths_and_table(B, w.seq_len, w.block_size, w.seed, lens)
        N = max(N, 1)
        k = cache((N, g, w.block_size, d), 16, k_scale if fp8 else None)
        v = cache((N, g, w.block_size, d), 16, v_scale if fp8 else None)
        bt = torch.from_numpy(table).to(device)
    else:
        lens_np = np.full(B, w.seq_len, dtype=np.int32) if lens is None else np.asarray(lens, dtype=np.int32)
        k = cache((B, g, w.seq_len, d), B, k_scale if fp8 else None)
        v = cache((B, g, w.seq_len, d), B, v_scale if fp8 else None)
        bt = None
    if poison_tail:
        _poison(k, v, lens_np, bt, w.block_size)
    inputs = {
        "q": q,
        "k": k,
        "v": v,
        "seq_lens": torch.from_numpy(lens_np.astype(np.int32)).to(device),
        "block_table": bt,
        "workload": w,
    }
    if fp8:
        inputs["k_scale"], inputs["v_scale"] = k_scale, v_scale
    return inputs


def make_mla_inputs(w, device="cpu", lens=None, poison_tail=False):
    """Inputs for one absorbed-MLA decode step: q [B,h,576], cache [B,S,576] or pool [N,bs,576]."""
    gen = torch.Generator(device=device).manual_seed(w.seed)
    dt = torch_dtype(w.dtype)
    B, h, width = w.batch, w.num_heads, w.d_latent + w.d_rope
    q = _randn((B, h, width), gen, device, dt)
    if w.paged:
        lens_np, table, N = ragged_lengths_and_table(B, w.seq_len, w.block_size, w.seed, lens)
        N = max(N, 1)
        cache = _randn((N, w.block_size, width), gen, device, dt, chunks=16)
        bt = torch.from_numpy(table).to(device)
    else:
        lens_np = np.full(B, w.seq_len, dtype=np.int32) if lens is None else np.asarray(lens, dtype=np.int32)
        cache = _randn((B, w.seq_len, width), gen, device, dt, chunks=B)
        bt = None
    if poison_tail:
        _poison(cache, None, lens_np, bt, w.block_size)
    return {
        "q": q,
        "cache": cache,
        "seq_lens": torch.from_numpy(lens_np.astype(np.int32)).to(device),
        "block_table": bt,
        "workload": w,
    }


def make_mla_explicit_inputs(w, device="cpu", lens=None, poison_tail=False):
    """Inputs for one reconstruct-then-attend MLA step (contiguous latent cache).

    q [B, h, d_head + d_rope] rows [q^C | q^R] ~ N(0,1); cache [B, S, 576] ~
    N(0,1); W_uk [h, d_latent, d_head] and W_uv [h, d_latent, d_v] ~
    N(0, 1/d_latent), so that rebuilt keys and values are ~ N(0,1) per
    component (and scale 1/sqrt(d_head + d_rope) keeps scores ~ N(0,1)).
    Drawn in that order, all bfloat16.  The pages give no weights; these are
    synthetic stand-ins of DeepSeek-V2's shapes.
    """
    gen = torch.Generator(device=device).manual_seed(w.seed)
    dt = torch_dtype(w.dtype)
    B, h, width = w.batch, w.num_heads, w.d_latent + w.d_rope
    q = _randn((B, h, w.d_head + w.d_rope), gen, device, dt)
    lens_np = np.full(B, w.seq_len, dtype=np.int32) if lens is None else np.asarray(lens, dtype=np.int32)
    cache = _randn((B, w.seq_len, width), gen, device, dt, chunks=B)
    std = 1.0 / math.sqrt(w.d_latent)
    w_uk = _randn((h, w.d_latent, w.d_head), gen, device, dt, std=std)
    w_uv = _randn((h, w.d_latent, w.d_v), gen, device, dt, std=std)
    if poison_tail:
        _poison(cache, None, lens_np, None, 0)
    return {
        "q": q,
        "cache": cache,
        "w_uk": w_uk,
        "w_uv": w_uv,
        "seq_lens": torch.from_numpy(lens_np.astype(np.int32)).to(device),
        "block_table": None,
        "workload": w,
    }


def _poison(k, v, lens_np, bt, block_size):
    """Fill every cache slot past each sequence's length with NaN (catches reads past the end).

    An fp8 (uint8) cache gets the E4M3 NaN code 0x7F."""
    nan = float("nan") if k.dtype != torch.uint8 else 0x7F
    for t in (k, v):
        if t is None:
            continue
        if bt is None:
            for b, n in enumerate(lens_np):
                if t.dim() == 4:
                    t[b, :, int(n):] = nan
                else:
                    t[b, int(n):] = nan
        else:
            table = bt.cpu().numpy()
            for b, n in enumerate(lens_np):
                n = int(n)
                if n % block_size:
                    blk = int(table[b, n // block_size])
                    if t.dim() == 4:
                        t[blk, :, n % block_size:] = nan
                    else:
                        t[blk, n % block_size:] = nan


def host_view(t):
    """Host copy in the form the CPU reference takes: float64 for f32, uint16 bit patterns for bf16, raw
    codes for an fp8 (uint8) cache."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.int32, torch.int64, torch.uint8):
        return t.numpy()
    return t.to(torch.float64).numpy()


def shrink(w, **kw):
    """Same workload with some fields replaced (smaller batch or length for CPU-sized checks)."""
    return replace(w, **kw)
