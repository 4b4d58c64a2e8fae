"""Seeded input generators: determinism and structural validity (CPU)."""

import numpy as np
import torch

from decode_attention_kv_03_amd import workloads as W


def test_named_workloads_have_expected_shapes():
    c = W.WORKLOADS
    assert c["gqa_h8_g2_d128_s512_b1_f32"].dtype == "f32"
    w70 = [c[n] for n in c if n.startswith("llama3_70b") and c[n].dtype == "bf16" and c[n].seq_len == 8192]
    assert sorted((w.num_kv_heads, w.batch) for w in w70) == [(1, 64), (8, 64), (64, 8)]
    long = [c[n] for n in c if c[n].seq_len == 131072]
    assert sorted((getattr(w, "num_kv_heads", 0), w.batch) for w in long) == [(0, 1), (1, 1), (8, 1)]
    f8 = c["llama3_70b_gqa_fp8_h64_g8_b64_s8192"]
    assert (f8.dtype, f8.num_q_heads, f8.num_kv_heads, f8.batch, f8.seq_len) == ("fp8", 64, 8, 64, 8192)
    m = c["deepseek_v2_mla_h128_b32_s8192"]
    assert (m.num_heads, m.d_latent + m.d_rope, m.batch, m.seq_len) == (128, 576, 32, 8192)
    assert abs(m.scale - 1 / np.sqrt(192)) < 1e-12


def test_ragged_lengths_and_table_are_valid():
    lens, table, N = W.ragged_lengths_and_table(128, 32768, 16, 4)
    assert lens.min() >= 1 and lens.max() <= 32768
    nblk = (lens + 15) // 16
    assert N == nblk.sum()
    used = np.concatenate([table[b, : nblk[b]] for b in range(128)])
    assert np.array_equal(np.sort(used), np.arange(N))  # every physical block exactly once
    for b in range(128):
        assert np.all(table[b, nblk[b]:] == -1)
    lens2, table2, _ = W.ragged_lengths_and_table(128, 32768, 16, 4)
    assert np.array_equal(lens, lens2) and np.array_equal(table, table2)


def test_generation_is_deterministic_and_poison_marks_tail():
    w = W.shrink(W.WORKLOADS["llama3_8b_gqa_h32_g8_b16_s8192"], batch=2, seq_len=40)
    a = W.make_gqa_inputs(w, "cpu", lens=[40, 17])
    b = W.make_gqa_inputs(w, "cpu", lens=[40, 17], poison_tail=True)
    assert a["q"].dtype == torch.bfloat16 and a["k"].shape == (2, 8, 40, 128)
    assert torch.equal(a["q"], b["q"])
    assert torch.equal(a["k"][1, :, :17], b["k"][1, :, :17])
    assert torch.isnan(b["k"][1, :, 17:].float()).all() and not torch.isnan(b["k"][0].float()).any()
    pw = W.shrink(W.WORKLOADS["paged_gqa_h64_g8_b128_bs16_len1_32768"], batch=3, seq_len=100)
    p = W.make_gqa_inputs(pw, "cpu", poison_tail=True)
    lens = p["seq_lens"].numpy()
    tab = p["block_table"].numpy()
    for bb, n in enumerate(lens):
        if n % 16:
            blk = tab[bb, n // 16]
            assert torch.isnan(p["k"][blk, :, n % 16:].float()).all()
            assert not torch.isnan(p["k"][blk, :, : n % 16].float()).any()


def test_host_view_round_trips_bits():
    t = torch.randn(5, 7).to(torch.bfloat16)
    h = W.host_view(t)
    assert h.dtype == np.uint16
    assert torch.equal(torch.from_numpy(h.view(np.int16)).view(torch.bfloat16), t)


def test_fp8_inputs_hold_codes_and_per_head_scales():
    w = W.GqaWorkload("f8", 2, 8, 2, 128, 300, "fp8", 11, 0.1)
    x = W.make_gqa_inputs(w, "cpu", lens=[300, 17], poison_tail=True)
    assert x["q"].dtype == torch.bfloat16 and x["k"].dtype == torch.uint8 and x["k_scale"].shape == (2,)
    assert torch.all((x["k_scale"] >= 1 / 32) & (x["k_scale"] < 2 / 32))
    # codes past each length are the E4M3 NaN code; none inside (no draw saturates)
    assert torch.all(x["k"][1, :, 17:] == 0x7F) and not torch.any(x["k"][0] == 0x7F)
    vals = x["v"][0].view(torch.float8_e4m3fn).float() * x["v_scale"][:, None, None]
    assert abs(float(vals.std()) - 1.0) < 0.05
    y = W.make_gqa_inputs(w, "cpu", lens=[300, 17], poison_tail=True)
    assert torch.equal(x["k"], y["k"]) and torch.equal(x["v_scale"], y["v_scale"])
