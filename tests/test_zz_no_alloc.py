"""kvattn_gqa_decode_noalloc (through the C ABI): the entry point that takes no
workspace and allocates nothing, its split-K partials in the library's fixed
per-GPU scratch array.

It must return exactly what kvattn_gqa_decode_window returns with a caller's
workspace (same kernels, same split plan), call after call, also when a
later call is smaller than an earlier one (the scratch keeps the last call's
contents), and match the fp64 oracle at the usual bar.
"""

import numpy as np
import pytest
import torch

import oracle
from decode_attention_kv_03_amd import gqa_decode, gqa_decode_noalloc
from decode_attention_kv_03_amd import workloads as W
from tests.tolerances import BF16_ATOL, BF16_RTOL, F32_ATOL, LSE_ATOL, LSE_ATOL_F32

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def setup_module(_):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def note(msg):
    print(f"\n[gpu-test] {msg}", flush=True)


def reference(x, window):
    w = x["workload"]
    q = W.host_view(x["q"])
    lens = W.host_view(x["seq_lens"])
    bf16 = w.dtype == "bf16"
    if w.paged:
        return oracle.paged_gqa_decode(q, W.host_view(x["k"]), W.host_view(x["v"]), W.host_view(x["block_table"]),
                                       lens, w.block_size, w.scale, bf16=bf16, window=window)
    return oracle.gqa_decode(q, W.host_view(x["k"]), W.host_view(x["v"]), lens, w.scale, bf16=bf16, window=window)


def both(x, split, window):
    w = x["workload"]
    B, h = w.batch, w.num_q_heads
    dt = W.torch_dtype(w.dtype)
    out_n = torch.empty((B, h, w.head_dim), dtype=dt, device=DEV)
    lse_n = torch.empty((B, h), dtype=torch.float32, device=DEV)
    gqa_decode_noalloc(x["q"], x["k"], x["v"], x["seq_lens"], w.scale, out_n, block_table=x["block_table"],
                       lse=lse_n, split_tokens=split, window=window)
    out_w, lse_w = gqa_decode(x["q"], x["k"], x["v"], x["seq_lens"], w.scale, block_table=x["block_table"],
                              return_lse=True, split_tokens=split, window=window)
    torch.cuda.synchronize()
    return out_n, lse_n, out_w, lse_w


def check(x, split, window=0):
    w = x["workload"]
    out_n, lse_n, out_w, lse_w = both(x, split, window)
    assert torch.equal(out_n, out_w) and torch.equal(lse_n, lse_w)
    ref, ref_lse = reference(x, window)
    got = out_n.double().cpu().numpy()
    err = np.abs(got - ref)
    if w.dtype == "f32":
        assert err.max() <= F32_ATOL
    else:
        assert not (err > BF16_ATOL + BF16_RTOL * np.abs(ref)).any(), f"max abs err {err.max():.3e}"
    l = lse_n.cpu().numpy()
    assert np.array_equal(np.isneginf(l), np.isneginf(ref_lse))
    fin = np.isfinite(ref_lse)
    np.testing.assert_allclose(l[fin], ref_lse[fin], atol=LSE_ATOL_F32 if w.dtype == "f32" else LSE_ATOL, rtol=1e-4)


def test_two_calls_in_a_row_second_smaller():
    big = W.GqaWorkload("noalloc_big", 6, 64, 8, 128, 1500, "bf16", 201, 1 / np.sqrt(128))
    small = W.GqaWorkload("noalloc_small", 2, 32, 8, 128, 700, "bf16", 202, 1 / np.sqrt(128))
    xb = W.make_gqa_inputs(big, DEV, lens=[1500, 3, 999, 64, 1200, 700], poison_tail=True)
    xs = W.make_gqa_inputs(small, DEV, lens=[700, 129], poison_tail=True)
    note("no-alloc: 6 x 1500 tokens at 64-token splits, then 2 x 700")
    check(xb, 64)
    check(xs, 64)
    check(xs, 0)


def test_paged_window_and_fp32():
    pw = W.GqaWorkload("noalloc_paged", 5, 32, 8, 128, 900, "bf16", 203, 1 / np.sqrt(128), block_size=16)
    xp = W.make_gqa_inputs(pw, DEV, poison_tail=True)
    note("no-alloc: paged, window 200")
    check(xp, 0, window=200)
    check(xp, 64)
    fw = W.GqaWorkload("noalloc_f32", 3, 8, 2, 128, 513, "f32", 204, 1 / np.sqrt(128))
    xf = W.make_gqa_inputs(fw, DEV, lens=[513, 1, 100], poison_tail=True)
    note("no-alloc: fp32, 64-token splits")
    check(xf, 64)


def test_full_size_paged_workload_bit_identical():
    w = W.WORKLOADS["paged_gqa_h64_g8_b128_bs16_len1_32768"]
    note(f"no-alloc: {w.name}")
    x = W.make_gqa_inputs(w, DEV)
    out_n, lse_n, out_w, lse_w = both(x, 0, 0)
    assert torch.equal(out_n, out_w) and torch.equal(lse_n, lse_w)
    del x
    torch.cuda.empty_cache()


def test_too_large_call_is_rejected():
    from decode_attention_kv_03_amd import kvattn

    w = W.GqaWorkload("noalloc_huge", 4, 128, 1, 128, 65536, "bf16", 205, 1 / np.sqrt(128))
    q = torch.zeros((4, 128, 128), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((4, 1, 65536, 128), dtype=torch.bfloat16, device=DEV)
    lens = torch.full((4,), 65536, dtype=torch.int32, device=DEV)
    out = torch.empty_like(q)
    with pytest.raises(ValueError, match="no-allocation"):
        gqa_decode_noalloc(q, k, k, lens, w.scale, out, split_tokens=64)
    assert kvattn.NOALLOC_SCRATCH_BYTES == 128 << 20
