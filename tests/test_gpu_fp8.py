"""GPU parity of kvattn_gqa_decode_fp8 (E4M3 cache, per-KV-head scales) against the fp64 oracle.

Tolerance: |gpu - ref| <= 2e-2 + 1e-2 |ref| elementwise, as for a bf16 cache:
every E4M3 value widens exactly to bf16, so the kernel's only roundings are
those of the bf16 path (probabilities fed to the matrix cores as bf16, fp32
accumulation, bf16 output) plus the fp32 product of the softmax scale and
the K scale.  Log-sum-exp: atol 4e-3 (derived in tests/tolerances.py), rtol 1e-4.
"""

import numpy as np
import pytest
import torch

from tests.tolerances import LSE_ATOL, LSE_ATOL_F32  # noqa: F401

import oracle
from decode_attention_kv_03_amd import gqa_decode_fp8
from decode_attention_kv_03_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ATOL, RTOL = 2e-2, 1e-2


def setup_module(_):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def note(msg):
    print(f"\n[gpu-test] {msg}", flush=True)


def assert_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} outside tolerance, max abs err {err.max():.3e}"


def reference(x, rows=None, window=0):
    w = x["workload"]
    q = W.host_view(x["q"])
    lens = W.host_view(x["seq_lens"])
    ks, vs = W.host_view(x["k_scale"]), W.host_view(x["v_scale"])
    if rows is None:
        rows = list(range(w.batch))
    if w.paged:
        bt = W.host_view(x["block_table"])
        return oracle.paged_gqa_decode_fp8(q[rows], W.host_view(x["k"]), W.host_view(x["v"]), ks, vs, bt[rows],
                                           lens[rows], w.block_size, w.scale, window=window)
    k = np.stack([W.host_view(x["k"][b]) for b in rows])
    v = np.stack([W.host_view(x["v"][b]) for b in rows])
    return oracle.gqa_decode_fp8(q[rows], k, v, ks, vs, lens[rows], w.scale, window=window)


def run(x, **kw):
    w = x["workload"]
    out, lse = gqa_decode_fp8(x["q"], x["k"], x["v"], x["k_scale"], x["v_scale"], x["seq_lens"], w.scale,
                              block_table=x["block_table"], return_lse=True, **kw)
    torch.cuda.synchronize()
    return out, lse


CASES = [
    # B, h, g, lens, split_tokens
    (1, 8, 8, [1], 0),
    (2, 4, 1, [17, 128], 0),
    (3, 32, 8, [1, 127, 129], 64),
    (2, 32, 8, [255, 256], 128),
    (2, 16, 2, [200, 129], 64),
    (2, 64, 64, [300, 1], 128),
    (2, 64, 8, [511, 512], 0),
    (2, 64, 1, [777, 64], 256),
    (2, 32, 1, [1000, 999], 0),
    (2, 48, 1, [333, 100], 64),
    (1, 128, 1, [700], 192),
    (2, 96, 1, [129, 500], 64),
    (3, 12, 4, [70, 1, 5], 0),
]


@pytest.mark.parametrize("B,h,g,lens,split", CASES)
def test_fp8_contiguous_ragged_with_poisoned_tail(B, h, g, lens, split):
    S = max(lens) + 3
    w = W.GqaWorkload(f"fp8_{B}_{h}_{g}", B, h, g, 128, S, "fp8", 3000 + h + g, 1 / np.sqrt(128))
    note(f"fp8 B={B} h={h} g={g} lens={lens} split={split}")
    x = W.make_gqa_inputs(w, DEV, lens=lens, poison_tail=True)
    ref, ref_lse = reference(x)
    out, lse = run(x, split_tokens=split)
    assert_close(out.float().cpu().numpy(), ref)
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, atol=LSE_ATOL, rtol=1e-4)


@pytest.mark.parametrize("B,h,g,lens,window,split", [
    (3, 32, 8, [300, 64, 5], 100, 64),
    (2, 64, 1, [777, 200], 129, 128),
    (1, 8, 8, [513], 1, 64),
    (2, 128, 1, [700, 333], 257, 0),
])
def test_fp8_sliding_window(B, h, g, lens, window, split):
    w = W.GqaWorkload(f"fp8win_{B}_{h}_{g}", B, h, g, 128, max(lens) + 3, "fp8", 4000 + h + window, 1 / np.sqrt(128))
    note(f"fp8 window={window} B={B} h={h} g={g} lens={lens} split={split}")
    x = W.make_gqa_inputs(w, DEV, lens=lens, poison_tail=True)
    ref, ref_lse = reference(x, window=window)
    out, lse = run(x, split_tokens=split, window=window)
    assert_close(out.float().cpu().numpy(), ref, f"window={window}")
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, atol=LSE_ATOL, rtol=1e-4)


@pytest.mark.parametrize("block_size", [0, 16])
def test_fp8_sliding_window_last_split_takes_the_aligned_start(block_size):
    """The automatic plan sizes its splits for the window (128 units); the last split of each
    sequence also takes the up to 63 tokens its 64-aligned start adds."""
    # a paged cache plans on ragged-length grounds: there a 4096-token window takes this plan
    B, h, g = 16, 32, 8
    S, window = (4400, 4096) if block_size else (2400, 2048)
    rng = np.random.default_rng(4096 + block_size)
    lens = rng.integers(window + 64, S + 1, size=B)
    lens[lens % 64 == 0] -= 1
    w = W.GqaWorkload(f"fp8win_last_{block_size}", B, h, g, 128, S, "fp8", 4200 + block_size, 1 / np.sqrt(128),
                      block_size=block_size)
    note(f"fp8 window={window} B={B} lens={lens.tolist()} block_size={block_size} auto split")
    x = W.make_gqa_inputs(w, DEV, lens=lens, poison_tail=True)
    ref, ref_lse = reference(x, window=window)
    out, lse = run(x, split_tokens=0, window=window)
    assert_close(out.float().cpu().numpy(), ref, "window, last split past n_split x split")
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, atol=LSE_ATOL, rtol=1e-4)


@pytest.mark.parametrize("B,h,g,max_len,block_size,window", [
    (5, 64, 8, 900, 16, 0),     # power-of-two blocks of >= 8 tokens: scalar table loads per 8 rows
    (4, 16, 4, 600, 8, 0),
    (4, 16, 4, 600, 4, 0),      # blocks smaller than one copy instruction's 8 rows
    (3, 32, 2, 500, 5, 0),      # non-power-of-two block size
    (5, 64, 8, 900, 16, 200),
    (4, 64, 1, 700, 32, 77),
])
def test_fp8_paged(B, h, g, max_len, block_size, window):
    w = W.GqaWorkload(f"fp8paged_{block_size}", B, h, g, 128, max_len, "fp8", 5000 + block_size + h, 0.09,
                      block_size=block_size)
    note(f"fp8 paged B={B} h={h} g={g} max_len={max_len} block_size={block_size} window={window}")
    x = W.make_gqa_inputs(w, DEV, poison_tail=True)
    ref, ref_lse = reference(x, window=window)
    for split in (0, 64, 256):
        out, lse = run(x, split_tokens=split, window=window)
        assert_close(out.float().cpu().numpy(), ref, f"split={split}")
        np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, atol=LSE_ATOL, rtol=1e-4)


def test_fp8_zero_lengths_and_scales():
    w = W.GqaWorkload("fp8zero", 3, 8, 2, 128, 300, "fp8", 6, 0.1)
    note("fp8 zero lengths")
    x = W.make_gqa_inputs(w, DEV, lens=[0, 300, 0])
    for split in (0, 64):
        out, lse = run(x, split_tokens=split)
        o = out.float().cpu().numpy()
        assert np.all(o[0] == 0) and np.all(o[2] == 0)
        assert torch.all(torch.isneginf(lse[0])) and torch.all(torch.isneginf(lse[2]))
        ref, _ = reference(x, rows=[1])
        assert_close(o[1:2], ref)
    # the V scale multiplies the output of its group only; the K scale acts as a softmax-scale factor
    x2 = dict(x)
    x2["v_scale"] = x["v_scale"] * torch.tensor([2.0, 1.0], device=DEV)
    x2["k_scale"] = x["k_scale"] * torch.tensor([1.0, 0.5], device=DEV)
    ref2, ref2_lse = reference(x2)
    out2, lse2 = run(x2)
    assert_close(out2.float().cpu().numpy(), ref2, "rescaled")
    np.testing.assert_allclose(lse2.cpu().numpy(), ref2_lse, atol=LSE_ATOL, rtol=1e-4)


def test_fp8_rerun_is_bit_identical():
    w = W.shrink(W.WORKLOADS["llama3_70b_gqa_fp8_h64_g8_b64_s8192"], batch=4, seq_len=2048)
    note("fp8 determinism")
    x = W.make_gqa_inputs(w, DEV)
    a, la = run(x)
    b, lb = run(x)
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_fp8_full_size_sampled():
    """The full 70B GQA-8 layer with an fp8 cache, library-chosen launch; oracle on sampled sequences."""
    w = W.WORKLOADS["llama3_70b_gqa_fp8_h64_g8_b64_s8192"]
    note(w.name)
    x = W.make_gqa_inputs(w, DEV)
    out, lse = run(x)
    rows = [0, 31, 63]
    ref, ref_lse = reference(x, rows=rows)
    assert_close(out[rows].float().cpu().numpy(), ref, w.name)
    np.testing.assert_allclose(lse[rows].cpu().numpy(), ref_lse, atol=LSE_ATOL, rtol=1e-4)
    assert torch.isfinite(out.float()).all()
    del x
    torch.cuda.empty_cache()
