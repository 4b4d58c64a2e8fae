"""Seeded random shapes against the fp64 oracle (GPU): every combination of the call's dials drawn at
random, so that paths meet in combinations the targeted tests do not name.

GQA: dtype (bf16, fp8, fp32), head-group size r = h/g from 1 to 64, batch 1-6, lengths from 0 to
3000 (zeros included), contiguous or paged (block sizes 1-32; fp32 contiguous only), with or without
a sliding window, automatic or requested split sizes.  MLA: 16-128 heads, batch 1-5, lengths up to
5000, contiguous or paged, automatic or requested pieces.  Each case compares every output element and
log-sum-exp with the oracle at the tolerances of the targeted tests.
"""

import numpy as np
import pytest
import torch

from decode_attention_kv_03_amd import workloads as W
from tests import test_gpu_fp8 as F8
from tests import test_gpu_gqa as G
from tests import test_gpu_mla as M
from tests.tolerances import LSE_ATOL, LSE_ATOL_F32

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def gqa_case(i):
    rng = np.random.default_rng(7000 + i)
    dtype = ["bf16", "bf16", "fp8", "f32"][i % 4]
    g = int(rng.choice([1, 2, 4, 8]))
    r = int(rng.choice([r for r in (1, 2, 4, 8, 16, 32, 64) if g * r <= 128]))
    B = int(rng.integers(1, 7))
    S = int(rng.integers(1, 3001))
    lens = rng.integers(0, S + 1, size=B)
    if B > 1 and rng.random() < 0.3:
        lens[rng.integers(0, B)] = 0
    block_size = 0 if dtype == "f32" else int(rng.choice([0, 0, 1, 3, 8, 16, 32]))
    window = int(rng.integers(1, S + 1)) if rng.random() < 0.4 else 0
    split = int(rng.choice([0, 0, 64, 128, 320]))
    return dtype, g * r, g, B, S, lens.astype(np.int64), block_size, window, split


def mla_case(i):
    rng = np.random.default_rng(8000 + i)
    h = int(rng.choice([16, 32, 128]))
    B = int(rng.integers(1, 6))
    S = int(rng.integers(1, 5001))
    lens = rng.integers(0, S + 1, size=B)
    block_size = int(rng.choice([0, 16, 64]))
    split = int(rng.choice([0, 0, 256]))
    return h, B, S, lens.astype(np.int64), block_size, split


@pytest.mark.parametrize("i", range(96))
def test_random_gqa_shape(i):
    dtype, h, g, B, S, lens, block_size, window, split = gqa_case(i)
    G.note(f"random GQA {i}: {dtype} h={h} g={g} B={B} S={S} lens={lens.tolist()} block_size={block_size} "
           f"window={window} split={split}")
    w = W.GqaWorkload(f"rand_{i}", B, h, g, 128, S, dtype, 7000 + i, 1 / np.sqrt(128), block_size=block_size)
    x = W.make_gqa_inputs(w, DEV, lens=lens, poison_tail=True)
    if dtype == "fp8":
        ref, ref_lse = F8.reference(x, window=window)
        out, lse = F8.run(x, split_tokens=split, window=window)
        F8.assert_close(out.float().cpu().numpy(), ref, f"random {i}")
    else:
        ref, ref_lse = G.reference(x, window=window)
        out, lse = G.run(x, split_tokens=split, window=window)
        G.assert_close(out.float().cpu().numpy(), ref, dtype, f"random {i}")
    tol = LSE_ATOL_F32 if dtype == "f32" else LSE_ATOL
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, atol=tol, rtol=1e-4)
    del x
    torch.cuda.empty_cache()


@pytest.mark.parametrize("i", range(24))
def test_random_mla_shape(i):
    h, B, S, lens, block_size, split = mla_case(i)
    G.note(f"random MLA {i}: h={h} B={B} S={S} lens={lens.tolist()} block_size={block_size} split={split}")
    w = W.MlaWorkload(f"rand_mla_{i}", B, h, S, 8000 + i, 1 / np.sqrt(192), block_size=block_size)
    x = W.make_mla_inputs(w, DEV, lens=lens, poison_tail=True)
    ref, ref_lse = M.reference(x)
    out, lse = M.run(x, split_tokens=split)
    M.assert_close(out.float().cpu().numpy(), ref, f"random mla {i}")
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, atol=LSE_ATOL, rtol=1e-4)
    del x
    torch.cuda.empty_cache()


def persistent_case(i):
    rng = np.random.default_rng(9000 + i)
    dtype = ["bf16", "fp8"][i % 2]
    g = int(rng.choice([4, 8]))
    h = g * int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(32, 65))
    S = int(rng.integers(1100, 2001))  # with B >= 32, g >= 4 and 64-token splits: more than 2048 splits
    lens = rng.integers(0, S + 1, size=B)
    # power-of-two blocks of at least one copy instruction's rows (4 bf16, 8 fp8), where full tiles need
    # no LDS table
    block_size = int(rng.choice([4, 8, 16, 32] if dtype == "bf16" else [8, 16, 32]))
    split = int(rng.choice([64, 128]))
    if B * g * -(-S // split) <= 2048:
        split = 64
    return dtype, h, g, B, S, lens.astype(np.int64), block_size, split


@pytest.mark.parametrize("i", range(16))
def test_random_persistent_shape(i):
    """Paged batches cut into more than 2048 splits: the persistent form with its device work list."""
    dtype, h, g, B, S, lens, block_size, split = persistent_case(i)
    slots = B * g * -(-S // split)
    assert slots > 2048, "the grid must be large enough for the persistent form"
    G.note(f"random persistent {i}: {dtype} h={h} g={g} B={B} S={S} block_size={block_size} split={split} "
           f"({slots} splits)")
    w = W.GqaWorkload(f"rand_pers_{i}", B, h, g, 128, S, dtype, 9000 + i, 1 / np.sqrt(128), block_size=block_size)
    x = W.make_gqa_inputs(w, DEV, lens=lens, poison_tail=True)
    if dtype == "fp8":
        ref, ref_lse = F8.reference(x)
        out, lse = F8.run(x, split_tokens=split)
        F8.assert_close(out.float().cpu().numpy(), ref, f"random persistent {i}")
    else:
        ref, ref_lse = G.reference(x)
        out, lse = G.run(x, split_tokens=split)
        G.assert_close(out.float().cpu().numpy(), ref, dtype, f"random persistent {i}")
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, atol=LSE_ATOL, rtol=1e-4)
    del x
    torch.cuda.empty_cache()
