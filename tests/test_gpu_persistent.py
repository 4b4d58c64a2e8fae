"""GPU parity of the persistent form of the grouped-query split kernel.

A bf16 or fp8 call whose grid of (sequence, KV head, split) workgroups would
hold more than 2048 of them (ragged or paged batches, short splits), on a
contiguous cache or on power-of-two blocks of at least one copy
instruction's rows, runs as 512 resident workgroups that take the splits
holding tokens from a device-side list.  Checked here through the C ABI:

* every group shape (h/g = 4, 8, 32, 64, 128), contiguous and paged (down to
  4-token bf16 and 8-token fp8 blocks), bf16 and fp8, a sliding window, zero
  and one-token lengths, fewer items than resident workgroups, and more units
  than the plan keeps in registers, against the fp64 oracle;
* bit-identical outputs to the grid-per-split form of the same call (a
  workspace with no room for the list keeps that form), over reruns, and
  through the no-allocation entry point.

Tolerances as elsewhere: |gpu - ref| <= 2e-2 + 1e-2 |ref|, lse atol 4e-3.
"""

import numpy as np
import pytest
import torch

from tests.tolerances import LSE_ATOL

from decode_attention_kv_03_amd import gqa_decode, gqa_decode_noalloc, kvattn
from decode_attention_kv_03_amd import workloads as W
from tests.test_gpu_edges import assert_close, gqa_call, gqa_reference

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
PERSISTENT_SLOTS = 4 * 512  # the library keeps one workgroup per split up to this many


def setup_module(_):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def note(msg):
    print(f"\n[gpu-test] {msg}", flush=True)


def n_split(w, max_len, split):
    s = kvattn.load_library().kvattn_gqa_split_tokens(w.batch, w.num_q_heads, w.num_kv_heads, max_len,
                                                      w.block_size, split)
    return 1 if max_len <= s else -(-max_len // s)


def inputs(name, B, h, g, S, dtype, seed, lens, bs=0):
    w = W.GqaWorkload(name, B, h, g, 128, S, dtype, seed, 1 / np.sqrt(128), block_size=bs)
    x = W.make_gqa_inputs(w, DEV, lens=lens, poison_tail=True)
    max_len = x["block_table"].shape[1] * bs if bs else S
    return w, x, max_len


def grid_form_call(x, max_len, split, window, ws_bytes):
    """The call through the C ABI with a workspace of exactly ws_bytes."""
    w = x["workload"]
    lib = kvattn.load_library()
    B, h = w.batch, w.num_q_heads
    out = torch.empty((B, h, 128), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, h), dtype=torch.float32, device=DEV)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    bt = x["block_table"]
    bs = w.block_size
    cache_len = x["k"].shape[0] if bs else x["k"].shape[2]
    max_blocks = bt.shape[1] if bs else 0
    P, S = kvattn._ptr, kvattn._stream(None)
    if w.dtype == "fp8":
        st = lib.kvattn_gqa_decode_fp8(P(x["q"]), P(x["k"]), P(x["v"]), P(x["k_scale"]), P(x["v_scale"]), P(bt),
                                       P(x["seq_lens"]), P(out), P(lse), B, h, w.num_kv_heads, 128, cache_len, bs,
                                       max_blocks, max_len, float(w.scale), int(window), int(split), P(ws), ws_bytes, S)
    else:
        st = lib.kvattn_gqa_decode_window(P(x["q"]), P(x["k"]), P(x["v"]), P(bt), P(x["seq_lens"]), P(out), P(lse),
                                          B, h, w.num_kv_heads, 128, cache_len, bs, max_blocks, max_len,
                                          float(w.scale), int(window), kvattn.KVATTN_BF16, int(split), P(ws),
                                          ws_bytes, S)
    assert st == 0, kvattn.load_library().kvattn_status_string(st)
    return out, lse


def lens_with_edges(rng, B, S):
    """Uniform lengths in [0, S] with the edge values planted at the front."""
    edge = [0, 1, 63, 64, 65, S]
    return np.concatenate([edge, rng.integers(0, S + 1, B - len(edge))]).astype(np.int32)[:B]


CASES = [
    # name, B, h, g, S, dtype, bs, split, window
    ("paged_r8", 64, 64, 8, 4096, "bf16", 16, 256, 0),
    ("contig_r4", 24, 32, 8, 2000, "bf16", 0, 64, 0),
    ("paged_r32", 32, 64, 2, 3000, "bf16", 32, 64, 0),
    ("contig_r64", 48, 64, 1, 3000, "bf16", 0, 64, 0),
    ("contig_r128", 48, 128, 1, 3000, "bf16", 0, 64, 0),
    ("paged_fp8_r4", 32, 32, 8, 4000, "fp8", 16, 128, 0),
    ("paged_window", 64, 32, 8, 6000, "bf16", 16, 64, 700),
    ("fp8_window", 40, 64, 8, 5000, "fp8", 0, 128, 900),
    # the smallest blocks that take the persistent form: one copy instruction's rows
    ("paged_bs4", 48, 32, 8, 2000, "bf16", 4, 64, 0),
    ("paged_fp8_bs8", 48, 32, 8, 2000, "fp8", 8, 128, 0),
]


@pytest.mark.parametrize("name,B,h,g,S,dtype,bs,split,window", CASES)
def test_persistent_matches_oracle_and_grid_form(name, B, h, g, S, dtype, bs, split, window):
    rng = np.random.default_rng(len(name) + B)
    lens = lens_with_edges(rng, B, S)
    w, x, max_len = inputs(name, B, h, g, S, dtype, 500 + B + h, lens, bs)
    span = min(max_len, window + 63) if window else max_len
    assert B * g * n_split(w, span, split) > PERSISTENT_SLOTS, "case does not reach the persistent form"
    note(f"{name}: B={B} h={h} g={g} S={S} {dtype} bs={bs} split={split} window={window}")
    out, lse = gqa_call(x, return_lse=True, split_tokens=split, window=window)
    torch.cuda.synchronize()
    ref, ref_lse = gqa_reference(x, window=window)
    assert_close(out.float().cpu().numpy(), ref, name)
    got = lse.cpu().numpy()
    assert np.array_equal(np.isneginf(got), np.isneginf(ref_lse))
    fin = np.isfinite(ref_lse)
    np.testing.assert_allclose(got[fin], ref_lse[fin], atol=LSE_ATOL, rtol=1e-4)

    # The same call in the grid-per-split form: a workspace that holds the bf16 partials and nothing more.
    nsp = n_split(w, span, split)
    out_g, lse_g = grid_form_call(x, max_len, split, window, B * h * nsp * (128 * 2 + 4))
    # ... and the persistent form again (items may be taken in another order)
    out_p, lse_p = gqa_call(x, return_lse=True, split_tokens=split, window=window)
    torch.cuda.synchronize()
    assert torch.equal(out_g, out) and torch.equal(out_p, out)
    assert torch.equal(lse_g, lse) and torch.equal(lse_p, lse)


def test_fewer_items_than_resident_workgroups():
    B, h, g, S = 300, 16, 8, 512
    lens = np.zeros(B, dtype=np.int32)
    lens[[0, 7, 150, 299]] = [512, 1, 65, 300]
    w, x, max_len = inputs("sparse", B, h, g, S, "bf16", 31, lens)
    assert B * g * n_split(w, max_len, 64) > PERSISTENT_SLOTS
    note("300 sequences, four of them non-empty, 64-token splits")
    out, lse = gqa_call(x, return_lse=True, split_tokens=64)
    torch.cuda.synchronize()
    o, lz = out.float().cpu().numpy(), lse.cpu().numpy()
    empty = lens == 0
    assert np.all(o[empty] == 0) and np.all(np.isneginf(lz[empty]))
    rows = [int(b) for b in np.nonzero(~empty)[0]]
    ref, ref_lse = gqa_reference(x, rows=rows)
    assert_close(o[rows], ref, "non-empty rows")
    np.testing.assert_allclose(lz[rows], ref_lse, atol=LSE_ATOL, rtol=1e-4)


def test_persistent_through_the_no_allocation_entry_point():
    B, h, g, S, bs = 64, 64, 8, 4096, 16
    rng = np.random.default_rng(5)
    lens = lens_with_edges(rng, B, S)
    w, x, max_len = inputs("noalloc_persistent", B, h, g, S, "bf16", 41, lens, bs)
    note("persistent form through the no-allocation entry point, twice, then a smaller call")
    ref_out = gqa_decode(x["q"], x["k"], x["v"], x["seq_lens"], w.scale, block_table=x["block_table"],
                         split_tokens=256)
    for _ in range(2):
        out = torch.empty_like(ref_out)
        gqa_decode_noalloc(x["q"], x["k"], x["v"], x["seq_lens"], w.scale, out, block_table=x["block_table"],
                           split_tokens=256)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out)
    # a smaller call of the grid-per-split form on the same scratch afterwards
    small = W.GqaWorkload("small_after", 2, 32, 8, 128, 700, "bf16", 77, 0.08)
    xs = W.make_gqa_inputs(small, DEV)
    out_s = torch.empty((2, 32, 128), dtype=torch.bfloat16, device=DEV)
    gqa_decode_noalloc(xs["q"], xs["k"], xs["v"], xs["seq_lens"], small.scale, out_s, split_tokens=64)
    torch.cuda.synchronize()
    ref_s, _ = gqa_reference(xs)
    assert_close(out_s.float().cpu().numpy(), ref_s, "after")


def test_more_units_than_the_plan_keeps_in_registers():
    """The plan keeps the spans of its first 4096 (sequence, KV head) units in registers and recomputes the rest."""
    B, h, g, S, bs, split = 520, 64, 8, 256, 16, 64
    assert B * g > 4 * 1024
    rng = np.random.default_rng(11)
    lens = lens_with_edges(rng, B, S)
    w, x, max_len = inputs("many_units", B, h, g, S, "bf16", 61, lens, bs)
    assert B * g * n_split(w, max_len, split) > PERSISTENT_SLOTS
    note(f"{B * g} units: B={B} h={h} g={g} S={S} bs={bs} split={split}")
    out, lse = gqa_call(x, return_lse=True, split_tokens=split)
    torch.cuda.synchronize()
    ref, ref_lse = gqa_reference(x)
    assert_close(out.float().cpu().numpy(), ref, "many_units")
    got = lse.cpu().numpy()
    assert np.array_equal(np.isneginf(got), np.isneginf(ref_lse))
    fin = np.isfinite(ref_lse)
    np.testing.assert_allclose(got[fin], ref_lse[fin], atol=LSE_ATOL, rtol=1e-4)
    out_g, lse_g = grid_form_call(x, max_len, split, 0, B * h * n_split(w, max_len, split) * (128 * 2 + 4))
    assert torch.equal(out_g, out) and torch.equal(lse_g, lse)


@pytest.mark.parametrize("window", [0, 700])
def test_work_list_holds_each_split_once_full_first_then_longest_first(window):
    """The device-side work list (16 bytes per slot after the partials, as kvattn.h places it).

    It must hold every split that holds tokens exactly once, as (unit b*g + j, split s, first token, end
    token) with the one-workgroup-per-split form's boundaries: the full splits first in unit order, then
    the shorter last splits by length class ceil(32 rest / split), longest first.  A missing split would
    show in the outputs; a duplicate or a misordered one would not, hence this check.
    """
    from decode_attention_kv_03_amd import gqa_workspace_bytes

    B, h, g, S, bs, split = 64, 32, 8, 6000, 16, 64
    rng = np.random.default_rng(19 + window)
    lens = lens_with_edges(rng, B, S)
    w, x, max_len = inputs("work_list", B, h, g, S, "bf16", 83, lens, bs)
    span = min(max_len, window + 63) if window else max_len
    nsp = n_split(w, span, split)
    assert B * g * nsp > PERSISTENT_SLOTS
    note(f"work list: B={B} g={g} split={split} window={window} splits per unit={nsp}")
    nbytes = gqa_workspace_bytes(B, h, g, 128, max_len, block_size=bs, split_tokens=split)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    gqa_call(x, split_tokens=split, window=window, workspace=ws)
    torch.cuda.synchronize()
    up = lambda v: -(-v // 256) * 256
    items_off = up(B * h * nsp * (128 * 2 + 4))
    ctl_off = items_off + up(B * g * nsp * 16)
    n_items = int(ws[ctl_off:ctl_off + 4].view(torch.int32).item())
    got = ws[items_off:items_off + 16 * n_items].view(torch.int32).reshape(-1, 4).cpu().numpy()

    full, last = [], []
    for b in range(B):
        n = int(min(max(lens[b], 0), max_len))
        base = (max(0, n - window) if window > 0 and n > window else 0) & ~63
        f = min((n - base) // split, nsp)
        for j in range(g):
            u = b * g + j
            full += [(u, s, base + s * split, base + (s + 1) * split) for s in range(f)]
            if f < nsp and n - base - f * split > 0:
                last.append((u, f, base + f * split, n))
    assert n_items == len(full) + len(last)
    assert [tuple(r) for r in got[:len(full)]] == full
    tail = [tuple(r) for r in got[len(full):]]
    assert sorted(tail) == sorted(last)
    classes = [-(-(t1 - t0) * 32 // split) for (_, _, t0, t1) in tail]
    assert all(a >= b for a, b in zip(classes, classes[1:])), "last splits not longest first"
