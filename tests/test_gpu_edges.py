"""GPU parity (through the C ABI, against the fp64 oracle) of the paths only
long, wide or unusual calls reach, and checks that a call writes nothing
outside its outputs and workspace.

* Paged caches with 1- and 2-token blocks and long splits: a split then
  needs more block-table entries than the kernels stage in LDS (2304), so the
  staged window of the table slides while the split streams (bf16 and fp8).
* One 65,536-token sequence: GQA with 64-token splits (1,024 splits) and the
  automatic plan (256 splits), fp8 with 512 splits, MLA on the automatic
  plan (256 pieces of one sequence) and with 64-token pieces (1,024): the
  merges then combine more than 64 partials per row.
* MLA with 600 sequences: the device plan keeps the first 512 lengths in
  registers and rereads the others.
* Guard bands: out, lse and the workspace sit inside bands of 0xFF bytes
  (NaN) that must come back untouched; out and lse start as NaN, so every
  element must be written.
* Out-of-range block-table entries: the sequence that holds one gets a
  finite (unspecified) output, and every other sequence still matches the
  oracle.

Tolerances as elsewhere: bf16 and fp8 caches |gpu - ref| <= 2e-2 + 1e-2
|ref|; fp32 max |gpu - ref| <= 1e-5; lse atol 4e-3 (fp32: 1e-5), derived in tests/tolerances.py.
"""

import numpy as np
import pytest
import torch

from tests.tolerances import LSE_ATOL, LSE_ATOL_F32  # noqa: F401

import oracle
from decode_attention_kv_03_amd import (gqa_decode, gqa_decode_fp8, gqa_workspace_bytes, mla_decode,
                                        mla_workspace_bytes)
from decode_attention_kv_03_amd import workloads as W
from tests.guard import fenced

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ATOL, RTOL = 2e-2, 1e-2


def setup_module(_):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def note(msg):
    print(f"\n[gpu-test] {msg}", flush=True)


def assert_close(got, ref, what="", f32=False):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    if f32:
        assert err.max() <= 1e-5, f"{what}: max abs err {err.max():.3e}"
        return
    bad = err > ATOL + RTOL * np.abs(ref)
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} outside tolerance, max abs err {err.max():.3e}"


def gqa_reference(x, rows=None, window=0):
    w = x["workload"]
    q = W.host_view(x["q"])
    lens = W.host_view(x["seq_lens"])
    rows = list(range(w.batch)) if rows is None else rows
    fp8 = w.dtype == "fp8"
    if w.paged:
        bt = W.host_view(x["block_table"])[rows]
        k, v = W.host_view(x["k"]), W.host_view(x["v"])
        if fp8:
            return oracle.paged_gqa_decode_fp8(q[rows], k, v, W.host_view(x["k_scale"]), W.host_view(x["v_scale"]),
                                               bt, lens[rows], w.block_size, w.scale, window=window)
        return oracle.paged_gqa_decode(q[rows], k, v, bt, lens[rows], w.block_size, w.scale, bf16=w.dtype == "bf16",
                                       window=window)
    k = np.stack([W.host_view(x["k"][b]) for b in rows])
    v = np.stack([W.host_view(x["v"][b]) for b in rows])
    if fp8:
        return oracle.gqa_decode_fp8(q[rows], k, v, W.host_view(x["k_scale"]), W.host_view(x["v_scale"]), lens[rows],
                                     w.scale, window=window)
    return oracle.gqa_decode(q[rows], k, v, lens[rows], w.scale, bf16=w.dtype == "bf16", window=window)


def mla_reference(x, rows=None):
    w = x["workload"]
    q = W.host_view(x["q"])
    lens = W.host_view(x["seq_lens"])
    rows = list(range(w.batch)) if rows is None else rows
    if w.paged:
        return oracle.paged_mla_absorbed_decode(q[rows], W.host_view(x["cache"]),
                                                W.host_view(x["block_table"])[rows], lens[rows], w.block_size,
                                                w.scale, bf16=True)
    c = np.stack([W.host_view(x["cache"][b]) for b in rows])
    return oracle.mla_absorbed_decode(q[rows], c, lens[rows], w.scale, bf16=True)


def gqa_call(x, **kw):
    w = x["workload"]
    if w.dtype == "fp8":
        return gqa_decode_fp8(x["q"], x["k"], x["v"], x["k_scale"], x["v_scale"], x["seq_lens"], w.scale,
                              block_table=x["block_table"], **kw)
    return gqa_decode(x["q"], x["k"], x["v"], x["seq_lens"], w.scale, block_table=x["block_table"], **kw)


# ---- sliding block-table window (tiny blocks, long splits) ----

@pytest.mark.parametrize("dtype,block_size,split,lens", [
    ("bf16", 1, 4096, [9000, 2500, 4097]),
    ("bf16", 1, 8192, [9000, 6000, 1]),
    ("bf16", 2, 8192, [9000, 5000, 8193]),
    ("bf16", 3, 8192, [9000, 7000, 64]),     # block size not a power of two: per-row lookups
    ("fp8", 1, 4096, [9000, 2500, 4097]),
    ("fp8", 2, 8192, [9000, 5000, 8193]),
])
def test_paged_tiny_blocks_slide_the_staged_table(dtype, block_size, split, lens):
    w = W.GqaWorkload(f"paged_tiny_{dtype}_{block_size}", len(lens), 16, 2, 128, 9000, dtype, 60 + block_size,
                      1 / np.sqrt(128), block_size=block_size)
    note(f"{dtype} block_size={block_size} split={split} lens={lens}")
    x = W.make_gqa_inputs(w, DEV, lens=lens, poison_tail=True)
    ref, ref_lse = gqa_reference(x)
    out, lse = gqa_call(x, return_lse=True, split_tokens=split)
    torch.cuda.synchronize()
    assert_close(out.float().cpu().numpy(), ref, f"split={split}")
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, atol=LSE_ATOL, rtol=1e-4)
    # and with the library's own split (at most 2048 tokens for a paged cache)
    out0 = gqa_call(x, split_tokens=0)
    torch.cuda.synchronize()
    assert_close(out0.float().cpu().numpy(), ref, "auto split")


# ---- one long sequence: more than 64 splits / pieces per row in the merges ----

LONG = 65536


@pytest.mark.parametrize("h,g,split,dtype", [(32, 8, 64, "bf16"), (8, 2, 0, "bf16"), (16, 2, 128, "fp8"),
                                             (8, 1, 0, "f32"), (64, 1, 0, "bf16")])
def test_long_single_sequence_gqa(h, g, split, dtype):
    w = W.GqaWorkload(f"long_{dtype}", 1, h, g, 128, LONG, dtype, 70 + h, 1 / np.sqrt(128))
    from decode_attention_kv_03_amd import kvattn

    lib = kvattn.load_library()
    chosen = lib.kvattn_gqa_split_tokens(1, h, g, LONG, 0, split)
    note(f"B=1 S={LONG} h={h} g={g} {dtype} split={split} -> {chosen}-token splits, {LONG // chosen} per row")
    assert LONG // chosen > 64
    x = W.make_gqa_inputs(w, DEV)
    ref, ref_lse = gqa_reference(x)
    out, lse = gqa_call(x, return_lse=True, split_tokens=split)
    torch.cuda.synchronize()
    assert_close(out.float().cpu().numpy(), ref, "long", f32=dtype == "f32")
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, atol=LSE_ATOL_F32 if dtype == "f32" else LSE_ATOL, rtol=1e-4)


@pytest.mark.parametrize("h,split", [(128, 0), (16, 64)])
def test_long_single_sequence_mla(h, split):
    w = W.MlaWorkload("long_mla", 1, h, LONG, 80 + h, 1 / np.sqrt(192))
    from decode_attention_kv_03_amd import kvattn

    lib = kvattn.load_library()
    piece = lib.kvattn_mla_split_tokens(1, h, LONG, 0, split)
    note(f"MLA B=1 S={LONG} h={h} split={split} -> {piece}-token pieces, {LONG // piece} of them")
    assert LONG // piece > 64
    x = W.make_mla_inputs(w, DEV)
    ref, ref_lse = mla_reference(x)
    out, lse = mla_decode(x["q"], x["cache"], x["seq_lens"], w.scale, return_lse=True, split_tokens=split)
    torch.cuda.synchronize()
    assert_close(out.float().cpu().numpy(), ref, "long mla")
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, atol=LSE_ATOL, rtol=1e-4)


# ---- many sequences in the MLA plan ----

@pytest.mark.parametrize("split,bs", [(0, 0), (64, 0), (0, 16)])
def test_mla_600_sequences(split, bs):
    rng = np.random.default_rng(600 + split + bs)
    lens = rng.integers(0, 200, size=600)
    lens[[3, 555]] = 0
    lens[[10, 599]] = 199
    w = W.MlaWorkload(f"mla600_{bs}", 600, 16, 199, 61 + bs, 1 / np.sqrt(192), block_size=bs)
    note(f"MLA B=600 split={split} block_size={bs} tokens={int(lens.sum())}")
    x = W.make_mla_inputs(w, DEV, lens=lens, poison_tail=True)
    ref, ref_lse = mla_reference(x)
    out, lse = mla_decode(x["q"], x["cache"], x["seq_lens"], w.scale, block_table=x["block_table"], return_lse=True,
                          split_tokens=split)
    torch.cuda.synchronize()
    assert_close(out.float().cpu().numpy(), ref, "B=600")
    got = lse.cpu().numpy()
    assert np.array_equal(np.isneginf(got), np.isneginf(ref_lse))
    fin = np.isfinite(ref_lse)
    np.testing.assert_allclose(got[fin], ref_lse[fin], atol=LSE_ATOL, rtol=1e-4)


# ---- guard bands around out, lse and the workspace ----

GQA_GUARD = [
    # dtype, B, h, g, lens, block_size, split, window
    ("bf16", 3, 32, 8, [700, 5, 333], 0, 64, 0),
    ("bf16", 2, 64, 1, [1000, 64], 0, 0, 0),
    ("bf16", 4, 16, 4, [600, 17, 0, 450], 16, 64, 0),
    ("bf16", 3, 32, 8, [900, 300, 77], 16, 0, 200),
    ("f32", 2, 8, 2, [513, 100], 0, 64, 0),
    ("fp8", 3, 32, 8, [700, 129, 1], 16, 128, 0),
    ("fp8", 2, 64, 8, [1000, 400], 0, 0, 300),
]


@pytest.mark.parametrize("dtype,B,h,g,lens,bs,split,window", GQA_GUARD)
def test_gqa_writes_nothing_outside_its_buffers(dtype, B, h, g, lens, bs, split, window):
    S = max(lens) + 7
    w = W.GqaWorkload(f"guard_{dtype}", B, h, g, 128, S, dtype, 90 + h + bs, 1 / np.sqrt(128), block_size=bs)
    note(f"guards {dtype} B={B} h={h} g={g} lens={lens} bs={bs} split={split} window={window}")
    x = W.make_gqa_inputs(w, DEV, lens=lens, poison_tail=True)
    out_dt = torch.float32 if dtype == "f32" else torch.bfloat16
    out = fenced((B, h, 128), out_dt)
    lse = fenced((B, h), torch.float32)
    max_len = x["block_table"].shape[1] * bs if bs else S
    nbytes = gqa_workspace_bytes(B, h, g, 128, max_len, bs, split, out_dt)
    ws = fenced((max(nbytes, 1),), torch.uint8)
    ws.raw[4096:4096 + nbytes].zero_()  # the workspace's own bytes may be anything; only the bands matter
    gqa_call(x, out=out.tensor, lse=lse.tensor, split_tokens=split, workspace=ws.tensor, window=window)
    torch.cuda.synchronize()
    assert out.bands_intact() and lse.bands_intact() and ws.bands_intact()
    ref, ref_lse = gqa_reference(x, window=window)
    assert_close(out.tensor.float().cpu().numpy(), ref, "guarded", f32=dtype == "f32")
    got = lse.tensor.cpu().numpy()
    assert np.array_equal(np.isneginf(got), np.isneginf(ref_lse))
    fin = np.isfinite(ref_lse)
    np.testing.assert_allclose(got[fin], ref_lse[fin], atol=LSE_ATOL_F32 if dtype == "f32" else LSE_ATOL, rtol=1e-4)


@pytest.mark.parametrize("B,h,lens,bs,split", [(3, 128, [2000, 31, 700], 0, 0), (4, 64, [900, 0, 65, 500], 16, 64),
                                               (2, 128, [40, 3000], 64, 256)])
def test_mla_writes_nothing_outside_its_buffers(B, h, lens, bs, split):
    S = max(lens) + 5
    w = W.MlaWorkload("guard_mla", B, h, S, 95 + h + bs, 1 / np.sqrt(192), block_size=bs)
    note(f"MLA guards B={B} h={h} lens={lens} bs={bs} split={split}")
    x = W.make_mla_inputs(w, DEV, lens=lens, poison_tail=True)
    out = fenced((B, h, 512), torch.bfloat16)
    lse = fenced((B, h), torch.float32)
    max_len = x["block_table"].shape[1] * bs if bs else S
    nbytes = mla_workspace_bytes(B, h, max_len, block_size=bs, split_tokens=split)
    ws = fenced((nbytes,), torch.uint8)
    mla_decode(x["q"], x["cache"], x["seq_lens"], w.scale, block_table=x["block_table"], out=out.tensor,
               lse=lse.tensor, split_tokens=split, workspace=ws.tensor)
    torch.cuda.synchronize()
    assert out.bands_intact() and lse.bands_intact() and ws.bands_intact()
    ref, ref_lse = mla_reference(x)
    assert_close(out.tensor.float().cpu().numpy(), ref, "guarded mla")
    got = lse.tensor.cpu().numpy()
    assert np.array_equal(np.isneginf(got), np.isneginf(ref_lse))
    fin = np.isfinite(ref_lse)
    np.testing.assert_allclose(got[fin], ref_lse[fin], atol=LSE_ATOL, rtol=1e-4)


# ---- out-of-range block-table entries ----

@pytest.mark.parametrize("kind,bs", [("bf16", 16), ("bf16", 5), ("fp8", 16), ("f32", 16), ("mla", 16), ("mla", 5)])
def test_out_of_range_table_entries_stay_contained(kind, bs):
    lens = [300, 250, 200]
    if kind == "mla":
        w = W.MlaWorkload(f"oob_mla_{bs}", 3, 32, 320, 120 + bs, 1 / np.sqrt(192), block_size=bs)
        x = W.make_mla_inputs(w, DEV, lens=lens)
    else:
        w = W.GqaWorkload(f"oob_{kind}_{bs}", 3, 16, 4, 128, 320, kind, 110 + bs, 1 / np.sqrt(128), block_size=bs)
        x = W.make_gqa_inputs(w, DEV, lens=lens)
    note(f"out-of-range table entries: {kind} block_size={bs}")
    ref, _ = mla_reference(x, rows=[0]) if kind == "mla" else gqa_reference(x, rows=[0])
    bt = x["block_table"].clone()
    bt[1, 3] = 1 << 30   # past the pool
    bt[2, 0] = -7        # negative
    x["block_table"] = bt
    for split in (0, 64):
        if kind == "mla":
            out = mla_decode(x["q"], x["cache"], x["seq_lens"], w.scale, block_table=bt, split_tokens=split)
        else:
            out = gqa_call(x, split_tokens=split)
        torch.cuda.synchronize()
        o = out.float()
        assert torch.isfinite(o).all()
        assert_close(o[0:1].cpu().numpy(), ref, "untouched sequence", f32=kind == "f32")


def test_read_probe_handles_buffers_smaller_than_its_grid():
    """The streaming-read probe reads what its whole tiles leave over with the whole grid: a buffer of
    less than one 16 KiB tile per workgroup finishes as fast as a tiled one."""
    import time

    from decode_attention_kv_03_amd import hbm_read_probe

    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    for nbytes, wgs in ((1 << 20, 4096), (48 * 1024 + 16, 8), (64 * 16384, 64)):
        note(f"read probe {nbytes} bytes, {wgs} workgroups")
        buf = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
        hbm_read_probe(buf, wgs, sink)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(10):
            hbm_read_probe(buf, wgs, sink)
        torch.cuda.synchronize()
        assert (time.perf_counter() - t0) / 10 < 0.05
