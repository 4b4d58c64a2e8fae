"""GPU parity of kvattn_mla_decode (through the C ABI) against the fp64 oracle.

bf16 inputs: |gpu - ref| <= 2e-2 + 1e-2 |ref| elementwise.
"""

import numpy as np
import pytest
import torch

from tests.tolerances import LSE_ATOL, LSE_ATOL_F32  # noqa: F401

import oracle
from decode_attention_kv_03_amd import mla_decode
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


def reference(x, rows=None):
    w = x["workload"]
    q = W.host_view(x["q"])
    lens = W.host_view(x["seq_lens"])
    if rows is None:
        rows = list(range(w.batch))
    if w.paged:
        return oracle.paged_mla_absorbed_decode(q[rows], W.host_view(x["cache"]), W.host_view(x["block_table"])[rows],
                                                lens[rows], w.block_size, w.scale, d_c=w.d_latent, bf16=True)
    c = np.stack([W.host_view(x["cache"][b]) for b in rows])
    return oracle.mla_absorbed_decode(q[rows], c, lens[rows], w.scale, d_c=w.d_latent, bf16=True)


def run(x, **kw):
    w = x["workload"]
    out, lse = mla_decode(x["q"], x["cache"], x["seq_lens"], w.scale, block_table=x["block_table"],
                          return_lse=True, **kw)
    torch.cuda.synchronize()
    return out, lse


CASES = [
    # B, h, lens, split
    (1, 128, [1], 0),
    (2, 128, [31, 33], 0),
    (2, 128, [32, 64], 64),
    (3, 128, [100, 1, 65], 64),
    (2, 64, [1000, 999], 256),
    (2, 16, [300, 17], 128),
    (2, 128, [2049, 777], 0),
    (1, 128, [96], 64),
]


@pytest.mark.parametrize("B,h,lens,split", CASES)
def test_contiguous_ragged_with_poisoned_tail(B, h, lens, split):
    w = W.MlaWorkload(f"mla_{B}_{h}", B, h, max(lens) + 5, 500 + h + B, 1 / np.sqrt(192))
    note(f"mla B={B} h={h} lens={lens} split={split}")
    x = W.make_mla_inputs(w, DEV, lens=lens, poison_tail=True)
    ref, ref_lse = reference(x)
    out, lse = run(x, split_tokens=split)
    assert_close(out.float().cpu().numpy(), ref)
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, atol=LSE_ATOL, rtol=1e-4)


def test_zero_lengths():
    w = W.MlaWorkload("mla_zero", 3, 128, 64, 8, 0.1)
    note("mla zero lengths")
    x = W.make_mla_inputs(w, DEV, lens=[0, 64, 0])
    for split in (0, 64):
        out, lse = run(x, split_tokens=split)
        o = out.float().cpu().numpy()
        assert np.all(o[0] == 0) and np.all(o[2] == 0)
        assert np.all(np.isneginf(lse.cpu().numpy()[[0, 2]]))
        ref, _ = reference(x, rows=[1])
        assert_close(o[1:2], ref)


@pytest.mark.parametrize("B,lens_seed,max_len,split,bs", [
    (5, 0, 2600, 0, 0),       # few tokens in all: shortest pieces, cuts away from sequence starts
    (300, 1, 120, 0, 0),      # more sequences than the plan kernel's threads (two scan rounds)
    (300, 2, 90, 64, 16),     # ... paged, requested piece length
    (40, 3, 3000, 0, 32),     # paged ragged batch, pieces spanning sequence boundaries
    (7, 4, 5000, 320, 0),     # requested piece length that is not a power of two
])
def test_device_plan_ragged_batches(B, lens_seed, max_len, split, bs):
    """The device-side piece plan on ragged batches: empty, one-token and multi-piece sequences."""
    rng = np.random.default_rng(lens_seed)
    lens = rng.integers(0, max_len + 1, size=B)
    lens[rng.integers(0, B)] = 0
    lens[rng.integers(0, B)] = 1
    h = 16
    if bs:
        w = W.MlaWorkload(f"mla_plan_paged_{B}", B, h, max_len, 900 + lens_seed, 1 / np.sqrt(192), block_size=bs)
        note(f"mla plan B={B} max_len={max_len} split={split} block_size={bs}")
        x = W.make_mla_inputs(w, DEV, poison_tail=True)
    else:
        w = W.MlaWorkload(f"mla_plan_{B}", B, h, max_len, 900 + lens_seed, 1 / np.sqrt(192))
        note(f"mla plan B={B} max_len={max_len} split={split} lens sum={int(lens.sum())}")
        x = W.make_mla_inputs(w, DEV, lens=lens, poison_tail=True)
    ref, ref_lse = reference(x)
    out, lse = run(x, split_tokens=split)
    assert_close(out.float().cpu().numpy(), ref, "plan")
    l_ref = np.where(np.isneginf(ref_lse), -np.inf, ref_lse)
    got = lse.cpu().numpy()
    assert np.array_equal(np.isneginf(got), np.isneginf(l_ref))
    fin = np.isfinite(l_ref)
    np.testing.assert_allclose(got[fin], l_ref[fin], atol=LSE_ATOL, rtol=1e-4)


@pytest.mark.parametrize("bs", [16, 5, 64, 8, 24])
def test_paged(bs):
    w = W.MlaWorkload(f"mla_paged_bs{bs}", 4, 128, 400, 40 + bs, 1 / np.sqrt(192), block_size=bs)
    note(f"mla paged bs={bs}")
    x = W.make_mla_inputs(w, DEV, poison_tail=True)
    ref, _ = reference(x)
    for split in (0, 64):
        out, _ = run(x, split_tokens=split)
        assert_close(out.float().cpu().numpy(), ref, f"split={split}")


def test_rerun_is_bit_identical():
    w = W.shrink(W.WORKLOADS["deepseek_v2_mla_h128_b32_s8192"], batch=4, seq_len=3000)
    note("mla determinism")
    x = W.make_mla_inputs(w, DEV)
    a, la = run(x)
    b, lb = run(x)
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_full_size_every_sequence():
    w = W.WORKLOADS["deepseek_v2_mla_h128_b32_s8192"]
    note(w.name)
    x = W.make_mla_inputs(w, DEV)
    out, lse = run(x)
    ref, ref_lse = reference(x)
    assert_close(out.float().cpu().numpy(), ref, w.name)
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, atol=LSE_ATOL, rtol=1e-4)
    del x
    torch.cuda.empty_cache()


def test_paged_full_size_sampled():
    w = W.WORKLOADS["deepseek_v2_mla_paged_h128_b32_bs64_len1_16384"]
    note(w.name)
    x = W.make_mla_inputs(w, DEV)
    out, lse = run(x)
    lens = x["seq_lens"].cpu().numpy()
    rows = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 5})
    ref, ref_lse = reference(x, rows=rows)
    assert_close(out[rows].float().cpu().numpy(), ref, w.name)
    np.testing.assert_allclose(lse[rows].cpu().numpy(), ref_lse, atol=LSE_ATOL, rtol=1e-4)
    assert torch.isfinite(out.float()).all()
    del x
    torch.cuda.empty_cache()


def test_clock_stamps_hook():
    """kvattn_clock_next_mla: the armed call stores sane counter stamps and computes the same output."""
    from decode_attention_kv_03_amd import clock_next_mla, shader_clock_ghz

    w = W.shrink(W.WORKLOADS["deepseek_v2_mla_h128_b32_s8192"], batch=8, seq_len=4000)
    note("mla clock stamps")
    x = W.make_mla_inputs(w, DEV)
    plain, plain_lse = run(x)
    stamps = torch.zeros(4, dtype=torch.int64, device=DEV)
    clock_next_mla(stamps)
    armed, armed_lse = run(x)
    assert torch.equal(plain, armed) and torch.equal(plain_lse, armed_lse)
    v = stamps.cpu().tolist()
    assert v[2] > v[0] > 0 and v[3] > v[1] > 0, v
    assert 0.3 < shader_clock_ghz(stamps.cpu()) < 3.0
    # Consumed by that call: the next one leaves a fresh buffer untouched.
    fresh = torch.zeros(4, dtype=torch.int64, device=DEV)
    run(x)
    assert int(fresh.abs().sum()) == 0


def _pieces_of(n, t):
    return -(-n // t) if n > 0 else 1


@pytest.mark.parametrize("B,seed,max_len,split,bs,mixed", [
    (40, 11, 3000, 0, 0, False),
    (40, 12, 3000, 0, 32, False),     # paged
    (600, 13, 1500, 0, 0, False),     # more sequences than the plan keeps in registers, more than 256 pieces
    (7, 14, 9000, 0, 0, False),       # few sequences: many pieces each
    (9, 15, 5000, 320, 0, False),     # a requested piece length
    (70, 16, 9000, 256, 0, True),     # first 64 at most 16 pieces each (per-sequence writes), the rest 17-36 (whole-wave)
])
def test_device_plan_matches_its_definition(B, seed, max_len, split, bs, mixed):
    """The plan the device leaves in the workspace (laid out as kvattn.h documents it).

    With split_tokens 0 the piece length t is the shortest multiple of 32, at least 256, that cuts the
    batch into at most max(256, B) pieces (an empty sequence keeps one empty piece); otherwise t is
    split_tokens.  A sequence of n tokens has ceil(n / t) consecutive pieces of ceil(n / count) tokens
    rounded up to 32, the last one shorter, flagged when a sequence has only one.  Results only show a
    plan that loses or doubles tokens; a longer t than needed, or pieces out of order, would not.
    """
    from decode_attention_kv_03_amd import mla_workspace_bytes

    rng = np.random.default_rng(seed)
    lens = rng.integers(0, max_len + 1, size=B).astype(np.int32)
    if mixed:
        lens[:64] = rng.integers(0, 16 * 256 + 1, size=64)
        lens[64:] = rng.integers(16 * 256 + 1, max_len + 1, size=B - 64)
    lens[0], lens[-1] = 0, 1
    h = 16
    w = W.MlaWorkload(f"mla_plan_def_{B}", B, h, max_len, 950 + seed, 1 / np.sqrt(192), block_size=bs)
    x = W.make_mla_inputs(w, DEV, lens=lens)
    len_cap = x["block_table"].shape[1] * bs if bs else max_len
    note(f"mla plan definition B={B} max_len={max_len} split={split} block_size={bs}")
    nbytes = mla_workspace_bytes(B, h, len_cap, block_size=bs, split_tokens=split)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    mla_decode(x["q"], x["cache"], x["seq_lens"], w.scale, block_table=x["block_table"], split_tokens=split,
               workspace=ws)
    torch.cuda.synchronize()

    up = lambda v: -(-v // 256) * 256
    P = max(256, B) if split == 0 else B * -(-len_cap // split)
    o_pieces = up(P * h * 512 * 2) + up(P * h * 4)
    o_seq = o_pieces + up(P * 16)
    o_count = o_seq + up(B * 8)
    host = ws.cpu()
    n_pieces, t = (int(v) for v in host[o_count:o_count + 8].view(torch.int32))
    seq = host[o_seq:o_seq + 8 * B].view(torch.int32).reshape(B, 2).numpy()
    pieces = host[o_pieces:o_pieces + 16 * n_pieces].view(torch.int32).reshape(-1, 4).numpy()

    n = [int(v) for v in lens]
    if split == 0:
        cap = max(256, B)
        assert t % 32 == 0 and t >= 256
        assert sum(_pieces_of(v, t) for v in n) <= cap
        assert t == 256 or sum(_pieces_of(v, t - 32) for v in n) > cap, "a shorter piece length fits"
    else:
        assert t == split
    first = 0
    for b, v in enumerate(n):
        count = _pieces_of(v, t)
        assert tuple(seq[b]) == (first, count), b
        plen = (-(-v // count) + 31) // 32 * 32 if v > 0 else 0
        for j in range(count):
            lo = j * plen
            assert tuple(pieces[first + j]) == (b, lo, min(lo + plen, v), int(count == 1)), (b, j)
        first += count
    assert n_pieces == first
