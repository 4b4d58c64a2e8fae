"""Pins for the oracle's FP8 (E4M3) KV-cache decode.

The pages say only that an fp8 cache halves the bytes and that GQA quantises
at the KV-head granularity ("Why GQA's KV Cache Savings Don't Fully Reduce
TPOT", section "When the Serving Engineer Doesn't Get to Choose").  The
oracle's readings (OCP E4M3, one scale per KV head for K and for V) are
pinned here against:

* torch's float8_e4m3fn dtype (a library decoder) on all 256 codes, and the
  format's closed forms (largest finite 448, smallest subnormal 2^-9, ...);
* torch's scaled_dot_product_attention in float64 over a cache dequantised
  with torch's decoder;
* closed-form invariances: a KV head's K scale acts as a softmax-scale
  multiplier for exactly that head's query group, its V scale multiplies
  exactly that group's outputs and leaves the log-sum-exp alone;
* paged == contiguous.

Planted mistakes (wrong exponent bias, subnormals read as normals, the
scales applied to the wrong heads) are caught.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as A
from oracle import fp8 as F8


def torch_e4m3(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_matches_torch_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    mine, ref = F8.e4m3_to_f64(codes), torch_e4m3(codes)
    nan = np.isnan(ref)
    assert list(np.flatnonzero(nan)) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])


@pytest.mark.parametrize(
    "code, value",
    [(0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x38, 1.0), (0x39, 1.125),
     (0x40, 2.0), (0x78, 256.0), (0x7E, 448.0), (0xB8, -1.0), (0xFE, -448.0), (0x81, -(2.0 ** -9))],
)
def test_closed_forms(code, value):
    assert F8.e4m3_to_f64(np.array([code]))[0] == value


def test_negative_zero_and_order():
    assert np.signbit(F8.e4m3_to_f64(np.array([0x80]))[0])
    pos = F8.e4m3_to_f64(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0) and pos[-1] == F8.E4M3_MAX
    assert np.array_equal(F8.e4m3_to_f64(np.arange(0x80, 0xFF)), -pos)


def _fp8_inputs(seed, B=3, h=8, g=2, S=40, d=16):
    gen = torch.Generator().manual_seed(seed)
    q = torch.randn((B, h, d), generator=gen).to(torch.bfloat16)
    k_scale = (1.0 + torch.rand(g, generator=gen, dtype=torch.float64)) / 32
    v_scale = (1.0 + torch.rand(g, generator=gen, dtype=torch.float64)) / 16
    K = (torch.randn((B, g, S, d), generator=gen, dtype=torch.float64) / k_scale[None, :, None, None])
    V = (torch.randn((B, g, S, d), generator=gen, dtype=torch.float64) / v_scale[None, :, None, None])
    Kc = K.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    Vc = V.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    qbits = q.view(torch.int16).numpy().view(np.uint16)
    return qbits, Kc, Vc, k_scale.numpy(), v_scale.numpy()


def sdpa_fp8(qbits, Kc, Vc, k_scale, v_scale, lens, scale):
    """float64 SDPA over a cache dequantised with torch's decoder, heads repeated per group."""
    q = torch.from_numpy(qbits.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    K = torch.from_numpy(torch_e4m3(Kc)) * torch.from_numpy(k_scale)[None, :, None, None]
    V = torch.from_numpy(torch_e4m3(Vc)) * torch.from_numpy(v_scale)[None, :, None, None]
    r = q.shape[1] // K.shape[1]
    K = K.repeat_interleave(r, dim=1)
    V = V.repeat_interleave(r, dim=1)
    out = np.zeros(q.shape, dtype=np.float64)
    for b, n in enumerate(lens):
        o = F.scaled_dot_product_attention(q[b][:, None, :], K[b, :, :n], V[b, :, :n], scale=scale)
        out[b] = o[:, 0].numpy()
    return out


@pytest.mark.parametrize("seed, g", [(1, 2), (2, 1), (3, 8)])
def test_fp8_decode_matches_sdpa(seed, g):
    qbits, Kc, Vc, ks, vs = _fp8_inputs(seed, g=g)
    lens = np.array([40, 17, 1])
    o, _ = F8.gqa_decode_fp8(qbits, Kc, Vc, ks, vs, lens, 0.25)
    np.testing.assert_allclose(o, sdpa_fp8(qbits, Kc, Vc, ks, vs, lens, 0.25), rtol=1e-12, atol=1e-12)


def test_k_scale_is_a_softmax_scale_for_its_group_only():
    qbits, Kc, Vc, ks, vs = _fp8_inputs(4, h=8, g=2)
    lens = np.array([40, 33, 5])
    o1, l1 = F8.gqa_decode_fp8(qbits, Kc, Vc, ks, vs, lens, 0.3)
    c = 1.75
    ks2 = ks.copy()
    ks2[1] *= c
    o2, l2 = F8.gqa_decode_fp8(qbits, Kc, Vc, ks2, vs, lens, 0.3)
    # group 0 (heads 0..3) unchanged, group 1 (heads 4..7) as if the softmax scale were c times larger
    assert np.array_equal(o1[:, :4], o2[:, :4]) and np.array_equal(l1[:, :4], l2[:, :4])
    o3, l3 = F8.gqa_decode_fp8(qbits, Kc, Vc, ks, vs, lens, 0.3 * c)
    np.testing.assert_allclose(o2[:, 4:], o3[:, 4:], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2[:, 4:], l3[:, 4:], rtol=1e-12, atol=1e-12)
    assert not np.allclose(o2[:, 4:], o1[:, 4:])


def test_v_scale_scales_its_group_outputs_only():
    qbits, Kc, Vc, ks, vs = _fp8_inputs(5, h=8, g=2)
    lens = np.array([40, 12, 3])
    o1, l1 = F8.gqa_decode_fp8(qbits, Kc, Vc, ks, vs, lens, 0.3)
    vs2 = vs.copy()
    vs2[0] *= 3.0
    o2, l2 = F8.gqa_decode_fp8(qbits, Kc, Vc, ks, vs2, lens, 0.3)
    np.testing.assert_allclose(o2[:, :4], 3.0 * o1[:, :4], rtol=1e-13, atol=1e-15)
    assert np.array_equal(o2[:, 4:], o1[:, 4:]) and np.array_equal(l1, l2)


def test_paged_fp8_equals_contiguous():
    qbits, Kc, Vc, ks, vs = _fp8_inputs(6, B=2, h=4, g=2, S=13, d=8)
    lens = np.array([13, 6])
    bs = 4
    rng = np.random.default_rng(6)
    nblk = [(int(n) + bs - 1) // bs for n in lens]
    perm = rng.permutation(sum(nblk))
    Kp = np.zeros((sum(nblk), 2, bs, 8), dtype=np.uint8)
    Vp = np.zeros_like(Kp)
    table = np.full((2, max(nblk)), -1, dtype=np.int64)
    off = 0
    for b in range(2):
        table[b, : nblk[b]] = perm[off: off + nblk[b]]
        off += nblk[b]
        for t in range(int(lens[b])):
            Kp[table[b, t // bs], :, t % bs] = Kc[b, :, t]
            Vp[table[b, t // bs], :, t % bs] = Vc[b, :, t]
    for window in (0, 3):
        op, lp = F8.paged_gqa_decode_fp8(qbits, Kp, Vp, ks, vs, table, lens, bs, 0.4, window=window)
        oc, lc = F8.gqa_decode_fp8(qbits, Kc, Vc, ks, vs, lens, 0.4, window=window)
        assert np.array_equal(op, oc) and np.array_equal(lp, lc)


def test_empty_sequence():
    qbits, Kc, Vc, ks, vs = _fp8_inputs(7, B=2)
    o, lse = F8.gqa_decode_fp8(qbits, Kc, Vc, ks, vs, np.array([0, 5]), 0.3)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0])) and np.all(np.isfinite(lse[1]))


# ---- planted mistakes ------------------------------------------------------------------------------------------


def _bias8(codes):
    c = np.asarray(codes).astype(np.int64)
    e = (c >> 3) & 0xF
    m = (c & 7) / 8.0
    v = np.where(e == 0, m * 2.0 ** -7, (1 + m) * np.exp2(e - 8.0))
    return np.where((c >> 7) & 1, -v, v)


def _subnormal_as_normal(codes):
    c = np.asarray(codes).astype(np.int64)
    e = (c >> 3) & 0xF
    m = (c & 7) / 8.0
    v = (1 + m) * np.exp2(e - 7.0)
    v = np.where((e == 15) & ((c & 7) == 7), np.nan, v)
    return np.where((c >> 7) & 1, -v, v)


@pytest.mark.parametrize("mutant", [_bias8, _subnormal_as_normal])
def test_planted_decoder_mistakes_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(F8, "e4m3_to_f64", mutant)
    with pytest.raises(AssertionError):
        test_decode_matches_torch_on_every_code()


def test_planted_scale_on_the_wrong_heads_is_caught(monkeypatch):
    orig = F8.dequantize_kv_heads

    def reversed_scales(codes, scales, head_axis):
        return orig(codes, np.asarray(scales)[::-1], head_axis)

    monkeypatch.setattr(F8, "dequantize_kv_heads", reversed_scales)
    with pytest.raises(AssertionError):
        test_fp8_decode_matches_sdpa(1, 2)
    with pytest.raises(AssertionError):
        test_v_scale_scales_its_group_outputs_only()


def test_oracle_uses_attention_module():
    # the dequantised cache goes through the same fp64 attention as the bf16/fp32 oracle
    assert F8.gqa_decode is A.gqa_decode
