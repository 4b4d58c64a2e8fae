"""Pins for the oracle's decode attention (GQA / MHA / MQA, paged gather, merge).

Each test ties the oracle to something other than itself: torch's
scaled_dot_product_attention in float64 on the CPU (a library routine), the
head-sharing figure of "MQA, GQA, and MLA" section 3, closed forms of special
cases, invariants of softmax attention, and brute force with scalar Python
arithmetic on tiny inputs.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import attention as A
from tests.conftest import read_tsv


def _rng(seed):
    return np.random.default_rng(seed)


def sdpa_decode(q, K, V, lens, scale):
    """Library reference: torch SDPA (float64, CPU) with GQA head sharing, one query per sequence."""
    B, h, _ = q.shape
    out = np.zeros((B, h, V.shape[3]))
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            continue
        qt = torch.from_numpy(q[b][None, :, None, :])
        kt = torch.from_numpy(np.ascontiguousarray(K[b][None, :, :n]))
        vt = torch.from_numpy(np.ascontiguousarray(V[b][None, :, :n]))
        o = F.scaled_dot_product_attention(qt, kt, vt, scale=scale, enable_gqa=True)
        out[b] = o[0, :, 0].numpy()
    return out


@pytest.mark.parametrize("h,g", [(8, 8), (8, 2), (8, 1), (32, 8), (64, 1), (12, 4)])
def test_gqa_matches_torch_sdpa(h, g):
    rng = _rng(h * 100 + g)
    B, S, d = 3, 37, 16
    q = rng.standard_normal((B, h, d))
    K = rng.standard_normal((B, g, S, d))
    V = rng.standard_normal((B, g, S, 24))
    lens = np.array([37, 1, 20])
    scale = 1 / math.sqrt(d)
    o, _ = oracle.gqa_decode(q, K, V, lens, scale)
    ref = sdpa_decode(q, K, V, lens, scale)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-13)


def test_gqa_equals_mha_on_repeated_heads():
    # "MQA, GQA, and MLA" section 8: repeating each KV head h/g times gives
    # the same numbers (only the bytes read differ).
    rng = _rng(7)
    B, h, g, S, d = 2, 16, 4, 29, 8
    q = rng.standard_normal((B, h, d))
    K = rng.standard_normal((B, g, S, d))
    V = rng.standard_normal((B, g, S, d))
    lens = np.array([29, 13])
    o, lse = oracle.gqa_decode(q, K, V, lens, 0.37)
    Kr = np.repeat(K, h // g, axis=1)
    Vr = np.repeat(V, h // g, axis=1)
    o2, lse2 = oracle.gqa_decode(q, Kr, Vr, lens, 0.37)
    np.testing.assert_allclose(o, o2, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, atol=1e-14)


@pytest.mark.parametrize("row", read_tsv("head_groups_figure.tsv"), ids=lambda r: r[0])
def test_head_groups_follow_figure(row):
    variant, g, mapping = row
    g = int(g)
    mapping = [int(x) for x in mapping.split(",")]
    h, S, d = 8, 5, 4
    # Give every KV head a constant, distinct value row so that each output
    # reveals which KV head it read.
    q = np.zeros((1, h, d))
    K = np.zeros((1, g, S, d))
    V = np.zeros((1, g, S, d))
    for j in range(g):
        V[0, j] = j + 1.0
    o, _ = oracle.gqa_decode(q, K, V, [S], 1.0)
    assert [int(round(o[0, i, 0])) - 1 for i in range(h)] == mapping, variant


def test_single_token_returns_its_value_row():
    rng = _rng(3)
    q = rng.standard_normal(16)
    K = rng.standard_normal((1, 16))
    V = rng.standard_normal((1, 9))
    o, lse = oracle.attend(q, K, V, 0.25)
    assert np.array_equal(o, V[0])
    assert lse == pytest.approx(0.25 * float(q @ K[0]), abs=1e-14)


@pytest.mark.parametrize("n", [1, 2, 7, 100])
def test_zero_query_averages_values(n):
    rng = _rng(n)
    K = rng.standard_normal((n, 8))
    V = rng.standard_normal((n, 5))
    o, lse = oracle.attend(np.zeros(8), K, V, 0.5)
    np.testing.assert_allclose(o, V.mean(axis=0), atol=1e-14)
    assert lse == pytest.approx(math.log(n), abs=1e-14)
    # scale 0 is the same case
    o2, _ = oracle.attend(rng.standard_normal(8), K, V, 0.0)
    np.testing.assert_allclose(o2, V.mean(axis=0), atol=1e-14)


def test_identical_keys_average_values_and_constant_values_pass_through():
    rng = _rng(11)
    n = 9
    k = rng.standard_normal(6)
    K = np.tile(k, (n, 1))
    V = rng.standard_normal((n, 4))
    o, lse = oracle.attend(rng.standard_normal(6), K, V, 0.7)
    np.testing.assert_allclose(o, V.mean(axis=0), atol=1e-14)
    Vc = np.tile(rng.standard_normal(4), (n, 1))
    o2, _ = oracle.attend(rng.standard_normal(6), rng.standard_normal((n, 6)), Vc, 0.7)
    np.testing.assert_allclose(o2, Vc[0], atol=1e-14)


def test_weights_are_a_distribution():
    # With V = identity the output is the softmax weight vector itself.
    rng = _rng(5)
    n = 12
    o, lse = oracle.attend(rng.standard_normal(8), rng.standard_normal((n, 8)) * 3, np.eye(n), 0.9)
    assert np.all(o > 0)
    assert abs(o.sum() - 1.0) < 1e-15
    # and lse is log of the softmax normaliser
    q = rng.standard_normal(8)
    K = rng.standard_normal((n, 8))
    _, lse = oracle.attend(q, K, np.eye(n), 0.9)
    s = 0.9 * K @ q
    assert lse == pytest.approx(math.log(sum(math.exp(x) for x in s)), abs=1e-13)


def test_brute_force_tiny():
    # Scalar Python arithmetic (math.exp, explicit sums) on S <= 4, d <= 3.
    rng = _rng(17)
    for n in range(1, 5):
        for d in range(1, 4):
            q = [float(x) for x in rng.standard_normal(d)]
            K = [[float(x) for x in rng.standard_normal(d)] for _ in range(n)]
            V = [[float(x) for x in rng.standard_normal(3)] for _ in range(n)]
            scale = 0.61
            s = [scale * sum(q[a] * K[t][a] for a in range(d)) for t in range(n)]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = sum(w)
            o = [sum(w[t] * V[t][c] for t in range(n)) / z for c in range(3)]
            got, lse = oracle.attend(np.array(q), np.array(K), np.array(V), scale)
            np.testing.assert_allclose(got, o, atol=1e-14)
            assert lse == pytest.approx(m + math.log(z), abs=1e-14)


def test_token_order_does_not_matter():
    rng = _rng(23)
    n = 50
    q, K, V = rng.standard_normal(16), rng.standard_normal((n, 16)), rng.standard_normal((n, 16))
    perm = rng.permutation(n)
    o1, l1 = oracle.attend(q, K, V, 0.3)
    o2, l2 = oracle.attend(q, K[perm], V[perm], 0.3)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    assert l1 == pytest.approx(l2, abs=1e-13)


def test_large_scores_do_not_overflow():
    rng = _rng(29)
    q = rng.standard_normal(8) * 100
    K = rng.standard_normal((20, 8)) * 100
    V = rng.standard_normal((20, 3))
    o, lse = oracle.attend(q, K, V, 1.0)
    assert np.all(np.isfinite(o)) and np.isfinite(lse)
    s = K @ q
    t = int(np.argmax(s))
    # the largest score dominates by hundreds of nats
    np.testing.assert_allclose(o, V[t], atol=1e-12)


def test_empty_cache():
    o, lse = oracle.attend(np.ones(4), np.zeros((0, 4)), np.zeros((0, 6)), 1.0)
    assert np.array_equal(o, np.zeros(6)) and lse == -np.inf
    q = np.ones((2, 4, 8))
    K = np.ones((2, 2, 3, 8))
    o, lse = oracle.gqa_decode(q, K, K, [0, 3], 0.5)
    assert np.all(o[0] == 0) and np.all(lse[0] == -np.inf)
    assert np.all(np.isfinite(lse[1]))


@pytest.mark.parametrize("n_parts", [1, 2, 3, 7])
def test_merge_of_any_partition_equals_whole(n_parts):
    rng = _rng(31 + n_parts)
    n = 40
    q, K, V = rng.standard_normal(16), rng.standard_normal((n, 16)), rng.standard_normal((n, 10))
    whole_o, whole_lse = oracle.attend(q, K, V, 0.4)
    cuts = np.sort(rng.choice(np.arange(0, n + 1), size=n_parts - 1, replace=True))
    bounds = [0, *cuts.tolist(), n]
    parts = [oracle.attend(q, K[a:b], V[a:b], 0.4) for a, b in zip(bounds[:-1], bounds[1:])]
    parts.append(oracle.attend(q, K[:0], V[:0], 0.4))  # an empty part weighs nothing
    o, lse = oracle.lse_merge(parts)
    np.testing.assert_allclose(o, whole_o, atol=1e-14)
    assert float(lse) == pytest.approx(whole_lse, abs=1e-13)


def test_merge_of_only_empty_parts():
    e = oracle.attend(np.ones(3), np.zeros((0, 3)), np.zeros((0, 5)), 1.0)
    o, lse = oracle.lse_merge([e, e])
    assert np.array_equal(o, np.zeros(5)) and lse == -np.inf


def test_paged_gather_places_tokens_by_table():
    # block_size 2, three physical blocks, table [2, 0, 1]: tokens 0,1 live in
    # block 2, tokens 2,3 in block 0, token 4 in block 1 slot 0.
    pool = np.arange(3 * 1 * 2 * 1, dtype=np.float64).reshape(3, 1, 2, 1)  # value = 2*block + slot
    rows = oracle.paged_gather(pool, [2, 0, 1], 5, 2, kv_head=0)
    assert rows[:, 0].tolist() == [4.0, 5.0, 0.0, 1.0, 2.0]


def test_paged_decode_equals_contiguous_after_gather():
    rng = _rng(37)
    B, h, g, d, bs = 3, 8, 2, 16, 4
    lens = np.array([13, 1, 8])
    nblk = [(n + bs - 1) // bs for n in lens]
    N = sum(nblk)
    perm = rng.permutation(N)
    table = -np.ones((B, 4), dtype=np.int64)
    off = 0
    for b in range(B):
        table[b, : nblk[b]] = perm[off : off + nblk[b]]
        off += nblk[b]
    Kp = rng.standard_normal((N, g, bs, d))
    Vp = rng.standard_normal((N, g, bs, d))
    q = rng.standard_normal((B, h, d))
    o, lse = oracle.paged_gqa_decode(q, Kp, Vp, table, lens, bs, 0.25)
    S = 16
    K = np.zeros((B, g, S, d))
    V = np.zeros((B, g, S, d))
    for b in range(B):
        for t in range(lens[b]):
            K[b, :, t] = Kp[table[b, t // bs], :, t % bs]
            V[b, :, t] = Vp[table[b, t // bs], :, t % bs]
    o2, lse2 = oracle.gqa_decode(q, K, V, lens, 0.25)
    np.testing.assert_allclose(o, o2, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, atol=1e-14)
    np.testing.assert_allclose(o, sdpa_decode(q, K, V, lens, 0.25), atol=1e-13)


def test_bf16_widening_is_exact():
    bits = np.array([0x3F80, 0xC000, 0x4049, 0x0001, 0x7F80, 0xFF80, 0x0000, 0x8000, 0x7F7F], dtype=np.uint16)
    got = oracle.bf16_bits_to_f64(bits)
    assert got[0] == 1.0 and got[1] == -2.0 and got[2] == 3.140625
    assert got[3] == 2.0**-133
    assert got[4] == np.inf and got[5] == -np.inf
    assert got[6] == 0.0 and math.copysign(1.0, got[7]) == -1.0
    assert got[8] == float.fromhex("0x1.fep127")
    # agrees with torch's own bfloat16 -> float64 conversion on random codes
    rng = _rng(41)
    codes = rng.integers(0, 2**16, size=4096, dtype=np.uint16)
    t = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    mine = oracle.bf16_bits_to_f64(codes)
    finite = np.isfinite(t)
    assert np.array_equal(mine[finite], t[finite])
    assert np.array_equal(np.isnan(mine), np.isnan(t))


def test_bf16_inputs_match_widened_float_inputs():
    rng = _rng(43)
    B, h, g, S, d = 2, 4, 2, 9, 8
    qf = torch.from_numpy(rng.standard_normal((B, h, d))).to(torch.bfloat16)
    Kf = torch.from_numpy(rng.standard_normal((B, g, S, d))).to(torch.bfloat16)
    Vf = torch.from_numpy(rng.standard_normal((B, g, S, d))).to(torch.bfloat16)
    bits = [t.view(torch.int16).numpy().view(np.uint16) for t in (qf, Kf, Vf)]
    o, _ = oracle.gqa_decode(*bits, [9, 4], 0.3, bf16=True)
    o2, _ = oracle.gqa_decode(*[t.double().numpy() for t in (qf, Kf, Vf)], [9, 4], 0.3)
    assert np.array_equal(o, o2)


def test_attention_module_exports():
    for name in ("attend", "gqa_decode", "paged_gather", "paged_gqa_decode", "mla_absorbed_decode",
                 "paged_mla_absorbed_decode", "mla_absorb_query", "mla_explicit_decode", "lse_merge"):
        assert getattr(A, name) is getattr(oracle, name)
