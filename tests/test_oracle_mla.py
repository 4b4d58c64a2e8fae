"""Pins for the oracle's absorbed MLA decode.

The main pin is Exercise D of "MQA, GQA, and MLA" (section 11): absorbed MLA
must equal the naive reconstruct-then-attend form.  Here both forms run on
tiny random float64 weights; the explicit form rebuilds per-head keys
``[c W_uk^(i) | k^R]`` and values ``c W_uv^(i)`` (section 5), the absorbed form
folds ``W_uk`` into the query and applies ``W_uv`` after the latent-space
average.  Further pins: torch SDPA in float64 on the absorbed layout, and
the reduction to MQA when there is no RoPE part and ``W_uk`` is the identity.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _weights(rng, h, d_c, d_h, d_v):
    W_uk = rng.standard_normal((h, d_c, d_h)) / math.sqrt(d_c)
    W_uv = rng.standard_normal((h, d_c, d_v)) / math.sqrt(d_c)
    return W_uk, W_uv


@pytest.mark.parametrize("h,d_c,d_r,d_h,d_v,n", [(4, 16, 4, 8, 8, 7), (3, 12, 2, 5, 6, 1), (8, 32, 8, 16, 16, 33)])
def test_absorbed_equals_explicit_reconstruction(h, d_c, d_r, d_h, d_v, n):
    rng = np.random.default_rng(h * 1000 + n)
    W_uk, W_uv = _weights(rng, h, d_c, d_h, d_v)
    q_c = rng.standard_normal((h, d_h))
    q_r = rng.standard_normal((h, d_r))
    c = rng.standard_normal((n, d_c))
    k_r = rng.standard_normal((n, d_r))
    scale = 1 / math.sqrt(d_h + d_r)

    o_exp, lse_exp = oracle.mla_explicit_decode(q_c, q_r, c, k_r, W_uk, W_uv, scale)

    q_abs = np.concatenate([oracle.mla_absorb_query(q_c, W_uk), q_r], axis=1)[None]
    cache = np.concatenate([c, k_r], axis=1)[None]
    o_lat, lse_abs = oracle.mla_absorbed_decode(q_abs, cache, [n], scale, d_c=d_c)
    o_abs = oracle.mla_up_project(o_lat, W_uv)[0]

    np.testing.assert_allclose(o_abs, o_exp, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_abs[0], lse_exp, rtol=0, atol=1e-12)


def test_batched_explicit_equals_absorbed_then_up_projected():
    """Exercise D over a batch of ragged sequences (one empty), in the layouts the library takes:
    q rows [q^C | q^R], cache rows [c | k^R], W_uk [h, d_c, d_h], W_uv [h, d_c, d_v]."""
    rng = np.random.default_rng(11)
    B, h, d_c, d_r, d_h, d_v, S = 3, 4, 16, 4, 8, 6, 9
    W_uk, W_uv = _weights(rng, h, d_c, d_h, d_v)
    q = rng.standard_normal((B, h, d_h + d_r))
    cache = rng.standard_normal((B, S, d_c + d_r))
    lens = [9, 0, 4]
    scale = 1 / math.sqrt(d_h + d_r)
    o_exp, lse_exp = oracle.mla_explicit_decode_batch(q, cache, lens, W_uk, W_uv, scale, d_c=d_c)
    q_abs = np.concatenate([np.stack([oracle.mla_absorb_query(q[b, :, :d_h], W_uk) for b in range(B)]),
                            q[..., d_h:]], axis=2)
    o_lat, lse_abs = oracle.mla_absorbed_decode(q_abs, cache, lens, scale, d_c=d_c)
    np.testing.assert_allclose(oracle.mla_up_project(o_lat, W_uv), o_exp, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(lse_exp), np.isneginf(lse_abs))
    fin = np.isfinite(lse_exp)
    np.testing.assert_allclose(lse_abs[fin], lse_exp[fin], rtol=0, atol=1e-12)
    assert np.all(o_exp[1] == 0) and np.all(np.isneginf(lse_exp[1]))
    # each sequence alone gives the same rows
    for b in range(B):
        o1, _ = oracle.mla_explicit_decode(q[b, :, :d_h], q[b, :, d_h:], cache[b, :lens[b], :d_c],
                                           cache[b, :lens[b], d_c:], W_uk, W_uv, scale)
        np.testing.assert_array_equal(o1, o_exp[b])


def test_up_projection_closed_forms():
    rng = np.random.default_rng(12)
    h, d_c = 3, 8
    o_lat = rng.standard_normal((2, h, d_c))
    # identity weights return the latent output itself
    eye = np.stack([np.eye(d_c)] * h)
    np.testing.assert_array_equal(oracle.mla_up_project(o_lat, eye), o_lat)
    # a weight that selects latent column j for value column k: out[..., i, k] = o_lat[..., i, j]
    W = np.zeros((h, d_c, 2))
    W[0, 5, 0] = 1.0
    W[1, 2, 1] = 1.0
    W[2, 7, 0] = 3.0
    out = oracle.mla_up_project(o_lat, W)
    np.testing.assert_array_equal(out[:, 0, 0], o_lat[:, 0, 5])
    np.testing.assert_array_equal(out[:, 1, 1], o_lat[:, 1, 2])
    np.testing.assert_array_equal(out[:, 2, 0], 3.0 * o_lat[:, 2, 7])
    assert np.all(out[:, 0, 1] == 0) and np.all(out[:, 1, 0] == 0)


def test_absorbed_query_scores_equal_reconstructed_key_scores():
    # q_i . (c W_uk^(i)) == (W_uk^(i) q_i) . c for every head and token.
    rng = np.random.default_rng(3)
    h, d_c, d_h, n = 5, 16, 8, 6
    W_uk, _ = _weights(rng, h, d_c, d_h, 4)
    q_c = rng.standard_normal((h, d_h))
    c = rng.standard_normal((n, d_c))
    qa = oracle.mla_absorb_query(q_c, W_uk)
    for i in range(h):
        np.testing.assert_allclose((c @ W_uk[i]) @ q_c[i], c @ qa[i], atol=1e-13)


def test_rope_part_enters_scores_but_not_values():
    rng = np.random.default_rng(5)
    h, d_c, d_r, n = 4, 16, 4, 9
    q = rng.standard_normal((1, h, d_c + d_r))
    cache = rng.standard_normal((1, n, d_c + d_r))
    o1, _ = oracle.mla_absorbed_decode(q, cache, [n], 0.3, d_c=d_c)
    assert o1.shape == (1, h, d_c)
    cache2 = cache.copy()
    cache2[..., d_c:] *= 5.0  # change only the RoPE keys
    o2, _ = oracle.mla_absorbed_decode(q, cache2, [n], 0.3, d_c=d_c)
    assert np.abs(o1 - o2).max() > 1e-3
    # the output is a convex combination of latent rows only
    q0 = q.copy()
    q0[..., d_c:] = 0.0
    cache3 = cache.copy()
    cache3[..., d_c:] = 1e6
    o3, _ = oracle.mla_absorbed_decode(q0, cache3, [n], 0.3, d_c=d_c)
    o4, _ = oracle.mla_absorbed_decode(q0, cache, [n], 0.3, d_c=d_c)
    np.testing.assert_allclose(o3, o4, atol=1e-13)
    assert np.abs(o3).max() < np.abs(cache[..., :d_c]).max() + 1e-12


def test_absorbed_matches_torch_sdpa():
    rng = np.random.default_rng(7)
    B, h, d_c, d_r, S = 2, 16, 64, 16, 21
    q = rng.standard_normal((B, h, d_c + d_r))
    cache = rng.standard_normal((B, S, d_c + d_r))
    lens = [21, 6]
    scale = 1 / math.sqrt(24)
    o, _ = oracle.mla_absorbed_decode(q, cache, lens, scale, d_c=d_c)
    for b in range(B):
        n = lens[b]
        qt = torch.from_numpy(q[b][None, :, None, :])
        kt = torch.from_numpy(np.ascontiguousarray(cache[b, None, None, :n]))
        vt = torch.from_numpy(np.ascontiguousarray(cache[b, None, None, :n, :d_c]))
        ref = F.scaled_dot_product_attention(qt, kt, vt, scale=scale, enable_gqa=True)[0, :, 0].numpy()
        np.testing.assert_allclose(o[b], ref, atol=1e-13)


def test_no_rope_identity_up_projection_is_mqa():
    # With d_r = 0 and W_uk = I the keys and values are the latent itself:
    # MLA becomes MQA with K = V = c.
    rng = np.random.default_rng(9)
    B, h, d, S = 2, 6, 12, 10
    q = rng.standard_normal((B, h, d))
    c = rng.standard_normal((B, S, d))
    o, lse = oracle.mla_absorbed_decode(q, c, [10, 3], 0.4, d_c=d)
    o2, lse2 = oracle.gqa_decode(q, c[:, None], c[:, None], [10, 3], 0.4)
    np.testing.assert_allclose(o, o2, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, atol=1e-14)
    qa = oracle.mla_absorb_query(q[0], np.stack([np.eye(d)] * h))
    np.testing.assert_allclose(qa, q[0], atol=0)


def test_paged_mla_equals_contiguous():
    rng = np.random.default_rng(13)
    B, h, w, d_c, bs = 2, 4, 20, 16, 3
    lens = [10, 4]
    nblk = [(n + bs - 1) // bs for n in lens]
    N = sum(nblk)
    perm = rng.permutation(N)
    table = -np.ones((B, 4), dtype=np.int64)
    table[0, :4] = perm[:4]
    table[1, :2] = perm[4:6]
    pool = rng.standard_normal((N, bs, w))
    q = rng.standard_normal((B, h, w))
    cache = np.zeros((B, 12, w))
    for b in range(B):
        for t in range(lens[b]):
            cache[b, t] = pool[table[b, t // bs], t % bs]
    o, lse = oracle.paged_mla_absorbed_decode(q, pool, table, lens, bs, 0.2, d_c=d_c)
    o2, lse2 = oracle.mla_absorbed_decode(q, cache, lens, 0.2, d_c=d_c)
    np.testing.assert_allclose(o, o2, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, atol=1e-14)
