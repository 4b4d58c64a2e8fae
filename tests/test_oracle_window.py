"""Pins for the oracle's sliding-window decode ("One dial, four settings",
the full ladder's SWA row and the sliding-window question: each token attends
only to the last W tokens; a token outside the window is not attended).

The oracle's window is pinned to torch's scaled_dot_product_attention in
float64 with an explicit boolean mask (a library routine), to closed forms
(W = 1 returns the last value row), and to invariances (tokens outside the
window can change arbitrarily).  A planted off-by-one window is caught.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import attention as A


def _inputs(seed, B=3, h=8, g=2, S=40, d=16):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, h, d))
    K = rng.standard_normal((B, g, S, d))
    V = rng.standard_normal((B, g, S, d))
    return q, K, V


def sdpa_window(q, K, V, lens, scale, window):
    """torch SDPA (float64, CPU) over the whole cache with a boolean mask that keeps only the window."""
    B, h, _ = q.shape
    S = K.shape[2]
    out = np.zeros((B, h, V.shape[3]))
    for b in range(B):
        n = int(lens[b])
        t = np.arange(S)
        keep = (t < n) & (t >= n - window)
        mask = torch.from_numpy(np.broadcast_to(keep, (1, h, 1, S)).copy())
        o = F.scaled_dot_product_attention(torch.from_numpy(q[b][None, :, None, :]), torch.from_numpy(K[b][None]),
                                           torch.from_numpy(V[b][None]), attn_mask=mask, scale=scale, enable_gqa=True)
        out[b] = o[0, :, 0].numpy()
    return out


@pytest.mark.parametrize("window", [1, 3, 7, 16, 39])
def test_window_matches_masked_sdpa(window):
    q, K, V = _inputs(window)
    lens = np.array([40, 25, 9])
    o, _ = oracle.gqa_decode(q, K, V, lens, 0.3, window=window)
    np.testing.assert_allclose(o, sdpa_window(q, K, V, lens, 0.3, window), rtol=1e-12, atol=1e-12)


def test_window_zero_or_at_least_the_length_is_full_attention():
    q, K, V = _inputs(5)
    lens = np.array([40, 25, 9])
    full = oracle.gqa_decode(q, K, V, lens, 0.2)
    for window in (0, 40, 1000):
        o, lse = oracle.gqa_decode(q, K, V, lens, 0.2, window=window)
        assert np.array_equal(o, full[0]) and np.array_equal(lse, full[1])


def test_window_of_one_returns_the_last_value_row():
    q, K, V = _inputs(6)
    lens = np.array([40, 25, 9])
    scale = 0.7
    o, lse = oracle.gqa_decode(q, K, V, lens, scale, window=1)
    r = q.shape[1] // K.shape[1]
    for b, n in enumerate(lens):
        for i in range(q.shape[1]):
            j = i // r
            np.testing.assert_allclose(o[b, i], V[b, j, n - 1], rtol=0, atol=1e-15)
            assert abs(lse[b, i] - scale * float(q[b, i] @ K[b, j, n - 1])) < 1e-12


def test_tokens_outside_the_window_do_not_matter():
    q, K, V = _inputs(7)
    lens = np.array([40, 25, 9])
    window = 6
    o1, l1 = oracle.gqa_decode(q, K, V, lens, 0.25, window=window)
    K2, V2 = K.copy(), V.copy()
    for b, n in enumerate(lens):
        K2[b, :, : n - window] = 1e3  # would dominate any softmax it took part in
        V2[b, :, : n - window] = -7.0
    o2, l2 = oracle.gqa_decode(q, K2, V2, lens, 0.25, window=window)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # ... while a change inside the window does
    K2[0, :, 40 - 1] += 1.0
    assert not np.allclose(oracle.gqa_decode(q, K2, V2, lens, 0.25, window=window)[0], o1)


def test_paged_window_equals_contiguous_window():
    rng = np.random.default_rng(8)
    B, h, g, d, bs = 2, 4, 2, 8, 4
    lens = np.array([13, 7])
    q = rng.standard_normal((B, h, d))
    nblk = [(int(n) + bs - 1) // bs for n in lens]
    pool_n = sum(nblk)
    perm = rng.permutation(pool_n)
    Kp = rng.standard_normal((pool_n, g, bs, d))
    Vp = rng.standard_normal((pool_n, g, bs, d))
    table = np.full((B, max(nblk)), -1, dtype=np.int64)
    off = 0
    for b in range(B):
        table[b, : nblk[b]] = perm[off: off + nblk[b]]
        off += nblk[b]
    S = max(lens)
    K = np.zeros((B, g, S, d))
    V = np.zeros((B, g, S, d))
    for b in range(B):
        for t in range(int(lens[b])):
            K[b, :, t] = Kp[table[b, t // bs], :, t % bs]
            V[b, :, t] = Vp[table[b, t // bs], :, t % bs]
    for window in (1, 5, 10):
        op, lp = oracle.paged_gqa_decode(q, Kp, Vp, table, lens, bs, 0.4, window=window)
        oc, lc = oracle.gqa_decode(q, K, V, lens, 0.4, window=window)
        np.testing.assert_allclose(op, oc, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lp, lc, rtol=1e-13, atol=1e-13)


def test_planted_off_by_one_window_is_caught(monkeypatch):
    orig = A.window_start

    def one_too_many(n, window):
        return max(0, n - window - 1) if window > 0 else 0

    monkeypatch.setattr(A, "window_start", one_too_many)
    with pytest.raises(AssertionError):
        test_window_of_one_returns_the_last_value_row()
    with pytest.raises(AssertionError):
        test_window_matches_masked_sdpa(7)
    monkeypatch.setattr(A, "window_start", orig)
