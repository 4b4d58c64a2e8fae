"""Planted mistakes in the oracle must be caught by its pins.

Each case swaps one oracle function for a copy with a plausible mistake
(a wrong head map, a dropped scale, a transposed operand, a swapped paged
index, a merge without log-sum-exp weights, a formula missing its factor 2)
and checks that at least one pin test then fails.  The mutants live only in
this file and only on the CPU.
"""

import numpy as np
import pytest

import oracle
from oracle import attention as A
from oracle import cache_bytes as CB
from tests import test_oracle_attention as TA
from tests import test_oracle_formulas as TF
from tests import test_oracle_mla as TM
from tests.conftest import read_tsv


def _patch(monkeypatch, name, fn, module=A):
    monkeypatch.setattr(module, name, fn)
    if hasattr(oracle, name):
        monkeypatch.setattr(oracle, name, fn)


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def gqa_modulo_map(q, K, V, seq_lens, scale, bf16=False):
    B, h, _ = q.shape
    g = K.shape[1]
    o = np.zeros((B, h, V.shape[3]))
    lse = np.full((B, h), -np.inf)
    for b in range(B):
        n = int(seq_lens[b])
        for i in range(h):
            j = i % g  # mistake: interleaved groups instead of contiguous ones
            o[b, i], lse[b, i] = A.attend(q[b, i], K[b, j, :n], V[b, j, :n], scale)
    return o, lse


def attend_no_scale(q, K, V, scale):
    return _attend_orig(q, K, V, 1.0)


def attend_keys_as_values(q, K, V, scale):
    if K.shape == V.shape:
        return _attend_orig(q, K, K, scale)
    return _attend_orig(q, K, V, scale)


def attend_no_max_shift_wrong_lse(q, K, V, scale):
    o, lse = _attend_orig(q, K, V, scale)
    if K.shape[0] == 0:
        return o, lse
    s = scale * (np.asarray(K) @ np.asarray(q))
    return o, lse - s.max()  # mistake: forgets to add the max back


_attend_orig = A.attend


def paged_gather_swapped(pool, table_row, n, block_size, kv_head=None):
    rows = []
    nb = len(table_row)
    for t in range(n):
        blk = int(table_row[t % nb])  # mistake: block and slot index swapped
        slot = (t // nb) % block_size
        rows.append(pool[blk, kv_head, slot] if kv_head is not None else pool[blk, slot])
    return np.stack(rows) if rows else np.zeros((0, pool.shape[-1]))


def lse_merge_plain_average(parts):
    os_ = np.stack([np.asarray(p[0], dtype=np.float64) for p in parts if np.isfinite(p[1]).all()])
    ls = np.stack([np.asarray(p[1], dtype=np.float64) for p in parts if np.isfinite(p[1]).all()])
    return os_.mean(axis=0), ls.max(axis=0)


def mla_values_with_rope(q_abs, cache, seq_lens, scale, d_c=512, bf16=False):
    B, h, _ = q_abs.shape
    o = np.zeros((B, h, d_c))
    lse = np.full((B, h), -np.inf)
    for b in range(B):
        n = int(seq_lens[b])
        rows = np.asarray(cache[b, :n], dtype=np.float64)
        for i in range(h):
            # mistake: values taken from the last d_c columns (includes k^R)
            o[b, i], lse[b, i] = A.attend(q_abs[b, i], rows, rows[:, -d_c:], scale)
    return o, lse


def absorb_without_transpose(q_c, W_uk):
    W = np.asarray(W_uk)
    if W.shape[1] == W.shape[2]:
        return np.stack([W[i].T @ q_c[i] for i in range(q_c.shape[0])])
    # shapes force the right contraction otherwise; transpose the weight rows instead
    return np.stack([W[i][::-1] @ q_c[i] for i in range(q_c.shape[0])])


def kv_bytes_no_factor_two(n_layers, n_kv_heads, d_head, bytes_per_elem):
    return n_layers * n_kv_heads * d_head * bytes_per_elem


def kv_cache_bytes_no_batch(n_layers, n_kv_heads, d_head, context_len, batch, bytes_per_elem):
    return n_layers * n_kv_heads * d_head * 2 * context_len * bytes_per_elem


def _any_gqa_pin_fails():
    return any(
        [
            _fails(TA.test_gqa_matches_torch_sdpa, 8, 2),
            _fails(TA.test_gqa_matches_torch_sdpa, 32, 8),
            *[_fails(TA.test_head_groups_follow_figure, row) for row in read_tsv("head_groups_figure.tsv")],
        ]
    )


def test_modulo_head_map_is_caught(monkeypatch):
    _patch(monkeypatch, "gqa_decode", gqa_modulo_map)
    assert _any_gqa_pin_fails()


def test_dropped_scale_is_caught(monkeypatch):
    _patch(monkeypatch, "attend", attend_no_scale)
    assert _fails(TA.test_gqa_matches_torch_sdpa, 8, 2)


def test_keys_used_as_values_is_caught(monkeypatch):
    _patch(monkeypatch, "attend", attend_keys_as_values)
    assert _fails(TA.test_gqa_matches_torch_sdpa, 8, 8) or _fails(TA.test_brute_force_tiny)


def test_wrong_lse_is_caught(monkeypatch):
    _patch(monkeypatch, "attend", attend_no_max_shift_wrong_lse)
    assert _fails(TA.test_weights_are_a_distribution) or _fails(TA.test_brute_force_tiny)


def test_swapped_paged_index_is_caught(monkeypatch):
    _patch(monkeypatch, "paged_gather", paged_gather_swapped)
    assert _fails(TA.test_paged_gather_places_tokens_by_table)
    assert _fails(TA.test_paged_decode_equals_contiguous_after_gather)


def test_unweighted_merge_is_caught(monkeypatch):
    _patch(monkeypatch, "lse_merge", lse_merge_plain_average)
    assert _fails(TA.test_merge_of_any_partition_equals_whole, 3)


def test_rope_in_values_is_caught(monkeypatch):
    _patch(monkeypatch, "mla_absorbed_decode", mla_values_with_rope)
    assert _fails(TM.test_absorbed_equals_explicit_reconstruction, 4, 16, 4, 8, 8, 7)
    assert _fails(TM.test_absorbed_matches_torch_sdpa)


def test_wrong_absorption_is_caught(monkeypatch):
    _patch(monkeypatch, "mla_absorb_query", absorb_without_transpose)
    assert _fails(TM.test_absorbed_equals_explicit_reconstruction, 4, 16, 4, 8, 8, 7)


@pytest.mark.parametrize(
    "name,mutant", [("kv_bytes_per_token", kv_bytes_no_factor_two), ("kv_cache_bytes", kv_cache_bytes_no_batch)]
)
def test_formula_mistakes_are_caught(monkeypatch, name, mutant):
    monkeypatch.setattr(CB, name, mutant)
    failed = [
        _fails(TF.test_printed_cache_bytes, row) for row in read_tsv("cache_bytes_printed.tsv") if row[1] == name
    ]
    assert any(failed)


def up_project_transposed(o_latent, W_uv):
    # plausible mistake: each head's weight read as [d_v, d_c] (reshaped, not transposed, when d_v != d_c)
    o_latent = np.asarray(o_latent, dtype=np.float64)
    h, d_c, d_v = W_uv.shape
    return np.stack([o_latent[..., i, :] @ np.asarray(W_uv[i]).reshape(d_v, d_c).T.reshape(d_c, d_v)
                     for i in range(h)], axis=-2)


def up_project_wrong_head(o_latent, W_uv):
    # plausible mistake: every head projected with head 0's weights
    o_latent = np.asarray(o_latent, dtype=np.float64)
    return np.stack([o_latent[..., i, :] @ W_uv[0] for i in range(o_latent.shape[-2])], axis=-2)


def test_up_projection_mistakes_are_caught(monkeypatch):
    _patch(monkeypatch, "mla_up_project", up_project_wrong_head)
    assert _fails(TM.test_absorbed_equals_explicit_reconstruction, 4, 16, 4, 8, 8, 7)
    assert _fails(TM.test_batched_explicit_equals_absorbed_then_up_projected)
    assert _fails(TM.test_up_projection_closed_forms)
    _patch(monkeypatch, "mla_up_project", up_project_transposed)
    assert _fails(TM.test_up_projection_closed_forms)


def test_explicit_batch_mistakes_are_caught(monkeypatch):
    orig = A.mla_explicit_decode_batch

    def values_from_keys(q, cache, seq_lens, W_uk, W_uv, scale, d_c=512, bf16=False):
        return orig(q, cache, seq_lens, W_uk, W_uk[:, :, :W_uv.shape[2]], scale, d_c=d_c, bf16=bf16)

    _patch(monkeypatch, "mla_explicit_decode_batch", values_from_keys)
    assert _fails(TM.test_batched_explicit_equals_absorbed_then_up_projected)
