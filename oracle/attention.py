"""fp64 reference for decode attention over a KV cache (oracle; test infrastructure).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use this module.

Sources (page title, then section):

* "MQA, GQA, and MLA" (learning-materials, Below the API track):
  section 2 "The three answers" and section 3 "The picture" define the head
  sharing of MHA / GQA / MQA; section 4 "The second benefit of GQA" states
  that a decode step computes scores plus attention-times-V for every query
  head; section 5 "MLA, mechanically" defines the latent ``c``, the per-head
  reconstruction ``k_i = c W_uk^(i)``, ``v_i = c W_uv^(i)``, the absorption of
  ``W_uk`` into the query, and the decoupled RoPE key cached next to ``c``;
  section 8 "Implementation notes" fixes the head map ``i // (h/g)``.
* "Why GQA's KV Cache Savings Don't Fully Reduce TPOT", section "What Makes
  MLA Different": the absorbed form needs no reconstruction, and the 64-wide
  RoPE part is kept and used explicitly (cache row width 512 + 64).
* "One dial, four settings" (runbooks, Document 07), the full ladder's SWA
  row and the question on sliding-window attention: with a window of W
  tokens each token attends only to the last W, and tokens outside the
  window are not attended at all (``window`` below; 0 means no window).
* "Compressing the KV Cache ... (MLA) vs. Meta's Grouped Queries (GQA)",
  section "KV-Cache Management Guardrails": caches live in fixed-size blocks
  (paged attention); the pages give no block layout, so the layout below is
  this library's reading (pool ``[num_blocks, g, block_size, d]``, token ``t``
  of a sequence in block ``table[t // block_size]`` at slot
  ``t % block_size``).

The pages never write the attention formula out; this oracle takes the
textbook one: for a query ``q`` and cached rows ``k_t, v_t`` (t < n),
``s_t = scale * <q, k_t>``, ``p = softmax(s)``, ``o = sum_t p_t v_t``, and the
log-sum-exp ``lse = log sum_t exp(s_t)``.  An empty cache (n = 0) gives
``o = 0`` and ``lse = -inf``.

All arithmetic is float64.  bfloat16 inputs arrive as their uint16 bit
patterns and are widened exactly (a bfloat16 is the top half of a float32).
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """Widen bfloat16 bit patterns (any integer array of 16-bit codes) to float64 exactly."""
    u = np.ascontiguousarray(np.asarray(bits)).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def _f64(x, bf16):
    return bf16_bits_to_f64(x) if bf16 else np.asarray(x, dtype=np.float64)


def attend(q, K, V, scale):
    """Scaled-softmax attention of one query over ``n`` cached rows.

    q: [d_k]; K: [n, d_k]; V: [n, d_v]; returns (o [d_v], lse scalar), fp64.
    The score is ``scale * <q, k_t>``; the output is the softmax-weighted sum
    of the value rows ("scores + attn@V", section 4 of "MQA, GQA, and MLA").
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    n = K.shape[0]
    if n == 0:
        return np.zeros(V.shape[1], dtype=np.float64), -np.inf
    s = scale * (K @ q)
    m = s.max()
    e = np.exp(s - m)
    z = e.sum()
    o = (e / z) @ V
    return o, m + np.log(z)


def window_start(n, window):
    """First attended token of a sequence of ``n`` tokens: the last ``window`` tokens (window 0: all)."""
    return max(0, n - window) if window > 0 else 0


def gqa_decode(q, K, V, seq_lens, scale, bf16=False, window=0):
    """Grouped-query decode: ``h`` query heads over ``g`` cached K/V heads.

    q: [B, h, d]; K: [B, g, S, d]; V: [B, g, S, d_v]; seq_lens: [B].
    Query head ``i`` reads KV head ``i // (h/g)`` (section 8 of "MQA, GQA,
    and MLA": index, never repeat), so the heads of one group are the
    contiguous run ``j*(h/g) .. (j+1)*(h/g)-1`` (section 3 figure).  ``g = h``
    is MHA, ``g = 1`` is MQA.  Sequence ``b`` attends to its first
    ``seq_lens[b]`` cached tokens, or with ``window`` > 0 to the last
    ``window`` of them.  Returns (o [B, h, d_v], lse [B, h]).
    With ``bf16=True`` the arrays hold bfloat16 bit patterns.
    """
    B, h, _ = q.shape
    g = K.shape[1]
    if h % g != 0:
        raise ValueError("h must be a multiple of g")
    r = h // g
    d_v = V.shape[3]
    o = np.zeros((B, h, d_v), dtype=np.float64)
    lse = np.full((B, h), -np.inf, dtype=np.float64)
    for b in range(B):
        n = int(seq_lens[b])
        t0 = window_start(n, window)
        qb = _f64(q[b], bf16)
        Kb = _f64(K[b, :, t0:n], bf16)
        Vb = _f64(V[b, :, t0:n], bf16)
        for i in range(h):
            j = i // r
            o[b, i], lse[b, i] = attend(qb[i], Kb[j], Vb[j], scale)
    return o, lse


def paged_gather(pool, table_row, n, block_size, kv_head=None):
    """Rows ``0..n-1`` of one sequence from a block pool.

    Token ``t`` lives in physical block ``table_row[t // block_size]`` at slot
    ``t % block_size``.  ``pool`` is [num_blocks, g, block_size, d] (pass
    ``kv_head``) or [num_blocks, block_size, d] (MLA latent pool).
    """
    rows = []
    for t in range(n):
        blk = int(table_row[t // block_size])
        slot = t % block_size
        rows.append(pool[blk, kv_head, slot] if kv_head is not None else pool[blk, slot])
    if not rows:
        width = pool.shape[-1]
        return np.zeros((0, width), dtype=pool.dtype)
    return np.stack(rows)


def paged_gqa_decode(q, K_pool, V_pool, block_table, seq_lens, block_size, scale, bf16=False, window=0):
    """``gqa_decode`` with K/V in a block pool addressed through ``block_table`` [B, max_blocks]."""
    B, h, _ = q.shape
    g = K_pool.shape[1]
    if h % g != 0:
        raise ValueError("h must be a multiple of g")
    r = h // g
    d_v = V_pool.shape[3]
    o = np.zeros((B, h, d_v), dtype=np.float64)
    lse = np.full((B, h), -np.inf, dtype=np.float64)
    for b in range(B):
        n = int(seq_lens[b])
        qb = _f64(q[b], bf16)
        t0 = window_start(n, window)
        Kb = [_f64(paged_gather(K_pool, block_table[b], n, block_size, j)[t0:], bf16) for j in range(g)]
        Vb = [_f64(paged_gather(V_pool, block_table[b], n, block_size, j)[t0:], bf16) for j in range(g)]
        for i in range(h):
            j = i // r
            o[b, i], lse[b, i] = attend(qb[i], Kb[j], Vb[j], scale)
    return o, lse


def mla_absorbed_decode(q_abs, cache, seq_lens, scale, d_c=512, bf16=False):
    """Absorbed MLA decode over a latent cache.

    q_abs: [B, h, d_c + d_r] absorbed queries ``[q^C_i W_uk^(i)T | q^R_i]``;
    cache: [B, S, d_c + d_r] rows ``[c_t | k^R_t]``.  Every head scores its
    absorbed query against the whole cached row (latent part plus the shared
    decoupled-RoPE key) and accumulates its output in latent space from the
    ``c_t`` part only: ``o_i = sum_t p_t c_t`` (``W_uv`` is applied
    downstream).  Sections 5 of "MQA, GQA, and MLA" and "What Makes MLA
    Different" of the TPOT page.  Returns (o [B, h, d_c], lse [B, h]).
    """
    B, h, _ = q_abs.shape
    o = np.zeros((B, h, d_c), dtype=np.float64)
    lse = np.full((B, h), -np.inf, dtype=np.float64)
    for b in range(B):
        n = int(seq_lens[b])
        rows = _f64(cache[b, :n], bf16)
        qb = _f64(q_abs[b], bf16)
        for i in range(h):
            o[b, i], lse[b, i] = attend(qb[i], rows, rows[:, :d_c], scale)
    return o, lse


def paged_mla_absorbed_decode(q_abs, pool, block_table, seq_lens, block_size, scale, d_c=512, bf16=False):
    """``mla_absorbed_decode`` with latent rows in a block pool [num_blocks, block_size, d_c + d_r]."""
    B, h, _ = q_abs.shape
    o = np.zeros((B, h, d_c), dtype=np.float64)
    lse = np.full((B, h), -np.inf, dtype=np.float64)
    for b in range(B):
        n = int(seq_lens[b])
        rows = _f64(paged_gather(pool, block_table[b], n, block_size), bf16)
        qb = _f64(q_abs[b], bf16)
        for i in range(h):
            o[b, i], lse[b, i] = attend(qb[i], rows, rows[:, :d_c], scale)
    return o, lse


def mla_absorb_query(q_c, W_uk):
    """Absorb the key up-projection into the query.

    q_c: [h, d_h] content queries; W_uk: [h, d_c, d_h] with ``k_i = c W_uk^(i)``.
    Since ``q_i . (c W_uk^(i)) = (q_i W_uk^(i)T) . c`` (section 5 of "MQA, GQA,
    and MLA"), the absorbed query of head ``i`` is ``W_uk^(i) q_i``, length d_c.
    """
    q_c = np.asarray(q_c, dtype=np.float64)
    W_uk = np.asarray(W_uk, dtype=np.float64)
    return np.stack([W_uk[i] @ q_c[i] for i in range(q_c.shape[0])])


def mla_explicit_decode(q_c, q_r, c, k_r, W_uk, W_uv, scale):
    """Reconstruct-then-attend MLA for one sequence (the naive form).

    q_c: [h, d_h]; q_r: [h, d_r]; c: [n, d_c]; k_r: [n, d_r] (shared by all
    heads); W_uk: [h, d_c, d_h]; W_uv: [h, d_c, d_v].  Head ``i`` rebuilds its
    keys ``[c W_uk^(i) | k^R]`` and values ``c W_uv^(i)`` and attends over
    them.  Returns (o [h, d_v], lse [h]) in the full per-head value space.
    """
    c = np.asarray(c, dtype=np.float64)
    k_r = np.asarray(k_r, dtype=np.float64)
    h = q_c.shape[0]
    outs, lses = [], []
    for i in range(h):
        k_i = np.concatenate([c @ W_uk[i], k_r], axis=1)
        v_i = c @ W_uv[i]
        q_i = np.concatenate([q_c[i], q_r[i]])
        o_i, lse_i = attend(q_i, k_i, v_i, scale)
        outs.append(o_i)
        lses.append(lse_i)
    return np.stack(outs), np.array(lses)


def mla_up_project(o_latent, W_uv):
    """Move absorbed MLA outputs from latent space to each head's value space.

    o_latent: [..., h, d_c] (the absorbed form's ``sum_t p_t c_t`` per head);
    W_uv: [h, d_c, d_v].  Since ``v_i = c W_uv^(i)`` (section 5 of "MQA, GQA,
    and MLA") and the attention average is linear, head ``i``'s output is
    ``o_latent_i W_uv^(i)``.  Returns [..., h, d_v].
    """
    o_latent = np.asarray(o_latent, dtype=np.float64)
    W_uv = np.asarray(W_uv, dtype=np.float64)
    h = o_latent.shape[-2]
    out = np.empty(o_latent.shape[:-1] + (W_uv.shape[2],), dtype=np.float64)
    for i in range(h):
        out[..., i, :] = o_latent[..., i, :] @ W_uv[i]
    return out


def mla_explicit_decode_batch(q, cache, seq_lens, W_uk, W_uv, scale, d_c=512, bf16=False):
    """``mla_explicit_decode`` for a batch over a contiguous latent cache.

    q: [B, h, d_h + d_r] rows ``[q^C_i | q^R_i]``; cache: [B, S, d_c + d_r]
    rows ``[c_t | k^R_t]``; W_uk: [h, d_c, d_h]; W_uv: [h, d_c, d_v].
    Sequence ``b`` attends over its first ``seq_lens[b]`` rows.  With
    ``bf16=True`` every array holds bfloat16 bit patterns.  Returns
    (o [B, h, d_v], lse [B, h]).
    """
    W_uk = _f64(W_uk, bf16)
    W_uv = _f64(W_uv, bf16)
    d_h = W_uk.shape[2]
    B, h, _ = q.shape
    o = np.zeros((B, h, W_uv.shape[2]), dtype=np.float64)
    lse = np.full((B, h), -np.inf, dtype=np.float64)
    for b in range(B):
        n = int(seq_lens[b])
        qb = _f64(q[b], bf16)
        rows = _f64(cache[b, :n], bf16)
        o[b], lse[b] = mla_explicit_decode(qb[:, :d_h], qb[:, d_h:], rows[:, :d_c], rows[:, d_c:], W_uk, W_uv, scale)
    return o, lse


def lse_merge(parts):
    """Combine attention results computed over disjoint token subsets.

    parts: list of (o_s [..., d_v], lse_s [...]) where ``o_s`` is already
    normalised over its subset.  With ``M = max_s lse_s`` and
    ``w_s = exp(lse_s - M)``: ``o = sum_s w_s o_s / sum_s w_s`` and
    ``lse = M + log sum_s w_s``.  Subsets with ``lse = -inf`` (empty) weigh 0;
    if every subset is empty the result is ``o = 0``, ``lse = -inf``.
    """
    os_ = np.stack([np.asarray(p[0], dtype=np.float64) for p in parts])
    ls = np.stack([np.asarray(p[1], dtype=np.float64) for p in parts])
    M = ls.max(axis=0)
    finite = np.isfinite(M)
    Msafe = np.where(finite, M, 0.0)
    w = np.where(np.isfinite(ls), np.exp(ls - Msafe), 0.0)
    W = w.sum(axis=0)
    Wsafe = np.where(W > 0, W, 1.0)
    o = (w[..., None] * os_).sum(axis=0) / Wsafe[..., None]
    o = np.where(finite[..., None], o, 0.0)
    lse = np.where(finite, Msafe + np.log(Wsafe), -np.inf)
    return o, lse
