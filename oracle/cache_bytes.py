"""KV-cache byte formulas and decode-attention intensity (oracle; test infrastructure).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use this module.

Exact integer arithmetic.  Sources (page title, then section):

* "Why GQA's KV Cache Savings Don't Fully Reduce TPOT", section "KV Cache
  Size by Attention Variant": whole-cache bytes are the product of layers,
  KV heads, head width, 2 (K and V), context length, batch and element size.
  On that page ``L`` is the context length.
* "MQA, GQA, and MLA", section 1 "The problem they solve": bytes per token
  are ``2 x layers x KV heads x head width x element size`` (there ``L`` is
  the layer count); section 5 "MLA, mechanically": an MLA cache keeps
  ``layers x (d_c + d_rope) x element size`` bytes per token.
* "MQA, GQA, and MLA", section 4 "The second benefit of GQA": one decode
  step of one sequence costs ``2 x h x S x d_head x 2`` FLOPs (scores and
  attention-times-V over all query heads) and reads
  ``2 x g x S x d_head x bytes`` of K and V; their ratio is the arithmetic
  intensity ``2 (h/g) / bytes``.
* "Compressing the KV Cache ...", section "Profiling KV-Cache Memory in
  TypeScript": the same two per-request formulas, with a 64-wide positional
  part added to the latent width for MLA.
"""


def kv_bytes_per_token(n_layers, n_kv_heads, d_head, bytes_per_elem):
    """Bytes one token adds to a K+V cache: 2 (K and V) x layers x KV heads x head width x element size."""
    return 2 * n_layers * n_kv_heads * d_head * bytes_per_elem


def kv_cache_bytes(n_layers, n_kv_heads, d_head, context_len, batch, bytes_per_elem):
    """Whole K+V cache of ``batch`` sequences of ``context_len`` tokens."""
    return n_layers * n_kv_heads * d_head * 2 * context_len * batch * bytes_per_elem


def mla_bytes_per_token(n_layers, d_latent, d_rope, bytes_per_elem):
    """Bytes one token adds to an MLA cache: the latent plus the decoupled RoPE key, per layer."""
    return n_layers * (d_latent + d_rope) * bytes_per_elem


def mla_cache_bytes(n_layers, d_latent, d_rope, context_len, batch, bytes_per_elem):
    """Whole MLA cache of ``batch`` sequences of ``context_len`` tokens."""
    return mla_bytes_per_token(n_layers, d_latent, d_rope, bytes_per_elem) * context_len * batch


def decode_attention_flops(n_q_heads, seq_len, d_head):
    """FLOPs of one decode step of one sequence: scores plus attention-times-V, 2 FLOPs per MAC."""
    return 2 * n_q_heads * seq_len * d_head * 2


def decode_attention_kv_bytes(n_kv_heads, seq_len, d_head, bytes_per_elem):
    """K and V bytes one decode step of one sequence reads when KV heads are indexed, not repeated."""
    return 2 * n_kv_heads * seq_len * d_head * bytes_per_elem


def decode_attention_intensity(n_q_heads, n_kv_heads, bytes_per_elem, seq_len=1, d_head=1):
    """FLOPs per KV byte of a decode step; independent of ``seq_len`` and ``d_head``."""
    return decode_attention_flops(n_q_heads, seq_len, d_head) / decode_attention_kv_bytes(
        n_kv_heads, seq_len, d_head, bytes_per_elem
    )
