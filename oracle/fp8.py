"""fp64 reference for decode attention over an FP8 KV cache (oracle; test infrastructure).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use this module.

Sources (page title, then section):

* "Why GQA's KV Cache Savings Don't Fully Reduce TPOT", section "When the
  Serving Engineer Doesn't Get to Choose": storing the KV cache in fp8 halves
  its bytes per sequence (the 70B GQA-8 example at 8K tokens), and a GQA
  cache quantises naturally at the granularity of one KV head.
* "One dial, four settings" (runbooks, Document 07), the question on what is
  a runtime flag: the cache dtype is a runtime choice whose saving multiplies
  with the model's head ratio.

The pages name neither the 8-bit format nor how values are scaled.  The
readings taken here:

* Format: OCP 8-bit floating point E4M3 (the "e4m3fn" variant): one sign
  bit, a 4-bit exponent with bias 7, a 3-bit mantissa; exponent field 0
  encodes subnormals ``m/8 * 2^-6``; the codes with all exponent and mantissa
  bits set (0x7F, 0xFF) are NaN; there are no infinities; the largest finite
  magnitude is 448.
* Scale: one float32 scale per KV head for K and one for V.  The value a
  cached code ``c`` of KV head ``j`` stands for is ``k_scale[j] * E4M3(c)``
  (``v_scale[j]`` for V).
* Attention then runs on the dequantised cache exactly as for a bf16 or fp32
  cache (``attention.gqa_decode``); the query stays bfloat16.
"""

import numpy as np

from .attention import bf16_bits_to_f64, gqa_decode, paged_gqa_decode

E4M3_MAX = 448.0


def e4m3_to_f64(codes):
    """Value of each E4M3 code (uint8 array) as float64, from the field definition above."""
    c = np.asarray(codes).astype(np.int64)
    if c.size and (c.min() < 0 or c.max() > 255):
        raise ValueError("E4M3 codes are bytes")
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    exp_field = (c >> 3) & 0xF
    mant = (c & 0x7).astype(np.float64)
    normal = (1.0 + mant / 8.0) * np.exp2(exp_field.astype(np.float64) - 7.0)
    subnormal = (mant / 8.0) * 2.0 ** -6
    mag = np.where(exp_field == 0, subnormal, normal)
    mag = np.where((exp_field == 0xF) & ((c & 0x7) == 0x7), np.nan, mag)
    return sign * mag


def dequantize_kv_heads(codes, scales, head_axis):
    """``scales[j] * E4M3(codes)`` with ``j`` the index along ``head_axis`` (one scale per KV head)."""
    vals = e4m3_to_f64(codes)
    s = np.asarray(scales, dtype=np.float64)
    if s.shape != (vals.shape[head_axis],):
        raise ValueError("one scale per KV head expected")
    shape = [1] * vals.ndim
    shape[head_axis] = -1
    return vals * s.reshape(shape)


def gqa_decode_fp8(q_bf16, K_codes, V_codes, k_scale, v_scale, seq_lens, scale, window=0):
    """Grouped-query decode over an E4M3 cache.

    q_bf16: [B, h, d] bfloat16 bit patterns; K_codes, V_codes: [B, g, S, d]
    uint8 codes; k_scale, v_scale: [g].  Dequantises every cached row with
    its KV head's scale, then attends as ``attention.gqa_decode`` (query head
    ``i`` reads KV head ``i // (h/g)``).  Returns (o [B, h, d], lse [B, h]).
    """
    K = dequantize_kv_heads(K_codes, k_scale, head_axis=1)
    V = dequantize_kv_heads(V_codes, v_scale, head_axis=1)
    return gqa_decode(bf16_bits_to_f64(q_bf16), K, V, seq_lens, scale, window=window)


def paged_gqa_decode_fp8(q_bf16, K_pool, V_pool, k_scale, v_scale, block_table, seq_lens, block_size, scale,
                         window=0):
    """``gqa_decode_fp8`` with the codes in a block pool [num_blocks, g, block_size, d]."""
    K = dequantize_kv_heads(K_pool, k_scale, head_axis=1)
    V = dequantize_kv_heads(V_pool, v_scale, head_axis=1)
    return paged_gqa_decode(bf16_bits_to_f64(q_bf16), K, V, block_table, seq_lens, block_size, scale,
                            window=window)
