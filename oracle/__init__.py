"""Plain fp64 CPU oracle for single-token decode attention over a KV cache.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite under ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import, call or execute anything in this package.  The GPU library
(``decode_attention_kv_03_amd``) never imports it, and this package never
imports the GPU library: the two share no code.  The only thing both sides
consume is the seeded input generator module, which holds random draws and
input layout only, none of the attention arithmetic.

Everything here is written from the definitions on the source pages, in
float64, with NumPy matrix products as the only library step:

* ``attention``   -- scaled-softmax decode attention for one query against
                     cached K/V rows; GQA/MHA/MQA head grouping; the paged
                     block-table gather; absorbed and explicit MLA; the
                     log-sum-exp merge of partial results.
* ``fp8``         -- the E4M3 code decoder and decode attention over an fp8
                     cache with one K and one V scale per KV head.
* ``cache_bytes`` -- the KV-cache byte formulas and the decode-attention
                     arithmetic-intensity formula.

Every function is pinned by tests under ``tests/`` against values the pages
print, closed forms, library routines (torch's scaled_dot_product_attention
in float64), and brute force on tiny inputs.
"""

from .attention import (  # noqa: F401
    bf16_bits_to_f64,
    attend,
    gqa_decode,
    paged_gather,
    paged_gqa_decode,
    mla_absorbed_decode,
    paged_mla_absorbed_decode,
    mla_absorb_query,
    mla_explicit_decode,
    mla_explicit_decode_batch,
    mla_up_project,
    lse_merge,
)
from .fp8 import (  # noqa: F401
    E4M3_MAX,
    e4m3_to_f64,
    dequantize_kv_heads,
    gqa_decode_fp8,
    paged_gqa_decode_fp8,
)
from .cache_bytes import (  # noqa: F401
    kv_cache_bytes,
    kv_bytes_per_token,
    mla_bytes_per_token,
    mla_cache_bytes,
    decode_attention_flops,
    decode_attention_kv_bytes,
    decode_attention_intensity,
)
