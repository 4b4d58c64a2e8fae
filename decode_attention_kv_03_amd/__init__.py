"""kvattn: single-token decode attention over a KV cache for MI355X (gfx950).

Two operations, both hand-written HIP kernels behind a C ABI
(``include/kvattn.h``, built into ``libkvattn.so`` next to this file):

* ``gqa_decode`` -- grouped-query decode: ``h`` query heads share ``g``
  cached K/V heads (MHA when ``g = h``, MQA when ``g = 1``), over a
  contiguous or block-table-paged cache with per-sequence lengths, optionally
  restricted to a sliding window of the last tokens.
* ``gqa_decode_fp8`` -- the same over an E4M3 (fp8) cache with one K and one
  V scale per KV head.
* ``mla_decode`` -- absorbed multi-head latent attention decode: every head
  scores an absorbed 576-wide query against cached ``[latent 512 | RoPE 64]``
  rows and accumulates its output in the 512-wide latent space.
* ``mla_up_project`` / ``mla_absorb_query`` (``mla_project``) -- the per-head
  projections out of and into the latent space on the matrix cores.
* ``mla_explicit_decode`` -- the naive reconstruct-then-attend MLA decode,
  which rebuilds per-head keys and values from the latent cache.

The Python layer only marshals arguments (device pointers, sizes, the
current HIP stream); every arithmetic step runs in the library's kernels.
Importing this package does not load the library; the first call does, and
raises if the library is missing or no GPU is present.
"""

from .kvattn import (  # noqa: F401
    KvattnError,
    gqa_decode,
    gqa_decode_fp8,
    gqa_decode_noalloc,
    gqa_workspace_bytes,
    hbm_read_probe,
    library_path,
    load_library,
    mla_absorb_query,
    mla_decode,
    mla_explicit_decode,
    mla_explicit_workspace_bytes,
    mla_project,
    mla_up_project,
    mla_workspace_bytes,
    time_next_kernel,
    clock_next_mla,
    shader_clock_ghz,
)
