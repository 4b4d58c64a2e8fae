"""ctypes binding of libkvattn's C ABI (include/kvattn.h).

Argument marshalling only: this module checks tensor placement, dtype,
shape and contiguity, takes device pointers, allocates output and
workspace tensors through torch when the caller passes none, and calls the
library on torch's current HIP stream.  Every step of the attention itself
runs in the library's kernels; there is no Python or CPU fallback.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libkvattn.so"

KVATTN_OK, KVATTN_ERR_INVALID, KVATTN_ERR_UNSUPPORTED, KVATTN_ERR_WORKSPACE, KVATTN_ERR_HIP = range(5)
KVATTN_F32, KVATTN_BF16 = 0, 1
SPLIT_ALIGN = 64

# Every symbol the header declares, with its ctypes signature.
_c_i32, _c_i64, _c_f32, _c_sz, _c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
SIGNATURES = {
    "kvattn_gqa_decode": (
        _c_i32,
        [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_i32, _c_i32,
         _c_i32, _c_f32, _c_i32, _c_i32, _c_vp, _c_sz, _c_vp],
    ),
    "kvattn_gqa_decode_window": (
        _c_i32,
        [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_i32, _c_i32,
         _c_i32, _c_f32, _c_i32, _c_i32, _c_i32, _c_vp, _c_sz, _c_vp],
    ),
    "kvattn_gqa_decode_noalloc": (
        _c_i32,
        [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_i32, _c_i32,
         _c_i32, _c_f32, _c_i32, _c_i32, _c_i32, _c_vp],
    ),
    "kvattn_gqa_decode_fp8": (
        _c_i32,
        [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64,
         _c_i32, _c_i32, _c_i32, _c_f32, _c_i32, _c_i32, _c_vp, _c_sz, _c_vp],
    ),
    "kvattn_gqa_workspace_bytes": (_c_sz, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32]),
    "kvattn_mla_decode": (
        _c_i32,
        [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_i32, _c_i32, _c_i32,
         _c_f32, _c_i32, _c_i32, _c_vp, _c_sz, _c_vp],
    ),
    "kvattn_mla_workspace_bytes": (_c_sz, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32]),
    "kvattn_mla_project": (
        _c_i32,
        [_c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_i64, _c_i64, _c_i64, _c_i32, _c_i64,
         _c_i64, _c_i64, _c_i32, _c_vp],
    ),
    "kvattn_mla_explicit_decode": (
        _c_i32,
        [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64,
         _c_i32, _c_f32, _c_i32, _c_i32, _c_vp, _c_sz, _c_vp],
    ),
    "kvattn_mla_explicit_workspace_bytes": (_c_sz, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32]),
    "kvattn_gqa_split_tokens": (_c_i32, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32]),
    "kvattn_mla_split_tokens": (_c_i32, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32]),
    "kvattn_time_next_kernel": (_c_i32, [_c_vp, _c_vp]),
    "kvattn_clock_next_mla": (_c_i32, [_c_vp]),
    "kvattn_hbm_read_probe": (_c_i32, [_c_vp, _c_sz, _c_vp, _c_i32, _c_vp]),
    "kvattn_status_string": (ctypes.c_char_p, [_c_i32]),
    "kvattn_last_error": (ctypes.c_char_p, []),
}

_lib = None


class KvattnError(RuntimeError):
    """A non-OK status from libkvattn (``status`` holds the code)."""

    def __init__(self, status, detail):
        self.status = status
        super().__init__(f"kvattn: {detail} (status {status})")


def library_path():
    return os.path.join(_HERE, _LIB_NAME)


def load_library():
    """Load libkvattn.so from the package directory; raise if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise KvattnError(-1, f"{path} is missing; build it with __graft_entry__.build() or "
                              "python decode_attention_kv_03_amd/build.py")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status):
    if status != KVATTN_OK:
        lib = load_library()
        detail = lib.kvattn_last_error().decode() or lib.kvattn_status_string(status).decode()
        exc = ValueError if status in (KVATTN_ERR_INVALID, KVATTN_ERR_WORKSPACE) else KvattnError
        if exc is ValueError:
            raise ValueError(f"kvattn: {detail} (status {status})")
        raise KvattnError(status, detail)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return KVATTN_F32
    if t.dtype == torch.bfloat16:
        return KVATTN_BF16
    raise ValueError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _need_gpu(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("kvattn: every tensor must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("kvattn: every tensor must be contiguous")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def hbm_read_probe(buf, workgroups, sink, stream=None):
    """Stream every byte of the GPU tensor `buf` once (measurement utility; see kvattn_hbm_read_probe)."""
    _need_gpu(buf, sink)
    lib = load_library()
    _check(lib.kvattn_hbm_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), int(workgroups),
                                     _stream(stream)))


def time_next_kernel(start_event, stop_event):
    """Arm two timing-enabled events (torch.cuda.Event) around the split-K kernel of this thread's next
    decode call (measurement utility; see kvattn_time_next_kernel).  None, None disarms."""
    lib = load_library()
    if start_event is None and stop_event is None:
        _check(lib.kvattn_time_next_kernel(None, None))
        return
    handles = []
    for ev in (start_event, stop_event):
        h = ev.cuda_event
        if not h:
            raise ValueError("time_next_kernel: record each event once first so that it exists")
        handles.append(ctypes.c_void_p(h))
    _check(lib.kvattn_time_next_kernel(*handles))


def clock_next_mla(stamps):
    """Arm the next mla_decode call on this thread to store {shader clock, 100 MHz real-time} counter pairs
    at the start and end of its split kernel's tile loop into ``stamps`` (a CUDA int64 tensor of at least 4
    elements; measurement utility, see kvattn_clock_next_mla).  None disarms."""
    lib = load_library()
    if stamps is None:
        _check(lib.kvattn_clock_next_mla(None))
        return
    if not stamps.is_cuda or stamps.dtype != torch.int64 or stamps.numel() < 4 or not stamps.is_contiguous():
        raise ValueError("clock_next_mla: stamps must be a contiguous CUDA int64 tensor of at least 4 elements")
    _check(lib.kvattn_clock_next_mla(ctypes.c_void_p(stamps.data_ptr())))


def shader_clock_ghz(stamps):
    """Shader clock in GHz from the four values clock_next_mla had stored."""
    v = [int(t) for t in stamps[:4].tolist()]
    return (v[2] - v[0]) / ((v[3] - v[1]) * 10.0)


def gqa_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len, block_size=0, split_tokens=0,
                        dtype=torch.bfloat16):
    lib = load_library()
    code = KVATTN_BF16 if dtype == torch.bfloat16 else KVATTN_F32
    n = lib.kvattn_gqa_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len, block_size,
                                       split_tokens, code)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("kvattn: arguments rejected by kvattn_gqa_workspace_bytes")
    return n


def mla_workspace_bytes(batch, num_heads, max_seq_len, d_latent=512, d_rope=64, block_size=0, split_tokens=0):
    lib = load_library()
    n = lib.kvattn_mla_workspace_bytes(batch, num_heads, d_latent, d_rope, max_seq_len, block_size, split_tokens,
                                       KVATTN_BF16)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("kvattn: arguments rejected by kvattn_mla_workspace_bytes")
    return n


def _workspace(nbytes, workspace, device):
    if nbytes == 0:
        return None
    if workspace is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)  # the library needs no initialised contents
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"kvattn: workspace needs {nbytes} bytes")
    return workspace


def _gqa_geometry(q, k_cache, block_table, max_seq_len):
    """(g, cache_len, block_size, max_blocks, max_seq_len) of a GQA cache, checked against q [B, h, d]."""
    B, h, d = q.shape
    if block_table is None:
        if k_cache.shape[0] != B or k_cache.shape[3] != d:
            raise ValueError("kvattn: contiguous cache must be [B, g, S, d]")
        g, cache_len, block_size, max_blocks = k_cache.shape[1], k_cache.shape[2], 0, 0
        default_max = cache_len
    else:
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
            raise ValueError("kvattn: block_table must be int32 [B, max_blocks]")
        if k_cache.shape[3] != d:
            raise ValueError("kvattn: paged cache must be [num_blocks, g, block_size, d]")
        g, cache_len, block_size, max_blocks = k_cache.shape[1], k_cache.shape[0], k_cache.shape[2], block_table.shape[1]
        default_max = max_blocks * block_size
    max_seq_len = default_max if max_seq_len is None else int(max_seq_len)
    return g, cache_len, block_size, max_blocks, max_seq_len


def gqa_decode(q, k_cache, v_cache, seq_lens, scale, *, block_table=None, max_seq_len=None, out=None,
               return_lse=False, lse=None, split_tokens=0, workspace=None, stream=None, window=0):
    """Grouped-query decode attention (MHA at g = h, MQA at g = 1).

    q [B, h, d]; contiguous k_cache/v_cache [B, g, S, d], or, with
    ``block_table`` (int32 [B, max_blocks]), block pools [N, g, block_size, d];
    seq_lens int32 [B].  ``max_seq_len`` bounds every length (default: S, or
    max_blocks * block_size).  ``window`` > 0 attends only to each sequence's
    last ``window`` tokens (kvattn_gqa_decode_window).  Returns out [B, h, d]
    (and lse [B, h] fp32 when ``return_lse``).
    """
    _need_gpu(q, k_cache, v_cache, seq_lens, block_table, out, lse, workspace)
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("kvattn: q must be [B, h, d] and the caches 4-d with equal shapes")
    code = _dtype_code(q)
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("kvattn: q, k_cache and v_cache must share a dtype")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (q.shape[0],):
        raise ValueError("kvattn: seq_lens must be int32 [B]")
    B, h, d = q.shape
    g, cache_len, block_size, max_blocks, max_seq_len = _gqa_geometry(q, k_cache, block_table, max_seq_len)
    if out is None:
        out = torch.empty((B, h, d), dtype=q.dtype, device=q.device)
    elif out.shape != (B, h, d) or out.dtype != q.dtype:
        raise ValueError("kvattn: out must be [B, h, d] with the dtype of q")
    if return_lse and lse is None:
        lse = torch.empty((B, h), dtype=torch.float32, device=q.device)
    lib = load_library()
    nbytes = lib.kvattn_gqa_workspace_bytes(B, h, g, d, max_seq_len, block_size, split_tokens, code)
    if nbytes == ctypes.c_size_t(-1).value:
        nbytes = 0  # the decode call reports the precise problem
    ws = _workspace(nbytes, workspace, q.device)
    if window:
        _check(lib.kvattn_gqa_decode_window(
            _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens), _ptr(out), _ptr(lse),
            B, h, g, d, cache_len, block_size, max_blocks, max_seq_len, float(scale), int(window), code,
            int(split_tokens), _ptr(ws), nbytes, _stream(stream)))
    else:
        _check(lib.kvattn_gqa_decode(
            _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens), _ptr(out), _ptr(lse),
            B, h, g, d, cache_len, block_size, max_blocks, max_seq_len, float(scale), code, int(split_tokens),
            _ptr(ws), nbytes, _stream(stream)))
    return (out, lse) if (return_lse or lse is not None) else out


NOALLOC_SCRATCH_BYTES = 128 << 20


def gqa_decode_noalloc(q, k_cache, v_cache, seq_lens, scale, out, *, block_table=None, max_seq_len=None, lse=None,
                       split_tokens=0, stream=None, window=0):
    """``gqa_decode`` through kvattn_gqa_decode_noalloc: no workspace, nothing allocated.

    The caller passes the output (and optionally lse) tensors; the split-K
    partials go to the library's fixed per-GPU scratch array
    (``NOALLOC_SCRATCH_BYTES``).  Calls that could overlap on one GPU race on
    that array.  Returns ``out`` (and ``lse`` when given).
    """
    _need_gpu(q, k_cache, v_cache, seq_lens, block_table, out, lse)
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("kvattn: q must be [B, h, d] and the caches 4-d with equal shapes")
    code = _dtype_code(q)
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("kvattn: q, k_cache and v_cache must share a dtype")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (q.shape[0],):
        raise ValueError("kvattn: seq_lens must be int32 [B]")
    B, h, d = q.shape
    g, cache_len, block_size, max_blocks, max_seq_len = _gqa_geometry(q, k_cache, block_table, max_seq_len)
    if out.shape != (B, h, d) or out.dtype != q.dtype:
        raise ValueError("kvattn: out must be [B, h, d] with the dtype of q")
    if lse is not None and (lse.shape != (B, h) or lse.dtype != torch.float32):
        raise ValueError("kvattn: lse must be float32 [B, h]")
    lib = load_library()
    _check(lib.kvattn_gqa_decode_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens), _ptr(out), _ptr(lse), B, h, g, d,
        cache_len, block_size, max_blocks, max_seq_len, float(scale), int(window), code, int(split_tokens),
        _stream(stream)))
    return (out, lse) if lse is not None else out


def gqa_decode_fp8(q, k_cache, v_cache, k_scale, v_scale, seq_lens, scale, *, block_table=None, max_seq_len=None,
                   out=None, return_lse=False, lse=None, split_tokens=0, workspace=None, stream=None, window=0):
    """Grouped-query decode over an E4M3 KV cache (kvattn_gqa_decode_fp8).

    q [B, h, d] bfloat16; k_cache/v_cache hold E4M3 codes (torch.uint8 or
    torch.float8_e4m3fn) in the layouts of ``gqa_decode``; k_scale and
    v_scale are float32 [g], one per KV head (a code c of head j stands for
    scale[j] * E4M3(c)).  Returns out [B, h, d] bfloat16 (and lse [B, h]).
    """
    _need_gpu(q, k_cache, v_cache, k_scale, v_scale, seq_lens, block_table, out, lse, workspace)
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("kvattn: q must be [B, h, d] and the caches 4-d with equal shapes")
    if q.dtype != torch.bfloat16:
        raise ValueError("kvattn: the fp8-cache decode takes a bfloat16 query")
    for c in (k_cache, v_cache):
        if c.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise ValueError("kvattn: fp8 caches must be uint8 or float8_e4m3fn")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (q.shape[0],):
        raise ValueError("kvattn: seq_lens must be int32 [B]")
    B, h, d = q.shape
    g, cache_len, block_size, max_blocks, max_seq_len = _gqa_geometry(q, k_cache, block_table, max_seq_len)
    for sc in (k_scale, v_scale):
        if sc.dtype != torch.float32 or sc.shape != (g,):
            raise ValueError("kvattn: k_scale and v_scale must be float32 [num_kv_heads]")
    if out is None:
        out = torch.empty((B, h, d), dtype=torch.bfloat16, device=q.device)
    elif out.shape != (B, h, d) or out.dtype != torch.bfloat16:
        raise ValueError("kvattn: out must be bfloat16 [B, h, d]")
    if return_lse and lse is None:
        lse = torch.empty((B, h), dtype=torch.float32, device=q.device)
    lib = load_library()
    nbytes = lib.kvattn_gqa_workspace_bytes(B, h, g, d, max_seq_len, block_size, split_tokens, KVATTN_BF16)
    if nbytes == ctypes.c_size_t(-1).value:
        nbytes = 0  # the decode call reports the precise problem
    ws = _workspace(nbytes, workspace, q.device)
    _check(lib.kvattn_gqa_decode_fp8(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(block_table), _ptr(seq_lens),
        _ptr(out), _ptr(lse), B, h, g, d, cache_len, block_size, max_blocks, max_seq_len, float(scale), int(window),
        int(split_tokens), _ptr(ws), nbytes, _stream(stream)))
    return (out, lse) if (return_lse or lse is not None) else out


def mla_decode(q, cache, seq_lens, scale, *, block_table=None, max_seq_len=None, out=None, return_lse=False,
               lse=None, split_tokens=0, workspace=None, stream=None, d_latent=512):
    """Absorbed MLA decode: q [B, h, 576] against cache rows [c (512) | k^R (64)].

    Contiguous cache [B, S, 576], or with ``block_table`` a pool
    [N, block_size, 576].  Returns out [B, h, 512] in latent space (and lse).
    """
    _need_gpu(q, cache, seq_lens, block_table, out, lse, workspace)
    if q.dim() != 3 or cache.shape[-1] != q.shape[2]:
        raise ValueError("kvattn: q must be [B, h, d_latent + d_rope] and match the cache row width")
    code = _dtype_code(q)
    if cache.dtype != q.dtype:
        raise ValueError("kvattn: q and cache must share a dtype")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (q.shape[0],):
        raise ValueError("kvattn: seq_lens must be int32 [B]")
    B, h, width = q.shape
    d_rope = width - d_latent
    if block_table is None:
        if cache.dim() != 3 or cache.shape[0] != B:
            raise ValueError("kvattn: contiguous MLA cache must be [B, S, d_latent + d_rope]")
        cache_len, block_size, max_blocks = cache.shape[1], 0, 0
        default_max = cache_len
    else:
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
            raise ValueError("kvattn: block_table must be int32 [B, max_blocks]")
        if cache.dim() != 3:
            raise ValueError("kvattn: paged MLA cache must be [num_blocks, block_size, d_latent + d_rope]")
        cache_len, block_size, max_blocks = cache.shape[0], cache.shape[1], block_table.shape[1]
        default_max = max_blocks * block_size
    max_seq_len = default_max if max_seq_len is None else int(max_seq_len)
    if out is None:
        out = torch.empty((B, h, d_latent), dtype=q.dtype, device=q.device)
    elif out.shape != (B, h, d_latent) or out.dtype != q.dtype:
        raise ValueError("kvattn: out must be [B, h, d_latent] with the dtype of q")
    if return_lse and lse is None:
        lse = torch.empty((B, h), dtype=torch.float32, device=q.device)
    lib = load_library()
    nbytes = lib.kvattn_mla_workspace_bytes(B, h, d_latent, d_rope, max_seq_len, block_size, split_tokens, code)
    if nbytes == ctypes.c_size_t(-1).value:
        nbytes = 0
    ws = _workspace(nbytes, workspace, q.device)
    _check(lib.kvattn_mla_decode(
        _ptr(q), _ptr(cache), _ptr(block_table), _ptr(seq_lens), _ptr(out), _ptr(lse), B, h, d_latent, d_rope,
        cache_len, block_size, max_blocks, max_seq_len, float(scale), code, int(split_tokens), _ptr(ws), nbytes,
        _stream(stream)))
    return (out, lse) if (return_lse or lse is not None) else out


def mla_project(x, w, y, *, outer, heads, rows, k_dim, n_dim, x_strides, w_head_stride, y_strides,
                w_transposed=False, stream=None):
    """kvattn_mla_project on raw strides: y[o, i, m] = x[o, i, m] W^(i) (or W^(i)^T).

    ``x_strides`` and ``y_strides`` are (outer, head, row) strides in elements;
    x, w and y are bfloat16 GPU tensors (their data pointers are used as-is).
    """
    _need_gpu(x, w, y)
    for t in (x, w, y):
        if t.dtype != torch.bfloat16:
            raise ValueError("kvattn: projections take bfloat16 tensors")
    lib = load_library()
    _check(lib.kvattn_mla_project(_ptr(x), _ptr(w), _ptr(y), int(outer), int(heads), int(rows), int(k_dim), int(n_dim),
                                  *[int(v) for v in x_strides], int(w_head_stride), int(bool(w_transposed)),
                                  *[int(v) for v in y_strides], KVATTN_BF16, _stream(stream)))
    return y


def mla_up_project(o_latent, w_uv, out=None, stream=None):
    """Per-head W_uv up-projection of absorbed MLA outputs: o_latent [B, h, d_c] x W_uv [h, d_c, d_v] -> [B, h, d_v]."""
    B, h, d_c = o_latent.shape
    if w_uv.dim() != 3 or w_uv.shape[0] != h or w_uv.shape[1] != d_c:
        raise ValueError("kvattn: w_uv must be [h, d_c, d_v]")
    d_v = w_uv.shape[2]
    if out is None:
        out = torch.empty((B, h, d_v), dtype=o_latent.dtype, device=o_latent.device)
    elif out.shape != (B, h, d_v):
        raise ValueError("kvattn: out must be [B, h, d_v]")
    return mla_project(o_latent, w_uv, out, outer=1, heads=h, rows=B, k_dim=d_c, n_dim=d_v,
                       x_strides=(0, d_c, h * d_c), w_head_stride=d_c * d_v, y_strides=(0, d_v, h * d_v),
                       stream=stream)


def mla_absorb_query(q_c, w_uk, out=None, stream=None):
    """Absorbed content queries q^C_i W_uk^(i)^T: q_c [B, h, d_h] with W_uk [h, d_c, d_h] -> [B, h, d_c].

    ``out`` may be a wider [B, h, d_c + d_r] tensor: the result fills its first d_c columns.
    """
    B, h, d_h = q_c.shape
    if w_uk.dim() != 3 or w_uk.shape[0] != h or w_uk.shape[2] != d_h:
        raise ValueError("kvattn: w_uk must be [h, d_c, d_h]")
    d_c = w_uk.shape[1]
    if out is None:
        out = torch.empty((B, h, d_c), dtype=q_c.dtype, device=q_c.device)
    if out.dim() != 3 or out.shape[:2] != (B, h) or out.shape[2] < d_c:
        raise ValueError("kvattn: out must be [B, h, >= d_c]")
    width = out.shape[2]
    return mla_project(q_c, w_uk, out, outer=1, heads=h, rows=B, k_dim=d_h, n_dim=d_c,
                       x_strides=(0, d_h, h * d_h), w_head_stride=d_c * d_h, y_strides=(0, width, h * width),
                       w_transposed=True, stream=stream)


def mla_explicit_workspace_bytes(batch, num_heads, max_seq_len, d_head=128, d_v=128, split_tokens=0):
    lib = load_library()
    n = lib.kvattn_mla_explicit_workspace_bytes(batch, num_heads, d_head, d_v, max_seq_len, split_tokens, KVATTN_BF16)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("kvattn: arguments rejected by kvattn_mla_explicit_workspace_bytes")
    return n


def mla_explicit_decode(q, cache, w_uk, w_uv, seq_lens, scale, *, max_seq_len=None, out=None, return_lse=False,
                        lse=None, split_tokens=0, workspace=None, stream=None, d_latent=512):
    """Reconstruct-then-attend MLA decode (kvattn_mla_explicit_decode).

    q [B, h, d_h + d_r] rows [q^C | q^R]; cache [B, S, d_latent + d_r]; w_uk [h, d_latent, d_h];
    w_uv [h, d_latent, d_v].  Returns out [B, h, d_v] (and lse [B, h]).
    """
    _need_gpu(q, cache, w_uk, w_uv, seq_lens, out, lse, workspace)
    if q.dim() != 3 or cache.dim() != 3 or cache.shape[0] != q.shape[0]:
        raise ValueError("kvattn: q must be [B, h, d_h + d_r] and cache [B, S, d_latent + d_r]")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (q.shape[0],):
        raise ValueError("kvattn: seq_lens must be int32 [B]")
    B, h, width = q.shape
    d_rope = cache.shape[2] - d_latent
    d_head = width - d_rope
    if w_uk.shape != (h, d_latent, d_head) or w_uv.dim() != 3 or w_uv.shape[:2] != (h, d_latent):
        raise ValueError("kvattn: w_uk must be [h, d_latent, d_head] and w_uv [h, d_latent, d_v]")
    d_v = w_uv.shape[2]
    code = _dtype_code(q)
    cache_len = cache.shape[1]
    max_seq_len = cache_len if max_seq_len is None else int(max_seq_len)
    if out is None:
        out = torch.empty((B, h, d_v), dtype=q.dtype, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty((B, h), dtype=torch.float32, device=q.device)
    lib = load_library()
    nbytes = lib.kvattn_mla_explicit_workspace_bytes(B, h, d_head, d_v, max_seq_len, split_tokens, code)
    if nbytes == ctypes.c_size_t(-1).value:
        nbytes = 0
    ws = _workspace(nbytes, workspace, q.device)
    _check(lib.kvattn_mla_explicit_decode(
        _ptr(q), _ptr(cache), _ptr(w_uk), _ptr(w_uv), _ptr(seq_lens), _ptr(out), _ptr(lse), B, h, d_latent, d_rope,
        d_head, d_v, cache_len, max_seq_len, float(scale), code, int(split_tokens), _ptr(ws), nbytes,
        _stream(stream)))
    return (out, lse) if (return_lse or lse is not None) else out
