"""C-ABI library checks that need no GPU: symbols, status strings, split
planning, workspace sizing, and host-side argument validation (every bad
argument is rejected before any HIP call, so these run on a CPU-only host)."""

import ctypes
import os
import re

import pytest

from decode_attention_kv_03_amd import kvattn as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvattn.h")
MEASURE_HEADER = os.path.join(ROOT, "include", "kvattn_measure.h")

lib = None


def setup_module(_):
    global lib
    if not os.path.exists(K.library_path()):
        pytest.skip("libkvattn.so not built (run __graft_entry__.build())")
    lib = K.load_library()


def header_functions(path=HEADER):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvattn_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported_and_bound():
    names = header_functions()
    measure = header_functions(MEASURE_HEADER)
    assert "kvattn_gqa_decode" in names and "kvattn_mla_decode" in names
    # the attention header holds the operations, sizing queries and error calls only
    assert not set(names) & set(measure)
    assert measure == ["kvattn_clock_next_mla", "kvattn_hbm_read_probe", "kvattn_time_next_kernel"]
    for n in names + measure:
        assert hasattr(lib, n), n
    assert sorted(K.SIGNATURES) == sorted(names + measure)


def test_status_strings():
    assert lib.kvattn_status_string(0) == b"ok"
    for s in range(1, 5):
        assert lib.kvattn_status_string(s) not in (b"ok", b"unknown status")
    assert lib.kvattn_status_string(99) == b"unknown status"


P = ctypes.c_void_p(16)  # a non-null pointer the library never dereferences on a rejected call


def gqa(**kw):
    a = dict(q=P, k=P, v=P, bt=None, lens=P, out=P, lse=None, B=2, h=8, g=2, d=128, cache_len=64, bs=0, maxb=0,
             maxlen=64, scale=0.1, dtype=K.KVATTN_BF16, split=0, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.kvattn_gqa_decode(a["q"], a["k"], a["v"], a["bt"], a["lens"], a["out"], a["lse"], a["B"], a["h"],
                                 a["g"], a["d"], a["cache_len"], a["bs"], a["maxb"], a["maxlen"], a["scale"],
                                 a["dtype"], a["split"], a["ws"], a["wsb"], a["stream"])


def mla(**kw):
    a = dict(q=P, c=P, bt=None, lens=P, out=P, lse=None, B=2, h=128, dc=512, dr=64, cache_len=64, bs=0, maxb=0,
             maxlen=64, scale=0.1, dtype=K.KVATTN_BF16, split=0, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.kvattn_mla_decode(a["q"], a["c"], a["bt"], a["lens"], a["out"], a["lse"], a["B"], a["h"], a["dc"],
                                 a["dr"], a["cache_len"], a["bs"], a["maxb"], a["maxlen"], a["scale"], a["dtype"],
                                 a["split"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(q=None), K.KVATTN_ERR_INVALID),
        (dict(v=None), K.KVATTN_ERR_INVALID),
        (dict(lens=None), K.KVATTN_ERR_INVALID),
        (dict(out=None), K.KVATTN_ERR_INVALID),
        (dict(B=0), K.KVATTN_ERR_INVALID),
        (dict(g=3), K.KVATTN_ERR_INVALID),          # h % g != 0
        (dict(g=0), K.KVATTN_ERR_INVALID),
        (dict(d=64), K.KVATTN_ERR_UNSUPPORTED),
        (dict(d=0), K.KVATTN_ERR_INVALID),
        (dict(dtype=7), K.KVATTN_ERR_INVALID),
        (dict(scale=float("nan")), K.KVATTN_ERR_INVALID),
        (dict(h=256, g=1, dtype=K.KVATTN_BF16), K.KVATTN_ERR_UNSUPPORTED),
        (dict(h=128, g=1, dtype=K.KVATTN_F32), K.KVATTN_ERR_UNSUPPORTED),
        (dict(maxlen=65), K.KVATTN_ERR_INVALID),    # beyond the contiguous cache
        (dict(maxlen=-1), K.KVATTN_ERR_INVALID),
        (dict(cache_len=0, maxlen=0), K.KVATTN_ERR_INVALID),
        (dict(split=100), K.KVATTN_ERR_INVALID),    # not a multiple of 64
        (dict(split=-64), K.KVATTN_ERR_INVALID),
        (dict(bt=P, bs=0, maxb=4), K.KVATTN_ERR_INVALID),   # paged without a block size
        (dict(bt=P, bs=16, maxb=0), K.KVATTN_ERR_INVALID),
        (dict(bt=P, bs=16, maxb=2, maxlen=64), K.KVATTN_ERR_INVALID),  # 2 blocks of 16 < 64 tokens
        (dict(B=70000), K.KVATTN_ERR_UNSUPPORTED),  # beyond the grid's batch dimension
    ],
)
def test_gqa_rejects_bad_arguments_before_touching_the_gpu(kw, status):
    assert gqa(**kw) == status
    assert lib.kvattn_last_error() != b""


def test_gqa_workspace_required_when_split():
    # 4096 tokens at split 256 means 16 splits: a workspace is required.
    need = lib.kvattn_gqa_workspace_bytes(2, 8, 2, 128, 4096, 0, 256, K.KVATTN_BF16)
    assert need == 2 * 8 * 16 * 129 * 4  # 16 splits of partial outputs and log-sum-exps
    assert gqa(cache_len=4096, maxlen=4096, split=256, ws=None, wsb=0) == K.KVATTN_ERR_WORKSPACE
    # the call needs the bytes of its own layout: bf16 partial outputs (fp32 ones for an fp32 call)
    need_bf16 = 2 * 8 * 16 * (128 * 2 + 4)
    assert gqa(cache_len=4096, maxlen=4096, split=256, ws=P, wsb=need_bf16 - 1) == K.KVATTN_ERR_WORKSPACE
    assert gqa(cache_len=4096, maxlen=4096, split=256, ws=P, wsb=need - 1, dtype=K.KVATTN_F32) == \
        K.KVATTN_ERR_WORKSPACE
    # a single split needs none
    assert lib.kvattn_gqa_workspace_bytes(2, 8, 2, 128, 256, 0, 256, K.KVATTN_BF16) == 0
    assert lib.kvattn_gqa_workspace_bytes(2, 8, 3, 128, 256, 0, 0, K.KVATTN_BF16) == ctypes.c_size_t(-1).value


def test_split_planner():
    f = lib.kvattn_gqa_split_tokens
    assert f(2, 8, 2, 4096, 0, 192) == 192          # an explicit request wins
    for B, h, g, S in [(16, 32, 8, 8192), (8, 64, 64, 8192), (64, 64, 8, 8192), (64, 64, 1, 8192),
                       (128, 64, 8, 32768), (1, 8, 2, 512), (3, 4, 4, 1)]:
        for bs in (0, 16):
            s = f(B, h, g, S, bs, 0)
            assert s > 0 and s % 64 == 0 and s <= max(S + 63, 256)
            if bs:
                assert s <= 2048  # paged: bounded split length for ragged sequences
    # contiguous: fewest splits giving 2 workgroups per CU (512 in all) on the measured shapes
    assert f(16, 32, 8, 8192, 0, 0) == 2048       # 128 (sequence, KV head) units x 4 splits
    assert f(64, 64, 1, 8192, 0, 0) == 1024       # 64 units x 8
    assert f(64, 64, 8, 8192, 0, 0) == 8192       # 512 units, no split
    assert f(8, 64, 64, 8192, 0, 0) == 8192
    assert f(128, 64, 8, 32768, 16, 0) == 2048    # paged
    # at least 16 r tokens per split (r = h / g partial rows), unless that leaves fewer than two
    # workgroups per CU: then at least 256
    assert f(4, 64, 1, 8192, 0, 0) == 256         # 16 r = 1024 would give 32 workgroups
    assert f(1, 64, 1, 131072, 0, 0) == 256       # one long MQA sequence: 512 splits
    assert f(1, 64, 1, 131072, 16, 0) == 256      # paged
    assert f(1, 32, 1, 131072, 0, 0) == 256       # 16 r = 512 would give 256
    assert f(2, 64, 1, 1 << 20, 0, 0) == 4096     # long enough: 256 splits each, above the floor
    m = lib.kvattn_mla_split_tokens
    assert m(32, 128, 8192, 0, 0) == 1024     # 32 x 8192 tokens over 256 compute units
    assert m(32, 128, 16384, 64, 0) == 2048
    assert m(1, 128, 1000, 0, 0) == 256       # shortest chosen piece
    assert m(32, 128, 8192, 0, 512) == 512


def _mla_workspace(batch, heads, pieces, d_c=512):
    def up(x):
        return (x + 255) // 256 * 256

    # bf16 partial outputs, fp32 partial log-sum-exps, the plan's pieces, per-sequence ranges, counts
    return up(pieces * heads * d_c * 2) + up(pieces * heads * 4) + up(pieces * 16) + up(batch * 8) + 256


def test_mla_workspace_bytes():
    # pieces of the device-side plan: at most max(256, batch) (one per compute unit, or per sequence),
    # each with bf16 partial outputs (512 wide) and fp32 log-sum-exps for every head, plus the plan itself
    assert lib.kvattn_mla_workspace_bytes(32, 128, 512, 64, 8192, 0, 0, K.KVATTN_BF16) == _mla_workspace(32, 128, 256)
    assert lib.kvattn_mla_workspace_bytes(300, 128, 512, 64, 64, 0, 0, K.KVATTN_BF16) == _mla_workspace(300, 128, 300)
    # a requested piece length bounds the pieces by ceil(max_seq_len / split) per sequence
    assert lib.kvattn_mla_workspace_bytes(32, 128, 512, 64, 1024, 0, 1024, K.KVATTN_BF16) == _mla_workspace(32, 128, 32)
    assert lib.kvattn_mla_workspace_bytes(32, 128, 512, 64, 1025, 0, 1024, K.KVATTN_BF16) == _mla_workspace(32, 128, 64)
    assert lib.kvattn_mla_workspace_bytes(32, 128, 512, 64, 1024, 0, 100, K.KVATTN_BF16) == ctypes.c_size_t(-1).value


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(q=None), K.KVATTN_ERR_INVALID),
        (dict(c=None), K.KVATTN_ERR_INVALID),
        (dict(B=0), K.KVATTN_ERR_INVALID),
        (dict(dc=256), K.KVATTN_ERR_UNSUPPORTED),
        (dict(dr=32), K.KVATTN_ERR_UNSUPPORTED),
        (dict(h=100), K.KVATTN_ERR_UNSUPPORTED),
        (dict(h=256), K.KVATTN_ERR_UNSUPPORTED),
        (dict(dtype=K.KVATTN_F32), K.KVATTN_ERR_UNSUPPORTED),
        (dict(maxlen=100), K.KVATTN_ERR_INVALID),
        (dict(split=32), K.KVATTN_ERR_INVALID),
        (dict(bt=P, bs=0, maxb=4), K.KVATTN_ERR_INVALID),
        (dict(cache_len=8192, maxlen=8192, split=256), K.KVATTN_ERR_WORKSPACE),
        (dict(), K.KVATTN_ERR_WORKSPACE),  # the plan always needs a workspace
    ],
)
def test_mla_rejects_bad_arguments_before_touching_the_gpu(kw, status):
    assert mla(**kw) == status
    assert lib.kvattn_last_error() != b""


def test_python_binding_rejects_cpu_tensors():
    import torch

    q = torch.zeros(1, 8, 128)
    kv = torch.zeros(1, 2, 16, 128)
    with pytest.raises(ValueError):
        K.gqa_decode(q, kv, kv, torch.zeros(1, dtype=torch.int32), 0.1)


def test_time_next_kernel_arms_both_events_or_none():
    """The timing hook only stores the two event handles; a half-armed pair is rejected on the host."""
    fake = ctypes.c_void_p(0x1000)
    assert lib.kvattn_time_next_kernel(fake, None) == K.KVATTN_ERR_INVALID
    assert lib.kvattn_time_next_kernel(None, fake) == K.KVATTN_ERR_INVALID
    assert lib.kvattn_time_next_kernel(None, None) == K.KVATTN_OK
    # A rejected decode call consumes (disarms) an armed pair without launching anything.
    assert lib.kvattn_time_next_kernel(fake, fake) == K.KVATTN_OK
    st = lib.kvattn_gqa_decode(None, None, None, None, None, None, None, 1, 8, 2, 128, 16, 0, 0, 16, 0.1,
                               K.KVATTN_BF16, 0, None, 0, None)
    assert st == K.KVATTN_ERR_INVALID


def test_clock_hook_checks_alignment_and_python_side_tensor():
    """The MLA clock hook stores a device pointer only; a misaligned one is rejected, and the binding
    refuses tensors that are not contiguous CUDA int64 of at least 4 elements."""
    import torch

    assert lib.kvattn_clock_next_mla(ctypes.c_void_p(0x1004)) == K.KVATTN_ERR_INVALID
    assert lib.kvattn_clock_next_mla(ctypes.c_void_p(0x1000)) == K.KVATTN_OK
    assert lib.kvattn_clock_next_mla(None) == K.KVATTN_OK
    with pytest.raises(ValueError):
        K.clock_next_mla(torch.zeros(4, dtype=torch.int64))
    assert K.shader_clock_ghz(torch.tensor([100, 10, 2100, 110])) == pytest.approx(2.0)


def test_noalloc_rejects_calls_beyond_its_scratch_before_touching_the_gpu():
    """A call whose partials exceed the fixed scratch fails on the host, with a message that says so."""
    cap = K.NOALLOC_SCRATCH_BYTES
    # 4 sequences x 128 heads x 1024 splits of 64 tokens x (2 x 128 + 4) bytes = 136 MB > 128 MiB
    B, h, g, S = 4, 128, 1, 65536
    assert B * h * (S // 64) * (2 * 128 + 4) > cap
    st = lib.kvattn_gqa_decode_noalloc(P, P, P, None, P, P, None, B, h, g, 128, S, 0, 0, S, 0.1, 0, K.KVATTN_BF16, 64,
                                       None)
    assert st == K.KVATTN_ERR_WORKSPACE
    assert b"no-allocation" in lib.kvattn_last_error()
    # argument errors come first, as for the other entry points
    st = lib.kvattn_gqa_decode_noalloc(P, P, P, None, P, P, None, B, h, 3, 128, S, 0, 0, S, 0.1, 0, K.KVATTN_BF16, 64,
                                       None)
    assert st == K.KVATTN_ERR_INVALID
