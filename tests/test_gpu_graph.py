"""Decode calls captured in a HIP graph (torch.cuda.CUDAGraph) replay like eager calls.

The library allocates, frees and synchronises nothing, and issues no memset,
so a call (split kernel, log-sum-exp merge and, for MLA, the plan kernel) can
be captured by a serving loop.  Each test captures one call with preallocated
outputs and workspace, then replays it several times with new queries
written in place and eager work on the same stream between replays, and
requires every replay to equal an eager call on the same inputs bit for bit
(the kernels are deterministic), and the last one to match the fp64 oracle.
"""

import numpy as np
import pytest
import torch

import oracle
from decode_attention_kv_03_amd import gqa_decode, mla_decode
from decode_attention_kv_03_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ATOL, RTOL = 2e-2, 1e-2
WS_BYTES = 64 << 20


def setup_module(_):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def note(msg):
    print(f"\n[gpu-test] {msg}", flush=True)


def _replay_matches_eager(call, q, n_replays=3, seed=0):
    """Capture call(q, out, lse, ws) once; replay with fresh q each time; compare with eager calls."""
    out_g, lse_g = call.alloc()
    ws_g = torch.empty(WS_BYTES, dtype=torch.uint8, device=DEV)
    out_e, lse_e = call.alloc()
    ws_e = torch.empty(WS_BYTES, dtype=torch.uint8, device=DEV)
    call(q, out_g, lse_g, ws_g)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(q, out_g, lse_g, ws_g)
    torch.cuda.synchronize()
    gen = torch.Generator(DEV).manual_seed(seed)
    for r in range(n_replays):
        q.copy_(torch.randn(q.shape, generator=gen, device=DEV, dtype=torch.float32).to(q.dtype))
        g.replay()
        call(q, out_e, lse_e, ws_e)  # eager work on the same stream between the replays
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {r}: output differs from the eager call"
        assert torch.equal(lse_g, lse_e), f"replay {r}: lse differs from the eager call"
    return out_g


class _Gqa:
    def __init__(self, x, w, split):
        self.x, self.w, self.split = x, w, split

    def alloc(self):
        B, h, d = self.x["q"].shape
        return (torch.empty((B, h, d), dtype=self.x["q"].dtype, device=DEV),
                torch.empty((B, h), dtype=torch.float32, device=DEV))

    def __call__(self, q, out, lse, ws):
        x = self.x
        gqa_decode(q, x["k"], x["v"], x["seq_lens"], self.w.scale, block_table=x["block_table"], out=out, lse=lse,
                   split_tokens=self.split, workspace=ws)


class _Mla:
    def __init__(self, x, w):
        self.x, self.w = x, w

    def alloc(self):
        B, h, _ = self.x["q"].shape
        return (torch.empty((B, h, self.w.d_latent), dtype=self.x["q"].dtype, device=DEV),
                torch.empty((B, h), dtype=torch.float32, device=DEV))

    def __call__(self, q, out, lse, ws):
        x = self.x
        mla_decode(q, x["cache"], x["seq_lens"], self.w.scale, block_table=x["block_table"], out=out, lse=lse,
                   workspace=ws)


def test_gqa_split_call_replays_in_a_graph():
    lens = [3000, 777, 1, 2049]
    w = W.shrink(W.WORKLOADS["llama3_8b_gqa_h32_g8_b16_s8192"], batch=len(lens), seq_len=max(lens))
    note(f"graph gqa bf16 h32 g8 lens={lens} split=512")
    x = W.make_gqa_inputs(w, DEV, lens=lens)
    out = _replay_matches_eager(_Gqa(x, w, 512), x["q"])
    ref, _ = oracle.gqa_decode(*(W.host_view(x[k]) for k in ("q", "k", "v")), lens, w.scale, bf16=True)
    got = out.double().cpu().numpy()
    assert np.all(np.abs(got - ref) <= ATOL + RTOL * np.abs(ref))


def test_mla_call_replays_in_a_graph():
    lens = [700, 33, 1500]
    w = W.shrink(W.WORKLOADS["deepseek_v2_mla_h128_b32_s8192"], batch=len(lens), seq_len=max(lens))
    note(f"graph mla h128 lens={lens}")
    x = W.make_mla_inputs(w, DEV, lens=lens)
    out = _replay_matches_eager(_Mla(x, w), x["q"])
    ref, _ = oracle.mla_absorbed_decode(W.host_view(x["q"]), W.host_view(x["cache"]), lens, w.scale, bf16=True)
    got = out.double().cpu().numpy()
    assert np.all(np.abs(got - ref) <= ATOL + RTOL * np.abs(ref))


def test_persistent_gqa_call_replays_in_a_graph():
    """The persistent form's claim counter sits in the workspace and is reset by its plan kernel on every replay."""
    from tests.test_gpu_edges import gqa_reference
    from tests.test_gpu_persistent import PERSISTENT_SLOTS, n_split

    B, h, g, S, bs, split = 40, 32, 8, 3000, 16, 64
    rng = np.random.default_rng(17)
    lens = np.concatenate([[0, 1, 64, S], rng.integers(0, S + 1, B - 4)]).astype(np.int32)
    w = W.GqaWorkload("graph_persistent", B, h, g, 128, S, "bf16", 23, 1 / np.sqrt(128), block_size=bs)
    x = W.make_gqa_inputs(w, DEV, lens=lens, poison_tail=True)
    max_len = x["block_table"].shape[1] * bs
    assert B * g * n_split(w, max_len, split) > PERSISTENT_SLOTS, "case does not reach the persistent form"
    note(f"graph gqa persistent form: paged bs={bs} B={B} h={h} g={g} split={split}")
    out = _replay_matches_eager(_Gqa(x, w, split), x["q"], n_replays=4, seed=3)
    ref, _ = gqa_reference(x)
    got = out.double().cpu().numpy()
    assert np.all(np.abs(got - ref) <= ATOL + RTOL * np.abs(ref))
