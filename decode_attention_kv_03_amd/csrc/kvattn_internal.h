// Host <-> kernel interface of libkvattn (not part of the public C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/kvattn.h"

namespace kvattn {

constexpr int kHeadDim = 128;      // GQA head width the kernels are built for
constexpr int kMlaLatent = 512;    // MLA latent width d_c
constexpr int kMlaRope = 64;       // MLA decoupled RoPE width
constexpr int kMlaRow = kMlaLatent + kMlaRope;
constexpr int kMaxGroupF32 = 64;   // largest h/g of the fp32 kernel
constexpr int kMaxGroupBf16 = 128; // largest h/g of the bf16 kernel
constexpr int kMaxMlaHeads = 128;
constexpr float kLog2eHost = 1.4426950408889634f;
constexpr int kPersistentWorkgroups = 512;  // persistent GQA grid: two resident workgroups per compute unit

// One decode call, as the kernels see it.  Cache addressing:
//   contiguous: row (b, j, t) at ((b * g + j) * cache_len + t) * width
//   paged:      block = table[b * max_blocks + t / block_size];
//               row at ((block * g + j) * block_size + t % block_size) * width
// (MLA uses g = 1.)
struct DecodeArgs {
  const void* q;
  const void* k;            // GQA K, or the MLA latent rows
  const void* v;            // GQA V (unused by MLA)
  const float* k_scale;     // fp8 GQA: per-KV-head scale of the K codes [g] (unused otherwise)
  const float* v_scale;     // fp8 GQA: per-KV-head scale of the V codes [g]
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* out;
  float* lse;               // may be null
  float* part_o;            // GQA: [B, h, n_split, d_v] fp32 partial outputs (normalised), null if n_split == 1;
                            // MLA: bf16, per piece (below)
  float* part_lse;          // [B, h, n_split] log2-domain log-sum-exp of each split
  int32_t batch;
  int32_t num_q_heads;      // h
  int32_t num_kv_heads;     // g (1 for MLA)
  int32_t group;            // h / g
  int64_t cache_len;        // contiguous: tokens per (b, j) row block; paged: number of blocks
  int32_t block_size;       // 0: contiguous
  int32_t block_shift;      // paged: log2(block_size) when it is a power of two, else -1
  int32_t max_blocks;       // paged: block_table row length
  int32_t len_cap;          // device lengths are clamped to [0, len_cap]
  int32_t window;           // GQA sliding window: attend to the last `window` tokens (0: all)
  int32_t split_tokens;     // tokens per split (multiple of 64)
  int32_t n_split;          // splits per sequence in the grid
  float scale_log2;         // softmax scale * log2(e): scores are kept in log2 units
  // MLA work plan, written on the device by the plan kernel:
  //   pieces[q] = (sequence, first token, end token, 1 if it is the sequence's only piece)
  //   seq_pieces[b] = (first piece, number of pieces); plan_count = {pieces, piece length}
  // Partials of piece q, head i: part_o[(q * h + i) * d_v] (bf16 for MLA), part_lse[q * h + i].
  const int4* pieces;
  const int2* seq_pieces;
  const int32_t* plan_count;
  int32_t max_pieces;       // grid bound: the plan never makes more pieces
  // Reconstruct-then-attend MLA: k and v hold the reconstructed per-head rows
  // [B, h, rec_len, 128]; `rope` is the latent cache [B, cache_len, 576],
  // whose columns 512.. hold the shared RoPE key.
  const void* rope;
  int32_t rec_len;
  // GQA work list of the persistent split kernel (null: one workgroup per
  // split), written on the device by the plan kernel (gqa_plan.hip):
  //   items[k] = (unit b * g + j, split, first token, end token), k < items_ctl[0];
  //   items_ctl[1] = the claim counter (zero when the split kernel starts).
  const int4* items;
  int32_t* items_ctl;
  // Measurement only (MLA): when non-null, the first wave of workgroup 0
  // stores {s_memtime, s_memrealtime} at the start and at the end of its tile
  // loop here (four uint64 values).
  uint64_t* clock_stamps;
};

// One batched per-head projection: for outer index o, head i and row m,
//   y[o, i, m, :] = x[o, i, m, :] W^(i)    (W^(i) [k_dim, n_dim] row-major at w + i * w_head)
// or, with w_transposed, x W^(i)^T (W^(i) [n_dim, k_dim]).  bf16, strides in elements.
struct ProjectArgs {
  const uint16_t* x;
  const uint16_t* w;
  uint16_t* y;
  int32_t outer, heads, rows, k_dim, n_dim;
  int64_t x_outer, x_head, x_row;
  int64_t w_head;
  int64_t y_outer, y_head, y_row;
  int32_t m_tiles, n_tiles;  // 128-row and 128-column tiles of y
  bool w_transposed;
};

// Arguments of the MLA plan kernel.
struct MlaPlanArgs {
  const int32_t* seq_lens;
  int32_t batch;
  int32_t len_cap;
  int32_t work_items;       // target number of pieces when the piece length is chosen
  int32_t min_chunk;        // shortest chosen piece length
  int32_t fixed_chunk;      // > 0: use this piece length instead
  int4* pieces;
  int2* seq_pieces;
  int32_t* plan_count;
};

// Arguments of the GQA plan kernel: the work list of the persistent split
// kernel for a call of `units` = batch * g (sequence, KV head) pairs cut into
// splits of `split` tokens (at most n_split per pair).
struct GqaPlanArgs {
  const int32_t* seq_lens;
  int32_t batch;
  int32_t g;
  int32_t len_cap;
  int32_t window;
  int32_t split;
  int32_t n_split;
  int4* items;
  int32_t* ctl;             // [0]: number of items, [1]: claim counter (set to 0)
};

// Optional events recorded when a launch's kernel starts and ends (null: none).
struct LaunchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// Where a call's split-K workspace comes from: the caller's buffer (ptr,
// bytes), or, when `resolve` is set, the library's fixed scratch of `bytes`
// bytes, looked up through `resolve` only after the call's size checks pass.
struct Workspace {
  void* ptr;
  size_t bytes;
  kvattn_status (*resolve)(void** ptr);
};

// kvattn_gqa_decode_window with its workspace taken from `ws` (api.cpp).
kvattn_status gqa_decode_with(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                              const int32_t* seq_lens, void* out, float* lse, int32_t batch, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int64_t cache_len, int32_t block_size,
                              int32_t max_blocks_per_seq, int32_t max_seq_len, float scale, int32_t window,
                              kvattn_dtype dtype, int32_t split_tokens, const Workspace& ws, void* stream);
// Record a failure (printf-style detail with up to two integers) / a HIP error as the thread's last error.
kvattn_status report(kvattn_status s, const char* what, long long a = 0, long long b = 0);
kvattn_status report_hip(hipError_t e, const char* what);

hipError_t launch_gqa_f32(const DecodeArgs& a, hipStream_t stream, const LaunchEvents& ev);
hipError_t launch_gqa_bf16(const DecodeArgs& a, hipStream_t stream, const LaunchEvents& ev);
hipError_t launch_gqa_fp8(const DecodeArgs& a, hipStream_t stream, const LaunchEvents& ev);
hipError_t launch_mla_bf16(const DecodeArgs& a, hipStream_t stream, const LaunchEvents& ev);
hipError_t launch_mla_plan(const MlaPlanArgs& p, hipStream_t stream);
hipError_t launch_gqa_plan(const GqaPlanArgs& p, hipStream_t stream);
hipError_t launch_mla_merge_pieces(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_latent_project(const ProjectArgs& p, hipStream_t stream);
// The same projection for the naive MLA form's K and V rebuild (transposed
// weights stacked over an even number of heads of 128 columns, y_head room
// for `rows` rounded up to 256: whole 256-row tiles are written), else as above.
hipError_t launch_latent_rebuild(const ProjectArgs& p, hipStream_t stream);
hipError_t launch_mla_explicit_attend(const DecodeArgs& a, hipStream_t stream, const LaunchEvents& ev);
// W^(i) [rows, cols] -> W^(i)^T [cols, rows] for every head (bf16; rows, cols multiples of 64).
hipError_t launch_transpose_heads(const void* src, void* dst, int heads, int rows, int cols, hipStream_t stream);
hipError_t launch_hbm_read_probe(const void* buf, int64_t n16, uint32_t* sink, int workgroups, hipStream_t stream);
// Log-sum-exp merge of the per-split GQA partials into out/lse (d_v = 128).
hipError_t launch_merge(const DecodeArgs& a, bool out_bf16, hipStream_t stream);

}  // namespace kvattn
