/*
 * kvattn.h -- C ABI of libkvattn: single-token decode attention that reads a
 * KV cache, on AMD Instinct MI355X (gfx950).
 *
 * The operation.  One decode step gives every sequence b one new query per
 * head; each head attends over the tokens already in the cache:
 *
 *     s_t = scale * <q, k_t>,  p = softmax(s),  o = sum_t p_t v_t,
 *     lse = log sum_t exp(s_t),       for t < seq_lens[b].
 *
 * The pages this library is written from never print that formula; they
 * describe a decode step as computing scores and then attention times V for
 * every query head ("MQA, GQA, and MLA", section 4 "The second benefit of
 * GQA").  The textbook scaled softmax above is the reading taken here.
 * No causal mask applies: the step's own key and value are expected to be in
 * the cache already.
 *
 * Two forms:
 *
 *  - Grouped-query decode (kvattn_gqa_decode).  h query heads share g cached
 *    K/V heads; query head i reads KV head i / (h/g), by index, never by
 *    copying ("MQA, GQA, and MLA", section 8 "Implementation notes", and the
 *    section 3 figure).  g = h is MHA and g = 1 is MQA (section 2).
 *
 *  - Absorbed multi-head latent attention decode (kvattn_mla_decode).  Each
 *    cached token is one row [c (d_latent) | k^R (d_rope)]; every head scores
 *    its absorbed query [q^C W_uk^T | q^R] against the whole row and
 *    accumulates its output from the c part only, so the output stays in
 *    latent space and W_uv is applied by the caller ("MQA, GQA, and MLA",
 *    section 5 "MLA, mechanically"; "Why GQA's KV Cache Savings Don't Fully
 *    Reduce TPOT", section "What Makes MLA Different").
 *
 * Conventions shared by every entry point:
 *
 *  - Pointers named q, k_cache, v_cache, cache, block_table, seq_lens, out,
 *    lse and workspace are DEVICE pointers on the current HIP device.  The
 *    caller owns and allocates all of them; the library never allocates,
 *    frees or synchronises.
 *  - Dense tensors are row-major and contiguous with the shapes given below.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL is the null
 *    stream).  A call returns after enqueueing its kernels.
 *  - Every argument is checked on the host before any HIP call; a bad
 *    argument returns a status and enqueues nothing.  kvattn_last_error()
 *    then describes the problem (thread-local).
 *  - Device-side preconditions are not checked on the host because they live
 *    in device memory: 0 <= seq_lens[b]; block table entries for the tokens a
 *    sequence uses lie in [0, num_blocks).  The kernels never read out of
 *    bounds when they are violated: lengths are clamped to [0, max_seq_len]
 *    and to the cache capacity, and a token whose table entry is out of
 *    range is read from an in-bounds stand-in row instead (zeros in the fp32
 *    GQA kernel; the pool's first rows in the bf16 and fp8 GQA kernels and in
 *    MLA), which still takes part in that sequence's softmax.  That
 *    sequence's output is then unspecified (but finite for finite cache
 *    contents); no other sequence's output is affected.
 *  - A sequence with length 0 gets out = 0 and lse = -inf.
 *  - Accumulation is fp32 for every input dtype.  `out` has the input dtype
 *    (rounded to nearest even for bf16); `lse` is fp32, natural log.
 *  - Split-K: a sequence's tokens are cut into splits of `split_tokens`
 *    tokens that run in parallel and are combined by a log-sum-exp merge.
 *    split_tokens = 0 lets the library choose; otherwise it must be a
 *    positive multiple of KVATTN_SPLIT_ALIGN.  Results do not depend on it
 *    beyond rounding: splits hand the merge partial outputs rounded to bf16
 *    (fp32 for an fp32 GQA call); their log-sum-exps and the merge stay
 *    fp32.
 *    The workspace holds the per-split partial
 *    results (and, for MLA, the work plan described at kvattn_mla_decode);
 *    its size comes from the matching *_workspace_bytes() call with the same
 *    shape arguments, and may be 0 for GQA (then workspace may be NULL).
 *    Its contents need no initialisation.  One workspace serves one call at
 *    a time: calls that share it must be ordered (for example, on one
 *    stream).
 *  - A bf16 or fp8 GQA call with more than 2048 (sequence, KV head, split)
 *    slots, on a contiguous cache or a paged one whose block size is a power
 *    of two of at least 4 (bf16) or 8 (fp8) tokens, runs in a persistent
 *    form when the workspace it is given also holds a list of the splits
 *    that hold tokens (16 bytes per slot, after the partials: the size
 *    kvattn_gqa_workspace_bytes reports always leaves room for it).  A
 *    device-side kernel makes the list from seq_lens, and 512 resident
 *    workgroups take its entries from a counter kept in the workspace.  Each
 *    split is computed as in the one-workgroup-per-split form, so the
 *    results are identical.
 */
#ifndef KVATTN_H
#define KVATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVATTN_SPLIT_ALIGN 64

typedef enum kvattn_status {
  KVATTN_OK = 0,
  KVATTN_ERR_INVALID = 1,     /* null pointer, non-positive size, h % g != 0, bad split_tokens ... */
  KVATTN_ERR_UNSUPPORTED = 2, /* well-formed but not provided: head_dim != 128, MLA widths != 512 + 64 ... */
  KVATTN_ERR_WORKSPACE = 3,   /* workspace smaller than the *_workspace_bytes() answer */
  KVATTN_ERR_HIP = 4          /* a HIP call failed; kvattn_last_error() holds HIP's message */
} kvattn_status;

typedef enum kvattn_dtype {
  KVATTN_F32 = 0, /* IEEE binary32 */
  KVATTN_BF16 = 1 /* bfloat16 */
} kvattn_dtype;

/*
 * Grouped-query decode attention (GQA; MHA at g = h, MQA at g = 1).
 *
 *  q            [batch, num_q_heads, head_dim], dtype.
 *  k_cache,     contiguous cache (block_table == NULL):
 *  v_cache        [batch, num_kv_heads, cache_len, head_dim], dtype; token t
 *                 of sequence b, KV head j is row (b, j, t).
 *               paged cache (block_table != NULL):
 *                 [cache_len (= number of physical blocks), num_kv_heads,
 *                  block_size, head_dim], dtype; token t of sequence b lives
 *                 in block block_table[b * max_blocks_per_seq + t / block_size]
 *                 at slot t % block_size.  The pages ask only for fixed-size
 *                 blocks ("Compressing the KV Cache ...", section "KV-Cache
 *                 Management Guardrails"); this layout keeps one (block, KV
 *                 head) as block_size * head_dim contiguous elements.
 *  block_table  NULL, or int32 [batch, max_blocks_per_seq]; unused entries
 *               may hold anything (-1 by convention).
 *  seq_lens     int32 [batch]: tokens of each sequence to attend over.
 *  out          [batch, num_q_heads, head_dim], dtype.
 *  lse          NULL, or fp32 [batch, num_q_heads]: natural-log log-sum-exp
 *               of the scaled scores.
 *  max_seq_len  host-side upper bound on every seq_lens[b]; sizes the grid.
 *               For a contiguous cache it must not exceed cache_len; for a
 *               paged one, max_blocks_per_seq * block_size.
 *  scale        multiplier of q.k (1/sqrt(head_dim) for the usual choice).
 *  Supported: head_dim == 128; dtype f32 with h/g <= 64; dtype bf16 with
 *  h/g <= 128.
 */
kvattn_status kvattn_gqa_decode(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_table, const int32_t* seq_lens, void* out,
                                float* lse, int32_t batch, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim, int64_t cache_len,
                                int32_t block_size, int32_t max_blocks_per_seq,
                                int32_t max_seq_len, float scale, kvattn_dtype dtype,
                                int32_t split_tokens, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * Grouped-query decode with a sliding window: each sequence attends only to
 * its last `window` cached tokens, t in [max(0, seq_lens[b] - window),
 * seq_lens[b]) ("One dial, four settings": the full ladder's SWA row and the
 * sliding-window question, where a token outside the window is not attended
 * at all).  window = 0 attends to every token and is kvattn_gqa_decode.
 * Arguments and layouts are those of kvattn_gqa_decode (token indices and
 * block-table lookups stay absolute); the workspace kvattn_gqa_workspace_bytes
 * reports for the same arguments is enough.  window < 0 is KVATTN_ERR_INVALID.
 * A window's tokens are read from the multiple of 64 at or below its first;
 * with split_tokens = 0 the library may size the splits for the window
 * itself, the last split of a sequence then holding up to 63 tokens more.
 */
kvattn_status kvattn_gqa_decode_window(const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_table, const int32_t* seq_lens, void* out,
                                       float* lse, int32_t batch, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int64_t cache_len,
                                       int32_t block_size, int32_t max_blocks_per_seq,
                                       int32_t max_seq_len, float scale, int32_t window,
                                       kvattn_dtype dtype, int32_t split_tokens, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * kvattn_gqa_decode_window without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  The split-K partials go to a
 * scratch array of KVATTN_NOALLOC_SCRATCH_BYTES bytes that the library keeps
 * in device memory, one per GPU it runs on, from the first call on that GPU
 * until the process ends.  The call allocates, frees and clears nothing
 * (the partials need no initialisation); the first call on a device looks up
 * the array's address there, a host-side query.
 *
 * Arguments, layouts, results and errors are those of
 * kvattn_gqa_decode_window (window 0: every token), with the same split
 * planning, so the results equal that call's bit for bit.  A call whose
 * partials need more than KVATTN_NOALLOC_SCRATCH_BYTES (bf16: batch *
 * num_q_heads * splits * (2 * head_dim + 4) bytes when it splits; fp32: 4 *
 * head_dim + 4 per row and split) returns KVATTN_ERR_WORKSPACE before any HIP
 * call; kvattn_gqa_split_tokens gives the split size it would use.
 *
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (on different streams, or from different threads without ordering)
 * race on it and must not be issued together.
 */
#define KVATTN_NOALLOC_SCRATCH_BYTES (128u << 20)

kvattn_status kvattn_gqa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                        const int32_t* block_table, const int32_t* seq_lens, void* out, float* lse,
                                        int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                        int64_t cache_len, int32_t block_size, int32_t max_blocks_per_seq,
                                        int32_t max_seq_len, float scale, int32_t window, kvattn_dtype dtype,
                                        int32_t split_tokens, void* stream);

/*
 * Grouped-query decode over an FP8 KV cache.  Storing the cache in fp8 halves
 * its bytes, and a GQA cache quantises at the granularity of one KV head
 * ("Why GQA's KV Cache Savings Don't Fully Reduce TPOT", section "When the
 * Serving Engineer Doesn't Get to Choose").  The pages name no format or
 * scale convention; this library reads them as:
 *
 *  k_cache,     uint8 codes of the OCP 8-bit float E4M3 ("e4m3fn": bias 7,
 *  v_cache        3 mantissa bits, subnormals, codes 0x7F/0xFF NaN, largest
 *                 finite 448), with the shapes and addressing of
 *                 kvattn_gqa_decode (one byte per element).
 *  k_scale,     DEVICE fp32 [num_kv_heads]: a K code c of KV head j stands
 *  v_scale        for k_scale[j] * E4M3(c), a V code for v_scale[j] * E4M3(c).
 *  q, out       bfloat16, as in kvattn_gqa_decode; lse fp32 or NULL.
 *
 * Attention is that of kvattn_gqa_decode_window over the dequantised cache
 * (window 0: every token).  Codes are widened exactly to bfloat16 and the
 * scales are applied in fp32 (k_scale[j] to the softmax scale, v_scale[j] to
 * the output), so results match a dequantise-then-attend reference to fp32
 * accumulation order.  Supported: head_dim == 128, h/g <= 128.  The workspace
 * kvattn_gqa_workspace_bytes reports for the same arguments (any dtype) is
 * enough.  NULL scales are KVATTN_ERR_INVALID.
 */
kvattn_status kvattn_gqa_decode_fp8(const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                                    const float* v_scale, const int32_t* block_table, const int32_t* seq_lens,
                                    void* out, float* lse, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int64_t cache_len, int32_t block_size,
                                    int32_t max_blocks_per_seq, int32_t max_seq_len, float scale, int32_t window,
                                    int32_t split_tokens, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes kvattn_gqa_decode needs for these arguments (0 when no split is needed).
 * block_size is 0 for a contiguous cache (block_table == NULL) and the pool's block size for a
 * paged one: the split planner treats the two differently.  Returns (size_t)-1 for arguments
 * kvattn_gqa_decode would reject. */
size_t kvattn_gqa_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t max_seq_len, int32_t block_size,
                                  int32_t split_tokens, kvattn_dtype dtype);

/*
 * Absorbed MLA decode attention.
 *
 *  q            [batch, num_heads, d_latent + d_rope], dtype: absorbed queries
 *               [q^C W_uk^T | q^R] ("MQA, GQA, and MLA", section 5).
 *  cache        contiguous (block_table == NULL):
 *                 [batch, cache_len, d_latent + d_rope], dtype, rows
 *                 [c_t | k^R_t]; one row per token shared by all heads.
 *               paged (block_table != NULL):
 *                 [cache_len (= number of physical blocks), block_size,
 *                  d_latent + d_rope], addressed as for kvattn_gqa_decode.
 *  out          [batch, num_heads, d_latent], dtype: o_i = sum_t p_t c_t.
 *  lse          NULL, or fp32 [batch, num_heads].
 *  scale        multiplier of the 576-wide dot product (1/sqrt(128 + 64)
 *               for DeepSeek-V2's head width plus RoPE width).
 *  Supported: dtype bf16, d_latent == 512, d_rope == 64, num_heads a
 *  multiple of 16 up to 128.
 *
 *  Work plan.  The call first enqueues a small kernel that reads seq_lens on
 *  the device and cuts every sequence into pieces of equal length (multiples
 *  of 32 tokens): with split_tokens = 0, the shortest piece length (at least
 *  256 tokens) that gives at most max(256, batch) pieces in all, so ragged
 *  batches keep every compute unit busy; otherwise at most split_tokens
 *  tokens per piece.  Each piece is one workgroup of the decode kernel;
 *  sequences with more than one piece are combined by a log-sum-exp merge.
 *  The plan lives in the workspace, which is therefore never empty.  With P
 *  the largest piece count the sizes allow, the workspace holds, each region
 *  starting at a multiple of 256 bytes: bf16 partial outputs [P, num_heads,
 *  d_latent], fp32 partial log2-sum-exps [P, num_heads], the pieces int32
 *  [P][4] = (sequence, first token, end token, 1 if it is its sequence's
 *  only piece), per sequence int32 [batch][2] = (first piece, piece count;
 *  an empty sequence keeps one empty piece), then int32 (number of pieces,
 *  piece length).  A sequence of n tokens cut for piece length t has
 *  ceil(n / t) pieces of ceil(n / count) tokens rounded up to 32 (the last
 *  one shorter).
 */
kvattn_status kvattn_mla_decode(const void* q, const void* cache, const int32_t* block_table,
                                const int32_t* seq_lens, void* out, float* lse, int32_t batch,
                                int32_t num_heads, int32_t d_latent, int32_t d_rope,
                                int64_t cache_len, int32_t block_size, int32_t max_blocks_per_seq,
                                int32_t max_seq_len, float scale, kvattn_dtype dtype,
                                int32_t split_tokens, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Workspace bytes kvattn_mla_decode needs for these arguments; (size_t)-1 if it would reject them. */
size_t kvattn_mla_workspace_bytes(int32_t batch, int32_t num_heads, int32_t d_latent,
                                  int32_t d_rope, int32_t max_seq_len, int32_t block_size,
                                  int32_t split_tokens, kvattn_dtype dtype);

/*
 * Per-head projection between MLA's latent space and a per-head space, on the
 * bf16 matrix cores (fp32 accumulation, bf16 result):
 *
 *     y[o][i][m][:] = x[o][i][m][:] . W^(i)            (w_transposed == 0)
 *     y[o][i][m][:] = x[o][i][m][:] . W^(i)^T          (w_transposed != 0)
 *
 * for every outer index o < outer, head i < heads and row m < rows.  W^(i)
 * starts at w + i * w_head_stride and is [k_dim, n_dim] row-major (the
 * layout of c W^(i) with c a row of k_dim latent values), or [n_dim, k_dim]
 * when transposed.  Row m of x for (o, i) starts at x + o * x_outer_stride +
 * i * x_head_stride + m * x_row_stride, and likewise for y; strides are in
 * elements.  This is the up-projection the absorbed form applies once to its
 * latent output, o_i = o_latent_i W_uv^(i) ("MQA, GQA, and MLA", section 5
 * "MLA, mechanically": v_i = c W_uv^(i), whose weights the absorbed form
 * moves past the attention sum); with x = q^C and W_uk transposed it forms
 * the absorbed query q^C_i W_uk^(i)^T, and kvattn_mla_explicit_decode uses
 * it to rebuild keys and values.
 *
 *  x, w, y      DEVICE pointers, bf16, 16-byte aligned; y must not overlap x or w.
 *  Supported:   dtype bf16, k_dim a multiple of 64, n_dim a multiple of 128,
 *               strides non-negative multiples of 8 elements, x_row_stride >=
 *               k_dim and y_row_stride >= n_dim (x_head_stride may be 0: one x
 *               shared by all heads).  rows == 0 enqueues nothing.
 */
kvattn_status kvattn_mla_project(const void* x, const void* w, void* y, int32_t outer, int32_t heads, int32_t rows,
                                 int32_t k_dim, int32_t n_dim, int64_t x_outer_stride, int64_t x_head_stride,
                                 int64_t x_row_stride, int64_t w_head_stride, int32_t w_transposed,
                                 int64_t y_outer_stride, int64_t y_head_stride, int64_t y_row_stride,
                                 kvattn_dtype dtype, void* stream);

/*
 * Non-absorbed ("reconstruct, then attend") MLA decode: the naive form the
 * pages set against absorption, which rebuilds per-head keys and values from
 * the latent cache and so turns it back into a cache of MHA's size before
 * attending ("One dial, four settings", "MLA - compress instead of shrink";
 * "MQA, GQA, and MLA", section 5 and exercise D of section 11, where the two
 * forms must agree).  Head i of sequence b computes
 *
 *     k_{i,t} = [c_t W_uk^(i) | k^R_t],   v_{i,t} = c_t W_uv^(i),
 *     s_t = scale * <[q^C_i | q^R_i], k_{i,t}>,  out_i = sum_t softmax(s)_t v_{i,t}
 *
 * over t < seq_lens[b], which equals kvattn_mla_decode on the absorbed query
 * followed by the W_uv up-projection (kvattn_mla_project), up to rounding.
 *
 *  q            [batch, num_heads, d_head + d_rope]: [q^C_i | q^R_i], bf16.
 *  cache        contiguous latent cache [batch, cache_len, d_latent + d_rope],
 *               rows [c_t | k^R_t], bf16 (as for kvattn_mla_decode).
 *  w_uk, w_uv   [num_heads, d_latent, d_head] and [num_heads, d_latent, d_v],
 *               bf16: k = c W_uk^(i), v = c W_uv^(i).
 *  out          [batch, num_heads, d_v], bf16; lse NULL or fp32 [batch, num_heads].
 *  workspace    kvattn_mla_explicit_workspace_bytes() bytes, 256-byte aligned:
 *               it holds both weights transposed ([num_heads, 128, d_latent]),
 *               the rebuilt keys (content part) and values,
 *               [batch, num_heads, R, 128] bf16 each with R = max_seq_len
 *               rounded up to a multiple of 256 (the naive form rebuilds every
 *               row below max_seq_len, in tiles of 256 rows; rows from
 *               max_seq_len on are never read), then the split partials.
 *  Supported: bf16, d_latent 512, d_rope 64, d_head = d_v = 128 (DeepSeek-V2's
 *  shapes).  The rebuilt rows are rounded to bf16 before attention, one more
 *  rounding than the absorbed path takes.
 */
kvattn_status kvattn_mla_explicit_decode(const void* q, const void* cache, const void* w_uk, const void* w_uv,
                                         const int32_t* seq_lens, void* out, float* lse, int32_t batch,
                                         int32_t num_heads, int32_t d_latent, int32_t d_rope, int32_t d_head,
                                         int32_t d_v, int64_t cache_len, int32_t max_seq_len, float scale,
                                         kvattn_dtype dtype, int32_t split_tokens, void* workspace,
                                         size_t workspace_bytes, void* stream);

/* Workspace bytes kvattn_mla_explicit_decode needs; (size_t)-1 if it would reject these sizes. */
size_t kvattn_mla_explicit_workspace_bytes(int32_t batch, int32_t num_heads, int32_t d_head, int32_t d_v,
                                           int32_t max_seq_len, int32_t split_tokens, kvattn_dtype dtype);

/* The split size (tokens per split) a call with these arguments uses (block_size 0 for a
 * contiguous cache, as for the workspace queries).  split_tokens = 0 asks for the library's choice:
 * for a contiguous GQA cache the fewest splits that still give every compute unit two resident
 * workgroups; for a paged one (ragged lengths assumed) about four workgroups per compute unit of
 * at most 2048 tokens each.  For MLA the piece length is chosen on the device from the actual
 * lengths (see kvattn_mla_decode); kvattn_mla_split_tokens returns the length chosen when every
 * sequence holds max_seq_len tokens. */
int32_t kvattn_gqa_split_tokens(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t max_seq_len, int32_t block_size, int32_t split_tokens);
int32_t kvattn_mla_split_tokens(int32_t batch, int32_t num_heads, int32_t max_seq_len,
                                int32_t block_size, int32_t split_tokens);

/* Static description of a status code. */
const char* kvattn_status_string(kvattn_status status);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* kvattn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVATTN_H */
