// C ABI of libkvattn: argument checks, split planning and kernel dispatch.
//
// Every check runs on the host before the first HIP call, so a rejected call
// touches no device state.  The library never allocates, frees or
// synchronises; it only enqueues kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdio>
#include <string>

#include "../../include/kvattn.h"
#include "../../include/kvattn_measure.h"
#include "kvattn_internal.h"
#include "plan.h"

namespace {

using namespace kvattn::plan;

thread_local std::string g_last_error;
// Events the next decode call on this thread records around its split-K kernel.
thread_local kvattn::LaunchEvents g_time_next;

kvattn::LaunchEvents take_timing_events() {
  const kvattn::LaunchEvents ev = g_time_next;
  g_time_next = kvattn::LaunchEvents{};
  return ev;
}

thread_local uint64_t* g_clock_next = nullptr;

uint64_t* take_clock_stamps() {
  uint64_t* const p = g_clock_next;
  g_clock_next = nullptr;
  return p;
}

kvattn_status fail(kvattn_status s, const char* fmt, long long a = 0, long long b = 0) {
  char buf[256];
  std::snprintf(buf, sizeof(buf), fmt, a, b);
  g_last_error = buf;
  return s;
}

kvattn_status ok() {
  g_last_error.clear();
  return KVATTN_OK;
}

constexpr int32_t kMaxGridYZ = 65535;  // largest y/z grid dimension the launches use

// Workspace regions of an MLA call: partial outputs (bf16), partial log-sum-exps (fp32), the plan's pieces,
// per-sequence piece ranges and the plan's counts, each 256-byte aligned.
struct MlaWorkspace {
  size_t part_o, part_lse, pieces, seq_pieces, plan_count, total;
};
MlaWorkspace mla_workspace(int64_t batch, int64_t heads, int64_t max_pieces, int64_t d_c) {
  MlaWorkspace w{};
  w.part_o = 0;
  w.part_lse = w.part_o + (size_t)round_up(max_pieces * heads * d_c * 2, 256);  // bf16 partial outputs
  w.pieces = w.part_lse + (size_t)round_up(max_pieces * heads * (int64_t)sizeof(float), 256);
  w.seq_pieces = w.pieces + (size_t)round_up(max_pieces * 16, 256);
  w.plan_count = w.seq_pieces + (size_t)round_up(batch * 8, 256);
  w.total = w.plan_count + 256;
  return w;
}


// Split-K partials: outputs of `part_elem` bytes per element, then one fp32 log-sum-exp per row.
size_t partial_bytes(int64_t batch, int64_t heads, int64_t nsplit, int64_t d_v, int64_t part_elem = 4) {
  if (nsplit <= 1) return 0;
  return (size_t)(batch * heads * nsplit * (d_v * part_elem + (int64_t)sizeof(float)));
}

kvattn_status check_split(int32_t split_tokens) {
  if (split_tokens < 0 || split_tokens % KVATTN_SPLIT_ALIGN != 0)
    return fail(KVATTN_ERR_INVALID, "split_tokens must be 0 or a positive multiple of 64 (got %lld)", split_tokens);
  return KVATTN_OK;
}

// log2(x) for a power of two x > 0, else -1.
int32_t pow2_shift(int32_t x) {
  if (x <= 0 || (x & (x - 1)) != 0) return -1;
  int32_t s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

kvattn_status check_cache_geometry(int64_t cache_len, int32_t block_size, int32_t max_blocks, int32_t max_seq_len,
                                   bool paged) {
  if (max_seq_len < 0) return fail(KVATTN_ERR_INVALID, "max_seq_len must be >= 0 (got %lld)", max_seq_len);
  if (max_seq_len > kMaxSeqLen)
    return fail(KVATTN_ERR_UNSUPPORTED, "max_seq_len %lld exceeds the supported %lld tokens", max_seq_len, kMaxSeqLen);
  if (cache_len < 1) return fail(KVATTN_ERR_INVALID, "cache_len must be >= 1 (got %lld)", cache_len);
  if (!paged) {
    if (max_seq_len > cache_len)
      return fail(KVATTN_ERR_INVALID, "max_seq_len %lld exceeds the contiguous cache length %lld", max_seq_len,
                  cache_len);
    return KVATTN_OK;
  }
  if (block_size < 1) return fail(KVATTN_ERR_INVALID, "block_size must be >= 1 for a paged cache (got %lld)", block_size);
  if (max_blocks < 1)
    return fail(KVATTN_ERR_INVALID, "max_blocks_per_seq must be >= 1 for a paged cache (got %lld)", max_blocks);
  if ((int64_t)max_seq_len > (int64_t)max_blocks * block_size)
    return fail(KVATTN_ERR_INVALID, "max_seq_len %lld exceeds max_blocks_per_seq * block_size = %lld", max_seq_len,
                (long long)max_blocks * block_size);
  return KVATTN_OK;
}

kvattn_status check_gqa(const void* q, const void* k, const void* v, const int32_t* lens, const void* out,
                        int32_t batch, int32_t h, int32_t g, int32_t d, kvattn_dtype dtype, float scale) {
  if (!q || !k || !v || !lens || !out) return fail(KVATTN_ERR_INVALID, "q, k_cache, v_cache, seq_lens and out must be non-null");
  if (batch < 1) return fail(KVATTN_ERR_INVALID, "batch must be >= 1 (got %lld)", batch);
  if (h < 1 || g < 1) return fail(KVATTN_ERR_INVALID, "head counts must be >= 1 (h=%lld, g=%lld)", h, g);
  if (h % g != 0) return fail(KVATTN_ERR_INVALID, "num_q_heads %lld is not a multiple of num_kv_heads %lld", h, g);
  if (d < 1) return fail(KVATTN_ERR_INVALID, "head_dim must be >= 1 (got %lld)", d);
  if (dtype != KVATTN_F32 && dtype != KVATTN_BF16) return fail(KVATTN_ERR_INVALID, "unknown dtype %lld", (int)dtype);
  if (!std::isfinite(scale)) return fail(KVATTN_ERR_INVALID, "scale must be finite");
  if (d != kvattn::kHeadDim) return fail(KVATTN_ERR_UNSUPPORTED, "head_dim %lld is not supported (only 128)", d);
  if (batch > kMaxGridYZ || g > kMaxGridYZ)
    return fail(KVATTN_ERR_UNSUPPORTED, "batch %lld and num_kv_heads %lld must be <= 65535", batch, g);
  const int32_t r = h / g;
  if (dtype == KVATTN_F32 && r > kvattn::kMaxGroupF32)
    return fail(KVATTN_ERR_UNSUPPORTED, "fp32 supports h/g <= 64 (got %lld)", r);
  if (dtype == KVATTN_BF16 && r > kvattn::kMaxGroupBf16)
    return fail(KVATTN_ERR_UNSUPPORTED, "bf16 supports h/g <= 128 (got %lld)", r);
  return KVATTN_OK;
}

kvattn_status check_mla(const void* q, const void* cache, const int32_t* lens, const void* out, int32_t batch,
                        int32_t h, int32_t d_c, int32_t d_r, kvattn_dtype dtype, float scale) {
  if (!q || !cache || !lens || !out) return fail(KVATTN_ERR_INVALID, "q, cache, seq_lens and out must be non-null");
  if (batch < 1) return fail(KVATTN_ERR_INVALID, "batch must be >= 1 (got %lld)", batch);
  if (h < 1) return fail(KVATTN_ERR_INVALID, "num_heads must be >= 1 (got %lld)", h);
  if (d_c < 1 || d_r < 0) return fail(KVATTN_ERR_INVALID, "bad MLA widths d_latent=%lld d_rope=%lld", d_c, d_r);
  if (dtype != KVATTN_F32 && dtype != KVATTN_BF16) return fail(KVATTN_ERR_INVALID, "unknown dtype %lld", (int)dtype);
  if (!std::isfinite(scale)) return fail(KVATTN_ERR_INVALID, "scale must be finite");
  if (d_c != kvattn::kMlaLatent || d_r != kvattn::kMlaRope)
    return fail(KVATTN_ERR_UNSUPPORTED, "MLA supports d_latent=512, d_rope=64 (got %lld, %lld)", d_c, d_r);
  if (dtype != KVATTN_BF16) return fail(KVATTN_ERR_UNSUPPORTED, "MLA supports bf16 only");
  if (batch > kMaxGridYZ) return fail(KVATTN_ERR_UNSUPPORTED, "batch %lld must be <= 65535", batch);
  if (h % 16 != 0 || h > kvattn::kMaxMlaHeads)
    return fail(KVATTN_ERR_UNSUPPORTED, "MLA supports num_heads a multiple of 16 up to 128 (got %lld)", h);
  return KVATTN_OK;
}

kvattn_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return KVATTN_ERR_HIP;
}

// Cache operands of a GQA call: element type, and the per-KV-head scales of an fp8 cache.
enum class CacheKind { kF32, kBf16, kFp8E4m3 };
struct GqaCache {
  const void* k;
  const void* v;
  const float* k_scale;
  const float* v_scale;
  CacheKind kind;
};

// Workspace of the persistent GQA form: the split partials (`partials`
// bytes), then the work list (one int4 per possible item), then its count and
// claim counter.  total = 0 when the call keeps one workgroup per split: an
// fp32 cache, a single split, a grid that fits in about two rounds of
// resident workgroups, or a paged layout whose full tiles need the LDS table
// (block size not a power of two, or below one copy instruction's rows: 4
// bf16 rows, 8 fp8 rows).
struct GqaPersistentLayout {
  size_t items, ctl, total;
};

GqaPersistentLayout gqa_persistent_layout(CacheKind kind, int64_t batch, int64_t g, int64_t nsplit, int32_t block_size,
                                          size_t partials) {
  GqaPersistentLayout l{0, 0, 0};
  const int64_t slots = batch * g * nsplit;
  const int32_t min_shift = kind == CacheKind::kFp8E4m3 ? 3 : 2;
  if (kind == CacheKind::kF32 || nsplit <= 1 || slots <= 4 * kvattn::kPersistentWorkgroups) return l;
  if (slots > INT32_MAX / 2) return l;  // the device plan counts items in 32-bit integers
  if (block_size > 0 && pow2_shift(block_size) < min_shift) return l;
  l.items = (size_t)round_up((int64_t)partials, 256);
  l.ctl = l.items + (size_t)round_up(slots * 16, 256);
  l.total = l.ctl + 256;
  return l;
}

// Geometry checks, split planning and launches shared by the GQA entry points
// (their operand checks have already run).
kvattn_status gqa_run(const kvattn::LaunchEvents& ev, const void* q, const GqaCache& cache,
                      const int32_t* block_table, const int32_t* seq_lens, void* out, float* lse, int32_t batch,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int64_t cache_len,
                      int32_t block_size, int32_t max_blocks_per_seq, int32_t max_seq_len, float scale,
                      int32_t window, int32_t split_tokens, const kvattn::Workspace& wsrc, void* stream) {
  kvattn_status st;
  if (window < 0) return fail(KVATTN_ERR_INVALID, "window must be >= 0 (0: attend to all tokens), got %lld", window);
  const bool paged = block_table != nullptr;
  if ((st = check_cache_geometry(cache_len, block_size, max_blocks_per_seq, max_seq_len, paged)) != KVATTN_OK)
    return st;
  if ((st = check_split(split_tokens)) != KVATTN_OK) return st;

  // Splits.  A window needs only the tokens from the 64-aligned token below
  // its start, at most window + 63 per sequence, so its splits are planned on
  // that span.  The automatic plan is not monotone in the span (a shorter
  // span can get more splits), so a window call never takes more splits than
  // the whole context would: the workspace kvattn_gqa_workspace_bytes reports
  // (it takes no window) then always suffices.
  const int32_t full_split = plan_gqa_split(batch, num_q_heads, num_kv_heads, max_seq_len, paged, split_tokens);
  const int32_t full_n = n_splits(max_seq_len, full_split);
  int32_t split = full_split, nsplit = full_n;
  bool absorb = false;  // the last split of a sequence may hold more than `split` tokens
  if (window > 0) {
    const int32_t span = (int32_t)std::min<int64_t>(max_seq_len, (int64_t)window + 63);
    split = plan_gqa_split(batch, num_q_heads, num_kv_heads, span, paged, split_tokens);
    nsplit = n_splits(span, split);
    if (nsplit > full_n) {
      split = (int32_t)round_up((span + full_n - 1) / full_n, KVATTN_SPLIT_ALIGN);
      nsplit = n_splits(span, split);
    }
    // The automatic plan may instead size the splits for the window itself,
    // the last split of a sequence also taking the up to 63 tokens of the
    // aligned start (every kernel ends a sequence's last split at its
    // length): an aligned 4096-token window in four splits then reads 16
    // tiles per split instead of 17.  Taken when that shortens the splits
    // without adding any, on grids of one workgroup per split (the
    // persistent form's work list cuts every split at `split` tokens).
    if (split_tokens == 0) {
      const int32_t wlen = std::min(max_seq_len, window);
      const int32_t s2 = plan_gqa_split(batch, num_q_heads, num_kv_heads, wlen, paged, 0);
      const int32_t n2 = n_splits(wlen, s2);
      if (s2 < split && n2 <= nsplit && (int64_t)n2 * s2 < span &&
          gqa_persistent_layout(cache.kind, batch, num_kv_heads, n2, paged ? block_size : 0, 0).total == 0) {
        split = s2;
        nsplit = n2;
        absorb = true;
      }
    }
  }
  // Partial outputs are fp32 for an fp32 cache and bf16 otherwise (the
  // workspace query sizes the fp32 layout, which bounds both).
  const size_t part_elem = cache.kind == CacheKind::kF32 ? sizeof(float) : sizeof(uint16_t);
  size_t need = partial_bytes(batch, num_q_heads, nsplit, head_dim, (int64_t)part_elem);
  // A grid of splits that would run in many rounds takes the persistent form
  // instead, with its work list after the partials, when the workspace holds
  // it (the bf16 partials leave room for it in the size the query reports).
  const GqaPersistentLayout pl =
      gqa_persistent_layout(cache.kind, batch, num_kv_heads, nsplit, paged ? block_size : 0, need);
  // (Its work list cuts every split at `split` tokens, so a plan whose last
  // split takes more keeps one workgroup per split.)
  const bool persistent =
      !absorb && pl.total > 0 && pl.total <= wsrc.bytes && (wsrc.resolve != nullptr || wsrc.ptr != nullptr);
  if (persistent) need = pl.total;
  void* workspace = wsrc.ptr;
  if (need > 0) {
    if (wsrc.resolve != nullptr) {
      // The library's own scratch: its size is checked before it is looked up.
      if (need > wsrc.bytes)
        return fail(KVATTN_ERR_WORKSPACE, "this call needs %lld bytes of scratch; the no-allocation entry point "
                    "holds %lld (use the entry point that takes a workspace)", (long long)need, (long long)wsrc.bytes);
      if ((st = wsrc.resolve(&workspace)) != KVATTN_OK) return st;
    } else if (workspace == nullptr || wsrc.bytes < need) {
      return fail(KVATTN_ERR_WORKSPACE, "workspace of %lld bytes needed, %lld given", (long long)need,
                  workspace == nullptr ? 0 : (long long)wsrc.bytes);
    }
  }

  kvattn::DecodeArgs a{};
  a.q = q;
  a.k = cache.k;
  a.v = cache.v;
  a.k_scale = cache.k_scale;
  a.v_scale = cache.v_scale;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.out = out;
  a.lse = lse;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_q_heads / num_kv_heads;
  a.cache_len = cache_len;
  a.block_size = paged ? block_size : 0;
  a.block_shift = paged ? pow2_shift(block_size) : -1;
  a.max_blocks = paged ? max_blocks_per_seq : 0;
  a.len_cap = max_seq_len;
  a.window = window;
  a.split_tokens = split;
  a.n_split = nsplit;
  a.scale_log2 = scale * kvattn::kLog2eHost;
  if (nsplit > 1) {
    // Partial outputs, then the fp32 log-sum-exps.
    const int64_t n_part = (int64_t)batch * num_q_heads * nsplit * head_dim;
    a.part_o = static_cast<float*>(workspace);
    a.part_lse = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + n_part * part_elem);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipErrorInvalidValue;
  if (persistent) {
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    kvattn::GqaPlanArgs p{};
    p.seq_lens = seq_lens;
    p.batch = batch;
    p.g = num_kv_heads;
    p.len_cap = max_seq_len;
    p.window = window;
    p.split = split;
    p.n_split = nsplit;
    p.items = reinterpret_cast<int4*>(ws + pl.items);
    p.ctl = reinterpret_cast<int32_t*>(ws + pl.ctl);
    a.items = p.items;
    a.items_ctl = p.ctl;
    e = kvattn::launch_gqa_plan(p, s);
    if (e != hipSuccess) return hip_status(e, "plan kernel launch");
  }
  switch (cache.kind) {
    case CacheKind::kF32: e = kvattn::launch_gqa_f32(a, s, ev); break;
    case CacheKind::kBf16: e = kvattn::launch_gqa_bf16(a, s, ev); break;
    case CacheKind::kFp8E4m3: e = kvattn::launch_gqa_fp8(a, s, ev); break;
  }
  if (e != hipSuccess) return hip_status(e, "split kernel launch");
  if (nsplit > 1) {
    e = kvattn::launch_merge(a, cache.kind != CacheKind::kF32, s);
    if (e != hipSuccess) return hip_status(e, "merge kernel launch");
  }
  return ok();
}

// Reconstruct-then-attend MLA: the two weights transposed ([h, 128, 512] bf16
// each, so that the projections read both operands row-wise), per-head K and
// V rows rebuilt from the latent cache ([B, h, R, 128] bf16 each, R =
// max_seq_len rounded up to the rebuild's 256-row tiles; rows from
// max_seq_len on are never read), then the split partials (bf16 outputs,
// fp32 log-sum-exps), each region 256-byte aligned.  Sizes in 128-bit
// arithmetic; total 0 when they overflow (the caller rejects it).
struct ExplicitWorkspace {
  size_t wt_k, wt_v, kc, v, part_o, part_lse, total;
};
constexpr int32_t kExplicitHead = 128;  // reconstructed content-key and value width
constexpr int32_t kRebuildRows = 256;   // rows per tile of the rebuild projection
int64_t rebuilt_rows(int64_t max_seq_len) { return round_up(max_seq_len, kRebuildRows); }
ExplicitWorkspace explicit_workspace(int64_t batch, int64_t heads, int64_t max_seq_len, int64_t nsplit) {
  typedef unsigned __int128 u128;
  auto up = [](u128 x) { return (x + 255) / 256 * 256; };
  const u128 wt = up((u128)heads * kvattn::kMlaLatent * kExplicitHead * 2);
  const u128 rows = (u128)batch * heads * (u128)rebuilt_rows(max_seq_len);
  const u128 rec = up(rows * kExplicitHead * 2);
  const u128 po = nsplit > 1 ? up((u128)batch * heads * nsplit * kExplicitHead * 2) : 0;
  const u128 pl = nsplit > 1 ? up((u128)batch * heads * nsplit * 4) : 0;
  const u128 total = 2 * wt + 2 * rec + po + pl;
  ExplicitWorkspace w{};
  if (total >= ((u128)1 << 56)) return w;
  w.wt_k = 0;
  w.wt_v = (size_t)wt;
  w.kc = (size_t)(2 * wt);
  w.v = (size_t)(2 * wt + rec);
  w.part_o = (size_t)(2 * wt + 2 * rec);
  w.part_lse = (size_t)(2 * wt + 2 * rec + po);
  w.total = (size_t)total;
  return w;
}

kvattn_status check_project(const void* x, const void* w, const void* y, int32_t outer, int32_t heads, int32_t rows,
                            int32_t k_dim, int32_t n_dim, int64_t xo, int64_t xh, int64_t xr, int64_t wh, int64_t yo,
                            int64_t yh, int64_t yr, kvattn_dtype dtype) {
  if (!x || !w || !y) return fail(KVATTN_ERR_INVALID, "x, w and y must be non-null");
  if (outer < 1 || heads < 1 || rows < 0)
    return fail(KVATTN_ERR_INVALID, "outer and heads must be >= 1 and rows >= 0 (outer=%lld, heads=%lld)", outer, heads);
  if (k_dim < 1 || n_dim < 1) return fail(KVATTN_ERR_INVALID, "k_dim and n_dim must be >= 1 (%lld, %lld)", k_dim, n_dim);
  if (dtype != KVATTN_F32 && dtype != KVATTN_BF16) return fail(KVATTN_ERR_INVALID, "unknown dtype %lld", (int)dtype);
  if (dtype != KVATTN_BF16) return fail(KVATTN_ERR_UNSUPPORTED, "projections are bf16 only");
  if (k_dim % 64 != 0 || n_dim % 128 != 0)
    return fail(KVATTN_ERR_UNSUPPORTED, "k_dim must be a multiple of 64 and n_dim of 128 (%lld, %lld)", k_dim, n_dim);
  const int64_t strides[] = {xo, xh, xr, wh, yo, yh, yr};
  for (int64_t st : strides)
    if (st < 0 || st % 8 != 0) return fail(KVATTN_ERR_INVALID, "strides must be non-negative multiples of 8 elements (got %lld)", st);
  if (xr < k_dim || yr < n_dim)
    return fail(KVATTN_ERR_INVALID, "row strides must cover a row (x_row_stride %lld, y_row_stride %lld)", xr, yr);
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(y)) % 16 != 0)
    return fail(KVATTN_ERR_INVALID, "x, w and y must be 16-byte aligned");
  const int64_t blocks = (int64_t)outer * heads * ((rows + 127) / 128) * (n_dim / 128);
  if (blocks > INT32_MAX) return fail(KVATTN_ERR_UNSUPPORTED, "projection of %lld tiles is too large for one launch", blocks);
  return KVATTN_OK;
}

kvattn::ProjectArgs project_args(const void* x, const void* w, void* y, int32_t outer, int32_t heads, int32_t rows,
                                 int32_t k_dim, int32_t n_dim, int64_t xo, int64_t xh, int64_t xr, int64_t wh,
                                 bool wt, int64_t yo, int64_t yh, int64_t yr) {
  kvattn::ProjectArgs p{};
  p.x = static_cast<const uint16_t*>(x);
  p.w = static_cast<const uint16_t*>(w);
  p.y = static_cast<uint16_t*>(y);
  p.outer = outer;
  p.heads = heads;
  p.rows = rows;
  p.k_dim = k_dim;
  p.n_dim = n_dim;
  p.x_outer = xo;
  p.x_head = xh;
  p.x_row = xr;
  p.w_head = wh;
  p.y_outer = yo;
  p.y_head = yh;
  p.y_row = yr;
  p.m_tiles = (rows + 127) / 128;
  p.n_tiles = n_dim / 128;
  p.w_transposed = wt;
  return p;
}

}  // namespace

namespace kvattn {

kvattn_status gqa_decode_with(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                              const int32_t* seq_lens, void* out, float* lse, int32_t batch, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int64_t cache_len, int32_t block_size,
                              int32_t max_blocks_per_seq, int32_t max_seq_len, float scale, int32_t window,
                              kvattn_dtype dtype, int32_t split_tokens, const Workspace& ws, void* stream) {
  const LaunchEvents ev = take_timing_events();  // armed for this call only, whatever its outcome
  kvattn_status st = check_gqa(q, k_cache, v_cache, seq_lens, out, batch, num_q_heads, num_kv_heads, head_dim, dtype,
                               scale);
  if (st != KVATTN_OK) return st;
  const GqaCache cache{k_cache, v_cache, nullptr, nullptr, dtype == KVATTN_BF16 ? CacheKind::kBf16 : CacheKind::kF32};
  return gqa_run(ev, q, cache, block_table, seq_lens, out, lse, batch, num_q_heads, num_kv_heads, head_dim,
                 cache_len, block_size, max_blocks_per_seq, max_seq_len, scale, window, split_tokens, ws, stream);
}

kvattn_status report(kvattn_status s, const char* what, long long a, long long b) { return fail(s, what, a, b); }

kvattn_status report_hip(hipError_t e, const char* what) { return hip_status(e, what); }

}  // namespace kvattn

extern "C" {

const char* kvattn_status_string(kvattn_status s) {
  switch (s) {
    case KVATTN_OK: return "ok";
    case KVATTN_ERR_INVALID: return "invalid argument";
    case KVATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVATTN_ERR_WORKSPACE: return "workspace too small";
    case KVATTN_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* kvattn_last_error(void) { return g_last_error.c_str(); }

int32_t kvattn_gqa_split_tokens(int32_t batch, int32_t h, int32_t g, int32_t max_seq_len, int32_t block_size,
                                int32_t split_tokens) {
  if (batch < 1 || h < 1 || g < 1 || h % g != 0 || split_tokens < 0 || max_seq_len > kMaxSeqLen) return -1;
  return plan_gqa_split(batch, h, g, max_seq_len, block_size > 0, split_tokens);
}

int32_t kvattn_mla_split_tokens(int32_t batch, int32_t h, int32_t max_seq_len, int32_t block_size,
                                int32_t split_tokens) {
  (void)block_size;
  if (batch < 1 || h < 1 || split_tokens < 0) return -1;
  return plan_mla_split(batch, max_seq_len, split_tokens);
}

size_t kvattn_gqa_workspace_bytes(int32_t batch, int32_t h, int32_t g, int32_t d, int32_t max_seq_len,
                                  int32_t block_size, int32_t split_tokens, kvattn_dtype dtype) {
  (void)dtype;
  if (batch < 1 || h < 1 || g < 1 || h % g != 0 || d < 1 || max_seq_len < 0 || max_seq_len > kMaxSeqLen ||
      split_tokens < 0 || split_tokens % KVATTN_SPLIT_ALIGN != 0)
    return (size_t)-1;
  const int32_t split = plan_gqa_split(batch, h, g, max_seq_len, block_size > 0, split_tokens);
  return partial_bytes(batch, h, n_splits(max_seq_len, split), d);
}

size_t kvattn_mla_workspace_bytes(int32_t batch, int32_t h, int32_t d_c, int32_t d_r, int32_t max_seq_len,
                                  int32_t block_size, int32_t split_tokens, kvattn_dtype dtype) {
  (void)dtype;
  (void)d_r;
  (void)block_size;
  if (batch < 1 || h < 1 || d_c < 1 || max_seq_len < 0 || max_seq_len > kMaxSeqLen || split_tokens < 0 ||
      split_tokens % KVATTN_SPLIT_ALIGN != 0)
    return (size_t)-1;
  const int64_t max_pieces = mla_max_pieces(batch, max_seq_len, split_tokens);
  if (max_pieces < 0) return (size_t)-1;
  return mla_workspace(batch, h, max_pieces, d_c).total;
}

kvattn_status kvattn_gqa_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                                const int32_t* seq_lens, void* out, float* lse, int32_t batch, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim, int64_t cache_len, int32_t block_size,
                                int32_t max_blocks_per_seq, int32_t max_seq_len, float scale, kvattn_dtype dtype,
                                int32_t split_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  return kvattn_gqa_decode_window(q, k_cache, v_cache, block_table, seq_lens, out, lse, batch, num_q_heads,
                                  num_kv_heads, head_dim, cache_len, block_size, max_blocks_per_seq, max_seq_len,
                                  scale, 0, dtype, split_tokens, workspace, workspace_bytes, stream);
}

kvattn_status kvattn_gqa_decode_window(const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_table, const int32_t* seq_lens, void* out, float* lse,
                                       int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int64_t cache_len, int32_t block_size, int32_t max_blocks_per_seq,
                                       int32_t max_seq_len, float scale, int32_t window, kvattn_dtype dtype,
                                       int32_t split_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  return kvattn::gqa_decode_with(q, k_cache, v_cache, block_table, seq_lens, out, lse, batch, num_q_heads,
                                 num_kv_heads, head_dim, cache_len, block_size, max_blocks_per_seq, max_seq_len, scale,
                                 window, dtype, split_tokens, kvattn::Workspace{workspace, workspace_bytes, nullptr},
                                 stream);
}

kvattn_status kvattn_gqa_decode_fp8(const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                                    const float* v_scale, const int32_t* block_table, const int32_t* seq_lens,
                                    void* out, float* lse, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int64_t cache_len, int32_t block_size,
                                    int32_t max_blocks_per_seq, int32_t max_seq_len, float scale, int32_t window,
                                    int32_t split_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  const kvattn::LaunchEvents ev = take_timing_events();  // armed for this call only, whatever its outcome
  // q/out are bf16: the bf16 checks (h/g <= 128) apply.
  kvattn_status st = check_gqa(q, k_cache, v_cache, seq_lens, out, batch, num_q_heads, num_kv_heads, head_dim,
                               KVATTN_BF16, scale);
  if (st != KVATTN_OK) return st;
  if (!k_scale || !v_scale) return fail(KVATTN_ERR_INVALID, "k_scale and v_scale must be non-null");
  const GqaCache cache{k_cache, v_cache, k_scale, v_scale, CacheKind::kFp8E4m3};
  return gqa_run(ev, q, cache, block_table, seq_lens, out, lse, batch, num_q_heads, num_kv_heads, head_dim,
                 cache_len, block_size, max_blocks_per_seq, max_seq_len, scale, window, split_tokens,
                 kvattn::Workspace{workspace, workspace_bytes, nullptr}, stream);
}

kvattn_status kvattn_mla_decode(const void* q, const void* cache, const int32_t* block_table, const int32_t* seq_lens,
                                void* out, float* lse, int32_t batch, int32_t num_heads, int32_t d_latent,
                                int32_t d_rope, int64_t cache_len, int32_t block_size, int32_t max_blocks_per_seq,
                                int32_t max_seq_len, float scale, kvattn_dtype dtype, int32_t split_tokens,
                                void* workspace, size_t workspace_bytes, void* stream) {
  const kvattn::LaunchEvents ev = take_timing_events();  // armed for this call only, whatever its outcome
  uint64_t* const clock_stamps = take_clock_stamps();     // likewise
  kvattn_status st = check_mla(q, cache, seq_lens, out, batch, num_heads, d_latent, d_rope, dtype, scale);
  if (st != KVATTN_OK) return st;
  const bool paged = block_table != nullptr;
  if ((st = check_cache_geometry(cache_len, block_size, max_blocks_per_seq, max_seq_len, paged)) != KVATTN_OK)
    return st;
  if ((st = check_split(split_tokens)) != KVATTN_OK) return st;

  const int64_t max_pieces = mla_max_pieces(batch, max_seq_len, split_tokens);
  if (max_pieces < 0)
    return fail(KVATTN_ERR_UNSUPPORTED, "batch %lld x max_seq_len %lld needs too many pieces for this split_tokens",
                batch, max_seq_len);
  const MlaWorkspace wl = mla_workspace(batch, num_heads, max_pieces, d_latent);
  if (workspace == nullptr || workspace_bytes < wl.total)
    return fail(KVATTN_ERR_WORKSPACE, "workspace of %lld bytes needed, %lld given", (long long)wl.total,
                workspace == nullptr ? 0 : (long long)workspace_bytes);
  unsigned char* ws = static_cast<unsigned char*>(workspace);

  kvattn::MlaPlanArgs pa{};
  pa.seq_lens = seq_lens;
  pa.batch = batch;
  pa.len_cap = max_seq_len;
  pa.work_items = kCUs;
  pa.min_chunk = kMlaMinChunk;
  pa.fixed_chunk = split_tokens;
  pa.pieces = reinterpret_cast<int4*>(ws + wl.pieces);
  pa.seq_pieces = reinterpret_cast<int2*>(ws + wl.seq_pieces);
  pa.plan_count = reinterpret_cast<int32_t*>(ws + wl.plan_count);

  kvattn::DecodeArgs a{};
  a.q = q;
  a.k = cache;
  a.v = nullptr;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.out = out;
  a.lse = lse;
  a.batch = batch;
  a.num_q_heads = num_heads;
  a.num_kv_heads = 1;
  a.group = num_heads;
  a.cache_len = cache_len;
  a.block_size = paged ? block_size : 0;
  a.block_shift = paged ? pow2_shift(block_size) : -1;
  a.max_blocks = paged ? max_blocks_per_seq : 0;
  a.len_cap = max_seq_len;
  a.scale_log2 = scale * kvattn::kLog2eHost;
  a.part_o = reinterpret_cast<float*>(ws + wl.part_o);
  a.part_lse = reinterpret_cast<float*>(ws + wl.part_lse);
  a.pieces = pa.pieces;
  a.seq_pieces = pa.seq_pieces;
  a.plan_count = pa.plan_count;
  a.max_pieces = (int32_t)max_pieces;
  a.clock_stamps = clock_stamps;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = kvattn::launch_mla_plan(pa, s);
  if (e != hipSuccess) return hip_status(e, "MLA plan kernel launch");
  e = kvattn::launch_mla_bf16(a, s, ev);
  if (e != hipSuccess) return hip_status(e, "MLA kernel launch");
  e = kvattn::launch_mla_merge_pieces(a, s);
  if (e != hipSuccess) return hip_status(e, "merge kernel launch");
  return ok();
}

kvattn_status kvattn_mla_project(const void* x, const void* w, void* y, int32_t outer, int32_t heads, int32_t rows,
                                 int32_t k_dim, int32_t n_dim, int64_t x_outer_stride, int64_t x_head_stride,
                                 int64_t x_row_stride, int64_t w_head_stride, int32_t w_transposed,
                                 int64_t y_outer_stride, int64_t y_head_stride, int64_t y_row_stride,
                                 kvattn_dtype dtype, void* stream) {
  kvattn_status st = check_project(x, w, y, outer, heads, rows, k_dim, n_dim, x_outer_stride, x_head_stride,
                                   x_row_stride, w_head_stride, y_outer_stride, y_head_stride, y_row_stride, dtype);
  if (st != KVATTN_OK) return st;
  if (rows == 0) return ok();
  const kvattn::ProjectArgs p =
      project_args(x, w, y, outer, heads, rows, k_dim, n_dim, x_outer_stride, x_head_stride, x_row_stride,
                   w_head_stride, w_transposed != 0, y_outer_stride, y_head_stride, y_row_stride);
  const hipError_t e = kvattn::launch_latent_project(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_status(e, "projection kernel launch");
  return ok();
}

size_t kvattn_mla_explicit_workspace_bytes(int32_t batch, int32_t num_heads, int32_t d_head, int32_t d_v,
                                           int32_t max_seq_len, int32_t split_tokens, kvattn_dtype dtype) {
  (void)dtype;
  if (batch < 1 || num_heads < 1 || d_head != kExplicitHead || d_v != kExplicitHead || max_seq_len < 0 ||
      max_seq_len > kMaxSeqLen || split_tokens < 0 || split_tokens % KVATTN_SPLIT_ALIGN != 0)
    return (size_t)-1;
  const int32_t split = plan_gqa_split(batch, num_heads, num_heads, max_seq_len, false, split_tokens);
  const ExplicitWorkspace w = explicit_workspace(batch, num_heads, max_seq_len, n_splits(max_seq_len, split));
  return w.total == 0 ? (size_t)-1 : w.total;
}

kvattn_status kvattn_mla_explicit_decode(const void* q, const void* cache, const void* w_uk, const void* w_uv,
                                         const int32_t* seq_lens, void* out, float* lse, int32_t batch,
                                         int32_t num_heads, int32_t d_latent, int32_t d_rope, int32_t d_head,
                                         int32_t d_v, int64_t cache_len, int32_t max_seq_len, float scale,
                                         kvattn_dtype dtype, int32_t split_tokens, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  const kvattn::LaunchEvents ev = take_timing_events();  // armed for this call only, whatever its outcome
  if (!q || !cache || !w_uk || !w_uv || !seq_lens || !out)
    return fail(KVATTN_ERR_INVALID, "q, cache, w_uk, w_uv, seq_lens and out must be non-null");
  if (batch < 1 || num_heads < 1)
    return fail(KVATTN_ERR_INVALID, "batch and num_heads must be >= 1 (got %lld, %lld)", batch, num_heads);
  if (d_latent < 1 || d_rope < 0 || d_head < 1 || d_v < 1)
    return fail(KVATTN_ERR_INVALID, "bad MLA widths (d_latent=%lld, d_head=%lld)", d_latent, d_head);
  if (dtype != KVATTN_F32 && dtype != KVATTN_BF16) return fail(KVATTN_ERR_INVALID, "unknown dtype %lld", (int)dtype);
  if (!std::isfinite(scale)) return fail(KVATTN_ERR_INVALID, "scale must be finite");
  if (d_latent != kvattn::kMlaLatent || d_rope != kvattn::kMlaRope)
    return fail(KVATTN_ERR_UNSUPPORTED, "MLA supports d_latent=512, d_rope=64 (got %lld, %lld)", d_latent, d_rope);
  if (d_head != kExplicitHead || d_v != kExplicitHead)
    return fail(KVATTN_ERR_UNSUPPORTED, "explicit MLA supports d_head = d_v = 128 (got %lld, %lld)", d_head, d_v);
  if (dtype != KVATTN_BF16) return fail(KVATTN_ERR_UNSUPPORTED, "MLA supports bf16 only");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(cache) | reinterpret_cast<uintptr_t>(w_uk) |
       reinterpret_cast<uintptr_t>(w_uv) | reinterpret_cast<uintptr_t>(out)) % 16 != 0)
    return fail(KVATTN_ERR_INVALID, "q, cache, w_uk, w_uv and out must be 16-byte aligned");
  kvattn_status st;
  if ((st = check_cache_geometry(cache_len, 0, 0, max_seq_len, false)) != KVATTN_OK) return st;
  if ((st = check_split(split_tokens)) != KVATTN_OK) return st;
  const int32_t split = plan_gqa_split(batch, num_heads, num_heads, max_seq_len, false, split_tokens);
  const int32_t nsplit = n_splits(max_seq_len, split);
  const ExplicitWorkspace wl = explicit_workspace(batch, num_heads, max_seq_len, nsplit);
  if (wl.total == 0) return fail(KVATTN_ERR_UNSUPPORTED, "batch %lld x max_seq_len %lld is too large", batch, max_seq_len);
  if ((int64_t)batch * num_heads * nsplit > INT32_MAX ||
      (int64_t)batch * num_heads * ((max_seq_len + 127) / 128) > INT32_MAX)
    return fail(KVATTN_ERR_UNSUPPORTED, "batch %lld x num_heads %lld is too large for one launch", batch, num_heads);
  if (workspace == nullptr || workspace_bytes < wl.total)
    return fail(KVATTN_ERR_WORKSPACE, "workspace of %lld bytes needed, %lld given", (long long)wl.total,
                workspace == nullptr ? 0 : (long long)workspace_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(KVATTN_ERR_INVALID, "workspace must be 256-byte aligned");
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  const int64_t row_elems = kvattn::kMlaRow;
  const int64_t rec = rebuilt_rows(max_seq_len) * kExplicitHead;  // elements of one (sequence, head) block
  if (max_seq_len > 0) {
    // k_i = c W_uk^(i) and v_i = c W_uv^(i) for every (sequence, head, row < max_seq_len), with the
    // weights first transposed to [h, 128, 512] so that both operands are read row-wise.
    if ((e = kvattn::launch_transpose_heads(w_uk, ws + wl.wt_k, num_heads, d_latent, kExplicitHead, s)) != hipSuccess ||
        (e = kvattn::launch_transpose_heads(w_uv, ws + wl.wt_v, num_heads, d_latent, kExplicitHead, s)) != hipSuccess)
      return hip_status(e, "transpose kernel launch");
    kvattn::ProjectArgs p = project_args(cache, ws + wl.wt_k, ws + wl.kc, batch, num_heads, max_seq_len, d_latent,
                                         kExplicitHead, cache_len * row_elems, 0, row_elems,
                                         (int64_t)d_latent * kExplicitHead, true, num_heads * rec, rec,
                                         kExplicitHead);
    if ((e = kvattn::launch_latent_rebuild(p, s)) != hipSuccess) return hip_status(e, "projection kernel launch");
    p.w = reinterpret_cast<const uint16_t*>(ws + wl.wt_v);
    p.y = reinterpret_cast<uint16_t*>(ws + wl.v);
    if ((e = kvattn::launch_latent_rebuild(p, s)) != hipSuccess) return hip_status(e, "projection kernel launch");
  }
  kvattn::DecodeArgs a{};
  a.q = q;
  a.k = ws + wl.kc;
  a.v = ws + wl.v;
  a.rope = cache;
  a.rec_len = (int32_t)rebuilt_rows(max_seq_len);
  a.seq_lens = seq_lens;
  a.out = out;
  a.lse = lse;
  a.batch = batch;
  a.num_q_heads = num_heads;
  a.num_kv_heads = num_heads;
  a.group = 1;
  a.cache_len = cache_len;
  a.len_cap = max_seq_len;
  a.window = 0;
  a.split_tokens = split;
  a.n_split = nsplit;
  a.scale_log2 = scale * kvattn::kLog2eHost;
  if (nsplit > 1) {
    a.part_o = reinterpret_cast<float*>(ws + wl.part_o);
    a.part_lse = reinterpret_cast<float*>(ws + wl.part_lse);
  }
  if ((e = kvattn::launch_mla_explicit_attend(a, s, ev)) != hipSuccess) return hip_status(e, "attention kernel launch");
  if (nsplit > 1 && (e = kvattn::launch_merge(a, true, s)) != hipSuccess) return hip_status(e, "merge kernel launch");
  return ok();
}

kvattn_status kvattn_time_next_kernel(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(KVATTN_ERR_INVALID, "start_event and stop_event must both be set or both be null");
  g_time_next.start = static_cast<hipEvent_t>(start_event);
  g_time_next.stop = static_cast<hipEvent_t>(stop_event);
  return ok();
}

kvattn_status kvattn_clock_next_mla(uint64_t* stamps) {
  if (reinterpret_cast<uintptr_t>(stamps) % 8 != 0) return fail(KVATTN_ERR_INVALID, "stamps must be 8-byte aligned");
  g_clock_next = stamps;
  return ok();
}

kvattn_status kvattn_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, int32_t workgroups,
                                    void* stream) {
  if (!buf || !sink) return fail(KVATTN_ERR_INVALID, "buf and sink must be non-null");
  if (bytes == 0 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return fail(KVATTN_ERR_INVALID, "bytes must be a positive multiple of 16 and buf 16-byte aligned (bytes=%lld)",
                (long long)bytes);
  if (workgroups < 1) return fail(KVATTN_ERR_INVALID, "workgroups must be >= 1 (got %lld)", workgroups);
  hipError_t e = kvattn::launch_hbm_read_probe(buf, (int64_t)(bytes / 16), sink, workgroups,
                                               static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_status(e, "probe launch");
  return ok();
}

}  // extern "C"
