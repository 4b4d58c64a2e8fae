// Host-side checks of libkvattn's C ABI, built from api.cpp with the launcher
// stand-ins of stub_launch.cpp (no GPU, no kernel code) so that the argument
// checks, the split planning and the workspace layout run under the address
// and undefined-behaviour sanitizers.  Prints one line per failed check and
// exits non-zero if any failed.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>

#include "../../include/kvattn.h"
#include "stub_launch.h"

static int g_failed = 0, g_checked = 0;
#define CHECK(cond, ...)                                  \
  do {                                                    \
    ++g_checked;                                          \
    if (!(cond)) {                                        \
      ++g_failed;                                         \
      std::printf("FAILED %s:%d: %s  ", __FILE__, __LINE__, #cond); \
      std::printf(__VA_ARGS__);                           \
      std::printf("\n");                                  \
    }                                                     \
  } while (0)

static void* const P = reinterpret_cast<void*>(16);  // never dereferenced: no kernel runs
static const int32_t* const PI = reinterpret_cast<const int32_t*>(16);
static const size_t kRejected = (size_t)-1;

static kvattn_status gqa_window(int32_t B, int32_t h, int32_t g, int32_t S, int32_t bs, int32_t window, int32_t split,
                                size_t ws, kvattn_dtype dt = KVATTN_BF16) {
  const bool paged = bs > 0;
  const int32_t maxb = paged ? (S + bs - 1) / bs : 0;
  const int64_t cache_len = paged ? (int64_t)B * maxb : (S > 0 ? S : 1);
  return kvattn_gqa_decode_window(P, P, P, paged ? PI : nullptr, PI, P, nullptr, B, h, g, 128, cache_len, bs, maxb, S,
                                  0.1f, window, dt, split, ws ? P : nullptr, ws, nullptr);
}

// The persistent form's work list: taken exactly when the grid of splits is large, for a bf16 cache with a
// layout whose full tiles need no LDS table; it lies inside the workspace after the partials, one int4 per
// possible item, then its count and claim counter; the plan kernel gets the call's split geometry.
static void check_work_list(const kvattn::DecodeArgs& a, int32_t B, int32_t h, int32_t g, int32_t bs, int32_t W,
                            int32_t S, size_t ws) {
  const int64_t slots = (int64_t)B * g * a.n_split;
  const bool pow2_ok = bs == 0 || (bs >= 4 && (bs & (bs - 1)) == 0);
  const bool expect = a.n_split > 1 && slots > 4 * kvattn::kPersistentWorkgroups && pow2_ok;
  CHECK((a.items != nullptr) == expect, "B=%d g=%d bs=%d n_split=%d: work list %d", B, g, bs, a.n_split,
        a.items != nullptr);
  CHECK(stub::last.gqa_plans == (expect ? 1 : 0), "plan launches %d", stub::last.gqa_plans);
  if (!expect) return;
  const auto* base = static_cast<const unsigned char*>(P);
  const auto* part_end = reinterpret_cast<const unsigned char*>(a.part_lse) + (size_t)B * h * a.n_split * 4;
  const auto* items = reinterpret_cast<const unsigned char*>(a.items);
  const auto* ctl = reinterpret_cast<const unsigned char*>(a.items_ctl);
  CHECK(reinterpret_cast<const unsigned char*>(a.part_o) == base, "partials first");
  CHECK(items >= part_end && items + slots * 16 <= ctl && ctl + 8 <= base + ws, "work list outside the workspace");
  CHECK((uintptr_t)(items - base) % 16 == 0 && (uintptr_t)(ctl - base) % 4 == 0, "alignment");
  const kvattn::GqaPlanArgs& p = stub::last.gqa_plan;
  CHECK(p.items == a.items && p.ctl == a.items_ctl && p.seq_lens == a.seq_lens, "plan pointers");
  CHECK(p.batch == B && p.g == g && p.split == a.split_tokens && p.n_split == a.n_split && p.window == W &&
            p.len_cap == S, "plan geometry");
}

static void window_sweep() {
  // A window call accepts exactly the bytes kvattn_gqa_workspace_bytes reports for the same arguments
  // (the query takes no window), and its splits cover the window's span.
  const int32_t Ss[] = {1, 64, 100, 1000, 2112, 4096, 8192, 32768, 65536};
  const int32_t Ws[] = {1, 63, 64, 100, 1730, 4096, 8191, 40000};
  const int32_t Bs[] = {1, 8, 64};
  const int32_t HG[][2] = {{8, 8}, {32, 8}, {64, 8}, {64, 1}, {128, 1}};
  const int32_t BSs[] = {0, 16, 1, 5};
  const int32_t splits[] = {0, 64, 1024};
  for (int32_t S : Ss)
    for (int32_t W : Ws)
      for (int32_t B : Bs)
        for (auto& hg : HG)
          for (int32_t bs : BSs)
            for (int32_t split : splits) {
              const size_t ws = kvattn_gqa_workspace_bytes(B, hg[0], hg[1], 128, S, bs, split, KVATTN_BF16);
              CHECK(ws != kRejected, "S=%d", S);
              stub::last = stub::Record{};
              const kvattn_status st = gqa_window(B, hg[0], hg[1], S, bs, W, split, ws);
              CHECK(st == KVATTN_OK, "S=%d W=%d B=%d h=%d g=%d bs=%d split=%d ws=%zu: %s", S, W, B, hg[0], hg[1], bs,
                    split, ws, kvattn_last_error());
              if (st != KVATTN_OK) continue;
              const kvattn::DecodeArgs& a = stub::last.args;
              const int64_t span = W < S ? (int64_t)W + 63 < S ? W + 63 : S : S;
              CHECK(a.split_tokens > 0 && a.split_tokens % 64 == 0, "split %d", a.split_tokens);
              // The last split runs to the sequence's end, taking up to 63 tokens of a window's aligned start.
              CHECK((int64_t)a.n_split * a.split_tokens + 63 >= span, "S=%d W=%d: %d x %d + 63 < %lld", S, W,
                    a.n_split, a.split_tokens, (long long)span);
              CHECK((int64_t)a.n_split * a.split_tokens >= span || W == 0 || stub::last.gqa_plans == 0,
                    "a persistent call whose last split would run past n_split x split");
              CHECK(a.n_split == 1 || (int64_t)(a.n_split - 1) * a.split_tokens < span, "empty split");
              const size_t need = a.n_split > 1 ? (size_t)B * hg[0] * a.n_split * 129 * 4 : 0;
              CHECK(need <= ws, "need %zu > queried %zu", need, ws);
              CHECK(stub::last.merges == (a.n_split > 1 ? 1 : 0), "merge count");
              check_work_list(a, B, hg[0], hg[1], bs, W, S, ws);
            }
}

static void gqa_rejections() {
  CHECK(gqa_window(2, 8, 3, 64, 0, 0, 0, 0) == KVATTN_ERR_INVALID, "h %% g");
  CHECK(gqa_window(2, 8, 2, 64, 0, -1, 0, 0) == KVATTN_ERR_INVALID, "negative window");
  CHECK(gqa_window(2, 8, 2, 64, 0, 0, 100, 0) == KVATTN_ERR_INVALID, "split not a multiple of 64");
  CHECK(gqa_window(0, 8, 2, 64, 0, 0, 0, 0) == KVATTN_ERR_INVALID, "batch 0");
  CHECK(gqa_window(2, 256, 1, 64, 0, 0, 0, 0) == KVATTN_ERR_UNSUPPORTED, "group 256");
  CHECK(gqa_window(2, 128, 1, 64, 0, 0, 0, 0, KVATTN_F32) == KVATTN_ERR_UNSUPPORTED, "fp32 group 128");
  const size_t need = kvattn_gqa_workspace_bytes(2, 8, 2, 128, 4096, 0, 256, KVATTN_BF16);
  CHECK(need == (size_t)2 * 8 * 16 * 129 * 4, "need %zu", need);
  // the call itself needs the bf16 layout: bf16 partial outputs and fp32 log-sum-exps
  const size_t need_bf16 = (size_t)2 * 8 * 16 * (128 * 2 + 4);
  CHECK(gqa_window(2, 8, 2, 4096, 0, 0, 256, need_bf16 - 1) == KVATTN_ERR_WORKSPACE, "short workspace");
  CHECK(gqa_window(2, 8, 2, 4096, 0, 0, 256, need_bf16) == KVATTN_OK, "%s", kvattn_last_error());
  CHECK(gqa_window(2, 8, 2, 4096, 0, 0, 256, need - 1, KVATTN_F32) == KVATTN_ERR_WORKSPACE, "short fp32 workspace");
  CHECK(gqa_window(2, 8, 2, 4096, 0, 0, 256, need) == KVATTN_OK, "%s", kvattn_last_error());
}

static void mla_sweep() {
  const int32_t Bs[] = {1, 5, 32, 300, 600, 5000};
  const int32_t Ss[] = {1, 100, 8192, 65536};
  const int32_t splits[] = {0, 64, 1024};
  const int32_t bss[] = {0, 64, 1};
  for (int32_t B : Bs)
    for (int32_t S : Ss)
      for (int32_t split : splits)
        for (int32_t bs : bss) {
          const size_t ws = kvattn_mla_workspace_bytes(B, 128, 512, 64, S, bs, split, KVATTN_BF16);
          CHECK(ws != kRejected && ws > 0, "B=%d S=%d", B, S);
          if (ws == kRejected) continue;
          const bool paged = bs > 0;
          const int32_t maxb = paged ? (S + bs - 1) / bs : 0;
          const int64_t cache_len = paged ? (int64_t)B * maxb : S;
          unsigned char* base = reinterpret_cast<unsigned char*>(1 << 20);
          stub::last = stub::Record{};
          const kvattn_status st =
              kvattn_mla_decode(P, P, paged ? PI : nullptr, PI, P, nullptr, B, 128, 512, 64, cache_len, bs, maxb, S,
                                0.07f, KVATTN_BF16, split, base, ws, nullptr);
          CHECK(st == KVATTN_OK, "B=%d S=%d split=%d: %s", B, S, split, kvattn_last_error());
          if (st != KVATTN_OK) continue;
          CHECK(kvattn_mla_decode(P, P, paged ? PI : nullptr, PI, P, nullptr, B, 128, 512, 64, cache_len, bs, maxb, S,
                                  0.07f, KVATTN_BF16, split, base, ws - 1, nullptr) == KVATTN_ERR_WORKSPACE,
                "short MLA workspace");
          const kvattn::DecodeArgs& a = stub::last.args;
          // The most pieces the device plan can make: max(256, B) when it chooses (one piece per sequence
          // always fits), B * ceil(S / split) for a requested length.
          const int64_t most = split > 0 ? (int64_t)B * ((S + split - 1) / split) : (B > 256 ? B : 256);
          CHECK(a.max_pieces >= most, "max_pieces %d < %lld", a.max_pieces, (long long)most);
          auto inside = [&](const void* p, int64_t bytes) {
            const unsigned char* c = static_cast<const unsigned char*>(p);
            return c >= base && c + bytes <= base + ws;
          };
          CHECK(inside(a.part_o, (int64_t)a.max_pieces * 128 * 512 * 2), "partials outside the workspace");
          CHECK(inside(a.part_lse, (int64_t)a.max_pieces * 128 * 4), "lse outside");
          CHECK(inside(a.pieces, (int64_t)a.max_pieces * 16), "pieces outside");
          CHECK(inside(a.seq_pieces, (int64_t)B * 8), "ranges outside");
          CHECK(inside(a.plan_count, 8), "count outside");
          CHECK(stub::last.plan.pieces == a.pieces && stub::last.plan.fixed_chunk == split, "plan args");
        }
}

static void fuzz() {
  // Random (also extreme) arguments: the size queries and the calls must agree, never overflow, and a
  // call given the queried workspace must not fail for lack of workspace.
  std::mt19937_64 rng(12345);
  auto pick = [&](std::initializer_list<int32_t> v) { return *(v.begin() + rng() % v.size()); };
  for (int i = 0; i < 20000; ++i) {
    const int32_t B = pick({1, 2, 7, 64, 4096, 65535, 70000, 0, -1});
    const int32_t g = pick({1, 2, 8, 64, 0});
    const int32_t h = g * pick({1, 4, 8, 64, 128, 3});
    const int32_t S = pick({0, 1, 63, 64, 65, 8192, 1 << 20, 1 << 28, (1 << 28) + 1, 2147483647, -5});
    const int32_t bs = pick({0, 0, 1, 16, 3, 1 << 20});
    const int32_t W = pick({0, 0, 1, 4096, 2147483647});
    const int32_t split = pick({0, 0, 64, 4096, 1 << 30, 100});
    const size_t ws = kvattn_gqa_workspace_bytes(B, h, g, 128, S, bs, split, KVATTN_BF16);
    if (B < 1 || g < 1 || h < 1 || S < 0 || split % 64 != 0) CHECK(ws == kRejected, "accepted bad sizes");
    if (ws == kRejected || ws > ((size_t)1 << 50)) continue;
    if (bs > 0 && (int64_t)((S + bs - 1) / bs) > 2147483647) continue;
    stub::last = stub::Record{};
    const kvattn_status st = gqa_window(B, h, g, S, bs, W, split, ws);
    CHECK(st != KVATTN_ERR_WORKSPACE, "B=%d h=%d g=%d S=%d bs=%d W=%d split=%d: %s", B, h, g, S, bs, W, split,
          kvattn_last_error());
    if (st == KVATTN_OK) {
      const kvattn::DecodeArgs& a = stub::last.args;
      CHECK(a.split_tokens > 0 && a.n_split >= 1, "split %d n %d", a.split_tokens, a.n_split);
      CHECK((int64_t)a.split_tokens * a.n_split < ((int64_t)1 << 31), "token arithmetic would overflow int");
    }
    const size_t mws = kvattn_mla_workspace_bytes(B, 128, 512, 64, S, bs, split, KVATTN_BF16);
    if (mws != kRejected && mws < ((size_t)1 << 50)) {
      const int32_t maxb = bs > 0 ? (S + bs - 1) / bs : 0;
      const kvattn_status ms = kvattn_mla_decode(P, P, bs > 0 ? PI : nullptr, PI, P, nullptr, B, 128, 512, 64,
                                                 bs > 0 ? 1 << 20 : (S > 0 ? S : 1), bs, maxb, S, 0.07f, KVATTN_BF16,
                                                 split, P, mws, nullptr);
      CHECK(ms != KVATTN_ERR_WORKSPACE, "MLA B=%d S=%d split=%d: %s", B, S, split, kvattn_last_error());
    }
  }
}

// The no-allocation path (kvattn_gqa_decode_noalloc) takes its workspace from a fixed scratch: the size
// check comes first, and the scratch is looked up only by a call that needs it and fits.
static int g_resolved = 0;
static kvattn_status fake_scratch(void** p) {
  ++g_resolved;
  *p = reinterpret_cast<void*>(1 << 24);
  return KVATTN_OK;
}

static void scratch_source() {
  const size_t cap = KVATTN_NOALLOC_SCRATCH_BYTES;
  struct Case {
    int32_t B, h, g, S, bs, split;
    kvattn_dtype dt;
  } cases[] = {{2, 8, 2, 64, 0, 0, KVATTN_BF16},          {16, 32, 8, 8192, 0, 0, KVATTN_BF16},
               {128, 64, 8, 32768, 16, 0, KVATTN_BF16},   {128, 64, 8, 32768, 16, 0, KVATTN_F32},
               {512, 64, 8, 32768, 16, 0, KVATTN_BF16},   {1, 128, 1, 65536, 0, 64, KVATTN_BF16},
               {64, 64, 1, 8192, 0, 64, KVATTN_F32}};
  for (const Case& c : cases) {
    const int32_t maxb = c.bs ? (c.S + c.bs - 1) / c.bs : 0;
    const int64_t cache_len = c.bs ? (int64_t)c.B * maxb : c.S;
    g_resolved = 0;
    stub::last = stub::Record{};
    const kvattn_status st = kvattn::gqa_decode_with(
        P, P, P, c.bs ? PI : nullptr, PI, P, nullptr, c.B, c.h, c.g, 128, cache_len, c.bs, maxb, c.S, 0.1f, 0, c.dt,
        c.split, kvattn::Workspace{nullptr, cap, fake_scratch}, nullptr);
    const int32_t split = kvattn_gqa_split_tokens(c.B, c.h, c.g, c.S, c.bs, c.split);
    const int64_t nsplit = c.S <= split ? 1 : (c.S + split - 1) / split;
    const int64_t elem = c.dt == KVATTN_F32 ? 4 : 2;
    const int64_t need = nsplit > 1 ? (int64_t)c.B * c.h * nsplit * (128 * elem + 4) : 0;
    if (need > (int64_t)cap) {
      CHECK(st == KVATTN_ERR_WORKSPACE && g_resolved == 0 && stub::last.launches == 0, "B=%d need %lld: st %d",
            c.B, (long long)need, st);
    } else {
      CHECK(st == KVATTN_OK, "B=%d S=%d: %s", c.B, c.S, kvattn_last_error());
      CHECK(g_resolved == (need > 0 ? 1 : 0), "looked up %d times", g_resolved);
      if (need > 0) CHECK(stub::last.args.part_o == reinterpret_cast<float*>(1 << 24), "partials not in the scratch");
    }
  }
}

// Reconstruct-then-attend MLA: workspace regions inside the queried size, the two projections cover every
// (sequence, head, row < max_seq_len) with the weights' head stride, and the attention reads what they wrote.
static void explicit_mla() {
  const int32_t Bs[] = {1, 3, 32};
  const int32_t Hs[] = {16, 128};
  const int32_t Ss[] = {0, 1, 300, 8192};
  const int32_t splits[] = {0, 64};
  for (int32_t B : Bs)
    for (int32_t h : Hs)
      for (int32_t S : Ss)
        for (int32_t split : splits) {
          const size_t ws = kvattn_mla_explicit_workspace_bytes(B, h, 128, 128, S, split, KVATTN_BF16);
          CHECK(ws != kRejected, "B=%d h=%d S=%d", B, h, S);
          unsigned char* base = reinterpret_cast<unsigned char*>(1 << 20);
          stub::last = stub::Record{};
          const int64_t cache_len = S > 0 ? S : 1;
          const kvattn_status st =
              kvattn_mla_explicit_decode(P, P, P, P, PI, P, nullptr, B, h, 512, 64, 128, 128, cache_len, S, 0.07f,
                                         KVATTN_BF16, split, base, ws, nullptr);
          CHECK(st == KVATTN_OK, "B=%d h=%d S=%d split=%d: %s", B, h, S, split, kvattn_last_error());
          if (st != KVATTN_OK) continue;
          CHECK(kvattn_mla_explicit_decode(P, P, P, P, PI, P, nullptr, B, h, 512, 64, 128, 128, cache_len, S, 0.07f,
                                           KVATTN_BF16, split, base, ws - 1, nullptr) == KVATTN_ERR_WORKSPACE,
                "short explicit workspace");
          const kvattn::DecodeArgs& a = stub::last.args;
          const int64_t R = (S + 255) / 256 * 256;  // rebuilt rows per (sequence, head): whole 256-row tiles
          const int64_t rec = (int64_t)B * h * R * 128 * 2;
          const int64_t wbytes = (int64_t)h * 512 * 128 * 2;
          auto inside = [&](const void* p, int64_t bytes) {
            const unsigned char* c = static_cast<const unsigned char*>(p);
            return bytes == 0 || (c >= base && c + bytes <= base + ws);
          };
          CHECK(inside(a.k, rec) && inside(a.v, rec), "rebuilt rows outside the workspace");
          CHECK(static_cast<const unsigned char*>(a.v) >= static_cast<const unsigned char*>(a.k) + rec || rec == 0,
                "keys and values overlap");
          if (a.n_split > 1) {
            CHECK(inside(a.part_o, (int64_t)B * h * a.n_split * 128 * 2), "partials outside");
            CHECK(inside(a.part_lse, (int64_t)B * h * a.n_split * 4), "lse outside");
          }
          CHECK((int64_t)a.n_split * a.split_tokens >= S, "splits do not cover the sequence");
          CHECK(stub::last.n_projects == (S > 0 ? 2 : 0), "projections %d", stub::last.n_projects);
          CHECK(stub::last.n_transposes == (S > 0 ? 2 : 0), "transposes %d", stub::last.n_transposes);
          if (S > 0) {
            const kvattn::ProjectArgs& pk = stub::last.projects[0];
            CHECK(pk.outer == B && pk.heads == h && pk.rows == S && pk.k_dim == 512 && pk.n_dim == 128, "shape");
            CHECK(pk.x_row == 576 && pk.x_head == 0 && pk.x_outer == cache_len * 576, "x strides");
            CHECK(pk.w_head == 512 * 128 && pk.w_transposed, "w stride");
            for (int tt = 0; tt < 2; ++tt) {
              const auto& tr = stub::last.transposes[tt];
              CHECK(tr.heads == h && tr.rows == 512 && tr.cols == 128 && inside(tr.dst, wbytes), "transpose");
              CHECK(reinterpret_cast<const void*>(stub::last.projects[tt].w) == tr.dst, "projection reads other weights");
            }
            CHECK(stub::last.transposes[0].dst != stub::last.transposes[1].dst, "weights share a region");
            CHECK(pk.y_row == 128 && pk.y_head == R * 128 && pk.y_outer == (int64_t)h * R * 128, "y strides");
            CHECK(reinterpret_cast<const void*>(pk.y) == a.k && reinterpret_cast<const void*>(stub::last.projects[1].y) == a.v,
                  "attention reads other rows than the projections wrote");
            CHECK(pk.m_tiles == (S + 127) / 128 && pk.n_tiles == 1, "tiles");
          }
          CHECK(a.rec_len == R && a.rope == P, "rope source");
        }
  // projections: rejected shapes and strides
  auto proj = [&](int32_t k, int32_t n, int64_t xr, int64_t yr, const void* y = P) {
    return kvattn_mla_project(P, P, const_cast<void*>(y), 1, 4, 10, k, n, 0, k, xr, k * n, 0, 0, n, yr, KVATTN_BF16,
                              nullptr);
  };
  CHECK(proj(512, 128, 512 * 4, 128 * 4) == KVATTN_OK, "%s", kvattn_last_error());
  CHECK(proj(500, 128, 512 * 4, 128 * 4) == KVATTN_ERR_UNSUPPORTED, "k not a multiple of 64");
  CHECK(proj(512, 100, 512 * 4, 128 * 4) == KVATTN_ERR_UNSUPPORTED, "n not a multiple of 128");
  CHECK(proj(512, 128, 100, 128 * 4) == KVATTN_ERR_INVALID, "row stride shorter than a row");
  CHECK(proj(512, 128, 512 * 4 + 4, 128 * 4) == KVATTN_ERR_INVALID, "stride not a multiple of 8");
  CHECK(proj(512, 128, 512 * 4, 128 * 4, reinterpret_cast<void*>(24)) == KVATTN_ERR_INVALID, "misaligned y");
  CHECK(kvattn_mla_project(P, P, P, 1, 4, 10, 512, 128, 0, 512, 2048, 65536, 0, 0, 128, 512, KVATTN_F32, nullptr) ==
            KVATTN_ERR_UNSUPPORTED,
        "fp32");
}

int main() {
  explicit_mla();
  scratch_source();
  gqa_rejections();
  window_sweep();
  mla_sweep();
  fuzz();
  std::printf("%d checks, %d failed\n", g_checked, g_failed);
  return g_failed == 0 ? 0 : 1;
}
