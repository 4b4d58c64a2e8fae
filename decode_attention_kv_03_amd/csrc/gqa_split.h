// The split-K grouped-query decode pipeline shared by the bf16 and fp8 cache
// kernels (gqa_bf16.hip, gqa_fp8.hip); the cache format supplies the tile
// geometry, the LDS swizzle and the score and value fragment routines.
//
// What it computes ("MQA, GQA, and MLA", sections 2-4 and 8): for sequence b
// and KV head j, the r = h/g query heads j*r .. j*r+r-1 attend over the
// cached K/V rows of head j; each K/V byte is fetched from HBM once per
// decode step and serves all r heads of its group (index, never repeat).
//
// Work decomposition.  One workgroup (4 waves) owns one (sequence, KV head,
// split) and walks the split's tokens in tiles of 16 KiB per tensor (64
// bf16 rows of 256 B, or 128 fp8 rows of 128 B):
//  * the 1-D grid is XCD-aware: workgroup w runs on XCD w % 8, and when the
//    (sequence, KV head) units divide evenly among the eight XCDs all splits
//    of a unit share that residue, so the group's queries are fetched into
//    one XCD's L2; otherwise (a single long sequence, say) consecutive
//    workgroups take consecutive splits, so that every XCD gets work;
//  * tiles stream from HBM straight into a two-stage LDS ring with
//    global_load_lds_dwordx4 carrying the non-temporal hint (the cache is
//    read once per step); one tile is in flight while the other is consumed.
//    The copies are issued as inline assembly and awaited with explicit
//    vmcnt counts, so the compiler never drains them before an LDS read;
//  * rows are stored unpadded with their 16-byte chunks XOR-swizzled by row
//    (the format's swz()), so that neither LDS read pattern stalls on bank
//    conflicts;
//  * a paged cache's block-table slice for the split is staged in LDS first,
//    so per-row block lookups never wait on the vector-memory counter; a
//    split that needs more entries than the LDS holds slides the staged
//    window when a tile reaches past it.  Power-of-two blocks of at least one
//    copy instruction's rows take one scalar table load per instruction;
//  * scores S^T = K_tile * Q^T on v_mfma_f32_16x16x32_bf16 (16 tokens x 16
//    query heads); the online softmax runs in the matrix-core output layout
//    (lane l: query head l%16, tokens 4*(l/16)+v), with lazy rescaling: the
//    reference max only moves when a tile's max exceeds it by more than 8
//    (log2 units);
//  * P V is accumulated as O^T = V^T * P^T with V^T from the row-major tile
//    through the gfx950 LDS transposing reads;
//  * waves split the tile's tokens when a group has at most 32 heads (each
//    keeps its own max/sum/accumulator, merged through LDS at the end) and
//    split the heads when it has more;
//  * the split's result is either the final output (one split) or a partial
//    rounded to bf16 plus its fp32 log2-domain log-sum-exp for the merge.
//
// A call whose grid of splits would run in many rounds (ragged or paged
// batches) takes the persistent form at the end of this file instead: 512
// resident workgroups take the splits that hold tokens from a device-side
// list (gqa_plan.hip) and compute each exactly as above, streaming from one
// split into the next without a start-up pause.
#pragma once

#include "device_common.h"
#include "kvattn_internal.h"
#include "lds_copy.h"

namespace kvattn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kGqaTileBytes = 16384;           // bytes per tensor and tile
constexpr int kGqaStageBytes = 2 * kGqaTileBytes;  // K tile, then V tile
constexpr int kGqaTblSlots = 2304;             // block-table entries staged in LDS
constexpr int kGqaRedFloatsPerWave = 34 * 64;  // 32 accumulators + max + sum, per lane
constexpr float kGqaRescaleSlack = 8.f;        // log2 units

// The (sequence, KV head, split) a workgroup owns, and its token range.
struct GqaWork {
  int b, j, split;
  int t_lo;     // tokens before t_lo lie before a sliding window (masked)
  int t_begin;  // first token of the split (a multiple of the tile size past window_base)
  int t_end;
  int n_tiles;
  bool final_out;
};

// Decode the workgroup's work item; false if the workgroup has nothing to do.
template <int kTile>
__device__ __forceinline__ bool gqa_work(const DecodeArgs& a, GqaWork& w) {
  const int units = a.batch * a.num_kv_heads;
  int unit;
  if ((units & 7) == 0) {
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    w.split = slot % a.n_split;
    unit = (slot / a.n_split) * 8 + xcd;
  } else {
    w.split = blockIdx.x % a.n_split;
    unit = blockIdx.x / a.n_split;
  }
  if (unit >= units) return false;
  w.b = unit / a.num_kv_heads;
  w.j = unit - w.b * a.num_kv_heads;
  const int len = clamp_len(a.seq_lens[w.b], a.len_cap);
  w.t_lo = window_first(len, a.window);
  w.t_begin = window_base(len, a.window) + w.split * a.split_tokens;
  w.final_out = (a.n_split == 1);
  if (!w.final_out && w.t_begin >= len) return false;  // the merge only reads splits that hold tokens
  // The last split ends at the sequence's end: a window's splits are sized
  // for the window, and the last one also takes the tokens of its aligned
  // start (otherwise n_split splits reach past the end anyway).
  w.t_end = w.split == a.n_split - 1 ? len : min(len, w.t_begin + a.split_tokens);
  const int ntok = w.t_end - w.t_begin;
  w.n_tiles = ntok > 0 ? (ntok + kTile - 1) / kTile : 0;
  return true;
}

// HBM -> LDS copies of the split's tiles.  A tile is 32 wave instructions
// (16 for K, 16 for V) of kRows rows x kChunks 16-byte chunks; wave w issues
// instructions 8w .. 8w+7.  Lane l of instruction i writes LDS slot (row
// kRows*(i%16) + l/kChunks, chunk l%kChunks), which holds logical chunk
// (l%kChunks) ^ swz(row).  Rows past the split's end re-read its last row
// (masked out of the softmax); an out-of-range table entry reads an
// in-bounds stand-in row.  Without an LDS table (tbl_lds null, the persistent
// kernel) the general path reads the block table from global memory.
template <class F>
struct GqaCopier {
  static constexpr int kRows = 1024 / F::kRowB;
  static constexpr int kChunks = F::kRowB / 16;
  static constexpr int kRowShift = kRows == 4 ? 2 : 3;
  static_assert(kRows == (1 << kRowShift), "rows per copy instruction");

  const DecodeArgs& a;
  const unsigned char* kbase;
  const unsigned char* vbase;
  const int32_t* table_row;
  int* tbl;
  int64_t head_rows;  // contiguous: first row of (b, j)
  int j, t_end, bs, win_first, wave, lane, tid;
  bool paged, paged_fast;
  uint32_t dpo[4];

  __device__ __forceinline__ GqaCopier(const DecodeArgs& args, const GqaWork& w, int* tbl_lds, int wave_, int tid_)
      : a(args), tbl(tbl_lds), j(w.j), t_end(w.t_end), wave(wave_), lane(tid_ & 63), tid(tid_) {
    kbase = static_cast<const unsigned char*>(a.k);
    vbase = static_cast<const unsigned char*>(a.v);
    paged = a.block_size != 0;
    bs = a.block_size;
    bind(w);
    win_first = 0;
    // Paged fast path: an instruction's rows start at a multiple of kRows
    // tokens and so lie in one block; the per-lane byte offset depends on
    // the instruction's row group mod 4 only (swz has period 4 in it).
    paged_fast = paged && a.block_shift >= kRowShift;
#pragma unroll
    for (int u4 = 0; u4 < 4; ++u4) {
      const int row = kRows * u4 + lane / kChunks;
      dpo[u4] = (uint32_t)((lane / kChunks) * F::kRowB + ((lane % kChunks) ^ F::swz(row)) * 16);
    }
  }

  // Point the copies at another work item (the persistent kernel).
  __device__ __forceinline__ void bind(const GqaWork& w) {
    j = w.j;
    t_end = w.t_end;
    table_row = paged ? a.block_table + (int64_t)w.b * a.max_blocks : nullptr;
    head_rows = (int64_t)(w.b * a.num_kv_heads + w.j) * a.cache_len;
  }

  __device__ __forceinline__ void load_window(int first) {
    const int last_needed = (t_end - 1) / bs;
    const int count = min(kGqaTblSlots, last_needed - first + 1);
    for (int i = tid; i < count; i += 256) tbl[i] = table_row[first + i];
    win_first = first;
  }

  // Stage the split's first block-table entries (plain loads, before any copy is in flight).
  __device__ __forceinline__ void stage_table(int t_begin, int n_tiles) {
    if (!paged) return;
    if (n_tiles > 0) load_window(t_begin / bs);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the table lands before any copy is addressed
    __syncthreads();
  }

  __device__ __forceinline__ void issue(int t0, uint32_t stage_base) {
    if (paged && tbl != nullptr && (min(t0 + F::kTile, t_end) - 1) / bs >= win_first + kGqaTblSlots) {
      // slide the table window (drains the copies in flight)
      __builtin_amdgcn_s_waitcnt(0x0070);
      __syncthreads();
      load_window(t0 / bs);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
    }
    if (paged_fast && t0 + F::kTile <= t_end) {
      // Full tile of a power-of-two paged cache: each instruction's table
      // entry is a wave-uniform scalar load (counted by lgkmcnt, so the
      // copies in flight are left alone) and its address one scalar base
      // plus a per-lane offset fixed for the kernel.
      const int tw = t0 + (F::kTile / 2) * (wave & 1);  // first token of this wave's 8 instructions
      const int32_t* ep[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) ep[u] = table_row + ((tw + kRows * u) >> a.block_shift);
      int e[8];
      asm volatile(
          "s_load_dword %0, %8, 0x0\n\ts_load_dword %1, %9, 0x0\n\ts_load_dword %2, %10, 0x0\n\t"
          "s_load_dword %3, %11, 0x0\n\ts_load_dword %4, %12, 0x0\n\ts_load_dword %5, %13, 0x0\n\t"
          "s_load_dword %6, %14, 0x0\n\ts_load_dword %7, %15, 0x0\n\ts_waitcnt lgkmcnt(0)"
          : "=&s"(e[0]), "=&s"(e[1]), "=&s"(e[2]), "=&s"(e[3]), "=&s"(e[4]), "=&s"(e[5]), "=&s"(e[6]), "=&s"(e[7])
          : "s"(ep[0]), "s"(ep[1]), "s"(ep[2]), "s"(ep[3]), "s"(ep[4]), "s"(ep[5]), "s"(ep[6]), "s"(ep[7])
          : "memory");
      const unsigned char* tbase = (wave >> 1) == 0 ? kbase : vbase;  // waves 0-1 copy K, 2-3 copy V
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int inst = wave * 8 + u;
        const int tg = tw + kRows * u;  // first token of the instruction's rows
        const int64_t row0 = (e[u] >= 0 && (int64_t)e[u] < a.cache_len)
                                 ? ((int64_t)e[u] * a.num_kv_heads + j) * bs + (tg & (bs - 1))
                                 : 0;  // out-of-range entry: in-bounds stand-in rows
        dma16s(dpo[u & 3], tbase + row0 * F::kRowB,
               stage_base + (inst >> 4) * kGqaTileBytes + (inst & 15) * 1024);
      }
      return;
    }
    // Table lookups first (all in flight together), then the source
    // addresses, then the copies.
    int tok[8], blk[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int row = kRows * ((wave * 8 + u) & 15) + lane / kChunks;
      tok[u] = min(t0 + row, t_end - 1);
      // The staged table window, or (no LDS table) the block table itself.
      if (paged) blk[u] = tbl != nullptr ? tbl[tok[u] / bs - win_first] : table_row[tok[u] / bs];
    }
    // Global table entries: one visible wait for all of them here, so that
    // no wait between the copies below drains the ones already issued.
    if (paged && tbl == nullptr) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int inst = wave * 8 + u;
      const int row = kRows * (inst & 15) + lane / kChunks;
      const int chunk = (lane % kChunks) ^ F::swz(row);
      int64_t row_index = head_rows + tok[u];
      if (paged) {
        const bool in_range = blk[u] >= 0 && (int64_t)blk[u] < a.cache_len;  // else an in-bounds stand-in row
        const int64_t b64 = in_range ? blk[u] : 0;
        row_index = in_range ? (b64 * a.num_kv_heads + j) * bs + tok[u] % bs : 0;
      }
      const unsigned char* src = ((inst >> 4) == 0 ? kbase : vbase) + row_index * F::kRowB + chunk * 16;
      dma16(src, stage_base + (inst >> 4) * kGqaTileBytes + (inst & 15) * 1024);
    }
  }
};

// The attention side of a workgroup on the 16x16 matrix-core tiling: HBW
// 16-head blocks per wave, WH waves sharing one head block by tokens.  The
// format F supplies the query fragments and the score and value products of
// one unit of kUnit tokens (16 or 32).
template <class F, int HBW, int WH>
struct GqaAttn16 {
  static_assert(WH == 1 || HBW == 1, "token-split waves own one head block");
  static constexpr int kUnit = F::template unit_tokens<WH>();
  static constexpr int kSub = kUnit / 16;

  typename F::template Frags<HBW> fr;
  f32x4 acc[HBW][8];
  float m_ref[HBW], l_run[HBW];
  float s_log2, v_scale;
  int hb0, ts, lane, n16, grp;

  __device__ __forceinline__ GqaAttn16(const DecodeArgs& a, const GqaWork& w, int wave, int lane_) : lane(lane_) {
    n16 = lane & 15;
    grp = lane >> 4;
    hb0 = (wave / WH) * HBW;  // first 16-head block of this wave
    ts = wave % WH;           // this wave's token slot within a tile
    s_log2 = a.scale_log2 * F::k_scale(a, w.j);
    v_scale = F::v_scale(a, w.j);
    const uint16_t* qg =
        static_cast<const uint16_t*>(a.q) + ((int64_t)w.b * a.num_q_heads + (int64_t)w.j * a.group) * kHeadDim;
    fr.init(qg, hb0, a.group, lane);
#pragma unroll
    for (int hbi = 0; hbi < HBW; ++hbi) {
      m_ref[hbi] = -INFINITY;
      l_run[hbi] = 0.f;
#pragma unroll
      for (int db = 0; db < 8; ++db) acc[hbi][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  // One landed tile: the wave's units of kUnit tokens.
  __device__ __forceinline__ void tile(const unsigned char* stage, int t0, int t_end, int t_lo) {
    for (int u0 = ts * kUnit; u0 < F::kTile; u0 += WH * kUnit) {
      if (t0 + u0 >= t_end) break;
      f32x4 s[HBW][kSub];
      fr.template scores<kSub>(stage, u0, s);
#pragma unroll
      for (int hbi = 0; hbi < HBW; ++hbi) {
        // s[hbi][sb][v] = q(head n16) . k(token t0 + u0 + 16*sb + 4*grp + v)
        float sv[4 * kSub];
#pragma unroll
        for (int sb = 0; sb < kSub; ++sb)
#pragma unroll
          for (int v = 0; v < 4; ++v) sv[4 * sb + v] = s[hbi][sb][v] * s_log2;
        if (t0 + u0 + kUnit > t_end || t0 + u0 < t_lo) {
#pragma unroll
          for (int e = 0; e < 4 * kSub; ++e) {
            const int t = t0 + u0 + 16 * (e >> 2) + 4 * grp + (e & 3);
            if (t >= t_end || t < t_lo) sv[e] = -INFINITY;
          }
        }
        float mt = sv[0];
#pragma unroll
        for (int e = 1; e < 4 * kSub; ++e) mt = fmaxf(mt, sv[e]);
        mt = max_over_row_groups(mt);
        const bool need = mt > m_ref[hbi] + kGqaRescaleSlack;  // also true while m_ref is -inf
        if (__any(need)) {
          const float m_new = need ? mt : m_ref[hbi];
          const float alpha = fast_exp2(m_ref[hbi] - m_new);
          m_ref[hbi] = m_new;
          l_run[hbi] *= alpha;
#pragma unroll
          for (int db = 0; db < 8; ++db) acc[hbi][db] *= alpha;
        }
        // m_ref stays -inf while every token so far lay before a sliding
        // window; its probabilities are then 0 (not -inf - -inf = NaN).
        const float m_use = m_ref[hbi] == -INFINITY ? 0.f : m_ref[hbi];
        uint32_t pk[2 * kSub];
#pragma unroll
        for (int e = 0; e < 2 * kSub; ++e) {
          pk[e] = pack_bf16x2(fast_exp2(sv[2 * e] - m_use), fast_exp2(sv[2 * e + 1] - m_use));
          l_run[hbi] = add_bf16x2(pk[e], l_run[hbi]);  // normalise with the weights the matrix core sees
        }
        fr.template values<kSub>(stage, u0, pk, acc[hbi]);
      }
    }
  }

  // Merge the token-split waves through `red` (an idle 32 KiB ring stage),
  // then write the output or the split's partial; the waves of a head block
  // other than its first only hand over their state.  Lane l holds
  // O^T[d = 16*db + 4*grp + v][head n16].
  __device__ __forceinline__ void finish(const DecodeArgs& a, const GqaWork& w, unsigned char* red_stage, int wave) {
#pragma unroll
    for (int hbi = 0; hbi < HBW; ++hbi) l_run[hbi] = sum_over_row_groups(l_run[hbi]);
    if constexpr (WH > 1) {
      static_assert((4 / WH) * (WH - 1) * kGqaRedFloatsPerWave * 4 <= kGqaStageBytes, "merge state fits a stage");
      // Slot of token slot t (1 .. WH-1) of this wave's head block.
      const int slot0 = (wave / WH) * (WH - 1) - 1;
      __syncthreads();
      float* red = reinterpret_cast<float*>(red_stage);
      if (ts != 0) {
        float* mine = red + (slot0 + ts) * kGqaRedFloatsPerWave;
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
          for (int v = 0; v < 4; ++v) mine[(db * 4 + v) * 64 + lane] = acc[0][db][v];
        mine[32 * 64 + lane] = m_ref[0];
        mine[33 * 64 + lane] = l_run[0];
      }
      __syncthreads();
      if (ts != 0) return;
#pragma unroll
      for (int w2 = 1; w2 < WH; ++w2) {
        const float* other = red + (slot0 + w2) * kGqaRedFloatsPerWave;
        const float m2 = other[32 * 64 + lane];
        const float l2 = other[33 * 64 + lane];
        const float M = fmaxf(m_ref[0], m2);
        if (M == -INFINITY) continue;
        const float a1 = fast_exp2(m_ref[0] - M);
        const float a2 = fast_exp2(m2 - M);
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[0][db][v] = acc[0][db][v] * a1 + other[(db * 4 + v) * 64 + lane] * a2;
        l_run[0] = l_run[0] * a1 + l2 * a2;
        m_ref[0] = M;
      }
    }
    const int r = a.group;
#pragma unroll
    for (int hbi = 0; hbi < HBW; ++hbi) {
      const int head = (hb0 + hbi) * 16 + n16;
      if (head >= r) continue;
      const int64_t row = (int64_t)w.b * a.num_q_heads + (int64_t)w.j * r + head;
      const float l = l_run[hbi];
      const bool empty = !(l > 0.f);
      const float inv = empty ? 0.f : v_scale / l;
      const float lse2 = empty ? -INFINITY : m_ref[hbi] + __log2f(l);
      // Final output, or the split's partial rounded to bf16 (the merge
      // weighs the splits in fp32 from their fp32 log-sum-exps).
      uint16_t* o = w.final_out
                        ? static_cast<uint16_t*>(a.out) + row * kHeadDim
                        : reinterpret_cast<uint16_t*>(a.part_o) + (row * a.n_split + w.split) * kHeadDim;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const uint32_t lo = pack_bf16x2(acc[hbi][db][0] * inv, acc[hbi][db][1] * inv);
        const uint32_t hi = pack_bf16x2(acc[hbi][db][2] * inv, acc[hbi][db][3] * inv);
        *reinterpret_cast<uint2*>(o + 16 * db + 4 * grp) = make_uint2(lo, hi);
      }
      if (grp == 0) {
        if (!w.final_out) a.part_lse[row * a.n_split + w.split] = lse2;
        else if (a.lse != nullptr) a.lse[row] = lse2 * kLn2;
      }
    }
  }
};

// The split-K kernel body for cache format F with attention side Attn.
template <class F, class Attn>
__device__ __forceinline__ void gqa_split_body(const DecodeArgs& a) {
  GqaWork w;
  if (!gqa_work<F::kTile>(a, w)) return;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: wave-derived values in SGPRs

  __shared__ __attribute__((aligned(1024))) unsigned char ring[2][kGqaStageBytes];
  __shared__ int tbl[kGqaTblSlots];

  Attn attn(a, w, wave, tid & 63);  // fetches the queries
  GqaCopier<F> cp(a, w, tbl, wave, tid);
  cp.stage_table(w.t_begin, w.n_tiles);

  if (w.n_tiles > 0) cp.issue(w.t_begin, (uint32_t)(uintptr_t)&ring[0][0]);
  // The queries and the first tile were fetched together (one HBM latency at
  // start-up, not two).  Let them all land here: the compiler cannot see the
  // copies in the vector-memory counter, and a wait it placed on the query
  // loads inside the loop would drain the copies in flight every tile.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  for (int it = 0; it < w.n_tiles; ++it) {
    // Tile `it` has landed (nothing else is in flight here); then the next
    // tile's copies go into the other stage, which every wave is done with.
    wait_copies_and_sync<0>();
    if (it + 1 < w.n_tiles)
      cp.issue(w.t_begin + (it + 1) * F::kTile, (uint32_t)(uintptr_t)&ring[(it + 1) & 1][0]);
    attn.tile(ring[it & 1], w.t_begin + it * F::kTile, w.t_end, w.t_lo);
  }
  attn.finish(a, w, &ring[0][0], wave);
}

// The work of one item of the device-side list (gqa_plan.hip).  The
// sliding window's first attended token is looked up only when `with_lo`.
template <int kTile>
__device__ __forceinline__ GqaWork gqa_item_work(const DecodeArgs& a, const int4& item, bool with_lo) {
  GqaWork w;
  w.b = item.x / a.num_kv_heads;
  w.j = item.x - w.b * a.num_kv_heads;
  w.split = item.y;
  w.t_begin = item.z;
  w.t_end = item.w;
  w.t_lo = with_lo && a.window > 0 ? window_first(clamp_len(a.seq_lens[w.b], a.len_cap), a.window) : 0;
  w.n_tiles = (w.t_end - w.t_begin + kTile - 1) / kTile;
  w.final_out = false;
  return w;
}

// Persistent form of the split kernel, for calls whose grid of splits would
// run in many rounds (ragged or paged batches).  Two resident workgroups per
// compute unit take the items of the device-side list one at a time from a
// counter (a vector atomic, one per item), in list order; an item is computed
// exactly as the grid-per-split body computes its split, so which workgroup
// takes it does not change any result.  A workgroup claims its next item
// three tiles before the current one ends (late enough that the items go to
// the workgroups that free up first, which keeps the longest-first order of
// the list effective at the end; early enough to hide the claim and the
// lookup), and its last tile iteration issues the copies of that item's
// first tile: the cache stream does not stop between items, and only the
// next queries' latency remains at an item boundary.  Only cache layouts
// whose full tiles need no LDS table take this form (contiguous, or paged
// with power-of-two blocks of at least one copy instruction's rows).
template <class F, class Attn>
__device__ __forceinline__ void gqa_persistent_body(const DecodeArgs& a) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: wave-derived values in SGPRs

  __shared__ __attribute__((aligned(1024))) unsigned char ring[2][kGqaStageBytes];
  __shared__ int4 s_item;

  const int n_items = a.items_ctl[0];
  int* const claim = a.items_ctl + 1;
  const int4 none = make_int4(-1, 0, 0, 0);
  auto lookup = [&](int t) __attribute__((always_inline)) { return t < n_items ? a.items[t] : none; };
  auto published = [&]() __attribute__((always_inline)) {
    const int4 v = s_item;
    return make_int4(__builtin_amdgcn_readfirstlane(v.x), __builtin_amdgcn_readfirstlane(v.y),
                     __builtin_amdgcn_readfirstlane(v.z), __builtin_amdgcn_readfirstlane(v.w));
  };

  if (tid == 0) s_item = lookup(atomicAdd(claim, 1));
  __syncthreads();
  int4 cur = published();
  if (cur.x < 0) return;

  auto stage = [&](uint32_t t) __attribute__((always_inline)) { return (uint32_t)(uintptr_t)&ring[t & 1][0]; };
  uint32_t gt = 0;          // tiles this workgroup has consumed; tile gt sits in stage gt & 1
  bool head_issued = false; // the current item's first tile is already in flight
  GqaCopier<F> cp(a, gqa_item_work<F::kTile>(a, cur, false), nullptr, wave, tid);
  while (true) {
    const GqaWork w = gqa_item_work<F::kTile>(a, cur, true);
    Attn attn(a, w, wave, tid & 63);  // fetches the queries
    cp.bind(w);
    if (!head_issued) cp.issue(w.t_begin, stage(gt));
    // Queries, the window bound and the first tile land here (a visible
    // wait, so that the compiler places none inside the loop).
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    // The next item: thread 0 claims it at iteration c, looks it up at c+1
    // and publishes it at c+2; every wave reads it at c+3, the last iteration
    // of an item of four tiles or more.
    const int n = w.n_tiles;
    const int c = n > 4 ? n - 4 : 0;
    int ticket = n_items;
    int4 looked = none, nxt = none;
    for (int it = 0; it < n; ++it) {
      wait_copies_and_sync<0>();
      __builtin_amdgcn_s_waitcnt(0x0F70);  // nothing is in flight: the claim and lookup below have landed
      if (it == c + 3) nxt = published();
      if (tid == 0) {
        if (it == c) ticket = atomicAdd(claim, 1);
        if (it == c + 1) looked = lookup(ticket);
        if (it == c + 2) s_item = looked;
      }
      if (it + 1 < n) {
        cp.issue(w.t_begin + (it + 1) * F::kTile, stage(gt + 1));
      } else if (nxt.x >= 0) {
        const GqaWork wn = gqa_item_work<F::kTile>(a, nxt, false);
        cp.bind(wn);
        cp.issue(wn.t_begin, stage(gt + 1));
      }
      attn.tile(ring[gt & 1], w.t_begin + it * F::kTile, w.t_end, w.t_lo);
      ++gt;
    }
    // The last tile's stage is free for the token-split merge; the other one
    // receives the next item's first tile.
    attn.finish(a, w, ring[(gt - 1) & 1], wave);
    head_issued = nxt.x >= 0;
    if (n < c + 4) {
      // An item of fewer than four tiles ends before the next one is known.
      if (tid == 0) {
        if (n < c + 2) looked = lookup(ticket);
        if (n < c + 3) s_item = looked;
      }
      __syncthreads();
      nxt = published();
      __syncthreads();  // s_item is rewritten during the next item
    }
    if (nxt.x < 0) break;
    cur = nxt;
  }
}

}  // namespace kvattn
