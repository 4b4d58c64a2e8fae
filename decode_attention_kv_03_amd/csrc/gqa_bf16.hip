// Grouped-query decode attention, bf16 cache, split-K flash-decode on the
// gfx950 matrix cores.
//
// What it computes ("MQA, GQA, and MLA", sections 2-4 and 8): for sequence b
// and KV head j, the r = h/g query heads j*r .. j*r+r-1 attend over the
// cached K/V rows of head j; each K/V byte is fetched from HBM once per
// decode step and serves all r heads of its group (index, never repeat).
//
// Work decomposition.  One workgroup (4 waves) owns one (sequence, KV head,
// split) and walks the split's tokens in 64-token tiles:
//  * tiles stream from HBM straight into a two-stage LDS ring with
//    global_load_lds_dwordx4 carrying the non-temporal hint (the cache is
//    read once per step); one tile is in flight while the other is consumed.
//    The copies are issued as inline assembly and awaited with explicit
//    vmcnt counts, so the compiler never drains them before an LDS read;
//  * rows are stored unpadded (256 B) with their 16-byte chunks XOR-swizzled
//    by row, and the score reads visit the dims in the order kchunk() below,
//    so neither LDS read pattern stalls on bank conflicts
//    (SQ_LDS_BANK_CONFLICT counts none for this kernel);
//  * a paged cache's block-table slice for the split is staged in LDS first,
//    so per-row block lookups never wait on the vector-memory counter;
//  * scores are S^T = K_tile * Q^T on v_mfma_f32_16x16x32_bf16 (16 tokens x 16
//    query heads, K from LDS, Q^T fragments in registers);
//  * the online softmax runs in the matrix-core output layout (lane l: query
//    head l%16, tokens 4*(l/16)+v), with lazy rescaling: the reference max
//    only moves when a tile's max exceeds it by more than 8 (log2 units);
//  * P V is accumulated as O^T = V^T * P^T; V^T comes from the row-major V
//    tile through the gfx950 LDS transpose read (ds_read_b64_tr_b16).  Waves
//    that own 32 tokens of a tile use 16x16x32 MFMAs (two transpose reads
//    per operand), waves that own 16 use 16x16x16;
//  * waves split the tile's tokens when a group has at most 32 heads (each
//    keeps its own max/sum/accumulator, merged through LDS at the end) and
//    split the heads when it has more;
//  * the split's result is either the final output (one split) or an fp32
//    partial (rounded to bf16) plus its fp32 log2-domain log-sum-exp for the
//    merge kernel.
#include <hip/hip_ext.h>

#include "device_common.h"
#include "kvattn_internal.h"
#include "lds_copy.h"

namespace kvattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;                   // tokens per tile
constexpr int kRowB = kHeadDim * 2;         // 256 B per K or V row
constexpr int kTileB = kTile * kRowB;       // 16 KiB per tensor and tile
constexpr int kStageB = 2 * kTileB;         // K tile, then V tile
constexpr int kTblSlots = 2304;             // block-table entries staged in LDS
constexpr int kRedFloatsPerWave = 34 * 64;  // 32 accumulators + max + sum, per lane
constexpr float kRescaleSlack = 8.f;        // log2 units

// Chunk swizzle of a 256-byte row: XOR of the 4-bit chunk index.  Rows r and
// r+16 share it; 16 consecutive rows get 16 distinct values and any 8
// consecutive rows 8 distinct pairs, which is what the two read patterns need.
__device__ __forceinline__ int swz(int row) { return ((row & 7) << 1) | ((row >> 3) & 1); }

// Logical 16-byte chunk (8 dims) that lane group grp reads at score step kk.
// The reduction over the 128 dims may visit them in any order shared by the
// K and Q^T operands.  Giving the four lane groups chunks that differ in bits
// 1-2 (and the steps bits 0 and 3) keeps lanes l and l+16, which read the
// same row, off the banks that the XOR with swz() aligns across rows r and
// r+8; the order 4*kk + grp measured 4 bank-conflict cycles per score read.
__device__ __forceinline__ int kchunk(int kk, int grp) { return (kk & 1) | (grp << 1) | ((kk >> 1) << 3); }

template <int HBW, int WH>
__global__ __launch_bounds__(256, 2) void gqa_split_bf16(DecodeArgs a) {
  static_assert(WH == 1 || HBW == 1, "token-split waves own one head block");
  constexpr int NST = 2;  // LDS ring stages
  constexpr int kUnit = WH == 4 ? 16 : 32;  // tokens a wave handles per step
  // 1-D grid, XCD-aware: workgroup w runs on XCD w % 8 and all splits of one
  // (sequence, KV head) group share a residue, so the group's queries are
  // fetched into one XCD's L2.
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int split = slot % a.n_split;
  const int unit = (slot / a.n_split) * 8 + xcd;
  if (unit >= a.batch * a.num_kv_heads) return;
  const int b = unit / a.num_kv_heads, j = unit - b * a.num_kv_heads;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: wave-derived values in SGPRs
  const int n16 = lane & 15, grp = lane >> 4;
  const int r = a.group, h = a.num_q_heads;

  const int len = clamp_len(a.seq_lens[b], a.len_cap);
  const int t_lo = window_first(len, a.window);  // tokens before t_lo are outside the window
  const int t_begin = window_base(len, a.window) + split * a.split_tokens;
  const bool final_out = (a.n_split == 1);
  if (!final_out && t_begin >= len) return;  // the merge only reads splits that hold tokens
  const int t_end = min(len, t_begin + a.split_tokens);
  const int ntok = t_end - t_begin;
  const int n_tiles = ntok > 0 ? (ntok + kTile - 1) / kTile : 0;

  __shared__ __attribute__((aligned(1024))) unsigned char ring[NST][kStageB];
  __shared__ int tbl[kTblSlots];

  const int hb0 = (wave / WH) * HBW;  // first 16-head block of this wave
  const int ts = wave % WH;           // this wave's token slot within a tile

  // Q^T fragments: lane l holds head (block*16 + l%16), dims 8*kchunk(kk, l/16) .. +7.
  const uint16_t* qg = static_cast<const uint16_t*>(a.q) + ((int64_t)b * h + (int64_t)j * r) * kHeadDim;
  bf16x8 qf[HBW][4];
#pragma unroll
  for (int hbi = 0; hbi < HBW; ++hbi) {
    const int head = (hb0 + hbi) * 16 + n16;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (head < r) v = *reinterpret_cast<const u32x4*>(qg + head * kHeadDim + 8 * kchunk(kk, grp));
      qf[hbi][kk] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // Paged cache: stage this split's block-table entries in LDS (plain loads,
  // before any copy is in flight).  A split whose slice exceeds the LDS table
  // reloads a window when a tile needs entries past it.
  const bool paged = a.block_size != 0;
  const int bs = a.block_size;
  const int32_t* table_row = paged ? a.block_table + (int64_t)b * a.max_blocks : nullptr;
  int win_first = 0;
  auto load_window = [&](int first) {
    const int last_needed = (t_end - 1) / bs;
    const int count = min(kTblSlots, last_needed - first + 1);
    for (int i = tid; i < count; i += 256) tbl[i] = table_row[first + i];
    win_first = first;
  };
  if (paged) {
    if (n_tiles > 0) load_window(t_begin / bs);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the table lands before any copy is addressed
    __syncthreads();
  }

  f32x4 acc[HBW][8];
  float m_ref[HBW], l_run[HBW];
#pragma unroll
  for (int hbi = 0; hbi < HBW; ++hbi) {
    m_ref[hbi] = -INFINITY;
    l_run[hbi] = 0.f;
#pragma unroll
    for (int db = 0; db < 8; ++db) acc[hbi][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const uint16_t* kbase = static_cast<const uint16_t*>(a.k);
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v);
  const int64_t head_rows = (int64_t)(b * a.num_kv_heads + j) * a.cache_len;  // contiguous: first row of (b, j)

  // Copies of one tile: 32 wave instructions (16 for K, 16 for V) of 4 rows
  // x 16 chunks; wave w issues instructions 8w .. 8w+7.  Lane l of
  // instruction i writes LDS slot (row 4*(i%16) + l/16, chunk l%16), which
  // holds logical chunk (l%16) ^ swz(row).  Rows past the split's end
  // re-read its last row (masked out of the softmax).
  // Per-lane byte offsets of the paged fast path: lane l of an instruction
  // with row group rg copies row 4*rg + l/16 (l/16-th of its four rows), slot
  // l%16, which holds logical chunk (l%16) ^ swz(row); swz depends on rg mod 4
  // only (rows of one wave's instructions are 32*(wave&1) + 4*u + l/16).
  const bool paged_fast = paged && a.block_shift >= 2;
  uint32_t dpo[4];
#pragma unroll
  for (int u4 = 0; u4 < 4; ++u4) {
    const int row = 4 * u4 + (lane >> 4);
    dpo[u4] = (uint32_t)(((lane >> 4) * kHeadDim + ((lane & 15) ^ swz(row)) * 8) * 2);
  }
  auto issue_tile = [&](int t0, int stage) __attribute__((always_inline)) {
    if (paged && (min(t0 + kTile, t_end) - 1) / bs >= win_first + kTblSlots) {
      // slow path: slide the table window (drains the copies in flight)
      __builtin_amdgcn_s_waitcnt(0x0070);
      __syncthreads();
      load_window(t0 / bs);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
    }
    const uint32_t stage_base = (uint32_t)(uintptr_t)&ring[stage][0];
    if (paged_fast && t0 + kTile <= t_end) {
      // Paged, full tile, power-of-two block size >= 4: an instruction's four
      // rows start at a multiple of 4 tokens and so lie in one block.  Its
      // table entry is a wave-uniform scalar load (counted by lgkmcnt, so the
      // copies in flight are left alone) and its address one scalar base plus
      // a per-lane offset fixed for the kernel (dpo, by instruction mod 4).
      const int tw = t0 + 32 * (wave & 1);  // first token of this wave's 8 instructions
      const int32_t* ep[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) ep[u] = table_row + ((tw + 4 * u) >> a.block_shift);
      int e[8];
      asm volatile(
          "s_load_dword %0, %8, 0x0\n\ts_load_dword %1, %9, 0x0\n\ts_load_dword %2, %10, 0x0\n\t"
          "s_load_dword %3, %11, 0x0\n\ts_load_dword %4, %12, 0x0\n\ts_load_dword %5, %13, 0x0\n\t"
          "s_load_dword %6, %14, 0x0\n\ts_load_dword %7, %15, 0x0\n\ts_waitcnt lgkmcnt(0)"
          : "=&s"(e[0]), "=&s"(e[1]), "=&s"(e[2]), "=&s"(e[3]), "=&s"(e[4]), "=&s"(e[5]), "=&s"(e[6]), "=&s"(e[7])
          : "s"(ep[0]), "s"(ep[1]), "s"(ep[2]), "s"(ep[3]), "s"(ep[4]), "s"(ep[5]), "s"(ep[6]), "s"(ep[7])
          : "memory");
      const uint16_t* tbase = (wave >> 1) == 0 ? kbase : vbase;  // waves 0-1 copy K, 2-3 copy V
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int inst = wave * 8 + u;
        const int tg = tw + 4 * u;  // first token of the instruction's four rows
        const int64_t row0 = (e[u] >= 0 && (int64_t)e[u] < a.cache_len)
                                 ? ((int64_t)e[u] * a.num_kv_heads + j) * bs + (tg & (bs - 1))
                                 : 0;  // out-of-range entry: in-bounds stand-in rows
        dma16s(dpo[u & 3], tbase + row0 * kHeadDim, stage_base + (inst >> 4) * kTileB + (inst & 15) * 1024);
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int inst = wave * 8 + u;
      const int tensor = inst >> 4, rg = inst & 15;
      const int row = 4 * rg + (lane >> 4);
      const int chunk = (lane & 15) ^ swz(row);
      const int t = min(t0 + row, t_end - 1);
      int64_t off;
      if (!paged) {
        off = (head_rows + t) * kHeadDim;
      } else {
        const int q = t / bs;
        const int blk = tbl[q - win_first];
        off = (blk >= 0 && (int64_t)blk < a.cache_len)
                  ? (((int64_t)blk * a.num_kv_heads + j) * bs + (t - q * bs)) * kHeadDim
                  : 0;  // out-of-range entry: an in-bounds stand-in row
      }
      const uint16_t* src = (tensor == 0 ? kbase : vbase) + off + chunk * 8;
      dma16(src, stage_base + tensor * kTileB + rg * 1024);
    }
  };

  // Per-lane LDS byte offsets inside a tile.  K reads (A operand of the
  // scores): row n16 of a 16-token subtile, chunk kchunk(kk, grp).  V transposing
  // reads: rows 4*grp + (n16/4) (+16 per subtile), 8-byte piece n16%4 of the
  // 16-column block db, i.e. chunk 2*db + (n16%4)/2.
  int koff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) koff[kk] = n16 * kRowB + 16 * (kchunk(kk, grp) ^ swz(n16));
  const int vrow = 4 * grp + (n16 >> 2);
  int voff[8];
#pragma unroll
  for (int db = 0; db < 8; ++db)
    voff[db] = kTileB + vrow * kRowB + 16 * ((2 * db + ((n16 & 3) >> 1)) ^ swz(vrow)) + 8 * (n16 & 1);

  if (n_tiles > 0) issue_tile(t_begin, 0);
  // The queries and the first tiles were fetched together (one HBM latency at
  // start-up, not two).  Let them all land here: the compiler cannot see the
  // copies in the vector-memory counter, and a wait it placed on the query
  // loads inside the loop would drain the copies in flight every tile.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  for (int it = 0; it < n_tiles; ++it) {
    // Tile `it` must have landed (nothing else is in flight here); then the
    // next tile's copies go into the other stage, which every wave is done with.
    wait_copies_and_sync<0>();
    if (it + 1 < n_tiles) issue_tile(t_begin + (it + 1) * kTile, (it + 1) % NST);

    const int t0 = t_begin + it * kTile;
    const unsigned char* stage = ring[it % NST];
    const auto* stage_lds = (const __attribute__((address_space(3))) unsigned char*)stage;

    for (int u0 = ts * kUnit; u0 < kTile; u0 += WH * kUnit) {
      if (t0 + u0 >= t_end) break;
      constexpr int kSub = kUnit / 16;
#pragma unroll
      for (int hbi = 0; hbi < HBW; ++hbi) {
        f32x4 s[kSub];
#pragma unroll
        for (int sb = 0; sb < kSub; ++sb) {
          s[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const u32x4 kraw = *reinterpret_cast<const u32x4*>(stage + (u0 + 16 * sb) * kRowB + koff[kk]);
            s[sb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kraw), qf[hbi][kk], s[sb],
                                                            0, 0, 0);
          }
        }
        // s[sb][v] = q(head n16) . k(token t0 + u0 + 16*sb + 4*grp + v)
        float sv[4 * kSub];
#pragma unroll
        for (int sb = 0; sb < kSub; ++sb)
#pragma unroll
          for (int v = 0; v < 4; ++v) sv[4 * sb + v] = s[sb][v] * a.scale_log2;
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
        const bool need = mt > m_ref[hbi] + kRescaleSlack;  // also true while m_ref is -inf
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
        const int vbase_off = u0 * kRowB;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(stage_lds + vbase_off + voff[db]));
          if constexpr (kSub == 1) {
            const i16x4 pb = __builtin_bit_cast(i16x4, (uint2){pk[0], pk[1]});
            acc[hbi][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v0, pb, acc[hbi][db], 0, 0, 0);
          } else {
            // second 16 tokens of the unit: slots 4..7 of the 32-deep operand
            const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4*)(stage_lds + vbase_off + 16 * kRowB + voff[db]));
            const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
            const bf16x8 pb = __builtin_bit_cast(bf16x8, (u32x4){pk[0], pk[1], pk[2], pk[3]});
            acc[hbi][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, acc[hbi][db], 0, 0, 0);
          }
        }
      }
    }
  }

  // Per-head sums: the four lane groups hold different tokens of the same head.
#pragma unroll
  for (int hbi = 0; hbi < HBW; ++hbi) l_run[hbi] = sum_over_row_groups(l_run[hbi]);

  if constexpr (WH > 1) {
    // Waves that split the tile's tokens merge (max, sum, accumulator) through LDS.
    __syncthreads();
    float* red = reinterpret_cast<float*>(&ring[0][0]);
    float* mine = red + wave * kRedFloatsPerWave;
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int v = 0; v < 4; ++v) mine[(db * 4 + v) * 64 + lane] = acc[0][db][v];
    mine[32 * 64 + lane] = m_ref[0];
    mine[33 * 64 + lane] = l_run[0];
    __syncthreads();
    if (ts != 0) return;
#pragma unroll
    for (int w2 = 1; w2 < WH; ++w2) {
      const float* other = red + (wave + w2) * kRedFloatsPerWave;
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

  // Lane l holds O^T[d = 16*db + 4*grp + v][head n16].
#pragma unroll
  for (int hbi = 0; hbi < HBW; ++hbi) {
    const int head = (hb0 + hbi) * 16 + n16;
    if (head >= r) continue;
    const int64_t row = (int64_t)b * h + (int64_t)j * r + head;
    const float l = l_run[hbi];
    const bool empty = !(l > 0.f);
    const float inv = empty ? 0.f : 1.f / l;
    const float lse2 = empty ? -INFINITY : m_ref[hbi] + __log2f(l);
    if (final_out) {
      uint16_t* o = static_cast<uint16_t*>(a.out) + row * kHeadDim;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const uint32_t lo = pack_bf16x2(acc[hbi][db][0] * inv, acc[hbi][db][1] * inv);
        const uint32_t hi = pack_bf16x2(acc[hbi][db][2] * inv, acc[hbi][db][3] * inv);
        *reinterpret_cast<uint2*>(o + 16 * db + 4 * grp) = make_uint2(lo, hi);
      }
      if (a.lse != nullptr && grp == 0) a.lse[row] = lse2 * kLn2;
    } else {
      // Partial output rounded to bf16 (the merge weighs the splits in fp32
      // from their fp32 log-sum-exps).
      uint16_t* po = reinterpret_cast<uint16_t*>(a.part_o) + (row * a.n_split + split) * kHeadDim;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const uint32_t lo = pack_bf16x2(acc[hbi][db][0] * inv, acc[hbi][db][1] * inv);
        const uint32_t hi = pack_bf16x2(acc[hbi][db][2] * inv, acc[hbi][db][3] * inv);
        *reinterpret_cast<uint2*>(po + 16 * db + 4 * grp) = make_uint2(lo, hi);
      }
      if (grp == 0) a.part_lse[row * a.n_split + split] = lse2;
    }
  }
}

}  // namespace

hipError_t launch_gqa_bf16(const DecodeArgs& a, hipStream_t stream, const LaunchEvents& ev) {
  const int64_t units = (int64_t)a.batch * a.num_kv_heads;
  const dim3 grid((unsigned)(8 * ((units + 7) / 8) * a.n_split));
  const dim3 block(256);
  const int head_blocks = (a.group + 15) / 16;
  if (head_blocks == 1) {
    hipExtLaunchKernelGGL((gqa_split_bf16<1, 4>), grid, block, 0, stream, ev.start, ev.stop, 0, a);
  } else if (head_blocks == 2) {
    hipExtLaunchKernelGGL((gqa_split_bf16<1, 2>), grid, block, 0, stream, ev.start, ev.stop, 0, a);
  } else if (head_blocks <= 4) {
    hipExtLaunchKernelGGL((gqa_split_bf16<1, 1>), grid, block, 0, stream, ev.start, ev.stop, 0, a);
  } else if (head_blocks <= 8) {
    hipExtLaunchKernelGGL((gqa_split_bf16<2, 1>), grid, block, 0, stream, ev.start, ev.stop, 0, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvattn
