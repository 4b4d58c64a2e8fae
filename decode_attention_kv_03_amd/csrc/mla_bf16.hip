// Absorbed MLA decode on the gfx950 matrix cores.
//
// What it computes ("MQA, GQA, and MLA", section 5 "MLA, mechanically";
// "Why GQA's KV Cache Savings Don't Fully Reduce TPOT", "What Makes MLA
// Different"): every token's cache row is [c (512) | k^R (64)], shared by
// all heads.  Head i scores its absorbed query [q^C W_uk^T | q^R] (576 wide)
// against the whole row and averages the c parts with the softmax weights;
// the output stays in the 512-wide latent space.  Nothing is reconstructed
// per head, so each cached byte leaves HBM once per decode step.
//
// Both products are dense contractions and run on v_mfma_f32_32x32x16_bf16,
// the shape that sustains the matrix cores' full bf16 rate on this part
// (the 16x16x32 shape issues at well under half of it):
//   S^T[32 tok x 32 heads] = C_tile[32 x 576] * Q^T[576 x 32]
//   O^T[32 cols x 32 heads] += C_tile[:, cols]^T * P^T[32 tok x 32 heads]
// A workgroup (8 waves, two per SIMD) owns one piece of a sequence (a run
// of its tokens, from the device-side plan in mla_plan.hip) and all heads.  Waves pair up per 32-head block: each wave of a pair holds the
// query for half of the 576 dims (18 reduction steps of 16) and the output
// accumulators for one half of the 512 latent columns (8 blocks of 32: the
// lower 256 columns for the first wave, the upper for the second), which
// keeps both under the 256 registers a wave has at two waves per SIMD.  The
// pair swaps partial scores through LDS once per tile.
//
// Data movement.  Tiles of 32 cache rows (36 KiB) stream from HBM straight
// into a three-stage LDS ring with global_load_lds_dwordx4 carrying the
// non-temporal hint (no register staging).  In LDS a tile is stored as
// 36 blocks of 1 KiB, [row half (16 rows)][slab of 4 chunks (64 bytes of
// each row)], one per copy instruction, with the four 16-byte chunks of each
// row XOR-swizzled by (row % 16) / 4.  Every copy instruction then reads one
// wave-uniform base plus the same per-lane offset (no per-tile vector
// address arithmetic), and both LDS read patterns spread over all banks
// (bank-conflict stalls are about 3 % of the kernel's LDS-busy cycles): the
// row-wise reads feeding the score product (16 rows, one chunk) and the
// transposing reads (ds_read_b64_tr_b16, 4 consecutive rows x 16 columns per
// 16-lane group) feeding the value product.  The copies are issued as inline
// assembly and awaited with explicit vmcnt counts followed by a bare
// s_barrier; a full workgroup fence, or the compiler's own alias-based
// waits, would drain every tile in flight.
//
// Online softmax in the matrix-core output layout (lane l: head l%32, tokens
// 8*(v/4) + 4*(l/32) + v%4 of the tile, v = 0..15), with lazy rescaling: the
// running reference max only moves when a tile's max exceeds it by more
// than 8 (log2 units), so the accumulators are rarely rescaled;
// probabilities stay below 2^8, exact in the fp32 accumulators and
// representable in bf16.  The value product reduces over tokens in the same
// per-lane order the scores come out in, so P^T needs no data movement.
#include <hip/hip_ext.h>

#include "device_common.h"
#include "kvattn_internal.h"
#include "lds_copy.h"

namespace kvattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kT = 32;                         // tokens per tile
constexpr int kRowElems = kMlaRow;             // 576 bf16
constexpr int kRowBytes = kRowElems * 2;       // 1152
constexpr int kChunks = kRowBytes / 16;        // 72 16-byte chunks per row
constexpr int kTileBytes = kT * kRowBytes;     // 36864
constexpr int kNBuf = 3;                       // LDS ring stages
constexpr int kWaves = 8;
constexpr int kTileInsts = kT * kChunks / 64;  // 36 wave-wide copies per tile
constexpr int kCopyWaves = kWaves / 2;        // the lagging group (waves 4-7) issues the copies
constexpr int kDmaPer = kTileInsts / kCopyWaves;  // 9 per copying wave
static_assert(kDmaPer * kCopyWaves == kTileInsts && kDmaPer == 9, "wait counts in the main loop assume 9 copies per wave");
constexpr int kSteps = kMlaRow / 16 / 2;       // 18 score reduction steps per wave
constexpr int kColBlocks = kMlaLatent / 32 / 2;  // 8 output column blocks per wave
constexpr int kSxFloats = kWaves * 16 * 64;    // partial-score exchange: 16 floats per lane
constexpr float kRescaleSlack = 8.f;           // log2 units
constexpr int kKDepth = 3;                     // LDS operand reads in flight, score product
constexpr int kVDepth = 3;                     // ... and value product

// LDS byte offset of 16-byte chunk `chunk` (0..71) of tile row `row` (0..31).
__device__ __forceinline__ int lds_chunk(int row, int chunk) {
  const int r = row & 15;
  return (row >> 4) * (kTileBytes / 2) + (chunk >> 2) * 1024 + r * 64 + (((chunk & 3) ^ (r >> 2)) << 4);
}

struct TagFalse { static constexpr bool value = false; };
struct TagTrue { static constexpr bool value = true; };

// Block-table index and in-block slot of token t (paged cache).
__device__ __forceinline__ int block_of(const DecodeArgs& a, int t) {
  return a.block_shift >= 0 ? t >> a.block_shift : t / a.block_size;
}
__device__ __forceinline__ int slot_of(const DecodeArgs& a, int t) {
  return a.block_shift >= 0 ? t & (a.block_size - 1) : t % a.block_size;
}

__global__ __launch_bounds__(kWaves * 64, 1) void mla_split_bf16(DecodeArgs a) {
  // One workgroup per piece of the device-side plan.  1-D grid, XCD-aware:
  // workgroup w runs on XCD w % 8, and XCD x takes the x-th eighth of the
  // pieces, a run of consecutive pieces (so about an eighth of all tokens,
  // and most of a sequence's pieces on one XCD, whose L2 then serves its
  // queries).
  const int n_pieces = a.plan_count[0];
  const int per_xcd = (n_pieces + 7) >> 3;
  const int slot = blockIdx.x >> 3;
  const int piece = (blockIdx.x & 7) * per_xcd + slot;
  if (slot >= per_xcd || piece >= n_pieces) return;
  const int4 pc = a.pieces[piece];
  const int b = pc.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps wave-derived values in SGPRs
  const int pair = wave >> 1, half = wave & 1;
  const int c32 = lane & 31, g = lane >> 5;
  const int h = a.num_q_heads;

  // The piece's tokens (t_begin a multiple of the tile), and whether it is
  // its sequence's only piece (then the output is final).
  const int t_begin = pc.y, t_end = pc.z;
  const bool final_out = pc.w != 0;

  __shared__ __attribute__((aligned(1024))) unsigned char tiles[kNBuf][kTileBytes];
  __shared__ __attribute__((aligned(16))) float sx[kSxFloats];

  // Q^T fragments of this wave's half of the 576 query dims for its pair's
  // 32 heads (B operand: lane l holds head l%32).  Step j of lane half g
  // covers the eight dims of 16-byte chunk 4*j + 2*half + g; the cache rows
  // are read with the same mapping.  Heads past h (h a multiple of 16) are
  // computed on a copy of the last head and never stored: branching around
  // the matrix work would cost more registers than it saves.
  const uint16_t* qb = static_cast<const uint16_t*>(a.q) + (int64_t)b * h * kRowElems;
  bf16x8 qf[kSteps];
  {
    const int head = min(32 * pair + c32, h - 1);
#pragma unroll
    for (int j = 0; j < kSteps; ++j)
      qf[j] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(qb + (int64_t)head * kRowElems + 8 * (4 * j + 2 * half + g)));
  }

  f32x16 acc[kColBlocks];
#pragma unroll
  for (int i = 0; i < kColBlocks; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;
  float m_ref = -INFINITY, l_run = 0.f;

  const uint16_t* cbase = static_cast<const uint16_t*>(a.k);
  // Copies of one tile: 36 wave instructions, 9 from each wave of the
  // lagging group (waves 4-7; see the tile loop).  Instruction `inst` fills LDS
  // block inst: rows 16*(inst/18) + (lane/4) of the tile, slab inst%18, and
  // lane l lands at physical chunk l%4 of its row's slab, which holds
  // logical chunk 4*slab + ((l%4) ^ (l/16)).
  const int inst0 = (wave - kCopyWaves) * kDmaPer;  // meaningful for the copying waves only
  const int drow = lane >> 2, dchunk = (lane & 3) ^ (lane >> 4);
  // Byte offset of the lane's source inside a 16-row run of cache rows (slab 0).
  const uint32_t doff = (uint32_t)((drow * kRowElems + dchunk * 8) * 2);
  // Contiguous rows of this sequence start here; a paged cache looks each row up.
  const uint16_t* seq_base = cbase + (a.block_size == 0 ? (int64_t)b * a.cache_len * kRowElems : 0);
  const int32_t* tbl = a.block_table + (int64_t)b * a.max_blocks;
  // Fast copies need each 16-row half of the tile to be one run of
  // consecutive cache rows: always true for a contiguous cache, and for a
  // paged one whose block size is a multiple of 16 (tiles start at
  // multiples of 32 tokens).  The ragged last tile of a piece takes the
  // general path, which clamps every row into the piece.
  const bool halves_contiguous = a.block_size == 0 || (a.block_size & 15) == 0;
  // First cache row of the 16-row run starting at token t (a multiple of 16;
  // fast path only).  A paged lookup is a scalar table load (counted by
  // lgkmcnt, so the copies in flight are left alone).
  auto half_base = [&](int t) __attribute__((always_inline)) -> const uint16_t* {
    if (a.block_size == 0) return seq_base + (int64_t)t * kRowElems;
    const int32_t* ep = tbl + block_of(a, t);
    int e;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=&s"(e) : "s"(ep) : "memory");
    // An out-of-range table entry reads the pool's first rows instead.
    return (e < 0 || (int64_t)e >= a.cache_len) ? cbase
                                                : cbase + ((int64_t)e * a.block_size + slot_of(a, t)) * kRowElems;
  };
  auto issue_tile = [&](int t0, int buf) __attribute__((always_inline)) {
    const uint32_t dst = (uint32_t)(uintptr_t)&tiles[buf][0];
    if (halves_contiguous && t0 + kT <= t_end) {
      // This wave's nine instructions lie in one 16-row half of the tile.
      const uint16_t* hb = half_base(t0 + 16 * (inst0 / 18));
#pragma unroll
      for (int u = 0; u < kDmaPer; ++u) {
        const int inst = inst0 + u;
        dma16s(doff, hb + (inst % 18) * 32, dst + inst * 1024);
      }
      return;
    }
    // General path: per-lane row addresses, rows past the end clamped to the
    // last valid row (their scores are masked).  Not unrolled: it is rare,
    // and the loop keeps its temporaries out of the registers the main loop
    // needs.
#pragma unroll 1
    for (int u = 0; u < kDmaPer; ++u) {
      {
        const int inst = inst0 + u;
        const int t = min(t0 + 16 * (inst / 18) + drow, t_end - 1);
        const int chunk = 4 * (inst % 18) + dchunk;
        int64_t off;
        if (a.block_size == 0) {
          off = (int64_t)t * kRowElems;
        } else {
          const int blk = tbl[block_of(a, t)];
          // An out-of-range table entry reads row 0 of the pool instead.
          off = (blk < 0 || (int64_t)blk >= a.cache_len) ? -(int64_t)(seq_base - cbase)
                                                          : ((int64_t)blk * a.block_size + slot_of(a, t)) * kRowElems;
        }
        dma16(seq_base + off + chunk * 8, dst + inst * 1024);
      }
    }
  };

  // Per-lane LDS byte offsets inside a tile.
  // Scores (A operand): lane l reads row l%32 at chunk 4*j + 2*half + l/32,
  // i.e. the per-lane offset below plus an immediate 1024 * j.
  const int koff = lds_chunk(c32, 2 * half + g);
  // Values (A operand): lane l needs column 32*cb + l%32 at the tokens of
  // step kk, two runs of four rows.  The transposing read returns to lane n
  // of a 16-lane group element n%4 of the 4-element piece addressed by lane
  // 4v + n/4, for rows v = 0..3; so lane n of group G addresses row
  // 4*(G/2) + n/4 (+8 for the second run, +16*kk) and the four columns
  // 32*cb + 16*(G%2) + 4*(n%4) .. +3 (chunk 4*cb + 2*(G%2) + (n%4)/2, byte
  // 8*(n%2)), and receives column 32*cb + 16*(G%2) + n.  Column block
  // cb = 8*half + i adds an immediate 1024 * i, step kk one of 16 rows.
  const int vn = lane & 15, vgrp = lane >> 4;
  const int vchunk = 32 * half + 2 * (vgrp & 1) + ((vn & 3) >> 1);
  const int vrow0 = 4 * (vgrp >> 1) + (vn >> 2);
  const int voff0 = lds_chunk(vrow0, vchunk) + 8 * (vn & 1);
  const int voff1 = lds_chunk(vrow0 + 8, vchunk) + 8 * (vn & 1);

  const int ntok = t_end - t_begin;
  const int n_tiles = ntok > 0 ? (ntok + kT - 1) / kT : 0;
  const bool lead = wave < kWaves - kCopyWaves;  // waves 0-3: the leading group (see the tile loop)
  if (!lead && n_tiles > 0) issue_tile(t_begin, 0);
  // The queries and the first tile were fetched together (one HBM latency at
  // start-up, not two).  Let both land here: the compiler cannot see the
  // copies in the vector-memory counter, and a wait it placed on the query
  // loads inside the loop would drain the copies in flight every tile.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  if (!lead && n_tiles > 1) issue_tile(t_begin + kT, 1);

  // Partial scores of tile `it` over this wave's half of the dims, published
  // in LDS for the other wave of the pair: each lane stores its 16 scores as
  // four 16-byte words, consecutive across lanes.  copy(u) runs after every
  // second matrix op (u = 0..8), so that a copying wave's nine copy
  // instructions are spread over its score products: issued in one burst
  // they hold the wave for about as long as the products take, since the
  // compute unit accepts copies only at the rate it moves their data.
  auto scores = [&](int it, auto copy) __attribute__((always_inline)) {
    const unsigned char* tile = tiles[it % kNBuf];
    f32x16 s;
#pragma unroll
    for (int v = 0; v < 16; ++v) s[v] = 0.f;
    auto read_k = [&](int j) __attribute__((always_inline)) {
      return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(tile + koff + 1024 * j));
    };
    bf16x8 ka[kKDepth];
#pragma unroll
    for (int j = 0; j + 1 < kKDepth; ++j) ka[j] = read_k(j);
#pragma unroll
    for (int j = 0; j < kSteps; ++j) {
      if (j + kKDepth - 1 < kSteps) ka[(j + kKDepth - 1) % kKDepth] = read_k(j + kKDepth - 1);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[j % kKDepth], qf[j], s, 0, 0, 0);
      if (j % 2 == 1) copy(j / 2);
      __builtin_amdgcn_sched_barrier(0);
    }
    f32x4* mine = reinterpret_cast<f32x4*>(sx) + wave * 4 * 64;
#pragma unroll
    for (int q = 0; q < 4; ++q) mine[q * 64 + lane] = f32x4{s[4 * q], s[4 * q + 1], s[4 * q + 2], s[4 * q + 3]};
    return s;
  };

  // Softmax and value product of tile `it`, from this wave's partial scores
  // `s` and the partner's published ones.  kLast marks the last tile of the
  // piece, the only one that can be ragged; the others are compiled without
  // any masking.
  auto softmax_values = [&](int it, const f32x16& s, auto last_tag) __attribute__((always_inline)) {
    constexpr bool kLast = decltype(last_tag)::value;
    const int t0 = t_begin + it * kT;
    const auto* tile_lds = (const __attribute__((address_space(3))) unsigned char*)tiles[it % kNBuf];
    const f32x4* other = reinterpret_cast<const f32x4*>(sx) + (wave ^ 1) * 4 * 64;
    float sv[16];  // raw scores q.k
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // Add in a fixed order (lower half first) so both waves get identical sums.
      const f32x4 o = other[q * 64 + lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) sv[4 * q + e] = half == 0 ? s[4 * q + e] + o[e] : o[e] + s[4 * q + e];
    }

    // Online softmax on c * score (c = scale * log2 e, log2 units); P^T is
    // packed straight into the B-operand layout.  The tile maximum of c * s
    // is c times the raw maximum (the minimum, for a negative scale).  Masked
    // scores of a ragged last tile are set to the neutral element of that
    // extremum and their probabilities to zero.
    const float c = a.scale_log2;
    const float neutral = c >= 0.f ? -INFINITY : INFINITY;
    if constexpr (kLast) {
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (t0 + 8 * (v >> 2) + 4 * g + (v & 3) >= t_end) sv[v] = neutral;
    }
    float ext;
    if (c >= 0.f) {
      ext = sv[0];
#pragma unroll
      for (int v = 1; v < 16; ++v) ext = fmaxf(ext, sv[v]);
    } else {
      ext = sv[0];
#pragma unroll
      for (int v = 1; v < 16; ++v) ext = fminf(ext, sv[v]);
    }
    const float mt = max_over_halves(ext * c);
    const bool need = mt > m_ref + kRescaleSlack;  // also true while m_ref is -inf
    if (__any(need)) {
      const float m_new = need ? mt : m_ref;
      const float alpha = fast_exp2(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < kColBlocks; ++i) acc[i] *= alpha;
    }
    float pv[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) pv[v] = fast_exp2(__builtin_fmaf(sv[v], c, -m_ref));
    if constexpr (kLast) {
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (t0 + 8 * (v >> 2) + 4 * g + (v & 3) >= t_end) pv[v] = 0.f;
    }
    // Reduction step kk of the value product takes the lane's scores
    // v = 8*kk .. 8*kk+7, i.e. tokens 16*kk + 8*(e/4) + 4*(l/32) + e%4.
    bf16x8 pp[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 packed;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        packed[e] = pack_bf16x2(pv[8 * kk + 2 * e], pv[8 * kk + 2 * e + 1]);
        l_run = add_bf16x2(packed[e], l_run);  // normalise with the weights the matrix core sees
      }
      pp[kk] = __builtin_bit_cast(bf16x8, packed);
    }

    // Values: O^T[32 cols x 32 heads] += V^T[32 cols x 16 tokens] * P^T per
    // step kk, for this wave's column blocks cb = 8*half + i (latent columns
    // 32*cb .. 32*cb+31).  Steps run kk-major, so consecutive matrix ops
    // accumulate into different blocks.
    auto read_v = [&](int i, int kk) __attribute__((always_inline)) {
      const int imm = 1024 * i + (kTileBytes / 2) * kk;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile_lds + voff0 + imm));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile_lds + voff1 + imm));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    constexpr int kVSteps = 2 * kColBlocks;
    bf16x8 va[kVDepth];
#pragma unroll
    for (int st = 0; st + 1 < kVDepth; ++st) va[st] = read_v(st % kColBlocks, st / kColBlocks);
#pragma unroll
    for (int st = 0; st < kVSteps; ++st) {
      const int nx = st + kVDepth - 1;
      if (nx < kVSteps) va[nx % kVDepth] = read_v(nx % kColBlocks, nx / kColBlocks);
      const int i = st % kColBlocks, kk = st / kColBlocks;
      acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[st % kVDepth], pp[kk], acc[i], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Two wave groups, one interval apart.  Waves 0-3 (pairs 0 and 1) and
  // waves 4-7 (pairs 2 and 3) share the SIMDs (wave w runs on SIMD w % 4).
  // A tile takes two intervals between workgroup barriers: the leading group
  // computes its partial scores in the first and its softmax and value
  // product in the second; the lagging group does its scores in the second
  // interval and the rest in the next tile's first.  On every SIMD one
  // wave's score products then run beside the other wave's softmax and value
  // products instead of all waves doing the same phase at once.  The
  // interval boundaries double as the pairs' partial-score swaps.  The
  // lagging group issues all copies: those of tile it+2 right after the
  // second barrier of tile it, when every wave is done with tile it-1, whose
  // stage they overwrite, and it waits for tile it's copies before the first
  // barrier of tile it.  Both groups pass the same barriers in the same
  // order: two per tile and one after the last.
  if (lead) {
    auto lead_tile = [&](int it, auto last_tag) __attribute__((always_inline)) {
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // tile it has landed
      const f32x16 s = scores(it, [](int) {});
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // partial scores published
      softmax_values(it, s, last_tag);
    };
    for (int it = 0; it + 1 < n_tiles; ++it) lead_tile(it, TagFalse{});
    if (n_tiles > 0) {
      lead_tile(n_tiles - 1, TagTrue{});
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
  } else {
    f32x16 s;
#pragma unroll
    for (int v = 0; v < 16; ++v) s[v] = 0.f;
    for (int it = 0; it < n_tiles; ++it) {
      // Tile it's copies have landed (tile it+1's may stay in flight).
      if (it + 1 < n_tiles) asm volatile("s_waitcnt vmcnt(9) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (it > 0) softmax_values(it - 1, s, TagFalse{});
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      // Copies of tile it+2, into the stage tile it-1 held.
      const int tn = t_begin + (it + 2) * kT;
      if (it + 2 < n_tiles && halves_contiguous && tn + kT <= t_end) {
        const uint16_t* hb = half_base(tn + 16 * (inst0 / 18));
        const uint32_t dst = (uint32_t)(uintptr_t)&tiles[(it + 2) % kNBuf][0] + inst0 * 1024;
        const int slab0 = inst0 % 18;
        s = scores(it, [&](int u) __attribute__((always_inline)) {
          dma16s(doff, hb + (slab0 + u) * 32, dst + u * 1024);
        });
      } else {
        if (it + 2 < n_tiles) issue_tile(tn, (it + 2) % kNBuf);
        s = scores(it, [](int) {});
      }
    }
    if (n_tiles > 0) {
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // partial scores of the last tile published
      softmax_values(n_tiles - 1, s, TagTrue{});
    }
  }

  // Lane l holds O^T[col = 32*cb + 8*(v/4) + 4*(l/32) + v%4][head 32*pair + l%32].
  const int head = 32 * pair + c32;
  const float l = sum_over_halves(l_run);
  const int64_t row = (int64_t)b * h + head;
  const bool empty = !(l > 0.f);
  const float inv = empty ? 0.f : 1.f / l;
  const float lse2 = empty ? -INFINITY : m_ref + __log2f(l);
  if (final_out) {
    if (head >= h) return;
    uint16_t* o = static_cast<uint16_t*>(a.out) + row * kMlaLatent + 4 * g;
#pragma unroll
    for (int i = 0; i < kColBlocks; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = pack_bf16x2(acc[i][4 * q] * inv, acc[i][4 * q + 1] * inv);
        const uint32_t hi = pack_bf16x2(acc[i][4 * q + 2] * inv, acc[i][4 * q + 3] * inv);
        *reinterpret_cast<uint2*>(o + 32 * (8 * half + i) + 8 * q) = make_uint2(lo, hi);
      }
    if (a.lse != nullptr && g == 0 && half == 0) a.lse[row] = lse2 * kLn2;
    return;
  }
  // Partial output, normalised and rounded to bf16 (the merge weighs the
  // pieces in fp32 from their fp32 log-sum-exps): staged through LDS so that
  // every store instruction writes whole 128-byte lines (the accumulator
  // layout would write 8-byte pieces of 32 head rows).  Each wave has its own
  // region of the (now idle) tile ring: 32 head rows of 128 columns (256
  // bytes), rows padded to 272 bytes (16-byte aligned, and the line-per-8-lanes
  // reads conflict-free).  Two rounds of four column blocks each, over the
  // wave's columns 256*half .. 256*half+255.
  constexpr int kStgPitch = 272;  // bytes
  __syncthreads();  // every wave is done with the tile ring
  unsigned char* stg = &tiles[0][0] + wave * (32 * kStgPitch);
  uint16_t* po = reinterpret_cast<uint16_t*>(a.part_o);
  const int64_t prow0 = (int64_t)piece * h + 32 * pair;  // partial row of this wave's first head
#pragma unroll
  for (int k = 0; k < kColBlocks / 4; ++k) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x16& x = acc[4 * k + jj];
        *reinterpret_cast<uint2*>(stg + c32 * kStgPitch + 2 * (32 * jj + 8 * q + 4 * g)) =
            make_uint2(pack_bf16x2(x[4 * q] * inv, x[4 * q + 1] * inv),
                       pack_bf16x2(x[4 * q + 2] * inv, x[4 * q + 3] * inv));
      }
    // Line 8*m + lane/8 of the round: head row line/2, columns 64*(line%2) .. +63 of the round's 128.
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int line = 8 * m + (lane >> 3);
      const int hh = line >> 1, jb = line & 1;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stg + hh * kStgPitch + 128 * jb + 16 * (lane & 7));
      if (32 * pair + hh < h)
        *reinterpret_cast<u32x4*>(po + (prow0 + hh) * kMlaLatent + 256 * half + 128 * k + 64 * jb +
                                  8 * (lane & 7)) = v;
    }
  }
  if (head < h && g == 0 && half == 0) a.part_lse[prow0 + c32] = lse2;
}

}  // namespace

hipError_t launch_mla_bf16(const DecodeArgs& a, hipStream_t stream, const LaunchEvents& ev) {
  if (a.num_q_heads % 16 != 0 || a.num_q_heads > kMaxMlaHeads) return hipErrorInvalidValue;
  const dim3 grid(8 * ((a.max_pieces + 7) / 8));
  hipExtLaunchKernelGGL(mla_split_bf16, grid, dim3(kWaves * 64), 0, stream, ev.start, ev.stop, 0, a);
  return hipGetLastError();
}

}  // namespace kvattn
