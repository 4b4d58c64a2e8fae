// Grouped-query decode attention over an FP8 (E4M3) KV cache, split-K
// flash-decode on the gfx950 matrix cores.
//
// What it computes: the grouped-query decode of the bf16 kernel ("MQA, GQA,
// and MLA", sections 2-4 and 8: query head i reads KV head i / (h/g), each
// cached byte fetched once per step for all heads of its group) over a cache
// whose K and V rows are E4M3 codes with one K scale and one V scale per KV
// head, the granularity at which a GQA cache quantises ("Why GQA's KV Cache
// Savings Don't Fully Reduce TPOT", section "When the Serving Engineer
// Doesn't Get to Choose").  The query and the output are bfloat16.
//
// Design.  Every E4M3 value is exactly a bfloat16 (3 mantissa bits, exponents
// inside bf16's range), so codes are widened to bf16 in registers with the
// gfx950 conversion (v_cvt_scalef32_pk_bf16_fp8, scale 1) and both products
// run on the bf16 matrix cores; the per-head scales are applied in fp32:
// k_scale[j] multiplies the softmax scale, v_scale[j] the final
// normalisation.  One workgroup (4 waves) owns one (sequence, KV head, split)
// and walks it in 128-token tiles (128 B per row, 16 KiB per tensor and tile):
//  * tiles stream into a 2-stage LDS ring with global_load_lds_dwordx4
//    (8 rows of one tensor per wave instruction, 32 per tile), awaited with
//    explicit vmcnt counts; 16-byte chunks are XOR-swizzled by row, and the
//    score reads take their chunks in an order (below) under which neither
//    LDS read pattern stalls on bank conflicts;
//  * scores S^T = K * Q^T on v_mfma_f32_16x16x32_bf16, 16 tokens x 16 heads
//    per product.  The 128 dims are dealt to the products so that a lane's
//    K bytes for all four are two 16-byte chunks of its row (two LDS reads),
//    with the query fragments dealt the same way;
//  * O^T += V^T * P^T, 32 tokens per product: V^T comes straight from the
//    row-major tile through the gfx950 8-bit transposing read
//    (ds_read_b64_tr_b8), whose lanes address the eight token rows the
//    probability operand holds;
//  * online softmax, lazy rescaling, head blocks, wave token slots and the
//    split output are those of the bf16 kernel.
#include <hip/hip_ext.h>

#include "device_common.h"
#include "kvattn_internal.h"
#include "lds_copy.h"

namespace kvattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int kTile = 128;                  // tokens per tile
constexpr int kRowB = kHeadDim;             // 128 B per K or V row
constexpr int kTileB = kTile * kRowB;       // 16 KiB per tensor and tile
constexpr int kStageB = 2 * kTileB;         // K tile, then V tile
constexpr int kNst = 2;                     // LDS ring stages
constexpr int kUnit = 32;                   // tokens per wave step
constexpr int kTblSlots = 2304;             // block-table entries staged in LDS
constexpr int kRedFloatsPerWave = 34 * 64;  // 32 accumulators + max + sum, per lane
constexpr float kRescaleSlack = 8.f;        // log2 units

// Chunk swizzle of a 128-byte row (8 chunks of 16 B).  Two rows share the 64
// LDS banks, so a read spreads over all banks when its rows give distinct
// (row parity, physical chunk) pairs: 16 consecutive rows (score reads) and the
// rows {0-3, 16-19} + 4k (transposing reads) both do with this XOR.
__device__ __forceinline__ int swz(int row) { return ((row >> 1) & 7) ^ (((row >> 4) & 1) << 2); }

// Four E4M3 codes (one dword) -> bf16 quadruple, exact.
__device__ __forceinline__ void widen4(uint32_t w, bf16x2& lo, bf16x2& hi) {
  lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true);
}

// Eight codes (two dwords) -> one bf16x8 matrix-core operand.
__device__ __forceinline__ bf16x8 widen8(uint32_t w0, uint32_t w1) {
  bf16x2 a, b, c, d;
  widen4(w0, a, b);
  widen4(w1, c, d);
  return __builtin_shufflevector(__builtin_shufflevector(a, b, 0, 1, 2, 3),
                                 __builtin_shufflevector(c, d, 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int HBW, int WH>
__global__ __launch_bounds__(256, 2) void gqa_split_fp8(DecodeArgs a) {
  static_assert(WH == 1 || HBW == 1, "token-split waves own one head block");
  // 1-D grid, XCD-aware as in the bf16 kernel: all splits of one (sequence,
  // KV head) run on one XCD.
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int split = slot % a.n_split;
  const int unit = (slot / a.n_split) * 8 + xcd;
  if (unit >= a.batch * a.num_kv_heads) return;
  const int b = unit / a.num_kv_heads, j = unit - b * a.num_kv_heads;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, grp = lane >> 4;
  const int r = a.group, h = a.num_q_heads;

  const int len = clamp_len(a.seq_lens[b], a.len_cap);
  const int t_lo = window_first(len, a.window);
  const int t_begin = window_base(len, a.window) + split * a.split_tokens;
  const bool final_out = (a.n_split == 1);
  if (!final_out && t_begin >= len) return;  // the merge only reads splits that hold tokens
  const int t_end = min(len, t_begin + a.split_tokens);
  const int ntok = t_end - t_begin;
  const int n_tiles = ntok > 0 ? (ntok + kTile - 1) / kTile : 0;

  __shared__ __attribute__((aligned(1024))) unsigned char ring[kNst][kStageB];
  __shared__ int tbl[kTblSlots];

  const int hb0 = (wave / WH) * HBW;  // first 16-head block of this wave
  const int ts = wave % WH;           // this wave's token slot within a tile

  // Per-head scales (KV head j): K's folds into the softmax scale, V's into
  // the final normalisation.
  const float s_log2 = a.scale_log2 * a.k_scale[j];
  const float v_sc = a.v_scale[j];

  // Q^T fragments.  Product kk of a score takes, in lane group grp, the dims
  // 64*(kk/2) + 16*grp + 8*(kk%2) .. +7 (the K fragment below takes the same
  // dims).
  const uint16_t* qg = static_cast<const uint16_t*>(a.q) + ((int64_t)b * h + (int64_t)j * r) * kHeadDim;
  bf16x8 qf[HBW][4];
#pragma unroll
  for (int hbi = 0; hbi < HBW; ++hbi) {
    const int head = (hb0 + hbi) * 16 + n16;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (head < r) v = *reinterpret_cast<const u32x4*>(qg + head * kHeadDim + 64 * (kk >> 1) + 16 * grp + 8 * (kk & 1));
      qf[hbi][kk] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // Paged cache: this split's block-table slice, staged in LDS.
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

  const uint8_t* kbase = static_cast<const uint8_t*>(a.k);
  const uint8_t* vbase = static_cast<const uint8_t*>(a.v);
  const int64_t head_rows = (int64_t)(b * a.num_kv_heads + j) * a.cache_len;  // contiguous: first row of (b, j)

  // Copies of one tile: 32 wave instructions (16 for K, 16 for V) of 8 rows
  // x 8 chunks; wave w issues instructions 8w .. 8w+7.  Lane l of
  // instruction i writes LDS slot (row 8*(i%16) + l/8, chunk l%8), which
  // holds logical chunk (l%8) ^ swz(row).  Rows past the split's end re-read
  // its last row (masked out of the softmax).
  // Paged fast path (power-of-two block size >= 8): an instruction's eight
  // rows start at a multiple of 8 tokens and so lie in one block; per-lane
  // offsets depend on the instruction's row group mod 4 only.
  const bool paged_fast = paged && a.block_shift >= 3;
  uint32_t dpo[4];
#pragma unroll
  for (int u4 = 0; u4 < 4; ++u4) {
    const int row = 8 * u4 + (lane >> 3);
    dpo[u4] = (uint32_t)((lane >> 3) * kRowB + ((lane & 7) ^ swz(row)) * 16);
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
      const int tw = t0 + 64 * (wave & 1);  // first token of this wave's 8 instructions
      const int32_t* ep[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) ep[u] = table_row + ((tw + 8 * u) >> a.block_shift);
      int e[8];
      asm volatile(
          "s_load_dword %0, %8, 0x0\n\ts_load_dword %1, %9, 0x0\n\ts_load_dword %2, %10, 0x0\n\t"
          "s_load_dword %3, %11, 0x0\n\ts_load_dword %4, %12, 0x0\n\ts_load_dword %5, %13, 0x0\n\t"
          "s_load_dword %6, %14, 0x0\n\ts_load_dword %7, %15, 0x0\n\ts_waitcnt lgkmcnt(0)"
          : "=&s"(e[0]), "=&s"(e[1]), "=&s"(e[2]), "=&s"(e[3]), "=&s"(e[4]), "=&s"(e[5]), "=&s"(e[6]), "=&s"(e[7])
          : "s"(ep[0]), "s"(ep[1]), "s"(ep[2]), "s"(ep[3]), "s"(ep[4]), "s"(ep[5]), "s"(ep[6]), "s"(ep[7])
          : "memory");
      const uint8_t* tbase = (wave >> 1) == 0 ? kbase : vbase;  // waves 0-1 copy K, 2-3 copy V
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int inst = wave * 8 + u;
        const int tg = tw + 8 * u;  // first token of the instruction's eight rows
        const int64_t row0 = (e[u] >= 0 && (int64_t)e[u] < a.cache_len)
                                 ? ((int64_t)e[u] * a.num_kv_heads + j) * bs + (tg & (bs - 1))
                                 : 0;  // out-of-range entry: in-bounds stand-in rows
        dma16s(dpo[u & 3], tbase + row0 * kRowB, stage_base + (inst >> 4) * kTileB + (inst & 15) * 1024);
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int inst = wave * 8 + u;
      const int tensor = inst >> 4, rg = inst & 15;
      const int row = 8 * rg + (lane >> 3);
      const int chunk = (lane & 7) ^ swz(row);
      const int t = min(t0 + row, t_end - 1);
      int64_t off;
      if (!paged) {
        off = (head_rows + t) * kRowB;
      } else {
        const int q = t / bs;
        const int blk = tbl[q - win_first];
        off = (blk >= 0 && (int64_t)blk < a.cache_len)
                  ? (((int64_t)blk * a.num_kv_heads + j) * bs + (t - q * bs)) * kRowB
                  : 0;  // out-of-range entry: an in-bounds stand-in row
      }
      const uint8_t* src = (tensor == 0 ? kbase : vbase) + off + chunk * 16;
      dma16(src, stage_base + tensor * kTileB + rg * 1024);
    }
  };

  // Per-lane LDS byte offsets inside a 32-token unit.  Score reads (A
  // operand): row 16*sb + n16, logical chunks grp and 4 + grp (dims 16*grp
  // .. +15 and 64 + 16*grp .. +15); the swizzle of rows 16..31 differs from
  // 0..15.  The order 2*grp + c measured 4 bank-conflict cycles per read: the
  // four lane groups read the same 16 rows, and chunks 2*grp + c put pairs of
  // groups on the banks that the XOR with swz() aligns across rows; chunks
  // 4*c + grp do not.
  // Transposing V reads: lane n16 of group grp addresses token row
  // R(grp, n16/2), R(grp, v) = 4*grp + v for v < 4 and 16 + 4*grp + v-4
  // otherwise, bytes 16*db + 8*(n16%2) .. +7; it then holds column
  // 16*db + n16 of rows R(grp, 0..7), the token order of its probabilities.
  int koff[2][2];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int row = 16 * sb + n16;
      koff[sb][c] = row * kRowB + 16 * ((4 * c + grp) ^ swz(row));
    }
  const int vv = n16 >> 1;
  const int vrow = (vv & 3) + 4 * grp + 16 * (vv >> 2);
  int voff[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) voff[db] = kTileB + vrow * kRowB + 16 * (db ^ swz(vrow)) + 8 * (n16 & 1);

  if (n_tiles > 0) issue_tile(t_begin, 0);
  // Queries, scales and the first tile were fetched together; let them all
  // land before the loop (a wait the compiler placed on the query loads
  // inside the loop would drain the copies in flight every tile).
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  for (int it = 0; it < n_tiles; ++it) {
    wait_copies_and_sync<0>();  // tile `it` has landed and every wave is done with the other stage
    if (it + 1 < n_tiles) issue_tile(t_begin + (it + 1) * kTile, (it + 1) % kNst);

    const int t0 = t_begin + it * kTile;
    const unsigned char* stage = ring[it % kNst];
    const auto* stage_lds = (const __attribute__((address_space(3))) unsigned char*)stage;

    for (int u0 = ts * kUnit; u0 < kTile; u0 += WH * kUnit) {
      if (t0 + u0 >= t_end) break;
      // K fragments of the unit, widened once and shared by the head blocks.
      bf16x8 kf[2][4];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const u32x4 kraw = *reinterpret_cast<const u32x4*>(stage + u0 * kRowB + koff[sb][c]);
          kf[sb][2 * c] = widen8(kraw[0], kraw[1]);
          kf[sb][2 * c + 1] = widen8(kraw[2], kraw[3]);
        }
#pragma unroll
      for (int hbi = 0; hbi < HBW; ++hbi) {
        f32x4 s[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          s[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
            s[sb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[sb][kk], qf[hbi][kk], s[sb], 0, 0, 0);
        }
        // s[sb][v] = q(head n16) . k(token t0 + u0 + 16*sb + 4*grp + v)
        float sv[8];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int v = 0; v < 4; ++v) sv[4 * sb + v] = s[sb][v] * s_log2;
        if (t0 + u0 + kUnit > t_end || t0 + u0 < t_lo) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int t = t0 + u0 + 16 * (e >> 2) + 4 * grp + (e & 3);
            if (t >= t_end || t < t_lo) sv[e] = -INFINITY;
          }
        }
        float mt = sv[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mt = fmaxf(mt, sv[e]);
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
        const float m_use = m_ref[hbi] == -INFINITY ? 0.f : m_ref[hbi];
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pk[e] = pack_bf16x2(fast_exp2(sv[2 * e] - m_use), fast_exp2(sv[2 * e + 1] - m_use));
          l_run[hbi] = add_bf16x2(pk[e], l_run[hbi]);  // normalise with the weights the matrix core sees
        }
        const bf16x8 pb = __builtin_bit_cast(bf16x8, (u32x4){pk[0], pk[1], pk[2], pk[3]});
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const i32x2 vr = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(stage_lds + u0 * kRowB + voff[db]));
          acc[hbi][db] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen8((uint32_t)vr[0], (uint32_t)vr[1]), pb, acc[hbi][db],
                                                      0, 0, 0);
        }
      }
    }
  }

#pragma unroll
  for (int hbi = 0; hbi < HBW; ++hbi) l_run[hbi] = sum_over_row_groups(l_run[hbi]);

  if constexpr (WH > 1) {
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

  // Lane l holds O^T[d = 16*db + 4*grp + v][head n16], in code units of V.
#pragma unroll
  for (int hbi = 0; hbi < HBW; ++hbi) {
    const int head = (hb0 + hbi) * 16 + n16;
    if (head >= r) continue;
    const int64_t row = (int64_t)b * h + (int64_t)j * r + head;
    const float l = l_run[hbi];
    const bool empty = !(l > 0.f);
    const float inv = empty ? 0.f : v_sc / l;
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

hipError_t launch_gqa_fp8(const DecodeArgs& a, hipStream_t stream, const LaunchEvents& ev) {
  const int64_t units = (int64_t)a.batch * a.num_kv_heads;
  const dim3 grid((unsigned)(8 * ((units + 7) / 8) * a.n_split));
  const dim3 block(256);
  const int head_blocks = (a.group + 15) / 16;
  if (head_blocks == 1) {
    hipExtLaunchKernelGGL((gqa_split_fp8<1, 4>), grid, block, 0, stream, ev.start, ev.stop, 0, a);
  } else if (head_blocks == 2) {
    hipExtLaunchKernelGGL((gqa_split_fp8<1, 2>), grid, block, 0, stream, ev.start, ev.stop, 0, a);
  } else if (head_blocks <= 4) {
    hipExtLaunchKernelGGL((gqa_split_fp8<1, 1>), grid, block, 0, stream, ev.start, ev.stop, 0, a);
  } else if (head_blocks <= 8) {
    hipExtLaunchKernelGGL((gqa_split_fp8<2, 1>), grid, block, 0, stream, ev.start, ev.stop, 0, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvattn
