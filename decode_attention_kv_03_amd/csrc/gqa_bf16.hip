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
//  * the tile's K and V rows (64 x 128 bf16 each, contiguous in HBM for a
//    contiguous cache, 16-token runs for a paged one) are fetched with
//    coalesced 16-byte loads into registers one tile ahead, then written to
//    LDS, so the HBM stream overlaps the math of the previous tile;
//  * scores are S^T = K_tile * Q^T on v_mfma_f32_16x16x32_bf16: 16 tokens x 16
//    query heads per matrix op, the K operand read from LDS (row = token,
//    eight consecutive head-dim values per lane) and Q^T held in registers;
//  * the online softmax runs in the matrix-core output layout: lane l owns
//    query head l%16 and tokens 4*(l/16)..+3, so per-head max/sum need two
//    cross-lane exchanges (xor 16, xor 32) and everything else is lane-local;
//  * P V is accumulated as O^T = V^T * P^T on v_mfma_f32_16x16x16_bf16: the
//    probabilities already sit in the B-operand layout, and V^T comes from
//    the row-major V tile through the gfx950 LDS transpose read
//    (ds_read_b64_tr_b16), one read per 16 head-dim columns;
//  * waves split the tile's tokens when a group has at most 32 heads
//    (each wave keeps its own max/sum/accumulator, merged through LDS at the
//    end) and split the heads when it has more;
//  * the split's result is either the final output (one split) or an fp32
//    partial plus its log2-domain log-sum-exp for the merge kernel.
#include "cache_addr.h"
#include "device_common.h"
#include "kvattn_internal.h"

namespace kvattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;                        // tokens per LDS tile
constexpr int kKStride = kHeadDim + 8;           // LDS row pitch of K (bf16): 272 B, conflict-free row reads
constexpr int kVStride = kHeadDim + 16;          // LDS row pitch of V (bf16): 288 B, conflict-free transpose reads
constexpr int kLdsK = kTile * kKStride * 2;      // bytes
constexpr int kLdsV = kTile * kVStride * 2;
constexpr int kLdsBytes = kLdsK + kLdsV;         // 35840 B
constexpr int kRedFloatsPerWave = 34 * 64;       // 32 accumulators + max + sum, per lane
static_assert(4 * kRedFloatsPerWave * 4 <= kLdsBytes, "cross-wave merge must fit in the tile buffer");

template <int HBW, int WH>
__global__ __launch_bounds__(256, 2) void gqa_split_bf16(DecodeArgs a) {
  static_assert(WH == 1 || HBW == 1, "token-split waves own one head block");
  const int split = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps wave-derived values in SGPRs
  const int n16 = lane & 15, grp = lane >> 4;
  const int r = a.group, h = a.num_q_heads;

  const int len = clamp_len(a.seq_lens[b], a.len_cap);
  const int t_begin = split * a.split_tokens;
  const bool final_out = (a.n_split == 1);
  if (!final_out && t_begin >= len) return;  // the merge only reads splits that hold tokens
  const int t_end = min(len, t_begin + a.split_tokens);

  __shared__ __attribute__((aligned(16))) unsigned char smem[kLdsBytes];
  uint16_t* ks = reinterpret_cast<uint16_t*>(smem);
  uint16_t* vs = reinterpret_cast<uint16_t*>(smem + kLdsK);
  auto* vs_lds = (__attribute__((address_space(3))) uint16_t*)vs;

  const int hb0 = (wave / WH) * HBW;  // first 16-head block of this wave
  const int ts = wave % WH;           // this wave's token slot within the tile

  // Q^T fragments: lane l holds head (block*16 + l%16), dims 32*kk + 8*(l/16) .. +7.
  const uint16_t* qg = static_cast<const uint16_t*>(a.q) + ((int64_t)b * h + (int64_t)j * r) * kHeadDim;
  bf16x8 qf[HBW][4];
#pragma unroll
  for (int hbi = 0; hbi < HBW; ++hbi) {
    const int head = (hb0 + hbi) * 16 + n16;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (head < r) v = *reinterpret_cast<const u32x4*>(qg + head * kHeadDim + 32 * kk + 8 * grp);
      qf[hbi][kk] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x4 acc[HBW][8];
  float m_run[HBW], l_run[HBW];
#pragma unroll
  for (int hbi = 0; hbi < HBW; ++hbi) {
    m_run[hbi] = -INFINITY;
    l_run[hbi] = 0.f;
#pragma unroll
    for (int db = 0; db < 8; ++db) acc[hbi][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const uint16_t* kbase = static_cast<const uint16_t*>(a.k);
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v);
  u32x4 kst[4], vst[4];
  // Thread tid fetches 16-byte chunks tid, tid+256, .. of the 64x256-byte tile:
  // four consecutive rows per wave instruction, fully coalesced.
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = tid + 256 * u;
      const int row = c >> 4, col = c & 15;
      const int t = t0 + row;
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (t < t_end) {
        const int64_t off = cache_row_offset(a, b, j, t, kHeadDim);
        if (off >= 0) {
          // read-once stream: non-temporal loads
          kv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + off + col * 8));
          vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vbase + off + col * 8));
        }
      }
      kst[u] = kv;
      vst[u] = vv;
    }
  };

  const int ntok = t_end - t_begin;
  const int n_tiles = ntok > 0 ? (ntok + kTile - 1) / kTile : 0;
  if (n_tiles > 0) load_tile(t_begin);

  for (int it = 0; it < n_tiles; ++it) {
    const int t0 = t_begin + it * kTile;
    __syncthreads();  // every wave is done with the previous tile
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = tid + 256 * u;
      const int row = c >> 4, col = c & 15;
      *reinterpret_cast<u32x4*>(ks + row * kKStride + col * 8) = kst[u];
      *reinterpret_cast<u32x4*>(vs + row * kVStride + col * 8) = vst[u];
    }
    __syncthreads();
    if (it + 1 < n_tiles) load_tile(t0 + kTile);  // in flight during this tile's math

    for (int st = ts; st < 4; st += WH) {
      const int row0 = st * 16;
      if (t0 + row0 >= t_end) break;
#pragma unroll
      for (int hbi = 0; hbi < HBW; ++hbi) {
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const u32x4 kraw = *reinterpret_cast<const u32x4*>(ks + (row0 + n16) * kKStride + 32 * kk + 8 * grp);
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kraw), qf[hbi][kk], s, 0, 0, 0);
        }
        // s[v] = q(head n16) . k(token t0 + row0 + 4*grp + v)
        float sv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int tok = t0 + row0 + 4 * grp + v;
          sv[v] = tok < t_end ? s[v] * a.scale_log2 : -INFINITY;
        }
        const float mt = max_over_row_groups(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
        const float m_new = fmaxf(m_run[hbi], mt);
        const float alpha = fast_exp2(m_run[hbi] - m_new);
        m_run[hbi] = m_new;
        const uint32_t p01 = pack_bf16x2(fast_exp2(sv[0] - m_new), fast_exp2(sv[1] - m_new));
        const uint32_t p23 = pack_bf16x2(fast_exp2(sv[2] - m_new), fast_exp2(sv[3] - m_new));
        // normalise with the weights the matrix core sees
        l_run[hbi] = add_bf16x2(p23, add_bf16x2(p01, l_run[hbi] * alpha));
        const i16x4 pb = __builtin_bit_cast(i16x4, (uint2){p01, p23});
        // Transpose-read rows (token) row0+4*grp .. +3, 16 columns per read:
        // lane n of a 16-lane group addresses row n/4, columns 4*(n%4)..+3 and
        // receives column n of the four rows.
        const int vrow = row0 + 4 * grp + (n16 >> 2);
        const int vcol = 4 * (n16 & 3);
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          acc[hbi][db] *= alpha;
          const i16x4 vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(vs_lds + vrow * kVStride + 16 * db + vcol));
          acc[hbi][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, pb, acc[hbi][db], 0, 0, 0);
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
    float* red = reinterpret_cast<float*>(smem);
    float* mine = red + wave * kRedFloatsPerWave;
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int v = 0; v < 4; ++v) mine[(db * 4 + v) * 64 + lane] = acc[0][db][v];
    mine[32 * 64 + lane] = m_run[0];
    mine[33 * 64 + lane] = l_run[0];
    __syncthreads();
    if (ts != 0) return;
#pragma unroll
    for (int w2 = 1; w2 < WH; ++w2) {
      const float* other = red + (wave + w2) * kRedFloatsPerWave;
      const float m2 = other[32 * 64 + lane];
      const float l2 = other[33 * 64 + lane];
      const float M = fmaxf(m_run[0], m2);
      if (M == -INFINITY) continue;
      const float a1 = fast_exp2(m_run[0] - M);
      const float a2 = fast_exp2(m2 - M);
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[0][db][v] = acc[0][db][v] * a1 + other[(db * 4 + v) * 64 + lane] * a2;
      l_run[0] = l_run[0] * a1 + l2 * a2;
      m_run[0] = M;
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
    const float lse2 = empty ? -INFINITY : m_run[hbi] + __log2f(l);
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
      float* po = a.part_o + (row * a.n_split + split) * kHeadDim;
#pragma unroll
      for (int db = 0; db < 8; ++db) *reinterpret_cast<f32x4*>(po + 16 * db + 4 * grp) = acc[hbi][db] * inv;
      if (grp == 0) a.part_lse[row * a.n_split + split] = lse2;
    }
  }
}

}  // namespace

hipError_t launch_gqa_bf16(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.n_split, a.num_kv_heads, a.batch);
  const dim3 block(256);
  const int head_blocks = (a.group + 15) / 16;
  if (head_blocks == 1) {
    gqa_split_bf16<1, 4><<<grid, block, 0, stream>>>(a);
  } else if (head_blocks == 2) {
    gqa_split_bf16<1, 2><<<grid, block, 0, stream>>>(a);
  } else if (head_blocks <= 4) {
    gqa_split_bf16<1, 1><<<grid, block, 0, stream>>>(a);
  } else if (head_blocks <= 8) {
    gqa_split_bf16<2, 1><<<grid, block, 0, stream>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvattn
