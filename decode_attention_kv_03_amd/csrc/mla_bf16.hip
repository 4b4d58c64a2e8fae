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
// Both products are dense contractions and run on v_mfma_f32_16x16x32_bf16:
//   S^T[32 tok x 16 heads] = C_tile[32 x 576] * Q^T[576 x 16]   (per head block)
//   O^T[512 x 16 heads]   += C_tile[:, :512]^T * P^T[32 x 16]
// One workgroup (4 waves) owns one (sequence, split) and all heads; each wave
// owns HPW blocks of 16 heads, keeps their queries in registers (Q^T
// fragments) and their 512-wide accumulators in the register file.
//
// Data movement.  Tiles of 32 cache rows (36 KiB) stream from HBM straight
// into LDS with global_load_lds_dwordx4 (no register staging), three tiles
// deep, so two tiles are in flight while one is consumed.  Rows are stored
// unpadded with their 16-byte chunks XOR-swizzled by row, which makes both
// LDS read patterns conflict-free: the row-wise reads feeding the score
// product (16 rows, same column chunk) and the transposing reads
// (ds_read_b64_tr_b16, 4 consecutive rows x 16 columns per lane group)
// feeding the value product.  Waits on the DMA are explicit vmcnt counts
// followed by a bare s_barrier; a full workgroup fence would drain every
// tile in flight.
//
// Online softmax in the matrix-core output layout (lane l: head l%16, tokens
// 4*(l/16)+v of each 16-token half), with lazy rescaling: the running
// reference max only moves when a tile's max exceeds it by more than 8 (log2
// units), so the 512-wide accumulators are rarely rescaled; probabilities
// stay below 2^8, exact in the fp32 accumulators and representable in bf16.
#include "cache_addr.h"
#include "device_common.h"
#include "kvattn_internal.h"

namespace kvattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kT = 32;                      // tokens per tile
constexpr int kRowElems = kMlaRow;          // 576 bf16
constexpr int kRowBytes = kRowElems * 2;    // 1152
constexpr int kChunks = kRowBytes / 16;     // 72 16-byte chunks per row
constexpr int kTileBytes = kT * kRowBytes;  // 36864
constexpr int kNBuf = 3;
constexpr int kThreads = 256;
constexpr int kDmaPerThread = kT * kChunks / kThreads;  // 9
static_assert(kT * kChunks % kThreads == 0, "tile must split evenly over the threads");
constexpr int kDB = kMlaLatent / 16;        // 32 output column blocks
constexpr int kKB = kMlaRow / 32;           // 18 score reduction blocks
constexpr float kRescaleSlack = 8.f;        // log2 units

// Chunk swizzle of row r: a permutation of the low three chunk-index bits.
__device__ __forceinline__ int swz(int row) {
  const int x = (row >> 1) & 7;
  return ((x & 1) << 2) | (x & 2) | (x >> 2);
}

template <int HPW>
__global__ __launch_bounds__(kThreads, 1) void mla_split_bf16(DecodeArgs a) {
  const int split = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, grp = lane >> 4;
  const int h = a.num_q_heads;

  const int len = clamp_len(a.seq_lens[b], a.len_cap);
  const int t_begin = split * a.split_tokens;
  const bool final_out = (a.n_split == 1);
  if (!final_out && t_begin >= len) return;
  const int t_end = min(len, t_begin + a.split_tokens);

  __shared__ __attribute__((aligned(1024))) unsigned char smem[kNBuf * kTileBytes];

  const int hb0 = wave * HPW;
  const uint16_t* qb = static_cast<const uint16_t*>(a.q) + (int64_t)b * h * kRowElems;
  bf16x8 qf[HPW][kKB];
#pragma unroll
  for (int hbi = 0; hbi < HPW; ++hbi) {
    const int head = (hb0 + hbi) * 16 + n16;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (head < h) v = *reinterpret_cast<const u32x4*>(qb + (int64_t)head * kRowElems + 32 * kb + 8 * grp);
      qf[hbi][kb] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x4 acc[HPW][kDB];
  float m_ref[HPW], l_run[HPW];
#pragma unroll
  for (int hbi = 0; hbi < HPW; ++hbi) {
    m_ref[hbi] = -INFINITY;
    l_run[hbi] = 0.f;
#pragma unroll
    for (int db = 0; db < kDB; ++db) acc[hbi][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const uint16_t* cbase = static_cast<const uint16_t*>(a.k);
  // DMA of one tile: wave instruction u of wave w fills LDS chunks
  // [(9w + u) * 64, +64) of the tile; lane l's chunk L sits in row L / 72 at
  // physical slot L % 72 and holds logical chunk (slot ^ swz(row)).
  auto issue_tile = [&](int t0, int buf) {
    unsigned char* dst = smem + buf * kTileBytes;
#pragma unroll
    for (int u = 0; u < kDmaPerThread; ++u) {
      const int inst = wave * kDmaPerThread + u;
      const int L = inst * 64 + lane;
      const int row = L / kChunks;
      const int slot = L - row * kChunks;
      const int chunk = slot ^ swz(row);
      int t = t0 + row;
      t = t < t_end ? t : t_end - 1;  // rows past the end re-read the last valid row (masked below)
      int64_t off = cache_row_offset(a, b, 0, t, kRowElems);
      off = off < 0 ? 0 : off;
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(cbase + off + chunk * 8),
                                       (lds_void*)(dst + inst * 1024), 16, 0, 0);
    }
  };

  const int ntok = t_end - t_begin;
  const int n_tiles = ntok > 0 ? (ntok + kT - 1) / kT : 0;
  if (n_tiles > 0) issue_tile(t_begin, 0);
  if (n_tiles > 1) issue_tile(t_begin + kT, 1);

  for (int it = 0; it < n_tiles; ++it) {
    if (it + 1 < n_tiles) {
      asm volatile("s_waitcnt vmcnt(9) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    if (it + 2 < n_tiles) issue_tile(t_begin + (it + 2) * kT, (it + 2) % kNBuf);
    const int t0 = t_begin + it * kT;
    const unsigned char* tile = smem + (it % kNBuf) * kTileBytes;
    const auto* tile_lds = (const __attribute__((address_space(3))) unsigned char*)tile;

    // Scores: S^T[16 tokens x 16 heads] per half and head block.
    f32x4 s[2][HPW];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int hbi = 0; hbi < HPW; ++hbi) s[st][hbi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int row = 16 * st + n16;
        const int phys = (4 * kb + grp) ^ swz(row);
        const u32x4 raw = *reinterpret_cast<const u32x4*>(tile + row * kRowBytes + phys * 16);
        const bf16x8 ka = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
        for (int hbi = 0; hbi < HPW; ++hbi)
          s[st][hbi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[hbi][kb], s[st][hbi], 0, 0, 0);
      }
    }

    // Online softmax; P^T packed straight into the B-operand layout.
    bf16x8 pp[HPW];
#pragma unroll
    for (int hbi = 0; hbi < HPW; ++hbi) {
      float sv[8];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int tok = t0 + 16 * st + 4 * grp + v;
          sv[4 * st + v] = tok < t_end ? s[st][hbi][v] * a.scale_log2 : -INFINITY;
        }
      float mt = sv[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mt = fmaxf(mt, sv[e]);
      mt = wave_max_xor(mt, 16);
      mt = wave_max_xor(mt, 32);
      const bool need = mt > m_ref[hbi] + kRescaleSlack;  // also true while m_ref is -inf
      if (__any(need)) {
        const float m_new = need ? mt : m_ref[hbi];
        const float alpha = fast_exp2(m_ref[hbi] - m_new);
        m_ref[hbi] = m_new;
        l_run[hbi] *= alpha;
#pragma unroll
        for (int db = 0; db < kDB; ++db) acc[hbi][db] *= alpha;
      }
      uint16_t pb[8];
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pb[e] = f32_to_bf16_bits(fast_exp2(sv[e] - m_ref[hbi]));
        psum += bf16_bits_to_f32(pb[e]);
      }
      l_run[hbi] += psum;
      u32x4 packed;
#pragma unroll
      for (int e = 0; e < 4; ++e) packed[e] = (uint32_t)pb[2 * e] | ((uint32_t)pb[2 * e + 1] << 16);
      pp[hbi] = __builtin_bit_cast(bf16x8, packed);
    }

    // Values: O^T[16 cols x 16 heads] += V^T[16 cols x 32 tokens] * P^T.
    // The transposing read of lane n in a 16-lane group addresses row
    // base + n/4, columns 4*(n%4)..+3 and returns column n of the 4 rows.
    const int r_lo = 4 * grp + (n16 >> 2);
    const int r_hi = 16 + r_lo;
    const int sz_lo = swz(r_lo), sz_hi = swz(r_hi);
    const int half = (n16 & 1) * 8;  // byte offset of the 4-column piece inside its 16-byte chunk
    const int csub = (n16 & 3) >> 1;
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      const int chunk = 2 * db + csub;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(tile_lds + r_lo * kRowBytes + ((chunk ^ sz_lo) * 16) + half));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(tile_lds + r_hi * kRowBytes + ((chunk ^ sz_hi) * 16) + half));
      const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int hbi = 0; hbi < HPW; ++hbi)
        acc[hbi][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pp[hbi], acc[hbi][db], 0, 0, 0);
    }
  }

  // Lane l holds O^T[col = 16*db + 4*grp + v][head (hb0+hbi)*16 + n16].
#pragma unroll
  for (int hbi = 0; hbi < HPW; ++hbi) {
    const int head = (hb0 + hbi) * 16 + n16;
    if (head >= h) continue;
    float l = wave_sum_xor(l_run[hbi], 16);
    l = wave_sum_xor(l, 32);
    const int64_t row = (int64_t)b * h + head;
    const bool empty = !(l > 0.f);
    const float inv = empty ? 0.f : 1.f / l;
    const float lse2 = empty ? -INFINITY : m_ref[hbi] + __log2f(l);
    if (final_out) {
      uint16_t* o = static_cast<uint16_t*>(a.out) + row * kMlaLatent;
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const uint32_t lo = f32_to_bf16_bits(acc[hbi][db][0] * inv) | ((uint32_t)f32_to_bf16_bits(acc[hbi][db][1] * inv) << 16);
        const uint32_t hi = f32_to_bf16_bits(acc[hbi][db][2] * inv) | ((uint32_t)f32_to_bf16_bits(acc[hbi][db][3] * inv) << 16);
        *reinterpret_cast<uint2*>(o + 16 * db + 4 * grp) = make_uint2(lo, hi);
      }
      if (a.lse != nullptr && grp == 0) a.lse[row] = lse2 * kLn2;
    } else {
      float* po = a.part_o + (row * a.n_split + split) * kMlaLatent;
#pragma unroll
      for (int db = 0; db < kDB; ++db) *reinterpret_cast<f32x4*>(po + 16 * db + 4 * grp) = acc[hbi][db] * inv;
      if (grp == 0) a.part_lse[row * a.n_split + split] = lse2;
    }
  }
}

}  // namespace

hipError_t launch_mla_bf16(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_q_heads % 16 != 0 || a.num_q_heads > kMaxMlaHeads) return hipErrorInvalidValue;
  const dim3 grid(a.n_split, a.batch);
  if (a.num_q_heads > 64) {
    mla_split_bf16<2><<<grid, dim3(kThreads), 0, stream>>>(a);
  } else {
    mla_split_bf16<1><<<grid, dim3(kThreads), 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace kvattn
