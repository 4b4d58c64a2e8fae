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
// One workgroup (8 waves) owns one (sequence, split) and all heads.  Waves
// come in pairs: pair p owns heads 32p .. 32p+31 (two 16-head blocks); the
// two waves of a pair each take half of the 576-wide score reduction (their
// half of the queries lives in registers), swap partial scores through LDS,
// and then each accumulates half of the 512 latent output columns.  So every
// wave holds 32 heads' worth of operands per LDS read (half the LDS traffic
// of 16-head waves) with half the registers of a 32-head wave.
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
// units), so the accumulators are rarely rescaled; probabilities stay below
// 2^8, exact in the fp32 accumulators and representable in bf16.  Both waves
// of a pair see identical scores, so they take identical softmax decisions.
#include "cache_addr.h"
#include "device_common.h"
#include "kvattn_internal.h"

namespace kvattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kT = 32;                      // tokens per tile
constexpr int kRowElems = kMlaRow;          // 576 bf16
constexpr int kRowBytes = kRowElems * 2;    // 1152
constexpr int kChunks = kRowBytes / 16;     // 72 16-byte chunks per row
constexpr int kTileBytes = kT * kRowBytes;  // 36864
constexpr int kNBuf = 3;
constexpr int kTileInsts = kT * kChunks / 64;  // 36 wave-wide DMA instructions per tile
constexpr int kKBHalf = kMlaRow / 32 / 2;   // 9 score reduction blocks per wave
constexpr int kDBHalf = kMlaLatent / 16 / 2;  // 16 output column blocks per wave
constexpr int kSxBytes = 32 * 1024;         // partial-score exchange: 8 waves x 16 or 4 waves x 32 floats per lane
constexpr float kRescaleSlack = 8.f;        // log2 units

// Chunk swizzle of row r: XOR of the low three chunk-index bits with a
// function of the row that makes both read patterns below conflict-free
// (16 rows x one chunk; 4 consecutive rows x 4 half-chunks).  Rows r and
// r+16 share it.
__device__ __forceinline__ int swz(int row) { return (((row >> 1) & 3) << 1) | ((row >> 3) & 1); }

// 16-byte global -> LDS copy of every lane: lane i's bytes land at
// lds_base + 16 * i (lds_base is wave-uniform, taken through M0).  The
// non-temporal hint marks the cache stream as read-once, which measurably
// raises the streaming rate on this part.  Issued as
// inline assembly so the compiler does not treat every later LDS read as a
// possible alias of the copy and drain all copies in flight; completion is
// awaited explicitly with vmcnt before the tile is read.  M0 is written here
// and nowhere else in this kernel.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}

// HBW: 16-head blocks per wave.  A pair of waves owns 16*HBW heads, so the
// workgroup has 2 * 8 / HBW waves for 128 heads (HBW = 4: 4 waves with the
// full 512-register budget each; HBW = 2: 8 waves, two per SIMD).
template <int HBW>
__global__ __launch_bounds__(2 * 8 / HBW * 64, 1) void mla_split_bf16(DecodeArgs a) {
  constexpr int kWaves = 2 * 8 / HBW;
  constexpr int kDmaPer = kTileInsts / kWaves, kDmaExtra = kTileInsts % kWaves;
  static_assert(kWaves * HBW * 16 * 4 * 4 <= kSxBytes / 16 * 16, "score exchange must fit");
  // 1-D grid, XCD-aware: workgroup w runs on XCD w % 8, and every split of
  // sequence b gets an id with the same residue, so a sequence's queries and
  // partials stay in one XCD's L2.
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int split = slot % a.n_split;
  const int b = (slot / a.n_split) * 8 + xcd;
  if (b >= a.batch) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps wave-derived values in SGPRs
  const int n16 = lane & 15, grp = lane >> 4;
  const int pair = wave >> 1, half = wave & 1;
  const int h = a.num_q_heads;

  const int len = clamp_len(a.seq_lens[b], a.len_cap);
  const int t_begin = split * a.split_tokens;
  const bool final_out = (a.n_split == 1);
  if (!final_out && t_begin >= len) return;
  const int t_end = min(len, t_begin + a.split_tokens);

  __shared__ __attribute__((aligned(1024))) unsigned char tiles[kNBuf][kTileBytes];
  __shared__ __attribute__((aligned(16))) float sx[kSxBytes / 4];

  // Q^T fragments of this wave's half of the 576 query dims, for its pair's
  // 32 heads.  Reduction step kk of lane group grp covers the eight dims of
  // 16-byte chunk 8*kk + 2*grp + half; the cache rows are read with the same
  // mapping, so the split between the two waves interleaves chunks.
  const uint16_t* qb = static_cast<const uint16_t*>(a.q) + (int64_t)b * h * kRowElems;
  bf16x8 qf[HBW][kKBHalf];
#pragma unroll
  for (int hbi = 0; hbi < HBW; ++hbi) {
    const int head = (HBW * pair + hbi) * 16 + n16;
#pragma unroll
    for (int kk = 0; kk < kKBHalf; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if ((HBW * pair + hbi) * 16 < h)  // h is a multiple of 16: whole head blocks are in or out
        v = *reinterpret_cast<const u32x4*>(qb + (int64_t)head * kRowElems + 8 * (8 * kk + 2 * grp + half));
      qf[hbi][kk] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // Let the query loads land now: the compiler cannot see the tile copies in
  // the vector-memory counter, and any wait it places on these loads inside
  // the loop would also drain the copies in flight.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  f32x4 acc[HBW][kDBHalf];
  float m_ref[HBW], l_run[HBW];
#pragma unroll
  for (int hbi = 0; hbi < HBW; ++hbi) {
    m_ref[hbi] = -INFINITY;
    l_run[hbi] = 0.f;
#pragma unroll
    for (int db = 0; db < kDBHalf; ++db) acc[hbi][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const uint16_t* cbase = static_cast<const uint16_t*>(a.k);
  // DMA of one tile: 36 wave instructions spread over the waves (the first
  // kDmaExtra waves take one more).  Instruction `inst` fills LDS chunks
  // [inst*64, +64) of the tile; lane l's chunk L sits in row L / 72 at
  // physical slot L % 72 and holds logical chunk (slot ^ swz(row)).
  const int inst0 = wave * kDmaPer + min(wave, kDmaExtra);
  const int ninst = kDmaPer + (wave < kDmaExtra ? 1 : 0);
  // Contiguous rows of this sequence start here; a paged cache looks each row up.
  const uint16_t* seq_base = cbase + (a.block_size == 0 ? (int64_t)b * a.cache_len * kRowElems : 0);
  auto issue_tile = [&](int t0, int buf) {
    const uint32_t dst = (uint32_t)(uintptr_t)&tiles[buf][0];
    // An opaque copy of the lane id: the per-lane DMA offsets are recomputed
    // here (a few integer ops) instead of being kept live across the loop.
    int ln;
    asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
    if (a.block_size == 0) {
#pragma unroll
      for (int u = 0; u < kDmaPer + (kDmaExtra ? 1 : 0); ++u) {
        if (u < ninst) {
          const int inst = inst0 + u;
          const int L = inst * 64 + ln;
          const int row = L / kChunks;
          const int chunk = (L - row * kChunks) ^ swz(row);
          const int t = min(t0 + row, t_end - 1);  // rows past the end re-read the last valid row (masked below)
          dma16(seq_base + (int64_t)t * kRowElems + chunk * 8, dst + inst * 1024);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < kDmaPer + (kDmaExtra ? 1 : 0); ++u) {
        if (u < ninst) {
          const int inst = inst0 + u;
          const int L = inst * 64 + ln;
          const int row = L / kChunks;
          const int chunk = (L - row * kChunks) ^ swz(row);
          const int t = min(t0 + row, t_end - 1);
          int64_t off = cache_row_offset(a, b, 0, t, kRowElems);
          off = off < 0 ? 0 : off;  // an out-of-range table entry reads row 0 of the pool instead
          dma16(cbase + off + chunk * 8, dst + inst * 1024);
        }
      }
    }
  };

  const int ntok = t_end - t_begin;
  const int n_tiles = ntok > 0 ? (ntok + kT - 1) / kT : 0;
  if (n_tiles > 0) issue_tile(t_begin, 0);
  if (n_tiles > 1) issue_tile(t_begin + kT, 1);


  for (int it = 0; it < n_tiles; ++it) {
    // Wait for this tile's DMA (the next tile's may stay in flight), then sync.
    if (it + 1 < n_tiles) {
      if constexpr (kWaves == 8) {
        static_assert(kDmaPer == 4 && kDmaExtra == 4, "wait counts below");
        if (wave < 4) asm volatile("s_waitcnt vmcnt(5) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      } else {
        static_assert(kWaves == 4 && kDmaPer == 9 && kDmaExtra == 0, "wait counts below");
        asm volatile("s_waitcnt vmcnt(9) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      }
    } else {
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    if (it + 2 < n_tiles) issue_tile(t_begin + (it + 2) * kT, (it + 2) % kNBuf);
    const int t0 = t_begin + it * kT;
    const unsigned char* tile = tiles[it % kNBuf];
    const auto* tile_lds = (const __attribute__((address_space(3))) unsigned char*)tile;
    // Per-lane LDS byte offsets inside a tile (see the read lambdas below),
    // recomputed per tile from an opaque lane id to keep them out of the
    // registers that live across the loop.
    int ln;
    asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
    const int ln16 = ln & 15, lgrp = ln >> 4;
    const int koff = ln16 * kRowBytes + 16 * ((2 * lgrp + half) ^ swz(ln16));

    // Partial scores over this wave's half of the 576 dims.
    f32x4 s[2][HBW];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int hbi = 0; hbi < HBW; ++hbi) s[st][hbi] = f32x4{0.f, 0.f, 0.f, 0.f};
    // One k-block of operands is read ahead of the matrix ops that use the
    // previous one; the scheduling barriers keep the compiler from hoisting
    // every read.  The swizzle only touches per-lane chunk bits, so the
    // step kk and the half st are immediate offsets.
    auto read_k = [&](int kk, int st) {
      return __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(tile + koff + st * 16 * kRowBytes + 128 * kk));
    };
    bf16x8 ka_next[2] = {read_k(0, 0), read_k(0, 1)};
#pragma unroll
    for (int kk = 0; kk < kKBHalf; ++kk) {
      const bf16x8 ka[2] = {ka_next[0], ka_next[1]};
      if (kk + 1 < kKBHalf) {
        ka_next[0] = read_k(kk + 1, 0);
        ka_next[1] = read_k(kk + 1, 1);
      }
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int hbi = 0; hbi < HBW; ++hbi)
          s[st][hbi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[st], qf[hbi][kk], s[st][hbi], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Swap partial scores with the other wave of the pair.
    // Each lane stores its four-score fragments as 16-byte words, consecutive
    // across lanes.
    f32x4* mine = reinterpret_cast<f32x4*>(sx) + wave * (2 * HBW) * 64;
    const f32x4* other = reinterpret_cast<const f32x4*>(sx) + (wave ^ 1) * (2 * HBW) * 64;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int hbi = 0; hbi < HBW; ++hbi) mine[(st * HBW + hbi) * 64 + lane] = s[st][hbi];
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int hbi = 0; hbi < HBW; ++hbi) {
        // Add in a fixed order (lower half first) so both waves get identical sums.
        const f32x4 o = other[(st * HBW + hbi) * 64 + lane];
        s[st][hbi] = half == 0 ? s[st][hbi] + o : o + s[st][hbi];
      }

    // Online softmax; P^T packed straight into the B-operand layout.  Only the
    // last tile of a split can hold tokens past its end.
    const bool ragged = t0 + kT > t_end;
    bf16x8 pp[HBW];
#pragma unroll
    for (int hbi = 0; hbi < HBW; ++hbi) {
      float sv[8];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int v = 0; v < 4; ++v) sv[4 * st + v] = s[st][hbi][v] * a.scale_log2;
      if (ragged) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (t0 + 16 * (e >> 2) + 4 * grp + (e & 3) >= t_end) sv[e] = -INFINITY;
      }
      float mt = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
      mt = max_over_row_groups(mt);
      const bool need = mt > m_ref[hbi] + kRescaleSlack;  // also true while m_ref is -inf
      if (__any(need)) {
        const float m_new = need ? mt : m_ref[hbi];
        const float alpha = fast_exp2(m_ref[hbi] - m_new);
        m_ref[hbi] = m_new;
        l_run[hbi] *= alpha;
#pragma unroll
        for (int db = 0; db < kDBHalf; ++db) acc[hbi][db] *= alpha;
      }
      u32x4 packed;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        packed[e] = pack_bf16x2(fast_exp2(sv[2 * e] - m_ref[hbi]), fast_exp2(sv[2 * e + 1] - m_ref[hbi]));
        l_run[hbi] = add_bf16x2(packed[e], l_run[hbi]);  // normalise with the weights the matrix core sees
      }
      pp[hbi] = __builtin_bit_cast(bf16x8, packed);
    }

    // Values: O^T[16 cols x 16 heads] += V^T[16 cols x 32 tokens] * P^T for
    // this wave's 256 latent columns.  The transposing read returns to lane n
    // of a 16-lane group element n%4 of the 4-element piece addressed by lane
    // 4v + n/4, for rows v = 0..3; lane L = 4v + c addresses token row
    // 4*grp + v (and +16) and piece c of the column block, so lane n receives
    // column start(db) + n.  Column block db covers latent columns
    // 64*(db/2) + 32*half + 16*(db%2) .. +15.
    const int vrow = 4 * lgrp + (ln16 >> 2);
    const int vc = ln16 & 3;
    const int voff_even = vrow * kRowBytes + 16 * ((4 * half + (vc >> 1)) ^ swz(vrow)) + 8 * (vc & 1);
    const int voff_odd = vrow * kRowBytes + 16 * ((4 * half + 2 + (vc >> 1)) ^ swz(vrow)) + 8 * (vc & 1);
    auto read_v = [&](int db) {
      const int off = ((db & 1) ? voff_odd : voff_even) + 128 * (db >> 1);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile_lds + off));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile_lds + off + 16 * kRowBytes));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8 va_next = read_v(0);
#pragma unroll
    for (int db = 0; db < kDBHalf; ++db) {
      const bf16x8 va = va_next;
      if (db + 1 < kDBHalf) va_next = read_v(db + 1);
#pragma unroll
      for (int hbi = 0; hbi < HBW; ++hbi)
        acc[hbi][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pp[hbi], acc[hbi][db], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Lane l holds O^T[col = start(db) + 4*grp + v][head (HBW*pair+hbi)*16 + n16].
#pragma unroll
  for (int hbi = 0; hbi < HBW; ++hbi) {
    const int head = (HBW * pair + hbi) * 16 + n16;
    if (head >= h) continue;
    const float l = sum_over_row_groups(l_run[hbi]);
    const int64_t row = (int64_t)b * h + head;
    const bool empty = !(l > 0.f);
    const float inv = empty ? 0.f : 1.f / l;
    const float lse2 = empty ? -INFINITY : m_ref[hbi] + __log2f(l);
    const int col0 = 32 * half + 4 * grp;
    if (final_out) {
      uint16_t* o = static_cast<uint16_t*>(a.out) + row * kMlaLatent + col0;
#pragma unroll
      for (int db = 0; db < kDBHalf; ++db) {
        const int start = 64 * (db >> 1) + 16 * (db & 1);
        const uint32_t lo = pack_bf16x2(acc[hbi][db][0] * inv, acc[hbi][db][1] * inv);
        const uint32_t hi = pack_bf16x2(acc[hbi][db][2] * inv, acc[hbi][db][3] * inv);
        *reinterpret_cast<uint2*>(o + start) = make_uint2(lo, hi);
      }
      if (a.lse != nullptr && grp == 0 && half == 0) a.lse[row] = lse2 * kLn2;
    } else {
      float* po = a.part_o + (row * a.n_split + split) * kMlaLatent + col0;
#pragma unroll
      for (int db = 0; db < kDBHalf; ++db)
        *reinterpret_cast<f32x4*>(po + 64 * (db >> 1) + 16 * (db & 1)) = acc[hbi][db] * inv;
      if (grp == 0 && half == 0) a.part_lse[row * a.n_split + split] = lse2;
    }
  }
}

}  // namespace

hipError_t launch_mla_bf16(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_q_heads % 16 != 0 || a.num_q_heads > kMaxMlaHeads) return hipErrorInvalidValue;
  const int seq_groups = (a.batch + 7) / 8;
  const dim3 grid(8 * seq_groups * a.n_split);
  mla_split_bf16<2><<<grid, dim3(512), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace kvattn
