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
// Both products are dense contractions on v_mfma_f32_16x16x32_bf16 (on this
// part the 16x16x32 shape sustains a higher rate than 32x32x16):
//   S^T[16 tok x 16 heads] += C[16 tok x 32 dims] * Q^T[32 dims x 16 heads]
//   O^T[16 cols x 16 heads] += C[32 tok, 16 cols]^T * P^T[32 tok x 16 heads]
// A workgroup owns one piece of a sequence (a run of its tokens, from the
// device-side plan in mla_plan.hip) and all heads; it has four waves, one per
// SIMD, and wave w owns heads 32w .. 32w+31 as two 16-head blocks.  A lone
// wave on a SIMD has the whole register file (512 per lane): its queries
// over all 576 dims take 144 registers and its output accumulators over all
// 512 latent columns 256, which leaves room for deep LDS prefetch and needs
// no exchange of partial scores between waves.  Every cache operand read
// from LDS feeds both head blocks (two matrix ops per read).
//
// Data movement.  Tiles of 32 cache rows (36 KiB) stream from HBM straight
// into a four-stage LDS ring with global_load_lds_dwordx4 carrying the
// non-temporal hint (no register staging); each wave issues nine of a tile's
// 36 copy instructions, spread over its score products.  In LDS a tile is
// stored as 36 blocks of 1 KiB, [row group (8 rows)][segment (128 bytes of
// each row)], one per copy instruction, so that every copy fetches whole
// 128-byte cache lines (with 16 rows x 64 bytes per instruction, each line
// was requested in two halves); the eight 16-byte chunks of row r are
// XOR-swizzled by swz(r % 16).  Score reads (16 rows x 64 bytes) and the
// transposing reads of the value product (ds_read_b64_tr_b16: 4 consecutive
// rows x 16 columns per 16-lane group) then spread over all banks.  The copies are issued as inline assembly
// and awaited with explicit vmcnt counts followed by a bare s_barrier; a
// full workgroup fence, or the compiler's own alias-based waits, would
// drain every tile in flight.
//
// Software pipeline.  Iteration it waits for tile it, issues the copies of
// tile it+2 (into the stage tile it-2 held), computes tile it's scores with
// the softmax of tile it-1 interleaved between the matrix ops (it depends
// only on tile it-1's scores), and then tile it-1's value product.
//
// Online softmax in the matrix-core output layout (lane l: head l%16 of a
// block, tokens 16*tb + 4*(l/16) + i of the tile for tb = 0, 1 and
// i = 0..3), with lazy rescaling: the running reference max only moves when
// a tile's max exceeds it by more than 8 (log2 units), so the accumulators
// are rarely rescaled; probabilities stay below 2^8, exact in the fp32
// accumulators and representable in bf16.  The value product reduces over
// tokens in the order the scores come out in (lane group g holds tokens
// 4g..4g+3 and 16+4g..16+4g+3), and the transposing reads fetch V rows in
// that order, so P^T needs no data movement.
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
constexpr int kHalfBytes = kTileBytes / 2;     // one 16-row half of a tile
constexpr int kNBuf = 4;                       // LDS ring stages
constexpr int kWaves = 4;
constexpr int kTileInsts = kT * kChunks / 64;  // 36 wave-wide copies per tile
constexpr int kDmaPer = kTileInsts / kWaves;   // 9 per wave
static_assert(kDmaPer * kWaves == kTileInsts && kDmaPer == 9, "wait counts in the main loop assume 9 copies per wave");
constexpr int kKSteps = kMlaRow / 32;          // 18 reduction steps of 32 dims
constexpr int kKReads = 2 * kKSteps;           // 36 cache-operand reads per tile (two 16-token halves)
constexpr int kColBlocks = kMlaLatent / 16;    // 32 output column blocks of 16
constexpr float kRescaleSlack = 8.f;           // log2 units
constexpr int kKDepth = 6;                     // LDS operand reads in flight, score product
constexpr int kVDepth = 6;                     // ... and value product
constexpr int kStgPitch = 2 * kMlaLatent + 32; // epilogue staging: bytes per head row
static_assert(kWaves * 32 * kStgPitch <= kNBuf * kTileBytes, "staging fits in the tile ring");

// Chunk swizzle of tile row r (r % 16 = rr), 128-byte rows of a segment:
// the physical chunk (0 .. 7) is the logical one XOR rr % 8.  Of the
// swizzles measured in the kernel (LDS bank-conflict stall cycles over
// LDS-busy cycles), this one gave 8 %, against 35-51 % for XORs with
// (rr / 2) % 8, 2 ((rr / 2) % 4) + rr / 8 and other mixes of the row bits,
// and 75 % for none, whose kernel ran a fifth slower.
__device__ __forceinline__ int swz(int rr) { return rr & 7; }

// Block-table index and in-block slot of token t (paged cache).
__device__ __forceinline__ int block_of(const DecodeArgs& a, int t) {
  return a.block_shift >= 0 ? t >> a.block_shift : t / a.block_size;
}
__device__ __forceinline__ int slot_of(const DecodeArgs& a, int t) {
  return a.block_shift >= 0 ? t & (a.block_size - 1) : t % a.block_size;
}

struct TagFalse { static constexpr bool value = false; };
struct TagTrue { static constexpr bool value = true; };

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
  const int n16 = lane & 15, g = lane >> 4;
  const int h = a.num_q_heads;

  // The piece's tokens (t_begin a multiple of the tile), and whether it is
  // its sequence's only piece (then the output is final).
  const int t_begin = pc.y, t_end = pc.z;
  const bool final_out = pc.w != 0;
  const int ntok = t_end - t_begin;
  const int n_tiles = ntok > 0 ? (ntok + kT - 1) / kT : 0;

  __shared__ __attribute__((aligned(1024))) unsigned char tiles[kNBuf][kTileBytes];

  const uint16_t* cbase = static_cast<const uint16_t*>(a.k);
  // Copies of one tile: 36 wave instructions, nine from each wave.
  // Instruction `inst` fills LDS block inst: row group inst/9 (rows 8*(inst/9)
  // + lane/8 of the tile), segment inst%9; lane l lands at physical chunk l%8
  // of its row's segment, which holds logical chunk 8*segment + ((l%8) ^
  // swz(row)).  Wave w's instructions 9w .. 9w+8 fill row group w.
  const int inst0 = wave * kDmaPer;
  const int drow = lane >> 3, dchunk = (lane & 7) ^ swz(8 * wave + drow);
  // Byte offset of the lane's source inside an 8-row run of cache rows (segment 0).
  const uint32_t doff = (uint32_t)((drow * kRowElems + dchunk * 8) * 2);
  // Contiguous rows of this sequence start here; a paged cache looks each row up.
  const uint16_t* seq_base = cbase + (a.block_size == 0 ? (int64_t)b * a.cache_len * kRowElems : 0);
  const int32_t* tbl = a.block_table + (int64_t)b * a.max_blocks;
  // Fast copies need each 8-row group of the tile to be one run of
  // consecutive cache rows: always true for a contiguous cache, and for a
  // paged one whose block size is a multiple of 8 (tiles start at multiples
  // of 32 tokens).  The ragged last tile of a piece takes the general path,
  // which clamps every row into the piece.
  const bool groups_contiguous = a.block_size == 0 || (a.block_size & 7) == 0;
  // First cache row of the 8-row run starting at token t (a multiple of 8;
  // fast path only).  A paged lookup is a scalar table load.
  auto group_base = [&](int t) __attribute__((always_inline)) -> const uint16_t* {
    if (a.block_size == 0) return seq_base + (int64_t)t * kRowElems;
    const int32_t* ep = tbl + block_of(a, t);
    int e;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=&s"(e) : "s"(ep) : "memory");
    // An out-of-range table entry reads the pool's first rows instead.
    return (e < 0 || (int64_t)e >= a.cache_len) ? cbase
                                                : cbase + ((int64_t)e * a.block_size + slot_of(a, t)) * kRowElems;
  };
  // General path: per-lane row addresses, rows past the end clamped to the
  // last valid row (their scores are masked).  Not unrolled: it is rare, and
  // the loop keeps its temporaries out of the registers the main loop needs.
  auto issue_tile_general = [&](int t0, int buf) __attribute__((always_inline)) {
    const uint32_t dst = (uint32_t)(uintptr_t)&tiles[buf][0];
#pragma unroll 1
    for (int u = 0; u < kDmaPer; ++u) {
      const int inst = inst0 + u;
      const int t = min(t0 + 8 * wave + drow, t_end - 1);
      const int chunk = 8 * u + dchunk;
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
  };
  auto fast_tile = [&](int t0) __attribute__((always_inline)) {
    return groups_contiguous && t0 + kT <= t_end;
  };
  auto issue_tile = [&](int t0, int buf) __attribute__((always_inline)) {
    if (fast_tile(t0)) {
      const uint16_t* gb = group_base(t0 + 8 * wave);
      const uint32_t dst = (uint32_t)(uintptr_t)&tiles[buf][0] + inst0 * 1024;
#pragma unroll
      for (int u = 0; u < kDmaPer; ++u) dma16s(doff, gb + u * 64, dst + u * 1024);
    } else {
      issue_tile_general(t0, buf);
    }
  };

  // Start-up: the first two tiles and the queries are fetched together (one
  // HBM latency, not two), and all of them are awaited here.  The compiler
  // cannot see the copies in the vector-memory counter; this visible full
  // wait also keeps it from placing a wait on the query loads inside the
  // loop, which would drain the copies in flight every tile.
  if (n_tiles > 0) issue_tile(t_begin, 0);
  if (n_tiles > 1) issue_tile(t_begin + kT, 1);

  // Q^T fragments (B operand: lane l holds head l%16 of its block, the eight
  // dims 32*ks + 8*(l/16) .. +7 of reduction step ks; the cache rows are
  // read with the same mapping).  Heads past h (h a multiple of 16) are
  // computed on a copy of the last head and never stored.
  const uint16_t* qb = static_cast<const uint16_t*>(a.q) + (int64_t)b * h * kRowElems;
  bf16x8 qf[2][kKSteps];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int head = min(32 * wave + 16 * hb + n16, h - 1);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks)
      qf[hb][ks] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(qb + (int64_t)head * kRowElems + 8 * (4 * ks + g)));
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  // Measurement hook (off unless armed): the first wave of workgroup 0
  // stamps the shader clock and real-time counters around its tile loop.
  const bool stamp = a.clock_stamps != nullptr && blockIdx.x == 0 && wave == 0 && n_tiles > 0;
  uint64_t clk0 = 0, rt0 = 0;
  if (stamp) {
    clk0 = __builtin_amdgcn_s_memtime();
    rt0 = __builtin_amdgcn_s_memrealtime();
  }

  f32x4 acc[kColBlocks][2];
#pragma unroll
  for (int i = 0; i < kColBlocks; ++i)
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) acc[i][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

  // Per-lane LDS byte offsets inside a tile.
  // Scores (A operand): lane l reads row 16*tb + l%16 (row group 2*tb +
  // l%16/8) at logical chunk 4*ks + l/16 (segment ks/2, chunk 4*(ks%2) +
  // l/16 within it): one of the two offsets below, by ks's parity, plus an
  // immediate kHalfBytes * tb + 1024 * (ks/2).
  const int kbase = (n16 >> 3) * 9 * 1024 + (n16 & 7) * 128;
  const int koff_even = kbase + ((g ^ swz(n16)) << 4);
  const int koff_odd = kbase + (((4 + g) ^ swz(n16)) << 4);
  // Values (A operand): lane l needs column 16*cb + l%16 at the tokens
  // 4g..4g+3 (first read) and 16+4g..16+4g+3 (second read), g = l/16.  The
  // transposing read returns to lane n of a 16-lane group element n%4 of the
  // 4-element piece addressed by lane 4v + n/4, for rows v = 0..3; so lane n
  // addresses row 4g + n/4 and the four columns 16*cb + 4*(n%4) .. +3
  // (logical chunk 2*cb + (n%4)/2, byte 8*(n%2)), and receives column
  // 16*cb + n.  The segment cb/4 is an immediate 1024 * (cb/4); the chunk
  // within the segment depends on cb % 4, hence four base offsets.
  const int vrr = 4 * g + (n16 >> 2);
  const int vbase = (vrr >> 3) * 9 * 1024 + (vrr & 7) * 128 + 8 * (n16 & 1);
  int voff[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) voff[m] = vbase + (((2 * m + ((n16 & 3) >> 1)) ^ swz(vrr)) << 4);

  const float c = a.scale_log2;
  const float neutral = c >= 0.f ? -INFINITY : INFINITY;

  // Scores of tile `it` into s; copy(u), u = 0..8, runs after
  // every fourth operand read, so that the wave's nine copy instructions are
  // spread over its matrix ops: issued in one burst they would hold the wave
  // for about as long as the products take, since the compute unit accepts
  // copies only at the rate it moves their data.
  //
  // The score products are written as inline assembly so that their
  // accumulators stay in VGPRs: the compiler gives every matrix op of a
  // kernel that uses AGPRs the AGPR form, and the 256 AGPRs hold the output
  // accumulators exactly.  The compiler does not know these instructions,
  // so the hazards it would otherwise cover are covered here.  Their
  // operands are written only by LDS reads (the cache fragments, awaited
  // through lgkmcnt) and by the query loads before the loop, never by a
  // VALU instruction, so no wait states are needed before a block (a test
  // checks the generated code for a VALU write of an operand just before
  // one); the first block of a tile starts with two, the wait a VALU write
  // of an operand would need.  The last block ends with 24, more than the
  // longest wait this instruction's result needs before a VALU or memory
  // instruction may read it.  Chains that accumulate into the same
  // registers need no wait states between their matrix ops.
  auto scores = [&](int it, f32x4 (&s)[2][2], auto copy) __attribute__((always_inline)) {
    const unsigned char* tile = tiles[it % kNBuf];
    // Read j: token half tb = j % 2, reduction step ks = j / 2.
    auto read_k = [&](int j) __attribute__((always_inline)) {
      return __builtin_bit_cast(bf16x8,
                                *reinterpret_cast<const u32x4*>(tile + (((j >> 1) & 1) ? koff_odd : koff_even) +
                                                                kHalfBytes * (j & 1) + 1024 * (j >> 2)));
    };
    bf16x8 ka[kKDepth];
#pragma unroll
    for (int j = 0; j + 1 < kKDepth; ++j) ka[j] = read_k(j);
#pragma unroll
    for (int j = 0; j < kKReads - 2; ++j) {
      if (j + kKDepth - 1 < kKReads) ka[(j + kKDepth - 1) % kKDepth] = read_k(j + kKDepth - 1);
      const int tb = j & 1, ks = j >> 1;
      if (ks == 0) {
        asm volatile("s_nop 1\n\t"
            "v_mfma_f32_16x16x32_bf16 %0, %2, %3, 0\n\t"
            "v_mfma_f32_16x16x32_bf16 %1, %2, %4, 0"
            : "=&v"(s[tb][0]), "=&v"(s[tb][1])
            : "v"(ka[j % kKDepth]), "v"(qf[0][ks]), "v"(qf[1][ks]));
      } else {
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %2, %3, %0\n\t"
            "v_mfma_f32_16x16x32_bf16 %1, %2, %4, %1"
            : "+v"(s[tb][0]), "+v"(s[tb][1])
            : "v"(ka[j % kKDepth]), "v"(qf[0][ks]), "v"(qf[1][ks]));
      }
      if (j % 4 == 3) copy(j / 4);
    }
    // The last reduction step of all four chains, then the wait states that
    // make their results safe to read.
    {
      constexpr int j = kKReads - 2, ks = kKSteps - 1;
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %4, %6, %0\n\t"
          "v_mfma_f32_16x16x32_bf16 %1, %4, %7, %1\n\t"
          "v_mfma_f32_16x16x32_bf16 %2, %5, %6, %2\n\t"
          "v_mfma_f32_16x16x32_bf16 %3, %5, %7, %3\n\t"
          "s_nop 15\n\t"
          "s_nop 7"
          : "+v"(s[0][0]), "+v"(s[0][1]), "+v"(s[1][0]), "+v"(s[1][1])
          : "v"(ka[j % kKDepth]), "v"(ka[(j + 1) % kKDepth]), "v"(qf[0][ks]), "v"(qf[1][ks]));
      copy(8);
    }
  };

  // Softmax of a tile from its raw scores s (q.k): updates the running max
  // and sum, returns P^T in the B-operand layout of the value product and
  // the factor by which the accumulators must be rescaled before that
  // product (1 when the reference max did not move).  With kMask, tokens at
  // or past `lim` (tile-relative; below 32 only in the ragged last tile of
  // the piece) are masked; the other tiles are compiled without masking.
  // Branch-free, so that it can be interleaved with matrix ops.
  auto softmax = [&](const f32x4 (&s)[2][2], int lim, auto mask_tag, bf16x8 (&pp)[2], float (&alpha)[2])
      __attribute__((always_inline)) -> bool {
    constexpr bool kMask = decltype(mask_tag)::value;
    bool valid[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) valid[e] = !kMask || 16 * (e >> 2) + 4 * g + (e & 3) < lim;
    bool need_any = false;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      // x[e]: token 16*(e/4) + 4g + e%4 of the tile; masked tokens hold the
      // neutral element of the extremum below.
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = valid[e] ? s[e >> 2][hb][e & 3] : neutral;
      // The tile maximum of c * s is c times the raw maximum (the minimum,
      // for a negative scale).  Both are taken and one selected, which keeps
      // the code free of branches.
      float hi = x[0], lo = x[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) {
        hi = fmaxf(hi, x[e]);
        lo = fminf(lo, x[e]);
      }
      const float mt = max_over_row_groups((c >= 0.f ? hi : lo) * c);
      const bool need = mt > m_ref[hb] + kRescaleSlack;  // also true while m_ref is -inf
      const float m_new = need ? mt : m_ref[hb];
      alpha[hb] = need ? fast_exp2(m_ref[hb] - m_new) : 1.f;
      m_ref[hb] = m_new;
      need_any |= need;
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = valid[e] ? fast_exp2(__builtin_fmaf(x[e], c, -m_new)) : 0.f;
      u32x4 packed;
      float l = l_run[hb] * alpha[hb];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        packed[k] = pack_bf16x2(p[2 * k], p[2 * k + 1]);
        l = add_bf16x2(packed[k], l);  // normalise with the weights the matrix core sees
      }
      l_run[hb] = l;
      pp[hb] = __builtin_bit_cast(bf16x8, packed);
    }
    return need_any;
  };

  // Rescale of the accumulators when a tile moved the reference max (rare).
  // The empty asm statements pin each block's round trip (AGPRs -> VGPRs,
  // multiply, back to AGPRs) to four VGPRs at a time: left to itself the
  // register allocator moves whole accumulators into VGPRs around this
  // branch and spills the queries to make room.
  auto rescale = [&](const float (&alpha)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kColBlocks; ++i)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        f32x4 t = acc[i][hb];
        asm volatile("" : "+v"(t));
        t *= alpha[hb];
        asm volatile("" : "+v"(t));
        acc[i][hb] = t;
        asm volatile("" : "+a"(acc[i][hb]));
      }
  };

  // Value product of tile `it` with its probabilities pp; `between` is
  // independent work (the next tile's softmax) for the scheduler to place
  // between the matrix ops.
  auto values = [&](int it, const bf16x8 (&pp)[2], auto between) __attribute__((always_inline)) {
    const auto* tile_lds = (const __attribute__((address_space(3))) unsigned char*)tiles[it % kNBuf];
    auto read_v = [&](int cb) __attribute__((always_inline)) {
      const int off = voff[cb & 3] + 1024 * (cb >> 2);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile_lds + off));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile_lds + off + kHalfBytes));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8 va[kVDepth];
#pragma unroll
    for (int cb = 0; cb + 1 < kVDepth; ++cb) va[cb] = read_v(cb);
    between();
#pragma unroll
    for (int cb = 0; cb < kColBlocks; ++cb) {
      if (cb + kVDepth - 1 < kColBlocks) va[(cb + kVDepth - 1) % kVDepth] = read_v(cb + kVDepth - 1);
      acc[cb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[cb % kVDepth], pp[0], acc[cb][0], 0, 0, 0);
      acc[cb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[cb % kVDepth], pp[1], acc[cb][1], 0, 0, 0);
    }
  };

  // Iteration it: wait for tile it (this wave's copies of tile it+1 may stay
  // in flight) and for every wave to finish iteration it-1, which read tile
  // it-2 last; issue tile it+2's copies into that stage while computing tile
  // it's scores; then tile it-1's value product with tile it's softmax
  // between its matrix ops.  pp, alpha and need carry a tile's softmax
  // results to its value product one iteration later; the rescale they may
  // call for runs right after the barrier, where few registers are live.
  bf16x8 pp[2];
  float alpha[2];
  bool need = false;
  auto iteration = [&](int it, auto first_tag, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool kFirst = decltype(first_tag)::value;
    if (it + 1 < n_tiles) asm volatile("s_waitcnt vmcnt(9) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // The accumulators are still zero while tile 0's probabilities wait.
    if (!kFirst && it > 1 && __builtin_expect(__any(need), 0)) rescale(alpha);
    const int tn = t_begin + (it + 2) * kT;
    f32x4 s[2][2];
    if (it + 2 < n_tiles && fast_tile(tn)) {
      const uint16_t* gb = group_base(tn + 8 * wave);
      const uint32_t dst = (uint32_t)(uintptr_t)&tiles[(it + 2) % kNBuf][0] + inst0 * 1024;
      scores(it, s, [&](int u) __attribute__((always_inline)) { dma16s(doff, gb + u * 64, dst + u * 1024); });
    } else {
      if (it + 2 < n_tiles) issue_tile_general(tn, (it + 2) % kNBuf);
      scores(it, s, [](int) {});
    }
    const int lim = min(t_end - (t_begin + it * kT), kT);
    if constexpr (kFirst) {
      need = softmax(s, lim, mask_tag, pp, alpha);
    } else {
      bf16x8 pn[2];
      float an[2];
      bool nn = false;
      values(it - 1, pp, [&]() __attribute__((always_inline)) { nn = softmax(s, lim, mask_tag, pn, an); });
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        pp[hb] = pn[hb];
        alpha[hb] = an[hb];
      }
      need = nn;
    }
  };
  if (n_tiles > 0) {
    iteration(0, TagTrue{}, TagTrue{});
    for (int it = 1; it + 1 < n_tiles; ++it) iteration(it, TagFalse{}, TagFalse{});
    if (n_tiles > 1) iteration(n_tiles - 1, TagFalse{}, TagTrue{});
    if (n_tiles > 1 && __builtin_expect(__any(need), 0)) rescale(alpha);
    values(n_tiles - 1, pp, []() {});
  }

  if (stamp) {
    const uint64_t clk1 = __builtin_amdgcn_s_memtime();
    const uint64_t rt1 = __builtin_amdgcn_s_memrealtime();
    if (lane == 0) {
      a.clock_stamps[0] = clk0;
      a.clock_stamps[1] = rt0;
      a.clock_stamps[2] = clk1;
      a.clock_stamps[3] = rt1;
    }
  }

  // Lane l holds O^T[col = 16*cb + 4*(l/16) + i][head 32*wave + 16*hb + l%16].
  float inv[2], lse2[2];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const float l = sum_over_row_groups(l_run[hb]);
    const bool empty = !(l > 0.f);
    inv[hb] = empty ? 0.f : 1.f / l;
    lse2[hb] = empty ? -INFINITY : m_ref[hb] + __log2f(l);
  }
  // The output (final) or the partial of the piece (normalised and rounded
  // to bf16; the merge weighs the pieces in fp32 from their fp32 log-sum-
  // exps) is staged through LDS so that every store instruction writes one
  // whole 1 KiB head row (the accumulator layout would write 8-byte pieces of
  // 16 head rows).  Each wave has its own region of the (now idle) tile
  // ring: its 32 head rows, 1056 bytes apart.
  __syncthreads();  // every wave is done with the tile ring
  unsigned char* stg = &tiles[0][0] + wave * (32 * kStgPitch);
#pragma unroll
  for (int cb = 0; cb < kColBlocks; ++cb)
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const f32x4& x = acc[cb][hb];
      *reinterpret_cast<uint2*>(stg + (16 * hb + n16) * kStgPitch + 2 * (16 * cb + 4 * g)) =
          make_uint2(pack_bf16x2(x[0] * inv[hb], x[1] * inv[hb]), pack_bf16x2(x[2] * inv[hb], x[3] * inv[hb]));
    }
  uint16_t* dst = static_cast<uint16_t*>(final_out ? a.out : a.part_o);
  const int64_t row0 = (final_out ? (int64_t)b : (int64_t)piece) * h + 32 * wave;  // row of the wave's first head
#pragma unroll 4
  for (int r = 0; r < 32; ++r) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * kStgPitch + 16 * lane);
    if (32 * wave + r < h) *reinterpret_cast<u32x4*>(dst + (row0 + r) * kMlaLatent + 8 * lane) = v;
  }
  if (g == 0) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int head = 32 * wave + 16 * hb + n16;
      if (head >= h) continue;
      if (!final_out) a.part_lse[row0 + 16 * hb + n16] = lse2[hb];
      else if (a.lse != nullptr) a.lse[row0 + 16 * hb + n16] = lse2[hb] * kLn2;
    }
  }
}

}  // namespace

hipError_t launch_mla_bf16(const DecodeArgs& a, hipStream_t stream, const LaunchEvents& ev) {
  if (a.num_q_heads % 16 != 0 || a.num_q_heads > kMaxMlaHeads) return hipErrorInvalidValue;
  const dim3 grid(8 * ((a.max_pieces + 7) / 8));
  hipExtLaunchKernelGGL(mla_split_bf16, grid, dim3(kWaves * 64), 0, stream, ev.start, ev.stop, 0, a);
  return hipGetLastError();
}

}  // namespace kvattn
