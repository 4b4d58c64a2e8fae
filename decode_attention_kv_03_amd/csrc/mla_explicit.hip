// Per-head projections between MLA's latent space and the per-head spaces,
// and the reconstruct-then-attend (non-absorbed) MLA decode built on them.
//
// What they compute ("MQA, GQA, and MLA", section 5 "MLA, mechanically";
// "One dial, four settings", "MLA - compress instead of shrink"): head i
// rebuilds its keys k_i = c W_uk^(i) and values v_i = c W_uv^(i) from the
// cached latent c, and attends with its query [q^C_i | q^R_i] over
// [k_i | k^R]; the decoupled RoPE key k^R is cached beside c and shared by
// all heads.  That is the naive form the pages contrast with absorption: it
// turns the latent cache back into one of MHA's size before attending.  The
// absorbed path instead scores against c directly and applies W_uv once to
// its latent output, o_i = o_latent_i W_uv^(i): the same projection kernel
// does that up-projection.
//
// latent_project: for every (outer index, head): Y = X W (W stored [K, N]
// row-major, the layout of c W^(i)) or Y = X W^T (W stored [N, K]), bf16 in,
// fp32 accumulation, bf16 out, on v_mfma_f32_32x32x16_bf16.  A workgroup (4
// waves) computes a 128 x 128 tile of Y, each wave a 64 x 64 quadrant, in
// 64-deep steps of K through a two-stage LDS buffer filled from registers
// (the loads of two steps ahead are in flight while a step computes).
// The products are computed transposed, Y^T = W^T X^T, so that each lane
// holds runs of four consecutive output columns of one row; the tile is
// staged through LDS and written as whole 128-byte rows.  X tile rows (and
// [N, K] weight rows) are stored with their 16-byte chunks XOR-swizzled by
// row pair; a [K, N] weight tile is stored as 8 column blocks of [64 k][16 cols]
// and read through the gfx950 transposing LDS read (ds_read_b64_tr_b16),
// which hands each lane one column and four consecutive k.
//
// mla_explicit_attend: attention of one head over its reconstructed rows,
// one workgroup per (sequence, head, split), on the VALU: a head has no other
// head sharing its rows, so there is nothing for the matrix cores to reuse.
// Lanes work in 16-lane groups, one token per group and step, each lane
// holding 8 of the 128 key dims, 4 of the 64 RoPE dims and 8 of the 128 value
// dims; the score is reduced across the group with DPP row operations.
#include <hip/hip_ext.h>

#include "device_common.h"
#include "kvattn_internal.h"

namespace kvattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kRowPitch = kBK * 2;             // bytes per X row (and per [N, K] weight row) in LDS
constexpr int kXBytes = kBM * kRowPitch;       // 16 KiB
constexpr int kNbPitch = kBK * 32 + 128;       // [K, N] weight tile: one 16-column block (padded)
constexpr int kWBytes = 8 * kNbPitch;          // 8 column blocks
constexpr int kStageBytes = kXBytes + kWBytes;
constexpr int kStgPitch = 144;                 // output staging row: 64 bf16 + 16 bytes of padding

// 16-byte chunk `chunk` of row `row` in a tile of 128-byte rows.  Two rows
// share one 256-byte line of the 64 banks, so the chunk index is XORed with
// (row / 2) % 8: any 16 consecutive rows read at one logical chunk (a
// fragment read's 16-lane group) then land on 16 distinct 16-byte bank slots.
__device__ __forceinline__ int swz_off(int row, int chunk) {
  return row * kRowPitch + ((chunk ^ ((row >> 1) & 7)) << 4);
}

template <bool kWT>
__global__ __launch_bounds__(256, 2) void latent_project(ProjectArgs p) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * kStageBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;  // quadrant: rows 64*wm.., columns 64*wn..
  // 1-D grid: column tile fastest, then head, then row tile, then the outer index, so
  // consecutive workgroups share the X tile.
  int L = blockIdx.x;
  const int nt = L % p.n_tiles;
  L /= p.n_tiles;
  const int head = L % p.heads;
  L /= p.heads;
  const int mt = L % p.m_tiles;
  const int o = L / p.m_tiles;
  const int m0 = mt * kBM, n0 = nt * kBN;
  const uint16_t* x = p.x + (int64_t)o * p.x_outer + (int64_t)head * p.x_head;
  const uint16_t* w = p.w + (int64_t)head * p.w_head;

  // Loads of K step kt: 1024 16-byte chunks of X and 1024 of W, four of each
  // per thread, into register set `set`; two sets, so the loads of step kt+2
  // are in flight while step kt computes.
  u32x4 xr[1][4], wr[1][4];
  auto load = [&](int kt, int set) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = tid + 256 * u;
      const int row = c >> 3, ch = c & 7;
      xr[set][u] = u32x4{0u, 0u, 0u, 0u};
      if (m0 + row < p.rows)
        xr[set][u] = *reinterpret_cast<const u32x4*>(x + (int64_t)(m0 + row) * p.x_row + kt * kBK + ch * 8);
      if constexpr (kWT) {
        wr[set][u] = *reinterpret_cast<const u32x4*>(w + (int64_t)(n0 + row) * p.k_dim + kt * kBK + ch * 8);
      } else {
        const int k = c >> 4, cc = c & 15;
        wr[set][u] = *reinterpret_cast<const u32x4*>(w + (int64_t)(kt * kBK + k) * p.n_dim + n0 + cc * 8);
      }
    }
  };
  auto store = [&](int stage, int set) __attribute__((always_inline)) {
    unsigned char* s = lds + stage * kStageBytes;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = tid + 256 * u;
      const int row = c >> 3, ch = c & 7;
      *reinterpret_cast<u32x4*>(s + swz_off(row, ch)) = xr[set][u];
      if constexpr (kWT) {
        *reinterpret_cast<u32x4*>(s + kXBytes + swz_off(row, ch)) = wr[set][u];
      } else {
        const int k = c >> 4, cc = c & 15;
        *reinterpret_cast<u32x4*>(s + kXBytes + (cc >> 1) * kNbPitch + k * 32 + (cc & 1) * 16) = wr[set][u];
      }
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int ni = 0; ni < 2; ++ni)
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[ni][mi][v] = 0.f;

  // Per-lane fragment offsets.  X (B operand of Y^T = W^T X^T): row 32*mi + lane%32 of the
  // quadrant, chunk 2*kk + lane/32.  W (A operand): column 32*ni + lane%32 with the same k.
  const int lrow = lane & 31, khalf = lane >> 5;
  const int G = lane >> 4, n16 = lane & 15;
  auto compute = [&](int stage) __attribute__((always_inline)) {
    const unsigned char* s = lds + stage * kStageBytes;
    const auto* s_lds = (const __attribute__((address_space(3))) unsigned char*)s;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      bf16x8 xf[2], wf[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int r = 64 * wm + 32 * mi + lrow;
        xf[mi] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(s + swz_off(r, 2 * kk + khalf)));
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        if constexpr (kWT) {
          const int r = 64 * wn + 32 * ni + lrow;
          wf[ni] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(s + kXBytes + swz_off(r, 2 * kk + khalf)));
        } else {
          // Lane n16 of group G receives column 16*(G%2) + n16 of the 32-column block and k =
          // 16*kk + 8*(G/2) + 0..3 (first read), + 4..7 (second read).
          const int nb = (64 * wn + 32 * ni + 16 * (G & 1)) >> 4;
          const int k = 16 * kk + 8 * (G >> 1) + (n16 >> 2);
          const int off = kXBytes + nb * kNbPitch + k * 32 + 8 * (n16 & 3);
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(s_lds + off));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(s_lds + off + 4 * 32));
          wf[ni] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
          acc[ni][mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ni], xf[mi], acc[ni][mi], 0, 0, 0);
    }
  };

  const int nk = p.k_dim / kBK;
  load(0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    // Stage kt&1 was last read by step kt-2, which every wave finished before
    // the barrier of step kt-1.
    store(kt & 1, 0);
    __syncthreads();
    if (kt + 1 < nk) load(kt + 1, 0);
    compute(kt & 1);
  }

  // acc[ni][mi][v] = Y[row 32*mi + lane%32][col 32*ni + 8*(v/4) + 4*(lane/32) + v%4] of the quadrant.
  __syncthreads();  // every wave is done with the operand buffers
  unsigned char* stg = lds + wave * (64 * kStgPitch);
#pragma unroll
  for (int ni = 0; ni < 2; ++ni)
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int r = 32 * mi + lrow, col = 32 * ni + 8 * g4 + 4 * khalf;
        const f32x16& a = acc[ni][mi];
        *reinterpret_cast<uint2*>(stg + r * kStgPitch + col * 2) =
            make_uint2(pack_bf16x2(a[4 * g4], a[4 * g4 + 1]), pack_bf16x2(a[4 * g4 + 2], a[4 * g4 + 3]));
      }
  __syncthreads();  // the staged rows have landed
  uint16_t* y = p.y + (int64_t)o * p.y_outer + (int64_t)head * p.y_head;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int c = lane + 64 * u;
    const int r = c >> 3, ch = c & 7;
    const int m = m0 + 64 * wm + r;
    const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * kStgPitch + ch * 16);
    if (m < p.rows) *reinterpret_cast<u32x4*>(y + (int64_t)m * p.y_row + n0 + 64 * wn + ch * 8) = v;
  }
}

// Rebuild projection of the naive form: Y[o, i, s, :] = X[o, s, :] W^(i) for
// every head i, with the weights already transposed to W^(i)^T [128, K] and
// stored one head after another.  Those rows are then one [heads * 128, K]
// operand, so the projection of one outer index is a single GEMM over all
// heads, and a 256 x 256 output tile spans two heads.  The tile size is what
// sets the rate here: with K = 512 a 128 x 128 tile reads 64 operand bytes
// per MFMA clock of a compute unit, as much as one compute unit can load;
// a 256 x 256 tile needs half of that.
//
// Persistent: one workgroup of eight waves (two per SIMD) per compute unit
// walks its share of the tiles.  It computes Y^T = W^T X^T on
// v_mfma_f32_16x16x32_bf16, wave w the 128 (columns) x 64 (rows) block at
// columns 128 (w / 4), rows 64 (w % 4): 32 accumulators of four per lane.
// K runs in steps of 64 through a two-stage LDS ring filled by direct
// global -> LDS copies (global_load_lds_dwordx4, with no cache hint: every
// operand tile is read by many workgroups), the next step in flight while a
// step computes, and the steps of consecutive tiles form one stream, so the
// next tile's first step is in flight while a tile's results are written.
// A copy instruction fetches 8 whole 128-byte rows of a step (64 k): copy
// lane l fills row l/8, physical chunk l%8, which holds logical chunk
// (l%8) ^ ((row / 2) % 8), so the fragment reads (16 rows at one logical
// chunk) fall on distinct bank slots.  (Steps of 32 k, half rows, fetched
// every cache line twice, half of it each time.)  The results leave through a staging area of 4 KiB per wave apart
// from the ring, 32 columns at a time, as 64-byte row pieces; their stores
// stay in flight during the next tile.  Every tile writes all of its 256
// rows (y holds `rows` rounded up to 256 per outer index and head; rows past
// `rows` are computed from copies of the last one), so each tile issues
// exactly 16 stores per wave, which the waits below count: loads, stores
// and LDS copies of a wave retire from the vector-memory counter in issue
// order (the compiler's own waits on this target rely on that too, e.g. a
// load's value used with a later store and load still outstanding).
//
// Tile order: XCD x (workgroups x, x + 8, ...) takes the x-th eighth of the
// tile sequence, its 32 workgroups in turn, so the tiles an XCD runs
// together are 32 consecutive ones.  The sequence runs over groups of four
// row tiles, column tiles outer and row tiles inner within a group, so those
// 32 tiles are four row tiles by eight column tiles, whose operands (1 MiB of
// X, 2 MiB of W) stay in the XCD's L2.
constexpr int kRbM = 256, kRbN = 256, kRbK = 64, kRbStages = 2;
constexpr int kRbOpBytes = kRbM * kRbK * 2;    // one operand's 256 rows for one K step: 32 KiB
constexpr int kRbStageBytes = 2 * kRbOpBytes;  // X rows, then W rows
constexpr int kRbWaves = 8;
constexpr int kRbStgBytes = 64 * 64;           // per wave: 64 rows x 32 bf16 columns
constexpr int kRbGroupM = 4;                   // row tiles per group of the tile order
constexpr int kRbSlots = 32;                   // workgroups per XCD (one per compute unit)
constexpr int kRbStores = 16;                  // output stores per wave and tile
constexpr int kRbCopies = 8;                   // copies per wave and K step

// 16-byte global -> LDS copy of every lane (lane i's bytes land at lds_base +
// 16 i; lds_base through M0, which nothing else in this kernel writes), with
// the default cache policy.  The compiler does not see it in the vector-
// memory counter; the loop waits for the copies explicitly.
__device__ __forceinline__ void rb_copy(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}

// At most n of this wave's vector-memory operations outstanding (0, or the
// 16 stores of a tile that ended after the awaited copies were issued), then
// a workgroup barrier.
__device__ __forceinline__ void rb_wait_sync(int n) {
  if (n == 0) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Staging address of 16-byte chunk `chunk` of row `row` (64-byte rows, the
// chunk XORed with (row / 4) % 4: 16 consecutive rows at one chunk, or 4
// rows at all four, fall on distinct bank slots).
__device__ __forceinline__ int rb_stg_off(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4); }

__global__ __launch_bounds__(kRbWaves * 64, 1) void latent_rebuild(ProjectArgs p) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kRbStages * kRbStageBytes + kRbWaves * kRbStgBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int m_per_outer = (p.rows + kRbM - 1) / kRbM;
  const int m_all = p.outer * m_per_outer;
  const int n_tiles = p.heads * p.n_dim / kRbN;
  const int64_t total = (int64_t)m_all * n_tiles;
  const int64_t per_xcd = (total + 7) / 8;
  const int64_t first = (int64_t)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  const int64_t end = min(total, (int64_t)((blockIdx.x & 7) + 1) * per_xcd);
  if (first >= end) return;
  const int my_tiles = (int)((end - first + kRbSlots - 1) / kRbSlots);  // tiles first, first + 32, ...
  const int nk = p.k_dim / kRbK;
  const int steps = my_tiles * nk;

  // Operand rows and output base of this workgroup's i-th tile.
  const int rr = lane >> 3;  // row within a copy's 8 rows: row 8 (4 wave + j) + rr of the tile
  const int wn = wave >> 2, wm = wave & 3;
  struct Tile {
    const uint16_t* xs[4];
    const uint16_t* ws[4];
    uint16_t* y;  // row m0 + 64 wm, column 0 of this wave's head
  };
  auto tile_of = [&](int i) __attribute__((always_inline)) {
    const int64_t t = first + (int64_t)kRbSlots * i;
    const int64_t group = (int64_t)kRbGroupM * n_tiles;
    const int first_m = (int)(t / group) * kRbGroupM;
    const int gm = min(m_all - first_m, kRbGroupM);
    const int r = (int)(t % group);
    const int mt = first_m + r % gm, nt = r / gm;
    const int o = mt / m_per_outer;
    const int m0 = (mt % m_per_outer) * kRbM, n0 = nt * kRbN;
    Tile T;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 8 * (4 * wave + j) + rr;
      const int lc = (lane & 7) ^ ((row >> 1) & 7);
      T.xs[j] = p.x + (int64_t)o * p.x_outer + (int64_t)min(m0 + row, p.rows - 1) * p.x_row + 8 * lc;
      T.ws[j] = p.w + (int64_t)(n0 + row) * p.k_dim + 8 * lc;
    }
    T.y = p.y + (int64_t)o * p.y_outer + (int64_t)((n0 + 128 * wn) / p.n_dim) * p.y_head +
          (int64_t)(m0 + 64 * wm) * p.y_row;
    return T;
  };

  // Step G (tile G / nk, K step G % nk) into stage G % 2: wave w fills rows
  // 32w .. 32w+31 of both operands, 8 rows per copy.
  Tile iss = tile_of(0);
  auto issue = [&](int G) __attribute__((always_inline)) {
    const int kt = G % nk;
    if (kt == 0 && G > 0) iss = tile_of(G / nk);
    const uint32_t base = (uint32_t)(uintptr_t)&lds[(G % kRbStages) * kRbStageBytes] + 4 * wave * 1024;
#pragma unroll
    for (int j = 0; j < 4; ++j) rb_copy(iss.xs[j] + kt * kRbK, base + j * 1024);
#pragma unroll
    for (int j = 0; j < 4; ++j) rb_copy(iss.ws[j] + kt * kRbK, base + kRbOpBytes + j * 1024);
  };

  // Fragments: for the k half kk of a step, lane l reads row l%16 of a
  // 16-row block at logical chunk 4 kk + l/16 (the eight k of
  // v_mfma_f32_16x16x32_bf16's A and B operands).
  const int n16 = lane & 15, g = lane >> 4;
  auto frag_off = [&](int block, int kk) __attribute__((always_inline)) {
    return (16 * block + n16) * 128 + (((4 * kk + g) ^ ((n16 >> 1) & 7)) << 4);
  };
  f32x4 acc[8][4];
  auto zero = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  auto compute = [&](int stage) __attribute__((always_inline)) {
    const unsigned char* s = lds + stage * kRbStageBytes;
#pragma unroll
    for (int kk = 0; kk < kRbK / 32; ++kk) {
      bf16x8 xf[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        xf[mb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(s + frag_off(4 * wm + mb, kk)));
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const bf16x8 wf =
            __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(s + kRbOpBytes + frag_off(8 * wn + nb, kk)));
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, xf[mb], acc[nb][mb], 0, 0, 0);
      }
    }
  };

  // acc[nb][mb][v] = Y^T[column 16 nb + 4 (lane/16) + v][row 16 mb + lane%16]
  // of the wave's block; written 32 columns (two nb) at a time through the
  // wave's own staging rows, 16 stores per wave.
  unsigned char* stg = lds + kRbStages * kRbStageBytes + wave * kRbStgBytes;
  auto write_tile = [&](uint16_t* y) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int nbi = 0; nbi < 2; ++nbi)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const f32x4& a = acc[2 * q + nbi][mb];
          *reinterpret_cast<uint2*>(stg + rb_stg_off(16 * mb + n16, 2 * nbi + (g >> 1)) + 8 * (g & 1)) =
              make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
        }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's staged rows have landed
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int row = 16 * u + (lane >> 2), c = lane & 3;
        const u32x4 v = *reinterpret_cast<const u32x4*>(stg + rb_stg_off(row, c));
        *reinterpret_cast<u32x4*>(y + (int64_t)row * p.y_row + 32 * q + 8 * c) = v;
      }
    }
  };

  // Step G: wait for its copies (the stores of a tile that ended after they
  // were issued, at step G-1, may stay in flight) and for every wave to
  // finish step G-1, whose stage then takes step G+1.
  zero();
  issue(0);
  for (int G = 0; G < steps; ++G) {
    rb_wait_sync(G >= nk && G % nk == 0 ? kRbStores : 0);
    if (G + 1 < steps) issue(G + 1);
    compute(G % kRbStages);
    if (G % nk == nk - 1) {
      write_tile(tile_of(G / nk).y);
      zero();
    }
  }
}

// W^(i) [rows, cols] -> W^(i)^T [cols, rows] for every head, through a
// 64 x 64 LDS tile (bf16; rows and cols multiples of 64).
__global__ __launch_bounds__(256) void transpose_heads(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                       int rows, int cols) {
  __shared__ uint16_t t[64][65];
  const int tiles_c = cols / 64, tiles_r = rows / 64;
  int L = blockIdx.x;
  const int tc = L % tiles_c;
  L /= tiles_c;
  const int tr = L % tiles_r;
  const int head = L / tiles_r;
  const uint16_t* s = src + (int64_t)head * rows * cols;
  uint16_t* d = dst + (int64_t)head * rows * cols;
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int e = tid + 256 * u;
    const int r = e >> 6, c = e & 63;
    t[r][c] = s[(int64_t)(64 * tr + r) * cols + 64 * tc + c];
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int e = tid + 256 * u;
    const int c = e >> 6, r = e & 63;
    d[(int64_t)(64 * tc + c) * rows + 64 * tr + r] = t[r][c];
  }
}

// Sum over the 16 lanes of a row (DPP row operations: swap neighbours, swap pairs, mirror
// within 8 lanes, mirror within 16); every lane of the row receives the sum.
__device__ __forceinline__ float row16_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
  return v;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc, false);
}

constexpr int kExHead = 128;  // reconstructed key (content part) and value width
constexpr int kExRope = 64;
constexpr int kExSteps = 4;   // tokens per lane group and loop step

__global__ __launch_bounds__(256) void mla_explicit_attend(DecodeArgs a) {
  const int L = blockIdx.x;
  const int split = L % a.n_split;
  const int row = L / a.n_split;  // b * h + head
  const int h = a.num_q_heads;
  const int b = row / h;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tg = lane >> 4, sub = lane & 15;

  const int len = clamp_len(a.seq_lens[b], a.len_cap);
  const int t_begin = split * a.split_tokens;
  const bool final_out = a.n_split == 1;
  if (!final_out && t_begin >= len) return;  // the merge reads only splits that hold tokens
  const int t_end = min(len, t_begin + a.split_tokens);

  // Query: content dims 8*sub .. +7, RoPE dims 4*sub .. +3.
  const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + (int64_t)row * (kExHead + kExRope);
  const u32x4 qc = *reinterpret_cast<const u32x4*>(qrow + 8 * sub);
  const uint2 qr = *reinterpret_cast<const uint2*>(qrow + kExHead + 4 * sub);

  const uint16_t* kc = static_cast<const uint16_t*>(a.k) + (int64_t)row * a.rec_len * kExHead + 8 * sub;
  const uint16_t* vr = static_cast<const uint16_t*>(a.v) + (int64_t)row * a.rec_len * kExHead + 8 * sub;
  const uint16_t* kr = static_cast<const uint16_t*>(a.rope) + (int64_t)b * a.cache_len * kMlaRow + kMlaLatent + 4 * sub;

  struct Step {
    u32x4 k[kExSteps], v[kExSteps];
    uint2 r[kExSteps];
  };
  // Tokens of one loop step for this lane's group: t0 + 4u + group (the last valid token stands in past the end).
  auto fetch = [&](int t0, Step& st) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kExSteps; ++u) {
      const int t = min(t0 + 4 * u + tg, t_end - 1);
      st.k[u] = *reinterpret_cast<const u32x4*>(kc + (int64_t)t * kExHead);
      st.v[u] = *reinterpret_cast<const u32x4*>(vr + (int64_t)t * kExHead);
      st.r[u] = *reinterpret_cast<const uint2*>(kr + (int64_t)t * kMlaRow);
    }
  };

  float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) acc[d] = 0.f;
  constexpr int kWaveTokens = 4 * kExSteps;  // tokens a wave takes per step
  Step cur, nxt;
  int t0 = t_begin + wave * kWaveTokens;
  if (t0 < t_end) fetch(t0, cur);
  for (; t0 < t_end; t0 += 4 * kWaveTokens) {
    const int tn = t0 + 4 * kWaveTokens;
    if (tn < t_end) fetch(tn, nxt);
    float s[kExSteps];
#pragma unroll
    for (int u = 0; u < kExSteps; ++u) {
      float d = dot2(qc[0], cur.k[u][0], 0.f);
      d = dot2(qc[1], cur.k[u][1], d);
      d = dot2(qc[2], cur.k[u][2], d);
      d = dot2(qc[3], cur.k[u][3], d);
      d = dot2(qr.x, cur.r[u].x, d);
      d = dot2(qr.y, cur.r[u].y, d);
      s[u] = row16_sum(d) * a.scale_log2;
      if (t0 + 4 * u + tg >= t_end) s[u] = -INFINITY;
    }
    const float m_new = fmaxf(m, fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
    const float m_use = m_new == -INFINITY ? 0.f : m_new;  // nothing attended yet: keep the weights at 0
    const float alpha = fast_exp2(m - m_use);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[d] *= alpha;
#pragma unroll
    for (int u = 0; u < kExSteps; ++u) {
      const float pu = fast_exp2(s[u] - m_use);
      l += pu;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += pu * bf16_lo(cur.v[u][e]);
        acc[2 * e + 1] += pu * bf16_hi(cur.v[u][e]);
      }
    }
    cur = nxt;
  }

  // Combine the wave's four lane groups (same dims, different tokens), then the four waves.
  auto merge_in = [&](float m2, float l2, const float* acc2) __attribute__((always_inline)) {
    const float M = fmaxf(m, m2);
    if (M == -INFINITY) return;
    const float a1 = fast_exp2(m - M), a2 = fast_exp2(m2 - M);
    l = l * a1 + l2 * a2;
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[d] = acc[d] * a1 + acc2[d] * a2;
    m = M;
  };
#pragma unroll
  for (int sh = 16; sh <= 32; sh <<= 1) {
    float o[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) o[d] = __shfl_xor(acc[d], sh, 64);
    const float m2 = __shfl_xor(m, sh, 64), l2 = __shfl_xor(l, sh, 64);
    merge_in(m2, l2, o);
  }
  __shared__ float red[4][16][10];
  if (lane < 16) {
    red[wave][sub][0] = m;
    red[wave][sub][1] = l;
#pragma unroll
    for (int d = 0; d < 8; ++d) red[wave][sub][2 + d] = acc[d];
  }
  __syncthreads();
  if (wave != 0 || lane >= 16) return;
#pragma unroll
  for (int w2 = 1; w2 < 4; ++w2) merge_in(red[w2][sub][0], red[w2][sub][1], &red[w2][sub][2]);

  const bool empty = !(l > 0.f);
  const float inv = empty ? 0.f : 1.f / l;
  const float lse2 = empty ? -INFINITY : m + __log2f(l);
  const u32x4 packed = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                        pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
  if (final_out) {
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.out) + (int64_t)row * kExHead + 8 * sub) = packed;
    if (a.lse != nullptr && sub == 0) a.lse[row] = lse2 * kLn2;
  } else {
    const int64_t prow = (int64_t)row * a.n_split + split;
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.part_o) + prow * kExHead + 8 * sub) = packed;
    if (sub == 0) a.part_lse[prow] = lse2;
  }
}


// Few-row projection with a [K, N] weight (rows <= 32: the decode batch, as
// in the absorbed layer's W_uv up-projection).  There the 128-row tiles above
// would compute mostly padding, and each workgroup's K loop waits on one
// load after another.  Here one workgroup owns (outer, head, 32 output
// columns) for all rows.  Every load it needs is issued before the first is
// used (one memory latency): the rows of x straight into the B fragments of
// v_mfma_f32_16x16x32_bf16 (contiguous along k), and the [kK, 32] weight
// slice through registers into LDS (rows padded by 16 bytes), from where the
// transposing reads deliver the A fragments.  Wave w computes the block
// Y^T[16 columns x 16 rows] = W^T X^T of column block w/2 and row block w%2;
// rows past `rows` are loaded as zeros and never stored.  A [N, K] weight
// (query absorption) has no such path: the tiled kernel above already runs
// it at the speed of a plain read of its bytes.
constexpr int kFewRows = 32;
constexpr int kFewNt = 32;                    // output columns per workgroup
constexpr int kFewWPitch = kFewNt * 2 + 16;   // bytes per staged weight row

template <int kK>
__global__ __launch_bounds__(256) void latent_project_few(ProjectArgs p) {
  constexpr int kSteps = kK / 32;
  __shared__ __attribute__((aligned(16))) unsigned char wst[kK * kFewWPitch];
  const int n_slices = p.n_dim / kFewNt;
  const int slice = blockIdx.x % n_slices;
  const int oi = blockIdx.x / n_slices;  // outer * heads + head
  const int head = oi % p.heads, o = oi / p.heads;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, g = lane >> 4;
  const int nb = wave >> 1, rb = wave & 1;
  const uint16_t* xg = p.x + (int64_t)o * p.x_outer + (int64_t)head * p.x_head;
  const uint16_t* wg = p.w + (int64_t)head * p.w_head + (int64_t)slice * kFewNt;

  // B operand X^T: lane l holds x row 16*rb + l%16 at k 32*ks + 8*(l/16) .. +7.
  const int row = 16 * rb + n16;
  bf16x8 xf[kSteps];
#pragma unroll
  for (int ks = 0; ks < kSteps; ++ks) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < p.rows) v = *reinterpret_cast<const u32x4*>(xg + (int64_t)row * p.x_row + 32 * ks + 8 * g);
    xf[ks] = __builtin_bit_cast(bf16x8, v);
  }
  // The weight slice: thread t moves 16-byte pieces t, t+256, ... (row piece/4, chunk piece%4).
  constexpr int kPer = kK * (kFewNt / 8) / 256;
  static_assert(kK * (kFewNt / 8) % 256 == 0, "whole pieces per thread");
  u32x4 wv[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int c = tid + 256 * u;
    wv[u] = *reinterpret_cast<const u32x4*>(wg + (int64_t)(c >> 2) * p.n_dim + 8 * (c & 3));
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int c = tid + 256 * u;
    *reinterpret_cast<u32x4*>(wst + (c >> 2) * kFewWPitch + 16 * (c & 3)) = wv[u];
  }
  __syncthreads();

  // A operand W^T: lane n of a 16-lane group addresses row 32*ks + 8*g + n/4
  // (and +4) at columns 16*nb + 4*(n%4) .. +3, and receives column 16*nb + n.
  const auto* wl = (const __attribute__((address_space(3))) unsigned char*)wst;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < kSteps; ++ks) {
    const int off = (32 * ks + 8 * g + (n16 >> 2)) * kFewWPitch + (16 * nb + 4 * (n16 & 3)) * 2;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(wl + off));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(wl + off + 4 * kFewWPitch));
    const bf16x8 aop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, xf[ks], acc, 0, 0, 0);
  }
  // Lane l holds Y^T[column 16*nb + 4*(l/16) + v][row 16*rb + l%16].
  if (row < p.rows) {
    uint16_t* y = p.y + (int64_t)o * p.y_outer + (int64_t)head * p.y_head + (int64_t)row * p.y_row +
                  slice * kFewNt + 16 * nb + 4 * g;
    *reinterpret_cast<uint2*>(y) = make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
  }
}

// The few-row path applies to [K, N] weights, rows <= 32 and the reduction
// lengths it is compiled for; it returns false (and launches nothing)
// otherwise.
bool launch_few(const ProjectArgs& p, hipStream_t stream, hipError_t& err) {
  if (p.w_transposed || p.rows > kFewRows || p.n_dim % kFewNt != 0) return false;
  const int64_t blocks = (int64_t)p.outer * p.heads * (p.n_dim / kFewNt);
  if (blocks <= 0 || blocks > 0x7fffffff) return false;
  const dim3 grid((unsigned)blocks), block(256);
  if (p.k_dim == 512) latent_project_few<512><<<grid, block, 0, stream>>>(p);
  else if (p.k_dim == 128) latent_project_few<128><<<grid, block, 0, stream>>>(p);
  else if (p.k_dim == 64) latent_project_few<64><<<grid, block, 0, stream>>>(p);
  else return false;
  err = hipGetLastError();
  return true;
}

}  // namespace

hipError_t launch_latent_project(const ProjectArgs& p, hipStream_t stream) {
  hipError_t few_err = hipSuccess;
  if (launch_few(p, stream, few_err)) return few_err;
  const int64_t blocks = (int64_t)p.outer * p.heads * p.m_tiles * p.n_tiles;
  if (blocks <= 0 || blocks > 0x7fffffff || p.k_dim % kBK != 0 || p.n_dim % kBN != 0) return hipErrorInvalidValue;
  if (p.w_transposed) latent_project<true><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(p);
  else latent_project<false><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_latent_rebuild(const ProjectArgs& p, hipStream_t stream) {
  // Stacked transposed weights of 128 columns per head, two heads per tile;
  // anything else takes the general projection.
  // y must hold whole 256-row tiles.
  const int64_t padded_rows = ((int64_t)p.rows + kRbM - 1) / kRbM * kRbM;
  if (!p.w_transposed || p.n_dim != 128 || p.heads % 2 != 0 || p.k_dim % kRbK != 0 ||
      p.w_head != (int64_t)p.n_dim * p.k_dim || p.rows < 1 || p.outer < 1 || p.y_head < padded_rows * p.y_row ||
      (int64_t)p.outer * ((p.rows + kRbM - 1) / kRbM) * (p.heads / 2) > INT32_MAX / 2)
    return launch_latent_project(p, stream);
  latent_rebuild<<<dim3(8 * kRbSlots), dim3(kRbWaves * 64), 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_transpose_heads(const void* src, void* dst, int heads, int rows, int cols, hipStream_t stream) {
  if (rows % 64 != 0 || cols % 64 != 0) return hipErrorInvalidValue;
  const int64_t blocks = (int64_t)heads * (rows / 64) * (cols / 64);
  transpose_heads<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(static_cast<const uint16_t*>(src),
                                                                   static_cast<uint16_t*>(dst), rows, cols);
  return hipGetLastError();
}

hipError_t launch_mla_explicit_attend(const DecodeArgs& a, hipStream_t stream, const LaunchEvents& ev) {
  const int64_t blocks = (int64_t)a.batch * a.num_q_heads * a.n_split;
  if (blocks <= 0 || blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipExtLaunchKernelGGL(mla_explicit_attend, dim3((unsigned)blocks), dim3(256), 0, stream, ev.start, ev.stop, 0, a);
  return hipGetLastError();
}

}  // namespace kvattn
