// Device-side work plan for MLA decode, and the merge of its pieces.
//
// An MLA split writes a partial as large as the output rows of all heads
// (128 heads x 513 fp32 for DeepSeek-V2, against 1152 cache bytes per
// token), so splits must stay long, and one 128-head workgroup fills a
// compute unit.  With ragged sequence lengths, fixed-size splits then leave
// either a few long workgroups that set the pace or a second round of
// workgroups.  The plan instead looks at the actual lengths (they live in
// device memory, so the plan is made on the device, by one wave, in the
// stream of the kernels that use it) and picks the shortest piece length t
// (a multiple of 32, at least min_chunk) for which the sequences, each cut
// into ceil(len / t) pieces, give at most max(work_items, batch) pieces: one
// round of workgroups with the longest piece as short as that allows.  A
// sequence's pieces are equal in length up to the 32-token tile (its cuts
// sit on multiples of 32), so a piece is a (sequence, first token, end
// token) triple and the pieces of a sequence are consecutive.  A caller's
// split_tokens fixes t instead.  A sequence covered by one piece gets its
// output written directly by the decode kernel; the others are combined by
// the log-sum-exp merge below.
#include <algorithm>

#include "device_common.h"
#include "kvattn_internal.h"

namespace kvattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The two bf16 values packed in a 32-bit word, widened to fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// The plan runs as one wave: lane l handles sequences l, l+64, ...; the
// lengths of the first kCached rounds stay in registers across the search.
constexpr int kCached = 8;

// Most waves in one workgroup of the piece merge.
constexpr int kMergeMaxWaves = 16;

__device__ __forceinline__ int64_t align32(int64_t x) { return (x + 31) & ~int64_t(31); }

// ceil(a / b) for 0 <= a, b < 2^31 in 32-bit unsigned arithmetic (a + b - 1
// stays below 2^32; the 64-bit division is several times slower).
__device__ __forceinline__ uint32_t ceil_div(uint32_t a, uint32_t b) { return (a + b - 1) / b; }

// Length of each piece of a sequence of `len` tokens cut for piece length t:
// ceil(len / t) pieces of equal length, rounded up to the tile.
__device__ __forceinline__ int64_t piece_len(int len, uint32_t t) {
  const uint32_t n = ceil_div((uint32_t)len, t);
  return align32(ceil_div((uint32_t)len, n));
}

// Pieces of a sequence of `len` tokens for piece length t (an empty sequence
// keeps one empty piece).
__device__ __forceinline__ int pieces_of(int len, uint32_t t) {
  return len > 0 ? (int)ceil_div((uint32_t)len, t) : 1;
}

__device__ __forceinline__ int64_t wave_sum_i64(int64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const int lo = __shfl_xor((int)(v & 0xffffffff), m, 64);
    const int hi = __shfl_xor((int)(v >> 32), m, 64);
    v += ((int64_t)hi << 32) | (uint32_t)lo;
  }
  return v;
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ int wave_max_int(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = max(v, __shfl_xor(v, m, 64));
  return v;
}

// Inclusive prefix sum over the wave.
__device__ __forceinline__ int wave_scan_int(int v) {
  const int lane = threadIdx.x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  return v;
}

__global__ __launch_bounds__(64) void mla_plan(MlaPlanArgs p) {
  const int lane = threadIdx.x;
  const int rounds = (p.batch + 63) / 64;  // wave-uniform
  int cl[kCached];
#pragma unroll
  for (int i = 0; i < kCached; ++i) {
    const int b = lane + 64 * i;
    cl[i] = b < p.batch ? clamp_len(p.seq_lens[b], p.len_cap) : -1;  // -1: no sequence
  }
  // Number of pieces for piece length t, saturated at cap + 1 (enough to compare with cap).
  auto pieces_for = [&](uint32_t t, int cap) {
    int n = 0;
#pragma unroll
    for (int i = 0; i < kCached; ++i)
      if (i < rounds && cl[i] >= 0) n = min(n + pieces_of(cl[i], t), cap + 1);
    for (int b = lane + 64 * kCached; b < p.batch && n <= cap; b += 64)
      n = min(n + pieces_of(clamp_len(p.seq_lens[b], p.len_cap), t), cap + 1);
    return wave_sum_int(n);
  };
  uint32_t t = p.fixed_chunk > 0 ? (uint32_t)p.fixed_chunk : 0u;  // piece length, up to 2^31
  if (t == 0) {
    // Shortest multiple of 32 in [min_chunk, len_cap rounded up] with at most
    // cap pieces (the count only falls as t grows, and the upper end gives
    // one piece per sequence).
    const int cap = p.work_items > p.batch ? p.work_items : p.batch;
    uint32_t lo = (uint32_t)p.min_chunk / 32;
    uint32_t hi = (uint32_t)(align32(p.len_cap > p.min_chunk ? p.len_cap : p.min_chunk) / 32);
    // Closed-form bounds narrow the search: sum ceil(len/t) >= total/t, and
    // <= total/t + (sequences), so t >= total/cap always and t = total/(cap -
    // sequences) is enough when cap exceeds the number of sequences.
    {
      int64_t tot = 0;
#pragma unroll
      for (int i = 0; i < kCached; ++i)
        if (i < rounds && cl[i] > 0) tot += cl[i];
      for (int b = lane + 64 * kCached; b < p.batch; b += 64) tot += clamp_len(p.seq_lens[b], p.len_cap);
      const int64_t total = wave_sum_i64(tot);
      const uint32_t lb = (uint32_t)(align32((total + cap - 1) / cap) / 32);
      if (lb > lo) lo = lb < hi ? lb : hi;
      if (cap > p.batch) {
        const uint32_t ub = (uint32_t)(align32((total + (cap - p.batch) - 1) / (cap - p.batch)) / 32);
        if (ub < hi) hi = ub > lo ? ub : lo;
      }
    }
    while (lo < hi) {
      const uint32_t mid = lo + (hi - lo) / 2;
      if (pieces_for(32u * mid, cap) <= cap) hi = mid;
      else lo = mid + 1;
    }
    t = 32u * lo;
  }

  // Sequences in rounds of 64; the first piece of each is an exclusive
  // prefix sum carried across rounds.  When no sequence of a round has more
  // than kOwnPieces pieces, each lane writes its own sequence's pieces;
  // otherwise (a long sequence has hundreds) the whole wave writes them,
  // piece q by lane q mod 64, which finds its sequence by a binary search
  // over the round's inclusive piece counts.
  constexpr int kOwnPieces = 16;
  __shared__ int s_incl[64], s_len[64];
  int carry = 0;
  for (int base = 0, i = 0; base < p.batch; base += 64, ++i) {
    const int b = base + lane;
    int len = -1;
#pragma unroll
    for (int k = 0; k < kCached; ++k)
      if (k == i) len = cl[k];
    if (i >= kCached && b < p.batch) len = clamp_len(p.seq_lens[b], p.len_cap);
    const int count = b < p.batch ? pieces_of(len, t) : 0;
    const int incl = wave_scan_int(count);
    const int round_total = __shfl(incl, 63, 64);
    const int first = carry + incl - count;
    if (b < p.batch) p.seq_pieces[b] = make_int2(first, count);
    if (wave_max_int(count) <= kOwnPieces) {
      const int64_t plen = len > 0 ? piece_len(len, t) : 0;
      for (int j = 0; j < count; ++j) {
        const int64_t lo = j * plen;
        const int64_t hi = lo + plen < len ? lo + plen : len;
        p.pieces[first + j] = make_int4(b, (int)lo, (int)hi, count == 1 ? 1 : 0);
      }
      carry += round_total;
      continue;
    }
    s_incl[lane] = incl;
    s_len[lane] = len;
    __syncthreads();
    for (int q = lane; q < round_total; q += 64) {
      // First k with s_incl[k] > q: the sequence holding piece q (sequences
      // with no pieces have s_incl[k] == s_incl[k - 1] and are skipped).
      int lo_k = 0, hi_k = 63;
      while (lo_k < hi_k) {
        const int mid = (lo_k + hi_k) >> 1;
        if (s_incl[mid] > q) hi_k = mid;
        else lo_k = mid + 1;
      }
      const int before = lo_k > 0 ? s_incl[lo_k - 1] : 0;
      const int cnt = s_incl[lo_k] - before, sl = s_len[lo_k], j = q - before;
      const int64_t plen = sl > 0 ? piece_len(sl, t) : 0;
      const int64_t lo = j * plen;
      const int64_t hi = lo + plen < sl ? lo + plen : sl;
      p.pieces[carry + q] = make_int4(base + lo_k, (int)lo, (int)hi, cnt == 1 ? 1 : 0);
    }
    __syncthreads();  // the next round rewrites s_incl and s_len
    carry += round_total;
  }
  if (lane == 0) {
    p.plan_count[0] = carry;
    p.plan_count[1] = (int)(t < 0x7fffffffu ? t : 0x7fffffffu);
  }
}

// Log-sum-exp merge of the pieces of each sequence with more than one.
// Piece q leaves o_q (normalised over its own tokens, rounded to bf16) and
// lse_q (fp32, log2 of its normaliser); M = max lse_q, w_q = 2^(lse_q - M), o = sum w_q o_q / sum w_q,
// lse = M + log2 sum w_q.  One workgroup per (sequence, head): one wave, or
// up to sixteen when sequences have many pieces (a long one): every wave then
// finds M and the normaliser over all pieces itself, sums the weighted
// partials of its share of the pieces, and the waves' sums are added
// through LDS.
__global__ __launch_bounds__(1024) void mla_merge_pieces(DecodeArgs a) {
  const int head = blockIdx.x, b = blockIdx.y, lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6, n_waves = blockDim.x >> 6;
  const int2 sp = a.seq_pieces[b];
  const int n = sp.y;
  if (n <= 1) return;  // written directly by the decode kernel
  const int h = a.num_q_heads;
  const int64_t row = (int64_t)b * h + head;
  const float* pl = a.part_lse + (int64_t)sp.x * h + head;  // piece s: pl[s * h]

  // Partial outputs are bf16 [piece, head, 512].  Lane l owns columns 8l ..
  // 8l+7 (one 16-byte load per piece); a round takes eight pieces, all of
  // whose loads are issued before any is used, and wave w takes rounds w,
  // w + n_waves, ...  The wave's first round is in flight while the maximum
  // and the normaliser are found.
  const uint16_t* po = reinterpret_cast<const uint16_t*>(a.part_o) + ((int64_t)sp.x * h + head) * kMlaLatent + 8 * lane;
  u32x4 x[8];
  float ls[8];
  auto load_round = [&](int s0) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = min(s0 + u, n - 1);  // past the last piece: reread it with weight 0
      ls[u] = pl[(int64_t)s * h];
      x[u] = *reinterpret_cast<const u32x4*>(po + (int64_t)s * h * kMlaLatent);
    }
  };
  if (n > 8 * wave) load_round(8 * wave);

  // Lane l keeps the log-sum-exps of pieces l, l + 64, l + 128, l + 192;
  // pieces past 256 are reread.
  float lv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) lv[i] = lane + 64 * i < n ? pl[(int64_t)(lane + 64 * i) * h] : -INFINITY;
  float M = fmaxf(fmaxf(lv[0], lv[1]), fmaxf(lv[2], lv[3]));
  for (int s = lane + 256; s < n; s += 64) M = fmaxf(M, pl[(int64_t)s * h]);
  M = wave_reduce_max(M);
  float L = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int i = 0; i < 4; ++i) L += fast_exp2(lv[i] - M);  // 2^-inf = 0 past the end
    for (int s = lane + 256; s < n; s += 64) L += fast_exp2(pl[(int64_t)s * h] - M);
  }
  L = wave_reduce_sum(L);
  const bool empty = !(L > 0.f);
  const float inv = empty ? 0.f : 1.f / L;

  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
  if (!empty) {
    for (int s0 = 8 * wave; s0 < n; s0 += 8 * n_waves) {
      if (s0 > 8 * wave) load_round(s0);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float w = s0 + u < n ? fast_exp2(ls[u] - M) : 0.f;
        acc0 += w * f32x4{bf16_lo(x[u][0]), bf16_hi(x[u][0]), bf16_lo(x[u][1]), bf16_hi(x[u][1])};
        acc1 += w * f32x4{bf16_lo(x[u][2]), bf16_hi(x[u][2]), bf16_lo(x[u][3]), bf16_hi(x[u][3])};
      }
    }
  }
  if (n_waves > 1) {
    // The other waves' sums, added by wave 0 (the launch sizes the LDS:
    // 2 x 64 float4 per wave past the first, none for a one-wave row).
    extern __shared__ f32x4 red[];
    if (wave > 0) {
      red[(wave - 1) * 128 + lane] = acc0;
      red[(wave - 1) * 128 + 64 + lane] = acc1;
    }
    __syncthreads();
    if (wave > 0) return;
    for (int w2 = 1; w2 < n_waves; ++w2) {
      acc0 += red[(w2 - 1) * 128 + lane];
      acc1 += red[(w2 - 1) * 128 + 64 + lane];
    }
  }
  acc0 *= inv;
  acc1 *= inv;
  uint16_t* o = static_cast<uint16_t*>(a.out) + row * kMlaLatent + 8 * lane;
  *reinterpret_cast<u32x4*>(o) = u32x4{pack_bf16x2(acc0[0], acc0[1]), pack_bf16x2(acc0[2], acc0[3]),
                                       pack_bf16x2(acc1[0], acc1[1]), pack_bf16x2(acc1[2], acc1[3])};
  if (lane == 0 && a.lse != nullptr) a.lse[row] = empty ? -INFINITY : (M + __log2f(L)) * kLn2;
}

}  // namespace

hipError_t launch_mla_plan(const MlaPlanArgs& p, hipStream_t stream) {
  mla_plan<<<1, 64, 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_mla_merge_pieces(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.num_q_heads, a.batch);
  // One wave per row, or, when the plan may give a sequence many pieces, one
  // per 16 of them (two rounds of loads each) up to kMergeMaxWaves.
  const int per_seq = (a.max_pieces + a.batch - 1) / a.batch;
  const int waves = per_seq > 16 ? std::min(kMergeMaxWaves, (per_seq + 15) / 16) : 1;
  mla_merge_pieces<<<grid, 64 * waves, (waves - 1) * 128 * sizeof(f32x4), stream>>>(a);
  return hipGetLastError();
}

}  // namespace kvattn
