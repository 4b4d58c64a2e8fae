// Log-sum-exp merge of split-K partial results.
//
// A sequence's tokens are cut into splits that run as separate workgroups.
// Split s leaves o_s (its output, already normalised over its own tokens)
// and lse_s (log2 of its softmax normaliser, in the same log2 units as the
// scaled scores).  The exact result over all tokens is
//     M = max_s lse_s,  w_s = 2^(lse_s - M),  o = sum_s w_s o_s / sum_s w_s,
//     lse = M + log2(sum_s w_s)
// (softmax over a union of token sets).  One workgroup per (sequence, head),
// of one wave, or of up to sixteen when a row has many splits (a long
// sequence): every wave then finds M and the normaliser over all splits
// itself (a few loads per lane), sums the weighted partials of its share of
// the splits, and the waves' sums are added through LDS.
// The splits of a bf16-output call (bf16 or fp8 cache) hand over bf16
// partial outputs, those of an fp32 call fp32 ones; log-sum-exps and the
// combination are fp32 throughout.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "kvattn_internal.h"

namespace kvattn {
namespace {

// The two bf16 values packed in a 32-bit word, widened to fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int DV, bool BF16>
__global__ __launch_bounds__(1024) void lse_merge(DecodeArgs a) {
  // Lane l handles float4 columns c = l % kRowLanes (+ kRowLanes * k) of
  // the splits s = l / kRowLanes + kSplitGroups * u.  Every load of a round
  // (the splits' log-sum-exps and partial outputs) is issued before any is
  // used, so a round costs one memory latency; one round covers up to
  // kSplitGroups * kU splits.
  constexpr int kVec = DV / 4;                        // float4 columns per row
  constexpr int kRowLanes = kVec < 64 ? kVec : 64;    // lanes across a row
  constexpr int kSplitGroups = 64 / kRowLanes;        // splits read side by side
  constexpr int kCols = kVec / kRowLanes;             // float4 columns per lane
  constexpr int kU = 8;                               // splits per lane and round
  const int head = blockIdx.x, b = blockIdx.y, lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6, n_waves = blockDim.x >> 6;
  const int c = lane % kRowLanes, sg = lane / kRowLanes;
  const int len = clamp_len(a.seq_lens[b], a.len_cap);
  int nv = (len - window_base(len, a.window) + a.split_tokens - 1) / a.split_tokens;
  nv = min(nv, a.n_split);
  const int64_t row = (int64_t)b * a.num_q_heads + head;
  const float* pl = a.part_lse + row * a.n_split;
  // Partial outputs: four columns per load, as loaded (bf16: 8 bytes, fp32: 16).
  using Part = std::conditional_t<BF16, uint16_t, float>;
  using Raw = std::conditional_t<BF16, uint2, f32x4>;
  const Part* po = reinterpret_cast<const Part*>(a.part_o) + row * a.n_split * DV;
  auto widen = [](const Raw& w) __attribute__((always_inline)) {
    if constexpr (BF16) return f32x4{bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
    else return w;
  };

  // Loads of one round: splits s0 + sg + kSplitGroups * u (past the last
  // split: the last one again, weighted 0 below).
  Raw x[kU][kCols];
  float ls[kU];
  auto load_round = [&](int s0) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int s = min(s0 + sg + kSplitGroups * u, nv - 1);
      ls[u] = pl[s];
#pragma unroll
      for (int k = 0; k < kCols; ++k)
        x[u][k] = *reinterpret_cast<const Raw*>(po + (int64_t)s * DV + 4 * (c + kRowLanes * k));
    }
  };
  constexpr int kRound = kSplitGroups * kU;  // splits per round of one wave; wave w takes rounds w, w + n_waves, ...
  if (nv > wave * kRound) load_round(wave * kRound);  // in flight while the maximum and the normaliser are found

  // Lane l keeps the log-sum-exps of splits l, l + 64, ..., l + 448, all
  // loaded before any is used; splits past 512 are reread.
  constexpr int kLse = 8;
  float lv[kLse];
#pragma unroll
  for (int i = 0; i < kLse; ++i) lv[i] = lane + 64 * i < nv ? pl[lane + 64 * i] : -INFINITY;
  float M = lv[0];
#pragma unroll
  for (int i = 1; i < kLse; ++i) M = fmaxf(M, lv[i]);
  for (int s = lane + 64 * kLse; s < nv; s += 64) M = fmaxf(M, pl[s]);
  M = wave_reduce_max(M);
  float L = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int i = 0; i < kLse; ++i) L += fast_exp2(lv[i] - M);  // 2^-inf = 0 past the end
    for (int s = lane + 64 * kLse; s < nv; s += 64) L += fast_exp2(pl[s] - M);
  }
  L = wave_reduce_sum(L);
  const bool empty = !(L > 0.f);
  const float inv = empty ? 0.f : 1.f / L;

  f32x4 acc[kCols];
#pragma unroll
  for (int k = 0; k < kCols; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (!empty) {
    for (int s0 = wave * kRound; s0 < nv; s0 += n_waves * kRound) {
      if (s0 > wave * kRound) load_round(s0);
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const float w = s0 + sg + kSplitGroups * u < nv ? fast_exp2(ls[u] - M) : 0.f;
#pragma unroll
        for (int k = 0; k < kCols; ++k) acc[k] += w * widen(x[u][k]);
      }
    }
  }
  // Lanes of the other split groups hold the other splits' sums for the same columns.
#pragma unroll
  for (int m = kRowLanes; m < 64; m <<= 1)
#pragma unroll
    for (int k = 0; k < kCols; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[k][e] += __shfl_xor(acc[k][e], m, 64);
  if (n_waves > 1) {
    // The other waves' sums, added by wave 0 (the launch sizes the LDS:
    // kRowLanes * kCols float4 per wave past the first, none for one wave).
    extern __shared__ f32x4 red[];
    constexpr int kRow = kRowLanes * kCols;
    if (wave > 0 && sg == 0) {
#pragma unroll
      for (int k = 0; k < kCols; ++k) red[(wave - 1) * kRow + c + kRowLanes * k] = acc[k];
    }
    __syncthreads();
    if (wave > 0) return;
    for (int w2 = 1; w2 < n_waves; ++w2)
#pragma unroll
      for (int k = 0; k < kCols; ++k) acc[k] += red[(w2 - 1) * kRow + c + kRowLanes * k];
  }
  if (sg == 0) {
#pragma unroll
    for (int k = 0; k < kCols; ++k) {
      const f32x4 o4 = acc[k] * inv;
      const int64_t off = row * DV + 4 * (c + kRowLanes * k);
      if constexpr (BF16) {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + off) =
            make_uint2(pack_bf16x2(o4[0], o4[1]), pack_bf16x2(o4[2], o4[3]));
      } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + off) = o4;
      }
    }
  }
  if (lane == 0 && a.lse != nullptr) a.lse[row] = empty ? -INFINITY : (M + __log2f(L)) * kLn2;
}

}  // namespace

hipError_t launch_merge(const DecodeArgs& a, bool out_bf16, hipStream_t stream) {
  const dim3 grid(a.num_q_heads, a.batch);
  // One wave per row, or one per 32 splits (two rounds of loads each) up to sixteen.
  const int waves = std::min(16, std::max(1, (a.n_split + 31) / 32));
  // LDS for the waves' sums: one row of kHeadDim floats per wave past the first.
  const size_t lds = (size_t)(waves - 1) * kHeadDim * sizeof(float);
  if (out_bf16) lse_merge<kHeadDim, true><<<grid, 64 * waves, lds, stream>>>(a);
  else lse_merge<kHeadDim, false><<<grid, 64 * waves, lds, stream>>>(a);
  return hipGetLastError();
}

}  // namespace kvattn
