// Log-sum-exp merge of split-K partial results.
//
// A sequence's tokens are cut into splits that run as separate workgroups.
// Split s leaves o_s (its output, already normalised over its own tokens)
// and lse_s (log2 of its softmax normaliser, in the same log2 units as the
// scaled scores).  The exact result over all tokens is
//     M = max_s lse_s,  w_s = 2^(lse_s - M),  o = sum_s w_s o_s / sum_s w_s,
//     lse = M + log2(sum_s w_s)
// (softmax over a union of token sets).  One wave per (sequence, head);
// lane l owns output columns 4l..4l+3 (and 4(l+64).. for d_v = 512).
#include "device_common.h"
#include "kvattn_internal.h"

namespace kvattn {
namespace {

template <int DV, bool BF16_OUT>
__global__ __launch_bounds__(64) void lse_merge(DecodeArgs a) {
  const int head = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int len = clamp_len(a.seq_lens[b], a.len_cap);
  int nv = (len - window_base(len, a.window) + a.split_tokens - 1) / a.split_tokens;
  nv = min(nv, a.n_split);
  const int64_t row = (int64_t)b * a.num_q_heads + head;
  const float* pl = a.part_lse + row * a.n_split;
  const float* po = a.part_o + row * a.n_split * DV;

  float M = -INFINITY;
  for (int s = lane; s < nv; s += 64) M = fmaxf(M, pl[s]);
  M = wave_reduce_max(M);
  float L = 0.f;
  if (M != -INFINITY)
    for (int s = lane; s < nv; s += 64) L += fast_exp2(pl[s] - M);
  L = wave_reduce_sum(L);
  const bool empty = !(L > 0.f);
  const float inv = empty ? 0.f : 1.f / L;

  for (int d4 = lane; d4 < DV / 4; d4 += 64) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (!empty) {
      for (int s = 0; s < nv; ++s) {
        const float w = fast_exp2(pl[s] - M);
        acc += w * *reinterpret_cast<const f32x4*>(po + (int64_t)s * DV + 4 * d4);
      }
    }
    acc *= inv;
    if constexpr (BF16_OUT) {
      uint16_t* o = static_cast<uint16_t*>(a.out) + row * DV + 4 * d4;
      const uint32_t lo = pack_bf16x2(acc[0], acc[1]);
      const uint32_t hi = pack_bf16x2(acc[2], acc[3]);
      *reinterpret_cast<uint2*>(o) = make_uint2(lo, hi);
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + row * DV + 4 * d4) = acc;
    }
  }
  if (lane == 0 && a.lse != nullptr) a.lse[row] = empty ? -INFINITY : (M + __log2f(L)) * kLn2;
}

}  // namespace

hipError_t launch_merge(const DecodeArgs& a, int d_v, bool out_bf16, hipStream_t stream) {
  const dim3 grid(a.num_q_heads, a.batch);
  const dim3 block(64);
  if (d_v == kHeadDim) {
    if (out_bf16) lse_merge<kHeadDim, true><<<grid, block, 0, stream>>>(a);
    else lse_merge<kHeadDim, false><<<grid, block, 0, stream>>>(a);
  } else if (d_v == kMlaLatent) {
    if (out_bf16) lse_merge<kMlaLatent, true><<<grid, block, 0, stream>>>(a);
    else lse_merge<kMlaLatent, false><<<grid, block, 0, stream>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvattn
