// Grouped-query decode attention, fp32 cache, split-K flash-decode on the
// vector ALUs.
//
// Same contract as the bf16 kernel ("MQA, GQA, and MLA", sections 2-4 and
// 8: query head i reads KV head i / (h/g), each K/V row is fetched once per
// decode step for all heads of its group).  fp32 has no matrix-core form that
// pays at these sizes, so the work is laid out for the VALUs, one workgroup
// per (sequence, KV head, split), 32-token tiles staged in LDS:
//  1. coalesced 16-byte loads bring the K and V rows of the tile into LDS;
//  2. one thread per (head, token) computes the 128-long dot product from LDS
//     (the group's queries sit in LDS for the whole split);
//  3. one thread per head updates its running max and sum and turns the
//     tile's scores into probabilities;
//  4. one thread per (head, pair of output columns) rescales its running
//     output and adds the tile's probability-weighted V rows.
#include "cache_addr.h"
#include <hip/hip_ext.h>

#include "device_common.h"
#include "kvattn_internal.h"

namespace kvattn {
namespace {

constexpr int kTileF = 32;                 // tokens per tile
constexpr int kRowF = kHeadDim + 4;        // LDS row pitch in floats (breaks bank aliasing between rows)
constexpr int kHeadsPerThread = kMaxGroupF32 / 4;

__global__ __launch_bounds__(256) void gqa_split_f32(DecodeArgs a) {
  const int split = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int r = a.group, h = a.num_q_heads;

  const int len = clamp_len(a.seq_lens[b], a.len_cap);
  const int t_lo = window_first(len, a.window);  // tokens before t_lo are outside the window
  const int t_begin = window_base(len, a.window) + split * a.split_tokens;
  const bool final_out = (a.n_split == 1);
  if (!final_out && t_begin >= len) return;
  // The last split ends at the sequence's end (it also takes a window's aligned start).
  const int t_end = split == a.n_split - 1 ? len : min(len, t_begin + a.split_tokens);

  __shared__ __attribute__((aligned(16))) float kt[kTileF * kRowF];
  __shared__ __attribute__((aligned(16))) float vt[kTileF * kRowF];
  __shared__ __attribute__((aligned(16))) float qs[kMaxGroupF32 * kHeadDim];
  __shared__ float sc[kMaxGroupF32][kTileF + 1];
  __shared__ float m_s[kMaxGroupF32], l_s[kMaxGroupF32], al_s[kMaxGroupF32];

  const float* qg = static_cast<const float*>(a.q) + ((int64_t)b * h + (int64_t)j * r) * kHeadDim;
  for (int e = tid; e < r * kHeadDim; e += 256) qs[e] = qg[e];
  if (tid < r) {
    m_s[tid] = -INFINITY;
    l_s[tid] = 0.f;
  }

  // Thread tid accumulates output columns dp, dp+1 of heads hg, hg+4, hg+8, ...
  const int dp = (tid & 63) * 2, hg = tid >> 6;
  float acc[kHeadsPerThread][2];
#pragma unroll
  for (int k = 0; k < kHeadsPerThread; ++k) acc[k][0] = acc[k][1] = 0.f;

  const float* kbase = static_cast<const float*>(a.k);
  const float* vbase = static_cast<const float*>(a.v);

  for (int t0 = t_begin; t0 < t_end; t0 += kTileF) {
    __syncthreads();
    // 32 rows x 128 floats per tensor = 1024 float4 chunks, 4 per thread.
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = tid + 256 * u;
      const int row = c >> 5, col = c & 31;
      const int t = t0 + row;
      float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
      if (t < t_end) {
        const int64_t off = cache_row_offset(a, b, j, t, kHeadDim);
        if (off >= 0) {
          kv = *reinterpret_cast<const float4*>(kbase + off + col * 4);
          vv = *reinterpret_cast<const float4*>(vbase + off + col * 4);
        }
      }
      *reinterpret_cast<float4*>(kt + row * kRowF + col * 4) = kv;
      *reinterpret_cast<float4*>(vt + row * kRowF + col * 4) = vv;
    }
    __syncthreads();

    for (int p = tid; p < r * kTileF; p += 256) {
      const int i = p / kTileF, tt = p % kTileF;
      const float* qi = qs + i * kHeadDim;
      const float* kr = kt + tt * kRowF;
      float dot = 0.f;
#pragma unroll 8
      for (int d = 0; d < kHeadDim; d += 4) {
        const float4 x = *reinterpret_cast<const float4*>(qi + d);
        const float4 y = *reinterpret_cast<const float4*>(kr + d);
        dot = fmaf(x.x, y.x, dot);
        dot = fmaf(x.y, y.y, dot);
        dot = fmaf(x.z, y.z, dot);
        dot = fmaf(x.w, y.w, dot);
      }
      sc[i][tt] = (t0 + tt < t_end && t0 + tt >= t_lo) ? dot * a.scale_log2 : -INFINITY;
    }
    __syncthreads();

    if (tid < r) {
      const int i = tid;
      float mt = -INFINITY;
      for (int tt = 0; tt < kTileF; ++tt) mt = fmaxf(mt, sc[i][tt]);
      const float m_old = m_s[i];
      const float m_new = fmaxf(m_old, mt);  // -inf only while every token so far was masked (sliding window)
      const float m_use = m_new == -INFINITY ? 0.f : m_new;  // then al and every p are 0, not NaN
      const float al = fast_exp2(m_old - m_use);
      float sum = 0.f;
      for (int tt = 0; tt < kTileF; ++tt) {
        const float p = fast_exp2(sc[i][tt] - m_use);
        sc[i][tt] = p;
        sum += p;
      }
      l_s[i] = l_s[i] * al + sum;
      m_s[i] = m_new;
      al_s[i] = al;
    }
    __syncthreads();

#pragma unroll
    for (int k = 0; k < kHeadsPerThread; ++k) {
      const int i = hg + 4 * k;
      if (i < r) {
        const float al = al_s[i];
        float x0 = acc[k][0] * al, x1 = acc[k][1] * al;
        for (int tt = 0; tt < kTileF; ++tt) {
          const float p = sc[i][tt];
          const float2 v = *reinterpret_cast<const float2*>(vt + tt * kRowF + dp);
          x0 = fmaf(p, v.x, x0);
          x1 = fmaf(p, v.y, x1);
        }
        acc[k][0] = x0;
        acc[k][1] = x1;
      }
    }
  }
  __syncthreads();

#pragma unroll
  for (int k = 0; k < kHeadsPerThread; ++k) {
    const int i = hg + 4 * k;
    if (i >= r) continue;
    const int64_t row = (int64_t)b * h + (int64_t)j * r + i;
    const float l = l_s[i];
    const bool empty = !(l > 0.f);
    const float inv = empty ? 0.f : 1.f / l;
    const float lse2 = empty ? -INFINITY : m_s[i] + __log2f(l);
    if (final_out) {
      float* o = static_cast<float*>(a.out) + row * kHeadDim + dp;
      o[0] = acc[k][0] * inv;
      o[1] = acc[k][1] * inv;
      if (a.lse != nullptr && dp == 0) a.lse[row] = lse2 * kLn2;
    } else {
      float* po = a.part_o + (row * a.n_split + split) * kHeadDim + dp;
      po[0] = acc[k][0] * inv;
      po[1] = acc[k][1] * inv;
      if (dp == 0) a.part_lse[row * a.n_split + split] = lse2;
    }
  }
}

}  // namespace

hipError_t launch_gqa_f32(const DecodeArgs& a, hipStream_t stream, const LaunchEvents& ev) {
  if (a.group > kMaxGroupF32) return hipErrorInvalidValue;
  const dim3 grid(a.n_split, a.num_kv_heads, a.batch);
  hipExtLaunchKernelGGL(gqa_split_f32, grid, dim3(256), 0, stream, ev.start, ev.stop, 0, a);
  return hipGetLastError();
}

}  // namespace kvattn
