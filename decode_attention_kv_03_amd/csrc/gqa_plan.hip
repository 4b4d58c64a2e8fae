// Device-side work list of the persistent grouped-query split kernel.
//
// A ragged or paged batch cut into fixed splits gives a grid of (sequence,
// KV head, split) workgroups that runs in many rounds, many of them empty
// (splits past a short sequence's end), and each workgroup pays its own
// start-up (lengths, queries, table entries, first tile) with its stream
// stopped.  For such calls the split kernel runs instead as resident
// workgroups that take items from a list made here, on the device, from the
// actual lengths.  An item is one split that holds tokens: (unit b * g + j,
// split s, first token, end token), the same token range the grid-per-split
// form gives split s, so partial outputs land in the same slots and the
// log-sum-exp merge is unchanged.  The list holds the full splits first, then
// the shorter last splits of the sequences, longest first (in 32 length
// classes): the items taken last are the shortest, so the workgroups finish
// close together.  Within a length class the order follows LDS atomics and
// may differ from call to call; which workgroup computes an item does not
// change its result.
#include "device_common.h"
#include "kvattn_internal.h"

namespace kvattn {
namespace {

constexpr int kThreads = 1024;
constexpr int kClasses = 32;
constexpr int kCachedRounds = 4;  // rounds of units whose spans stay in registers between the passes

// Length class of a last split holding `rest` tokens, 0 < rest < split:
// ceil(32 * rest / split), in 1 .. 32.
__device__ __forceinline__ int length_class(int rest, int split) {
  return (int)(((int64_t)rest * kClasses + split - 1) / split);
}

// Exclusive prefix sum of v over the workgroup; the sum of all v in `total`.
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_wave, int& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(x, d, 64);
    if (lane >= d) x += u;
  }
  if (lane == 63) s_wave[wv] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) {
    const int t = s_wave[i];
    before += i < wv ? t : 0;
    all += t;
  }
  __syncthreads();  // s_wave is reused by the next call
  total = all;
  return before + x - v;
}

// The splits of unit u: tokens [base, len) cut at base + s * split.
struct UnitSpan {
  int len, base, full, rest;
};

__device__ __forceinline__ UnitSpan unit_span(const GqaPlanArgs& p, int u) {
  UnitSpan r;
  r.len = clamp_len(p.seq_lens[u / p.g], p.len_cap);
  r.base = window_base(r.len, p.window);
  const int span = r.len - r.base;
  r.full = min(span / p.split, p.n_split);
  r.rest = r.full < p.n_split ? span - r.full * p.split : 0;
  return r;
}

__global__ __launch_bounds__(kThreads) void gqa_plan(GqaPlanArgs p) {
  __shared__ int s_wave[kThreads / 64];
  __shared__ int s_next[kClasses + 1];  // per length class: count, then next free slot
  const int tid = threadIdx.x;
  const int units = p.batch * p.g;
  for (int i = tid; i <= kClasses; i += kThreads) s_next[i] = 0;
  __syncthreads();

  // Full splits, in unit order; the short last splits are counted per class.
  // The spans of the first kCachedRounds rounds of units stay in registers.
  UnitSpan cached[kCachedRounds];
  int carry = 0;
  for (int u0 = 0, i = 0; u0 < units; u0 += kThreads, ++i) {
    const int u = u0 + tid;
    UnitSpan r{0, 0, 0, 0};
    if (u < units) {
      r = unit_span(p, u);
      if (r.rest > 0) atomicAdd(&s_next[length_class(r.rest, p.split)], 1);
    }
#pragma unroll
    for (int k = 0; k < kCachedRounds; ++k)
      if (k == i) cached[k] = r;
    int total;
    const int first = carry + block_exclusive_scan(r.full, s_wave, total);
    for (int s = 0; s < r.full; ++s) {
      const int t0 = r.base + s * p.split;
      p.items[first + s] = make_int4(u, s, t0, t0 + p.split);
    }
    carry += total;
  }
  __syncthreads();
  // Slots of the short splits, the longest class first: an exclusive scan
  // over the classes in descending order, on the first wave.
  if (tid < 64) {
    const int c = kClasses - tid;  // lanes 0 .. 31: classes 32 .. 1
    const int n = c >= 1 ? s_next[c] : 0;
    int x = n;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(x, d, 64);
      if (tid >= d) x += y;
    }
    if (c >= 1) s_next[c] = carry + x - n;
    if (tid == 63) {
      p.ctl[0] = carry + x;
      p.ctl[1] = 0;
    }
  }
  __syncthreads();
  for (int u0 = 0, i = 0; u0 < units; u0 += kThreads, ++i) {
    const int u = u0 + tid;
    UnitSpan r{0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < kCachedRounds; ++k)
      if (k == i) r = cached[k];
    if (i >= kCachedRounds && u < units) r = unit_span(p, u);
    if (u < units && r.rest > 0) {
      const int slot = atomicAdd(&s_next[length_class(r.rest, p.split)], 1);
      const int t0 = r.base + r.full * p.split;
      p.items[slot] = make_int4(u, r.full, t0, r.len);
    }
  }
}

}  // namespace

hipError_t launch_gqa_plan(const GqaPlanArgs& p, hipStream_t stream) {
  gqa_plan<<<1, kThreads, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace kvattn
