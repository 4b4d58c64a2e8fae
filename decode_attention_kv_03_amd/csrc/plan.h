// Split planning of libkvattn (host side): how a call's tokens are cut into
// the splits or pieces that run as separate workgroups.  It decides the grid
// of every split-K kernel, and with it the partials each call writes.
#pragma once

#include <stdint.h>

#include <algorithm>
#include <climits>

#include "../../include/kvattn.h"

namespace kvattn {
namespace plan {

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

constexpr int kCUs = 256;          // MI355X compute units
// Longest sequence a call takes: token indices, split ends and piece ends stay
// well inside 32-bit arithmetic on the device.
constexpr int32_t kMaxSeqLen = 1 << 28;

// Tokens per split for GQA.  A contiguous cache is taken to hold sequences of
// similar length: the fewest splits that still give every CU two resident
// workgroups (longer splits amortise each workgroup's start-up and need fewer
// partials; measured best on all four contiguous workloads).  A paged cache
// is taken to hold ragged lengths: about four workgroups per CU in all, each
// at most 2048 tokens, so that long sequences do not leave a tail.
inline int32_t plan_gqa_split(int32_t batch, int32_t h, int32_t g, int32_t max_seq_len, bool paged, int32_t requested) {
  const int64_t S = max_seq_len > 0 ? max_seq_len : 1;
  // A requested split longer than the longest sequence is one split either way.
  if (requested > 0) return (int32_t)std::min<int64_t>(requested, round_up(S, KVATTN_SPLIT_ALIGN));
  const int64_t units = (int64_t)batch * g;
  const int64_t r = h / g;
  // A split writes r partial rows: at least 16 r tokens keep them small next
  // to the split's own reads, unless that leaves the chip short of
  // workgroups (few sequences and KV heads with many query heads each, e.g.
  // one long MQA sequence); then the floor is 256 tokens.
  const int64_t min_chunk = std::max<int64_t>(256, 16 * r);
  int64_t even;
  if (paged) {
    even = round_up((S * units + 4 * kCUs - 1) / (4 * kCUs), KVATTN_SPLIT_ALIGN);
  } else {
    const int64_t want_splits = std::max<int64_t>(1, (2 * kCUs + units - 1) / units);
    even = round_up((S + want_splits - 1) / want_splits, KVATTN_SPLIT_ALIGN);
  }
  int64_t chunk = std::max(even, min_chunk);
  if (units * ((S + chunk - 1) / chunk) < 2 * kCUs) chunk = std::max<int64_t>(even, 256);
  if (paged) chunk = std::min<int64_t>(chunk, 2048);
  return (int32_t)std::min(chunk, round_up(S, KVATTN_SPLIT_ALIGN));
}

// MLA work plan.  The decode kernel's workgroups take pieces of the
// sequences, cut on the device from the actual lengths (mla_plan.hip): the
// shortest piece length (a multiple of 32, at least kMlaMinChunk) that gives
// at most max(kCUs, batch) pieces (one 128-head workgroup fills a CU), or the
// caller's split_tokens.  The host only bounds the number of pieces.
constexpr int32_t kMlaMinChunk = 256;

// Piece length the plan chooses when every sequence holds max_seq_len tokens.
inline int32_t plan_mla_split(int32_t batch, int32_t max_seq_len, int32_t requested) {
  if (requested > 0) return requested;
  const int64_t S = std::max<int32_t>(max_seq_len, 1);
  const int64_t per_seq = std::max<int64_t>(kCUs, batch) / batch;  // pieces each sequence may take
  const int64_t t = round_up((S + per_seq - 1) / per_seq, 32);
  return (int32_t)std::min<int64_t>(std::max<int64_t>(t, kMlaMinChunk), INT32_MAX);
}

// Upper bound on the number of pieces, or -1 if it overflows.
inline int64_t mla_max_pieces(int32_t batch, int32_t max_seq_len, int32_t requested) {
  const int64_t S = std::max<int32_t>(max_seq_len, 1);
  const int64_t n = requested > 0 ? (int64_t)batch * ((S + requested - 1) / requested)
                                  : std::max<int64_t>(kCUs, batch);
  return n > (int64_t)INT32_MAX / 8 ? -1 : n;
}

// Splits of a sequence of max_seq_len tokens at `split` tokens each (at least one).
inline int32_t n_splits(int32_t max_seq_len, int32_t split) {
  if (max_seq_len <= split) return 1;
  return (int32_t)(((int64_t)max_seq_len + split - 1) / split);
}

}  // namespace plan
}  // namespace kvattn
