// Grouped-query decode attention over an FP8 (E4M3) KV cache: the split-K
// pipeline of gqa_split.h with 128-token tiles of 128-byte rows.
//
// What it computes: the grouped-query decode of the bf16 kernel ("MQA, GQA,
// and MLA", sections 2-4 and 8) over a cache whose K and V rows are E4M3
// codes with one K scale and one V scale per KV head, the granularity at
// which a GQA cache quantises ("Why GQA's KV Cache Savings Don't Fully
// Reduce TPOT", section "When the Serving Engineer Doesn't Get to Choose").
// The query and the output are bfloat16.
//
// Format specifics.  Every E4M3 value is exactly a bfloat16 (3 mantissa
// bits, exponents inside bf16's range), so codes are widened to bf16 in
// registers with the gfx950 conversion (v_cvt_scalef32_pk_bf16_fp8, scale 1)
// and both products run on the bf16 matrix cores; the per-head scales are
// applied in fp32: k_scale[j] multiplies the softmax scale, v_scale[j] the
// final normalisation.
//  * a row's eight 16-byte chunks are XOR-swizzled by row (swz below), and
//    the score reads take their chunks in an order under which neither LDS
//    read pattern stalls on bank conflicts;
//  * scores: the 128 dims are dealt to the four 16x16x32 products so that a
//    lane's K bytes for all four are two 16-byte chunks of its row (two LDS
//    reads, widened once and shared by the head blocks), with the query
//    fragments dealt the same way;
//  * values: 32 tokens per product; V^T comes straight from the row-major
//    tile through the 8-bit transposing read (ds_read_b64_tr_b8), whose
//    lanes address the eight token rows the probability operand holds.
#include <hip/hip_ext.h>

#include "gqa_split.h"

namespace kvattn {
namespace {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// Four E4M3 codes (one dword) -> bf16 quadruple, exact.
__device__ __forceinline__ void widen4(uint32_t w, bf16x2& lo, bf16x2& hi) {
  lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true);
}

// Eight codes (two dwords) -> one bf16x8 matrix-core operand.
__device__ __forceinline__ bf16x8 widen8(uint32_t w0, uint32_t w1) {
  bf16x2 a, b, c, d;
  widen4(w0, a, b);
  widen4(w1, c, d);
  return __builtin_shufflevector(__builtin_shufflevector(a, b, 0, 1, 2, 3),
                                 __builtin_shufflevector(c, d, 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
}

struct Fp8Format {
  static constexpr int kRowB = kHeadDim;  // 128 B per K or V row
  static constexpr int kTile = kGqaTileBytes / kRowB;  // 128 tokens

  // Chunk swizzle of a 128-byte row (8 chunks of 16 B).  Two rows share the
  // 64 LDS banks, so a read spreads over all banks when its rows give
  // distinct (row parity, physical chunk) pairs: 16 consecutive rows (score
  // reads) and the rows {0-3, 16-19} + 4k (transposing reads) both do with
  // this XOR.
  __device__ static __forceinline__ int swz(int row) { return ((row >> 1) & 7) ^ (((row >> 4) & 1) << 2); }
  template <int WH>
  static constexpr int unit_tokens() { return 32; }
  __device__ static __forceinline__ float k_scale(const DecodeArgs& a, int j) { return a.k_scale[j]; }
  __device__ static __forceinline__ float v_scale(const DecodeArgs& a, int j) { return a.v_scale[j]; }

  template <int HBW>
  struct Frags {
    bf16x8 qf[HBW][4];
    int koff[2][2];
    int voff[8];

    __device__ __forceinline__ void init(const uint16_t* qg, int hb0, int r, int lane) {
      const int n16 = lane & 15, grp = lane >> 4;
      // Q^T fragments.  Product kk of a score takes, in lane group grp, the
      // dims 64*(kk/2) + 16*grp + 8*(kk%2) .. +7 (the K fragment below takes
      // the same dims).
#pragma unroll
      for (int hbi = 0; hbi < HBW; ++hbi) {
        const int head = (hb0 + hbi) * 16 + n16;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          u32x4 v = {0u, 0u, 0u, 0u};
          if (head < r)
            v = *reinterpret_cast<const u32x4*>(qg + head * kHeadDim + 64 * (kk >> 1) + 16 * grp + 8 * (kk & 1));
          qf[hbi][kk] = __builtin_bit_cast(bf16x8, v);
        }
      }
      // Score reads: row 16*sb + n16, logical chunks grp and 4 + grp (dims
      // 16*grp .. +15 and 64 + 16*grp .. +15); the swizzle of rows 16..31
      // differs from 0..15.  The order 2*grp + c measured 4 bank-conflict
      // cycles per read: the four lane groups read the same 16 rows, and
      // chunks 2*grp + c put pairs of groups on the banks that the XOR with
      // swz() aligns across rows; chunks 4*c + grp do not.
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int row = 16 * sb + n16;
          koff[sb][c] = row * kRowB + 16 * ((4 * c + grp) ^ swz(row));
        }
      // Transposing V reads: lane n16 of group grp addresses token row
      // R(grp, n16/2), R(grp, v) = 4*grp + v for v < 4 and 16 + 4*grp + v-4
      // otherwise, bytes 16*db + 8*(n16%2) .. +7; it then holds column
      // 16*db + n16 of rows R(grp, 0..7), the token order of its probabilities.
      const int vv = n16 >> 1;
      const int vrow = (vv & 3) + 4 * grp + 16 * (vv >> 2);
#pragma unroll
      for (int db = 0; db < 8; ++db) voff[db] = kGqaTileBytes + vrow * kRowB + 16 * (db ^ swz(vrow)) + 8 * (n16 & 1);
    }

    // K fragments of the unit, widened once and shared by the head blocks.
    template <int kSub>
    __device__ __forceinline__ void scores(const unsigned char* stage, int u0, f32x4 (&s)[HBW][kSub]) {
      static_assert(kSub == 2, "32-token units");
      bf16x8 kf[2][4];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const u32x4 kraw = *reinterpret_cast<const u32x4*>(stage + u0 * kRowB + koff[sb][c]);
          kf[sb][2 * c] = widen8(kraw[0], kraw[1]);
          kf[sb][2 * c + 1] = widen8(kraw[2], kraw[3]);
        }
#pragma unroll
      for (int hbi = 0; hbi < HBW; ++hbi)
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          s[hbi][sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
            s[hbi][sb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[sb][kk], qf[hbi][kk], s[hbi][sb], 0, 0, 0);
        }
    }

    template <int kSub>
    __device__ __forceinline__ void values(const unsigned char* stage, int u0, const uint32_t* pk, f32x4 (&acc)[8]) {
      const auto* stage_lds = (const __attribute__((address_space(3))) unsigned char*)stage;
      const bf16x8 pb = __builtin_bit_cast(bf16x8, (u32x4){pk[0], pk[1], pk[2], pk[3]});
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const i32x2 vr = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(stage_lds + u0 * kRowB + voff[db]));
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen8((uint32_t)vr[0], (uint32_t)vr[1]), pb, acc[db], 0, 0, 0);
      }
    }
  };
};

template <int HBW, int WH>
__global__ __launch_bounds__(256, 2) void gqa_split_fp8(DecodeArgs a) {
  gqa_split_body<Fp8Format, GqaAttn16<Fp8Format, HBW, WH>>(a);
}

template <int HBW, int WH>
__global__ __launch_bounds__(256, 2) void gqa_split_fp8_persistent(DecodeArgs a) {
  gqa_persistent_body<Fp8Format, GqaAttn16<Fp8Format, HBW, WH>>(a);
}

// One workgroup per (sequence, KV head, split), or, with a work list, the
// resident workgroups of the persistent form.
template <int HBW, int WH>
hipError_t launch_shape(const DecodeArgs& a, hipStream_t stream, const LaunchEvents& ev) {
  const dim3 block(256);
  if (a.items != nullptr) {
    hipExtLaunchKernelGGL((gqa_split_fp8_persistent<HBW, WH>), dim3(kPersistentWorkgroups), block, 0, stream,
                          ev.start, ev.stop, 0, a);
  } else {
    const int64_t units = (int64_t)a.batch * a.num_kv_heads;
    const dim3 grid((unsigned)(8 * ((units + 7) / 8) * a.n_split));
    hipExtLaunchKernelGGL((gqa_split_fp8<HBW, WH>), grid, block, 0, stream, ev.start, ev.stop, 0, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gqa_fp8(const DecodeArgs& a, hipStream_t stream, const LaunchEvents& ev) {
  const int head_blocks = (a.group + 15) / 16;
  if (head_blocks == 1) return launch_shape<1, 4>(a, stream, ev);
  if (head_blocks == 2) return launch_shape<1, 2>(a, stream, ev);
  if (head_blocks <= 4) return launch_shape<1, 1>(a, stream, ev);
  if (head_blocks <= 8) return launch_shape<2, 1>(a, stream, ev);
  return hipErrorInvalidValue;
}

}  // namespace kvattn
