// Grouped-query decode attention over a bf16 cache: the split-K pipeline of
// gqa_split.h with 64-token tiles of 256-byte rows.
//
// Format specifics:
//  * each row's sixteen 16-byte chunks are XOR-swizzled by row (swz below);
//    the score reads visit the 128 dims in the order kchunk() below, so that
//    neither LDS read pattern stalls on bank conflicts (SQ_LDS_BANK_CONFLICT
//    counts none for this kernel);
//  * scores: K fragments straight from LDS into v_mfma_f32_16x16x32_bf16
//    against Q^T fragments held in registers;
//  * values: V^T through the 16-bit transposing read (ds_read_b64_tr_b16);
//    waves that own 32 tokens of a tile use 16x16x32 products (two
//    transposing reads per operand), waves that own 16 use 16x16x16.
#include <hip/hip_ext.h>

#include "gqa_split.h"

namespace kvattn {
namespace {

// Logical 16-byte chunk (8 dims) that lane group grp reads at score step kk.
// The reduction over the 128 dims may visit them in any order shared by the
// K and Q^T operands.  Giving the four lane groups chunks that differ in bits
// 1-2 (and the steps bits 0 and 3) keeps lanes l and l+16, which read the
// same row, off the banks that the XOR with swz() aligns across rows r and
// r+8; the order 4*kk + grp measured 4 bank-conflict cycles per score read.
__device__ __forceinline__ int kchunk(int kk, int grp) { return (kk & 1) | (grp << 1) | ((kk >> 1) << 3); }

struct Bf16Format {
  static constexpr int kRowB = kHeadDim * 2;  // 256 B per K or V row
  static constexpr int kTile = kGqaTileBytes / kRowB;  // 64 tokens

  // Chunk swizzle of a 256-byte row: XOR of the 4-bit chunk index.  Rows r
  // and r+16 share it; 16 consecutive rows get 16 distinct values and any 8
  // consecutive rows 8 distinct pairs, which is what the two read patterns need.
  __device__ static __forceinline__ int swz(int row) { return ((row & 7) << 1) | ((row >> 3) & 1); }
  template <int WH>
  static constexpr int unit_tokens() { return WH == 4 ? 16 : 32; }
  __device__ static __forceinline__ float k_scale(const DecodeArgs&, int) { return 1.f; }
  __device__ static __forceinline__ float v_scale(const DecodeArgs&, int) { return 1.f; }

  template <int HBW>
  struct Frags {
    bf16x8 qf[HBW][4];
    int koff[4];  // K reads: row n16 of a 16-token subtile, chunk kchunk(kk, grp)
    int voff[8];  // V^T reads: rows 4*grp + n16/4 (+16 per subtile), 8-byte piece n16%4 of column block db

    __device__ __forceinline__ void init(const uint16_t* qg, int hb0, int r, int lane) {
      const int n16 = lane & 15, grp = lane >> 4;
      // Q^T fragments: lane l holds head (block*16 + l%16), dims 8*kchunk(kk, l/16) .. +7.
#pragma unroll
      for (int hbi = 0; hbi < HBW; ++hbi) {
        const int head = (hb0 + hbi) * 16 + n16;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          u32x4 v = {0u, 0u, 0u, 0u};
          if (head < r) v = *reinterpret_cast<const u32x4*>(qg + head * kHeadDim + 8 * kchunk(kk, grp));
          qf[hbi][kk] = __builtin_bit_cast(bf16x8, v);
        }
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) koff[kk] = n16 * kRowB + 16 * (kchunk(kk, grp) ^ swz(n16));
      const int vrow = 4 * grp + (n16 >> 2);
#pragma unroll
      for (int db = 0; db < 8; ++db)
        voff[db] = kGqaTileBytes + vrow * kRowB + 16 * ((2 * db + ((n16 & 3) >> 1)) ^ swz(vrow)) + 8 * (n16 & 1);
    }

    // s[hbi][sb] = K(tokens u0 + 16*sb ..) Q^T(head block hbi); each K fragment feeds every head block.
    template <int kSub>
    __device__ __forceinline__ void scores(const unsigned char* stage, int u0, f32x4 (&s)[HBW][kSub]) {
#pragma unroll
      for (int hbi = 0; hbi < HBW; ++hbi)
#pragma unroll
        for (int sb = 0; sb < kSub; ++sb) s[hbi][sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int sb = 0; sb < kSub; ++sb)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const u32x4 kraw = *reinterpret_cast<const u32x4*>(stage + (u0 + 16 * sb) * kRowB + koff[kk]);
#pragma unroll
          for (int hbi = 0; hbi < HBW; ++hbi)
            s[hbi][sb] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kraw), qf[hbi][kk], s[hbi][sb], 0, 0, 0);
        }
    }

    // acc[db] += V^T(column block db, tokens of the unit) P^T, P packed as bf16 pairs in token order.
    template <int kSub>
    __device__ __forceinline__ void values(const unsigned char* stage, int u0, const uint32_t* pk, f32x4 (&acc)[8]) {
      const auto* stage_lds = (const __attribute__((address_space(3))) unsigned char*)stage;
      const int vbase_off = u0 * kRowB;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(stage_lds + vbase_off + voff[db]));
        if constexpr (kSub == 1) {
          const i16x4 pb = __builtin_bit_cast(i16x4, (uint2){pk[0], pk[1]});
          acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v0, pb, acc[db], 0, 0, 0);
        } else {
          // second 16 tokens of the unit: slots 4..7 of the 32-deep operand
          const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(stage_lds + vbase_off + 16 * kRowB + voff[db]));
          const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
          const bf16x8 pb = __builtin_bit_cast(bf16x8, (u32x4){pk[0], pk[1], pk[2], pk[3]});
          acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, acc[db], 0, 0, 0);
        }
      }
    }
  };
};

template <int HBW, int WH>
__global__ __launch_bounds__(256, 2) void gqa_split_bf16(DecodeArgs a) {
  gqa_split_body<Bf16Format, GqaAttn16<Bf16Format, HBW, WH>>(a);
}

template <int HBW, int WH>
__global__ __launch_bounds__(256, 2) void gqa_split_bf16_persistent(DecodeArgs a) {
  gqa_persistent_body<Bf16Format, GqaAttn16<Bf16Format, HBW, WH>>(a);
}

// One workgroup per (sequence, KV head, split), or, with a work list, the
// resident workgroups of the persistent form.
template <int HBW, int WH>
hipError_t launch_shape(const DecodeArgs& a, hipStream_t stream, const LaunchEvents& ev) {
  const dim3 block(256);
  if (a.items != nullptr) {
    hipExtLaunchKernelGGL((gqa_split_bf16_persistent<HBW, WH>), dim3(kPersistentWorkgroups), block, 0, stream,
                          ev.start, ev.stop, 0, a);
  } else {
    const int64_t units = (int64_t)a.batch * a.num_kv_heads;
    const dim3 grid((unsigned)(8 * ((units + 7) / 8) * a.n_split));
    hipExtLaunchKernelGGL((gqa_split_bf16<HBW, WH>), grid, block, 0, stream, ev.start, ev.stop, 0, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gqa_bf16(const DecodeArgs& a, hipStream_t stream, const LaunchEvents& ev) {
  const int head_blocks = (a.group + 15) / 16;
  if (head_blocks == 1) return launch_shape<1, 4>(a, stream, ev);
  if (head_blocks == 2) return launch_shape<1, 2>(a, stream, ev);
  if (head_blocks <= 4) return launch_shape<1, 1>(a, stream, ev);
  if (head_blocks <= 8) return launch_shape<2, 1>(a, stream, ev);
  return hipErrorInvalidValue;
}

}  // namespace kvattn
