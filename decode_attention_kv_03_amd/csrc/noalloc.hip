// kvattn_gqa_decode_noalloc: grouped-query decode whose split-K partials go
// to a fixed scratch array in device memory that the library owns, so the
// call needs no workspace from its caller and allocates nothing.
//
// The array is a file-scope __device__ variable: each GPU the library runs on
// holds its own copy, at its own address, from the first use until the
// process ends.  In host code the variable's name is only a stand-in for the
// symbol, not a device address, so the address is taken once per device with
// hipGetSymbolAddress (with that device current) and kept; kernels receive
// that address, exactly as they receive a caller's workspace.  The partials
// need no initialisation (every split that the merge reads writes its rows
// first), so no memset is issued either.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/kvattn.h"
#include "kvattn_internal.h"

namespace kvattn {
namespace {

static_assert(KVATTN_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");

__device__ __align__(256) unsigned char scratch[KVATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];  // device address of `scratch`, per device (null: not looked up yet)
std::mutex g_lookup;

// Device address of the current device's scratch array, looked up on its first use.
kvattn_status current_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return report_hip(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return report(KVATTN_ERR_UNSUPPORTED, "device %lld is beyond the %lld supported",
                                                   dev, kMaxDevices);
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_lookup);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return report_hip(e, "hipGetSymbolAddress(scratch)");
      if (p == nullptr) return report(KVATTN_ERR_HIP, "hipGetSymbolAddress(scratch) returned no address");
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return KVATTN_OK;
}

}  // namespace
}  // namespace kvattn

extern "C" kvattn_status kvattn_gqa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                                   const int32_t* block_table, const int32_t* seq_lens, void* out,
                                                   float* lse, int32_t batch, int32_t num_q_heads,
                                                   int32_t num_kv_heads, int32_t head_dim, int64_t cache_len,
                                                   int32_t block_size, int32_t max_blocks_per_seq,
                                                   int32_t max_seq_len, float scale, int32_t window,
                                                   kvattn_dtype dtype, int32_t split_tokens, void* stream) {
  return kvattn::gqa_decode_with(q, k_cache, v_cache, block_table, seq_lens, out, lse, batch, num_q_heads,
                                 num_kv_heads, head_dim, cache_len, block_size, max_blocks_per_seq, max_seq_len,
                                 scale, window, dtype, split_tokens,
                                 kvattn::Workspace{nullptr, KVATTN_NOALLOC_SCRATCH_BYTES, kvattn::current_scratch},
                                 stream);
}
