// mla_decode_noalloc: mla_decode with its workspace taken from a device array
// the library owns, for callers that cannot allocate device memory (code under
// graph capture, tight serving loops, harnesses that forbid allocation).
//
// The array `scratch` is a file-scope __device__ array: every GPU the library
// runs on holds its own copy, at its own address, until the process ends.  In
// host code the array's name is only a host-side stand-in, so its device
// address is looked up once per device with hipGetSymbolAddress (on the first
// call made with that device current) and kept; kernels receive that address
// as their workspace pointer, exactly as they receive a caller's workspace.
//
// The array keeps whatever the previous call left in it.  No kernel of the
// decode path reads workspace memory it has not written in the same call, so
// nothing is cleared between calls.  Calls that overlap on one GPU share the
// array and race.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/mla.h"

namespace {

constexpr size_t kScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "the scratch size keeps 256-byte alignment");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of the current device's copy of `scratch` (looked up once per
// device, under a lock, then read lock-free).
mla_status current_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_UNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
      void* q = nullptr;
      if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr)
        return MLA_ERR_HIP;
      g_scratch_ptr[dev].store(q, std::memory_order_release);
      p = q;
    }
  }
  *out = p;
  return MLA_OK;
}

}  // namespace

extern "C" mla_status mla_decode_noalloc(const mla_cache* cache, int32_t layer_idx,
                                         const mla_attn* attn, const void* q_nope,
                                         int64_t q_nope_stride_b, int64_t q_nope_stride_h,
                                         const void* q_pe, int64_t q_pe_stride_b,
                                         int64_t q_pe_stride_h, const int32_t* block_tables,
                                         int32_t max_blocks_per_seq, const int32_t* context_lens,
                                         int32_t batch, void* out, float* lse_or_null,
                                         void* stream) {
  const size_t need = mla_decode_workspace_size(cache, attn, batch, max_blocks_per_seq);
  if (need == 0) {
    // invalid arguments (or no device): mla_decode reports which, and with no
    // workspace it enqueues nothing
    return mla_decode(cache, layer_idx, attn, q_nope, q_nope_stride_b, q_nope_stride_h, q_pe,
                      q_pe_stride_b, q_pe_stride_h, block_tables, max_blocks_per_seq, context_lens,
                      batch, out, lse_or_null, nullptr, 0, stream);
  }
  if (need > kScratchBytes) return MLA_ERR_WORKSPACE;
  void* ws = nullptr;
  const mla_status st = current_scratch(&ws);
  if (st != MLA_OK) return st;
  return mla_decode(cache, layer_idx, attn, q_nope, q_nope_stride_b, q_nope_stride_h, q_pe,
                    q_pe_stride_b, q_pe_stride_h, block_tables, max_blocks_per_seq, context_lens,
                    batch, out, lse_or_null, ws, kScratchBytes, stream);
}
