// mla_write_kv kernels: scatter new tokens' [c_kv | k_pe] rows into one layer
// of the paged latent cache through the slot mapping.
//
// Cites "feat(serving): DeepSeek-V2/V3 paged-attention shim (MLA)", Root causes
// item 2 and Changes (KV written for decode tokens as well as prefill tokens),
// and "[unified-memory] Let Kimi-Linear use the paged MLA attention backends",
// Cuda-graph safety (pad rows must not scatter into live pages: slot < 0 is
// skipped).  The fp8 layout (uint8 E4M3 codes plus a per-token fp32 scale)
// follows "[Models] Support MLA_SWA functionality", Modifications (uint8 MLA
// cache); the scale rule is this library's reading: scale = amax / 448.
//
// One wavefront per token.  The write is a tiny, latency-bound scatter; rows
// are copied with 16-byte accesses when the row pointers allow it.
#include "device_utils.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kWavesPerBlock = 4;

__global__ __launch_bounds__(256) void write_kv_bf16_kernel(
    uint16_t* __restrict__ cache, int64_t num_slots, int32_t R, int32_t Dr,
    const uint16_t* __restrict__ c_kv, int64_t c_stride, const uint16_t* __restrict__ k_pe,
    int64_t k_stride, const int64_t* __restrict__ slots, int32_t T, bool vec) {
  const int lane = threadIdx.x & 63;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
  if (i >= T) return;
  const int64_t s = slots[i];
  if (s < 0 || s >= num_slots) return;
  const int D = R + Dr;
  uint16_t* dst = cache + s * D;
  const uint16_t* src_c = c_kv + i * c_stride;
  const uint16_t* src_r = k_pe + i * k_stride;
  if (vec) {
    // R and Dr multiples of 8, all row starts 16-byte aligned
    for (int j = lane; j < R / 8; j += 64)
      reinterpret_cast<uint4*>(dst)[j] = reinterpret_cast<const uint4*>(src_c)[j];
    for (int j = lane; j < Dr / 8; j += 64)
      reinterpret_cast<uint4*>(dst + R)[j] = reinterpret_cast<const uint4*>(src_r)[j];
  } else {
    for (int j = lane; j < R; j += 64) dst[j] = src_c[j];
    for (int j = lane; j < Dr; j += 64) dst[R + j] = src_r[j];
  }
}

// Per-token fp8 quantisation: amax over the token's R + Dr values, scale =
// amax / 448 as a correctly rounded fp32 quotient, code = E4M3
// round-to-nearest-even of x / scale (also a correctly rounded fp32
// quotient), saturating.  hipcc's fp32 division is IEEE correctly rounded
// unless fast-math options are given, and the build gives none.
__global__ __launch_bounds__(256) void write_kv_fp8_kernel(
    uint8_t* __restrict__ cache, float* __restrict__ scale_out, int64_t num_slots, int32_t R,
    int32_t Dr, const uint16_t* __restrict__ c_kv, int64_t c_stride,
    const uint16_t* __restrict__ k_pe, int64_t k_stride, const int64_t* __restrict__ slots,
    int32_t T) {
  const int lane = threadIdx.x & 63;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
  if (i >= T) return;
  const int64_t s = slots[i];
  if (s < 0 || s >= num_slots) return;
  const int D = R + Dr;
  const uint16_t* src_c = c_kv + i * c_stride;
  const uint16_t* src_r = k_pe + i * k_stride;
  constexpr int kMaxPerLane = 16;  // D <= 1024
  float v[kMaxPerLane];
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxPerLane; ++k) {
    const int j = lane + 64 * k;
    float x = 0.f;
    if (j < R) x = bf16_to_f32(src_c[j]);
    else if (j < D) x = bf16_to_f32(src_r[j - R]);
    v[k] = x;
    amax = fmaxf(amax, fabsf(x));
  }
  amax = wave_max(amax);
  const float scale = amax == 0.f ? 1.0f : amax / 448.0f;
  uint8_t* dst = cache + s * D;
#pragma unroll
  for (int k = 0; k < kMaxPerLane; ++k) {
    const int j = lane + 64 * k;
    if (j < D) dst[j] = static_cast<uint8_t>(f32_to_e4m3_satfinite(v[k] / scale));
  }
  if (lane == 0) scale_out[s] = scale;
}

}  // namespace

hipError_t launch_write_kv(void* cache_layer, float* scale_layer, int32_t dtype, int64_t num_slots,
                           int32_t R, int32_t Dr, const uint16_t* c_kv, int64_t c_stride,
                           const uint16_t* k_pe, int64_t k_stride, const int64_t* slots,
                           int32_t num_tokens, hipStream_t s) {
  const dim3 grid((num_tokens + kWavesPerBlock - 1) / kWavesPerBlock);
  const dim3 block(64 * kWavesPerBlock);
  if (dtype == kKvBf16) {
    const auto aligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    const bool vec = (R % 8 == 0) && (Dr % 8 == 0) && (c_stride % 8 == 0) && (k_stride % 8 == 0) &&
                     aligned(cache_layer) && aligned(c_kv) && aligned(k_pe);
    hipLaunchKernelGGL(write_kv_bf16_kernel, grid, block, 0, s,
                       static_cast<uint16_t*>(cache_layer), num_slots, R, Dr, c_kv, c_stride, k_pe,
                       k_stride, slots, num_tokens, vec);
  } else {
    hipLaunchKernelGGL(write_kv_fp8_kernel, grid, block, 0, s, static_cast<uint8_t*>(cache_layer),
                       scale_layer, num_slots, R, Dr, c_kv, c_stride, k_pe, k_stride, slots,
                       num_tokens);
  }
  return hipGetLastError();
}

}  // namespace mla
