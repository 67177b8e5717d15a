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
#include "write_device.h"

namespace mla {
namespace {

constexpr int kWavesPerBlock = 4;

__global__ __launch_bounds__(256) void write_kv_kernel(TokenWrite w) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
  if (i < w.T) write_token(w, i, threadIdx.x & 63);
}

// The write with the latent's RMSNorm and the rope part's rotation folded in
// ("Support dsv4 model", Model Architecture and Inference: fused
// normalization/RoPE and packed KV writers; "[Attention] MLA with chunked
// prefill", Future work: the cache holds kv_c_normed).  One wavefront per
// token, element j of the row in lane j % 64, slot j / 64 of the lane's
// registers:
//   latent  y = x * (1 / sqrt(sum(x^2) / R + eps)) * w    (fp32, wave-wide sum)
//   rope    (a, b) -> (a cos - b sin, b cos + a sin), the pair's partner read
//           from the input row, angle i of the token's position in the table
// Each result is rounded to bf16 (nearest even), then written exactly as
// write_kv writes a bf16 row: a bit copy, or the per-token E4M3 quantisation.

// The same token in the 16-byte chunk layout (lane l: the row's 8-element
// chunks l and l + 64, chunk c < R / 8 of the latent, else of the rope part;
// R and Dr multiples of 8, Dr of 16 for half-split pairs, R + Dr <= 1024,
// rows, weight and table 16-byte aligned): one 16-byte load per chunk, its
// norm weights in one more, an interleaved pair inside one chunk (a
// half-split pair's partner chunk is loaded whole), and one 16- (bf16) or
// 8-byte (E4M3) store, where the lane-strided form moves 2 bytes (1 for a
// code) per lane and access.  The arithmetic is the lane-strided form's; only
// the order of the sum of squares differs.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Eight values rounded to bf16, nearest even, and back to fp32: the packed
// hardware convert, two values per instruction (measured equal to
// f32_to_bf16 on every non-NaN input tried, subnormals, ties and overflow
// included); a group holding a NaN takes f32_to_bf16 itself, so a NaN becomes
// 0x7FC0 as in the lane-strided form.
__device__ __forceinline__ void round_bf16x8(float (&v)[8]) {
  bool nan = false;
#pragma unroll
  for (int e = 0; e < 8; ++e) nan |= v[e] != v[e];
  if (nan) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = bf16_to_f32(f32_to_bf16(v[e]));
    return;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const f32x2_t p = {v[2 * k], v[2 * k + 1]};
    const uint32_t u = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2_t));
    v[2 * k] = __uint_as_float(u << 16);
    v[2 * k + 1] = __uint_as_float(u & 0xFFFF0000u);
  }
}

template <bool kFp8>
__device__ __forceinline__ void fused_token_chunks(void* __restrict__ cache, float* __restrict__ scale_out,
                                                   int64_t s, int32_t R, int32_t Dr,
                                                   const uint16_t* __restrict__ src_c,
                                                   const uint16_t* __restrict__ src_r, const KvTransform& tf,
                                                   int64_t i, int lane) {
  const int rc = R >> 3, nc = (R + Dr) >> 3;
  float v[2][8];
  load_row_chunks(src_c, src_r, rc, nc, lane, v);
  if (tf.norm_weight != nullptr) {
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < 2; ++q)
      if (lane + 64 * q < rc)
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(v[q][e], v[q][e], ss);
    const float r = 1.0f / sqrtf(wave_sum(ss) / static_cast<float>(R) + tf.eps);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int c = lane + 64 * q;
      if (c < rc) {
        float wf[8];
        unpack_bf16x8(reinterpret_cast<const uint4*>(tf.norm_weight)[c], wf);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[q][e] = v[q][e] * r * wf[e];
        round_bf16x8(v[q]);
      }
    }
  }
  if (tf.cos_sin != nullptr) {
    const int64_t pos = min(max(tf.positions[i], int64_t{0}), static_cast<int64_t>(tf.max_position - 1));
    const float* cs = tf.cos_sin + pos * Dr;
    const int h = Dr >> 1;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int c = lane + 64 * q;
      if (c >= rc && c < nc) {
        const int j0 = 8 * (c - rc);  // first rope element of the chunk
        float y[8];
        if (tf.interleaved) {
          // pairs (j0 + 2p, j0 + 2p + 1), angle j0 / 2 + p
          const float4 co = *reinterpret_cast<const float4*>(cs + j0 / 2);
          const float4 si = *reinterpret_cast<const float4*>(cs + h + j0 / 2);
          const float cf[4] = {co.x, co.y, co.z, co.w}, sf[4] = {si.x, si.y, si.z, si.w};
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const float a = v[q][2 * p], b = v[q][2 * p + 1];
            y[2 * p] = a * cf[p] - b * sf[p];
            y[2 * p + 1] = b * cf[p] + a * sf[p];
          }
        } else {
          // pairs (u, u + h): the chunk lies wholly in one half (h % 8 == 0)
          const bool first = j0 < h;
          const int f0 = first ? j0 : j0 - h;
          float xp[8];
          unpack_bf16x8(reinterpret_cast<const uint4*>(src_r)[(first ? j0 + h : j0 - h) >> 3], xp);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float cf = cs[f0 + e], sf = cs[h + f0 + e];
            y[e] = first ? v[q][e] * cf - xp[e] * sf : v[q][e] * cf + xp[e] * sf;
          }
        }
        round_bf16x8(y);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[q][e] = y[e];
      }
    }
  }
  const int D = R + Dr;
  if constexpr (!kFp8) {
    uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(cache) + s * D);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int c = lane + 64 * q;
      if (c < nc) {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          w[k] = (__float_as_uint(v[q][2 * k]) >> 16) | (__float_as_uint(v[q][2 * k + 1]) & 0xFFFF0000u);
        dst[c] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  } else {
    store_fp8_chunks(static_cast<uint8_t*>(cache) + s * D, scale_out, s, nc, v, lane);
  }
}

template <bool kFp8>
__global__ __launch_bounds__(256) void write_kv_fused_kernel(
    void* __restrict__ cache, float* __restrict__ scale_out, int64_t num_slots, int32_t R,
    int32_t Dr, const uint16_t* __restrict__ c_kv, int64_t c_stride,
    const uint16_t* __restrict__ k_pe, int64_t k_stride, const int64_t* __restrict__ slots,
    int32_t T, KvTransform tf, int32_t vec) {
  const int lane = threadIdx.x & 63;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
  if (i >= T) return;
  const int64_t s = slots[i];
  if (s < 0 || s >= num_slots) return;
  const int D = R + Dr;
  const uint16_t* src_c = c_kv + i * c_stride;
  const uint16_t* src_r = k_pe + i * k_stride;
  if (vec) {
    fused_token_chunks<kFp8>(cache, scale_out, s, R, Dr, src_c, src_r, tf, i, lane);
    return;
  }
  constexpr int kMaxPerLane = 16;  // D <= 1024
  float v[kMaxPerLane];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxPerLane; ++k) {
    const int j = lane + 64 * k;
    float x = 0.f;
    if (j < R) {
      x = bf16_to_f32(src_c[j]);
      ss = fmaf(x, x, ss);
    } else if (j < D) {
      x = bf16_to_f32(src_r[j - R]);
    }
    v[k] = x;
  }
  if (tf.norm_weight != nullptr) {
    const float r = 1.0f / sqrtf(wave_sum(ss) / static_cast<float>(R) + tf.eps);
#pragma unroll
    for (int k = 0; k < kMaxPerLane; ++k) {
      const int j = lane + 64 * k;
      if (j < R) v[k] = bf16_to_f32(f32_to_bf16(v[k] * r * bf16_to_f32(tf.norm_weight[j])));
    }
  }
  if (tf.cos_sin != nullptr) {
    const int64_t pos = min(max(tf.positions[i], int64_t{0}), static_cast<int64_t>(tf.max_position - 1));
    const float* cs = tf.cos_sin + pos * Dr;
    const int h = Dr >> 1;
#pragma unroll
    for (int k = 0; k < kMaxPerLane; ++k) {
      const int j = lane + 64 * k;
      if (j >= R && j < D) {
        const int jr = j - R;
        int fi, partner;
        bool first;
        if (tf.interleaved) {
          fi = jr >> 1;
          partner = jr ^ 1;
          first = (jr & 1) == 0;
        } else {
          first = jr < h;
          fi = first ? jr : jr - h;
          partner = first ? jr + h : jr - h;
        }
        const float c = cs[fi], sn = cs[h + fi];
        const float xp = bf16_to_f32(src_r[partner]);
        const float y = first ? v[k] * c - xp * sn : v[k] * c + xp * sn;
        v[k] = bf16_to_f32(f32_to_bf16(y));
      }
    }
  }
  if (!kFp8) {
    uint16_t* dst = static_cast<uint16_t*>(cache) + s * D;
#pragma unroll
    for (int k = 0; k < kMaxPerLane; ++k) {
      const int j = lane + 64 * k;
      if (j < D) dst[j] = static_cast<uint16_t>(__float_as_uint(v[k]) >> 16);
    }
    return;
  }
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxPerLane; ++k) amax = fmaxf(amax, fabsf(v[k]));
  amax = wave_max(amax);
  const float scale = amax == 0.f ? 1.0f : amax / 448.0f;
  uint8_t* dst = static_cast<uint8_t*>(cache) + s * D;
#pragma unroll
  for (int k = 0; k < kMaxPerLane; ++k) {
    const int j = lane + 64 * k;
    if (j < D) dst[j] = static_cast<uint8_t>(f32_to_e4m3_satfinite(v[k] / scale));
  }
  if (lane == 0) scale_out[s] = scale;
}

}  // namespace

hipError_t launch_write_kv_fused(void* cache_layer, float* scale_layer, int32_t dtype,
                                 int64_t num_slots, int32_t R, int32_t Dr, const uint16_t* c_kv,
                                 int64_t c_stride, const uint16_t* k_pe, int64_t k_stride,
                                 const int64_t* slots, int32_t num_tokens, const KvTransform& tf,
                                 hipStream_t s) {
  const dim3 grid((num_tokens + kWavesPerBlock - 1) / kWavesPerBlock);
  const dim3 block(64 * kWavesPerBlock);
  const auto aligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  // the 16-byte chunk layout when the shapes and pointers allow it
  const int32_t vec = (R % 8 == 0) && (Dr % 8 == 0) && R + Dr <= 1024 && (c_stride % 8 == 0) &&
                      (k_stride % 8 == 0) && aligned(cache_layer) && aligned(c_kv) && aligned(k_pe) &&
                      (tf.norm_weight == nullptr || aligned(tf.norm_weight)) &&
                      (tf.cos_sin == nullptr || (aligned(tf.cos_sin) && (tf.interleaved || Dr % 16 == 0)));
  if (dtype == kKvBf16) {
    hipLaunchKernelGGL(write_kv_fused_kernel<false>, grid, block, 0, s, cache_layer, nullptr,
                       num_slots, R, Dr, c_kv, c_stride, k_pe, k_stride, slots, num_tokens, tf, vec);
  } else {
    hipLaunchKernelGGL(write_kv_fused_kernel<true>, grid, block, 0, s, cache_layer, scale_layer,
                       num_slots, R, Dr, c_kv, c_stride, k_pe, k_stride, slots, num_tokens, tf, vec);
  }
  return hipGetLastError();
}

TokenWrite make_token_write(void* cache_layer, float* scale_layer, int32_t dtype, int64_t num_slots, int32_t R,
                            int32_t Dr, const uint16_t* c_kv, int64_t c_stride, const uint16_t* k_pe,
                            int64_t k_stride, const int64_t* slots, int32_t num_tokens) {
  const auto aligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  TokenWrite w;
  w.cache = cache_layer;
  w.scale = scale_layer;
  w.num_slots = num_slots;
  w.c_kv = c_kv;
  w.c_stride = c_stride;
  w.k_pe = k_pe;
  w.k_stride = k_stride;
  w.slots = slots;
  w.dtype = dtype;
  w.R = R;
  w.Dr = Dr;
  w.T = num_tokens;
  w.vec = (R % 8 == 0) && (Dr % 8 == 0) && (c_stride % 8 == 0) && (k_stride % 8 == 0) && aligned(cache_layer) &&
          aligned(c_kv) && aligned(k_pe) && (dtype == kKvBf16 || R + Dr <= 1024);
  return w;
}

hipError_t launch_write_kv(void* cache_layer, float* scale_layer, int32_t dtype, int64_t num_slots,
                           int32_t R, int32_t Dr, const uint16_t* c_kv, int64_t c_stride,
                           const uint16_t* k_pe, int64_t k_stride, const int64_t* slots,
                           int32_t num_tokens, hipStream_t s) {
  const TokenWrite w = make_token_write(cache_layer, scale_layer, dtype, num_slots, R, Dr, c_kv, c_stride, k_pe,
                                        k_stride, slots, num_tokens);
  const dim3 grid((num_tokens + kWavesPerBlock - 1) / kWavesPerBlock);
  hipLaunchKernelGGL(write_kv_kernel, grid, dim3(64 * kWavesPerBlock), 0, s, w);
  return hipGetLastError();
}

}  // namespace mla
