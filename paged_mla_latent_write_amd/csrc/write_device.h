// One token of mla_write_kv, written by one wavefront (lane = its lane index):
// the bodies of the write kernels (write_kv.hip), also run by the extra
// workgroups of the absorb launch when a decode call writes its new tokens
// (mla_decode_write).
//
// Cites "feat(serving): DeepSeek-V2/V3 paged-attention shim (MLA)", Root causes
// item 2 and Changes (KV written for decode tokens as well as prefill tokens),
// and "[unified-memory] Let Kimi-Linear use the paged MLA attention backends",
// Cuda-graph safety (slot < 0 is a pad row and writes nothing).  The fp8 layout
// follows "[Models] Support MLA_SWA functionality", Modifications (uint8 MLA
// cache); scale = amax / 448 is this library's reading.
#pragma once

#include "device_utils.h"
#include "mla_internal.h"

namespace mla {

// bf16 cache: a bit copy of [c_kv | k_pe] (16-byte pieces when `vec`).
__device__ __forceinline__ void write_token_bf16(uint16_t* __restrict__ cache, int64_t num_slots, int32_t R,
                                                 int32_t Dr, const uint16_t* __restrict__ c_kv, int64_t c_stride,
                                                 const uint16_t* __restrict__ k_pe, int64_t k_stride,
                                                 const int64_t* __restrict__ slots, int64_t i, bool vec,
                                                 int lane) {
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

// The eight bf16 values of a 16-byte piece, as floats.
__device__ __forceinline__ void unpack_bf16x8(const uint4& x, float (&f)[8]) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f[2 * k] = __uint_as_float(w[k] << 16);
    f[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
  }
}

// Row chunks of the 16-byte layout: lane l holds the row's 8-element chunks
// l and l + 64 (chunk c < R / 8 of the latent, else of the rope part), so a
// load moves 16 bytes per lane.  The chunks of one token, as floats (zeros
// for a lane's missing chunk).
__device__ __forceinline__ void load_row_chunks(const uint16_t* __restrict__ src_c,
                                                const uint16_t* __restrict__ src_r, int rc, int nc, int lane,
                                                float (&v)[2][8]) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int c = lane + 64 * q;
    uint4 x = make_uint4(0u, 0u, 0u, 0u);
    if (c < rc) x = reinterpret_cast<const uint4*>(src_c)[c];
    else if (c < nc) x = reinterpret_cast<const uint4*>(src_r)[c - rc];
    unpack_bf16x8(x, v[q]);
  }
}

// The E4M3 row of one token from its chunks (the rule of write_token_fp8
// below: the same amax, scale and codes), eight codes per 8-byte store.
__device__ __forceinline__ void store_fp8_chunks(uint8_t* __restrict__ dst_row, float* __restrict__ scale_out,
                                                 int64_t s, int nc, const float (&v)[2][8], int lane) {
  float amax = 0.f;
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[q][e]));
  amax = wave_max(amax);
  const float scale = amax == 0.f ? 1.0f : amax / 448.0f;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int c = lane + 64 * q;
    if (c < nc) {
      uint32_t lo = 0u, hi = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo |= f32_to_e4m3_satfinite(v[q][e] / scale) << (8 * e);
        hi |= f32_to_e4m3_satfinite(v[q][4 + e] / scale) << (8 * e);
      }
      reinterpret_cast<uint2*>(dst_row)[c] = make_uint2(lo, hi);
    }
  }
  if (lane == 0) scale_out[s] = scale;
}

// fp8 cache: amax over the token's R + Dr values, scale = amax / 448 as a
// correctly rounded fp32 quotient (1 when amax is 0), code = E4M3
// round-to-nearest-even of x / scale (also a correctly rounded fp32
// quotient), saturating.  hipcc's fp32 division is IEEE correctly rounded
// unless fast-math options are given, and the build gives none.  `vec`: the
// 16-byte chunk layout (R and Dr multiples of 8, R + Dr <= 1024, rows 16-byte
// aligned); else element j of the row in lane j % 64.
__device__ __forceinline__ void write_token_fp8(uint8_t* __restrict__ cache, float* __restrict__ scale_out,
                                                int64_t num_slots, int32_t R, int32_t Dr,
                                                const uint16_t* __restrict__ c_kv, int64_t c_stride,
                                                const uint16_t* __restrict__ k_pe, int64_t k_stride,
                                                const int64_t* __restrict__ slots, int64_t i, bool vec,
                                                int lane) {
  const int64_t s = slots[i];
  if (s < 0 || s >= num_slots) return;
  const int D = R + Dr;
  const uint16_t* src_c = c_kv + i * c_stride;
  const uint16_t* src_r = k_pe + i * k_stride;
  if (vec) {
    float v[2][8];
    load_row_chunks(src_c, src_r, R >> 3, D >> 3, lane, v);
    store_fp8_chunks(cache + s * D, scale_out, s, D >> 3, v, lane);
    return;
  }
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

// Token i of a TokenWrite (i < w.T).
__device__ __forceinline__ void write_token(const TokenWrite& w, int64_t i, int lane) {
  if (w.dtype == kKvBf16)
    write_token_bf16(static_cast<uint16_t*>(w.cache), w.num_slots, w.R, w.Dr, w.c_kv, w.c_stride, w.k_pe,
                     w.k_stride, w.slots, i, w.vec != 0, lane);
  else
    write_token_fp8(static_cast<uint8_t*>(w.cache), w.scale, w.num_slots, w.R, w.Dr, w.c_kv, w.c_stride,
                    w.k_pe, w.k_stride, w.slots, i, w.vec != 0, lane);
}

}  // namespace mla
