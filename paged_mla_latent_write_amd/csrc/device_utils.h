// Small device helpers: bf16 / E4M3 conversions and wave reductions (gfx950,
// wave64).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// OCP E4M3 code -> float (bias 7, no infinities, S.1111.111 is NaN).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t sign = (c & 0x80u) << 24;
  const uint32_t e = (c >> 3) & 0xFu;
  const uint32_t m = c & 0x7u;
  if (e == 0) {
    // subnormal: m * 2^-9, exact in fp32
    return __uint_as_float(__float_as_uint(static_cast<float>(m) * 0.001953125f) | sign);
  }
  if (e == 0xF && m == 0x7) return __uint_as_float(0x7FC00000u);
  return __uint_as_float(sign | ((e + 120u) << 23) | (m << 20));
}

// float -> OCP E4M3 code: round to nearest, ties to even; magnitudes >= 448
// (and infinities) saturate to +-448; the sign is kept; NaN -> 0x7F.
// Integer arithmetic only, so the result does not depend on the GPU's
// floating-point modes.
__device__ __forceinline__ uint32_t f32_to_e4m3_satfinite(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0x7Fu;
  if (a >= 0x43E00000u) return sign | 0x7Eu;  // >= 448
  if (a >= 0x3C800000u) {                     // >= 2^-6: normal E4M3
    const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
    return sign | (r - ((127u - 7u) << 3));
  }
  // below 2^-6: E4M3 subnormal k * 2^-9 with k = round_half_even(|x| * 2^9)
  const uint32_t e = a >> 23;
  if (e == 0) return sign;  // fp32 subnormal: far below 2^-10
  const uint32_t M = (a & 0x7FFFFFu) | 0x800000u;  // |x| = M * 2^(e - 150)
  const uint32_t s = 141u - e;                     // |x| * 2^9 = M >> s (s >= 21)
  if (s > 24u) return sign;
  uint32_t q = M >> s;
  const uint32_t rem = M & ((1u << s) - 1u);
  const uint32_t half = 1u << (s - 1u);
  q += (rem > half || (rem == half && (q & 1u))) ? 1u : 0u;
  return sign | q;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace mla
