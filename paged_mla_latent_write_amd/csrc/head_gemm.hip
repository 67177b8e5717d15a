// Per-head projections of absorbed MLA on matrix cores (gfx950):
//   absorb      q_lat[i,h,:] = W_UK[h]^T q_nope[i,h,:]      (K = qk_nope, N = kv_lora_rank)
//   up-project  out[i,h,:]   = W_UV[h] (o_lat[i,h,:] / l)   (K = kv_lora_rank, N = v_head)
// The up-projection kv_b_proj is named by "[Attention] MLA with chunked
// prefill", Future work; reading it as k_nope = W_UK[h] c and v = W_UV[h] c is
// this library's, as is folding W_UK into the query and W_UV into the output.
//
// Both are batched (one GEMM per head) with M = query items.  A workgroup of
// four waves owns one head and 32 * MT items (absorb: and 128 of the R output
// columns); each wave computes 32 output columns with v_mfma_f32_32x32x16_bf16.
//  * absorb: the W_UK[h] column block is staged in LDS (rows padded to 288 B)
//    and read as the B operand with ds_read_b64_tr_b16 (W_UK rows run along
//    the output dimension, the MFMA wants runs along K).  bf16 in, fp32
//    accumulate, bf16 out.
//  * up-project: W_UV rows already run along K, so B fragments come straight
//    from global memory.  o_lat is fp32; each A fragment is split into a bf16
//    high part and a bf16 remainder and both are multiplied (two MFMAs), which
//    keeps the product accurate to about 2^-16 relative.
#include "device_utils.h"
#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(T) __attribute__((address_space(3))) T*

constexpr int kAbsCols = 128;              // W_UK columns staged per chunk
constexpr int kAbsPitch = kAbsCols * 2 + 32;  // bytes per staged row (padded)
constexpr int kAbsMaxDn = 128;

template <int MT>
__global__ __launch_bounds__(256) void absorb_mfma_kernel(const uint16_t* __restrict__ q_nope,
                                                          int64_t st, int64_t sh,
                                                          const uint16_t* __restrict__ w_uk,
                                                          int32_t Nq, int32_t H, int32_t Dn,
                                                          int32_t R, uint16_t* __restrict__ q_lat) {
  __shared__ __attribute__((aligned(16))) char wt[kAbsMaxDn * kAbsPitch];
  const int c0 = blockIdx.x * kAbsCols;  // this workgroup's 128 output columns
  const int h = blockIdx.y;
  const int m0 = blockIdx.z * 32 * MT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 5, n32 = lane & 31;
  const int ksteps = Dn / 16;

  // A fragments: q_nope rows of this wave's M tiles (all waves hold the same)
  i16x8 af[MT][kAbsMaxDn / 16];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int item = m0 + 32 * mt + n32;
#pragma unroll
    for (int k = 0; k < kAbsMaxDn / 16; ++k) {
      i16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
      if (k < ksteps && item < Nq)
        v = *reinterpret_cast<const i16x8*>(q_nope + item * st + h * sh + 16 * k + 8 * g);
      af[mt][k] = v;
    }
  }

  // transposed-read lane offsets (see the attention kernel for the layout)
  const int q = lane >> 4, jj = lane & 15, rr = jj >> 2, c4 = jj & 3;
  const int tr_off = (8 * g + rr) * kAbsPitch + (32 * wave + 16 * (q & 1) + 4 * c4) * 2;
  const uint16_t* wh = w_uk + static_cast<int64_t>(h) * Dn * R;

  {
    // stage W_UK[h][0:Dn][c0 : c0 + 128]: all loads first (16 B per thread
    // per step), then the LDS stores
    constexpr int kStage = kAbsMaxDn * (kAbsCols / 8) / 256;
    i16x8 wv[kStage];
#pragma unroll
    for (int j = 0; j < kStage; ++j) {
      const int idx = threadIdx.x + 256 * j;
      const int d = idx / (kAbsCols / 8), c = idx % (kAbsCols / 8);
      if (d < Dn) wv[j] = *reinterpret_cast<const i16x8*>(wh + static_cast<int64_t>(d) * R + c0 + 8 * c);
    }
#pragma unroll
    for (int j = 0; j < kStage; ++j) {
      const int idx = threadIdx.x + 256 * j;
      const int d = idx / (kAbsCols / 8), c = idx % (kAbsCols / 8);
      if (d < Dn) *reinterpret_cast<i16x8*>(wt + d * kAbsPitch + c * 16) = wv[j];
    }
    __syncthreads();
    f32x16 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16{};
#pragma unroll
    for (int k = 0; k < kAbsMaxDn / 16; ++k) {
      if (k < ksteps) {
        const LDS_PTR(char) base = (LDS_PTR(char))(wt) + tr_off + 16 * k * kAbsPitch;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(i16x4))(base));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(i16x4))(base + 4 * kAbsPitch));
        const i16x8 b = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af[mt][k]),
                                                            __builtin_bit_cast(bf16x8, b), acc[mt],
                                                            0, 0, 0);
      }
    }
    const int col = c0 + 32 * wave + n32;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int item = m0 + 32 * mt + 8 * (i >> 2) + 4 * g + (i & 3);
        if (item < Nq) q_lat[(static_cast<int64_t>(item) * H + h) * R + col] = f32_to_bf16(acc[mt][i]);
      }
    }
  }
}

template <int MT>
__global__ __launch_bounds__(256) void up_project_mfma_kernel(const float* __restrict__ o_lat,
                                                              const float* __restrict__ o_scale,
                                                              const uint16_t* __restrict__ w_uv,
                                                              int32_t Nq, int32_t H, int32_t R,
                                                              int32_t Dv,
                                                              uint16_t* __restrict__ out) {
  const int h = blockIdx.y;
  const int m0 = blockIdx.x * 32 * MT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 5, n32 = lane & 31;
  const int v = 32 * wave + n32;  // output column of this lane's B fragment
  if (32 * wave >= Dv) return;
  const uint16_t* wrow = w_uv + (static_cast<int64_t>(h) * Dv + v) * R;
  const float* orow[MT];
  float sc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int item = m0 + 32 * mt + n32;
    const int it = item < Nq ? item : Nq - 1;
    orow[mt] = o_lat + (static_cast<int64_t>(it) * H + h) * R;
    sc[mt] = item < Nq ? o_scale[static_cast<int64_t>(it) * H + h] : 0.f;
  }
  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16{};
  // K in chunks of kU 16-wide steps: every load of a chunk is issued before
  // its first MFMA, so the loop waits for memory once per chunk, not per step
  constexpr int kU = 4;
  for (int k0 = 0; k0 < R; k0 += 16 * kU) {
    i16x8 b[kU];
    f32x4 x0[MT][kU], x1[MT][kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const bool in = k0 + 16 * u < R;
      const int k = in ? k0 + 16 * u : k0;
      b[u] = *reinterpret_cast<const i16x8*>(wrow + k + 8 * g);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        x0[mt][u] = *reinterpret_cast<const f32x4*>(orow[mt] + k + 8 * g);
        x1[mt][u] = *reinterpret_cast<const f32x4*>(orow[mt] + k + 8 * g + 4);
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (k0 + 16 * u >= R) break;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        bf16x8 hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = (e < 4 ? x0[mt][u][e] : x1[mt][u][e - 4]) * sc[mt];
          const __bf16 xh = static_cast<__bf16>(x);
          hi[e] = xh;
          lo[e] = static_cast<__bf16>(x - static_cast<float>(xh));
        }
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hi, __builtin_bit_cast(bf16x8, b[u]), acc[mt],
                                                          0, 0, 0);
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lo, __builtin_bit_cast(bf16x8, b[u]), acc[mt],
                                                          0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int item = m0 + 32 * mt + 8 * (i >> 2) + 4 * g + (i & 3);
      if (item < Nq) out[(static_cast<int64_t>(item) * H + h) * Dv + v] = f32_to_bf16(acc[mt][i]);
    }
  }
}

int pick_mt(int Nq) { return Nq <= 32 ? 1 : (Nq <= 64 ? 2 : 4); }

// The up-projection streams W_UV once per 32 * MT items; small batches take
// one 32-item tile per workgroup so that the grid still covers the chip.
int pick_mt_up(int Nq) { return Nq <= 128 ? 1 : (Nq <= 512 ? 2 : 4); }

}  // namespace

bool absorb_mfma_supported(int32_t Dn, int32_t R) {
  return Dn % 16 == 0 && Dn <= kAbsMaxDn && R % kAbsCols == 0;
}

bool up_project_mfma_supported(int32_t R, int32_t Dv) {
  return R % 16 == 0 && Dv % 32 == 0 && Dv <= 128;
}

hipError_t launch_absorb_mfma(const uint16_t* q_nope, int64_t st, int64_t sh, const uint16_t* w_uk,
                              int32_t num_items, int32_t H, int32_t Dn, int32_t R, uint16_t* q_lat,
                              hipStream_t s) {
  const int mt = pick_mt(num_items);
  const dim3 grid(R / kAbsCols, H, (num_items + 32 * mt - 1) / (32 * mt));
  switch (mt) {
    case 1: hipLaunchKernelGGL(absorb_mfma_kernel<1>, grid, dim3(256), 0, s, q_nope, st, sh, w_uk, num_items, H, Dn, R, q_lat); break;
    case 2: hipLaunchKernelGGL(absorb_mfma_kernel<2>, grid, dim3(256), 0, s, q_nope, st, sh, w_uk, num_items, H, Dn, R, q_lat); break;
    default: hipLaunchKernelGGL(absorb_mfma_kernel<4>, grid, dim3(256), 0, s, q_nope, st, sh, w_uk, num_items, H, Dn, R, q_lat); break;
  }
  return hipGetLastError();
}

hipError_t launch_up_project_mfma(const float* o_lat, const float* o_scale, const uint16_t* w_uv,
                                  int32_t num_items, int32_t H, int32_t R, int32_t Dv, uint16_t* out,
                                  hipStream_t s) {
  const int mt = pick_mt_up(num_items);
  const dim3 grid((num_items + 32 * mt - 1) / (32 * mt), H);
  switch (mt) {
    case 1: hipLaunchKernelGGL(up_project_mfma_kernel<1>, grid, dim3(256), 0, s, o_lat, o_scale, w_uv, num_items, H, R, Dv, out); break;
    case 2: hipLaunchKernelGGL(up_project_mfma_kernel<2>, grid, dim3(256), 0, s, o_lat, o_scale, w_uv, num_items, H, R, Dv, out); break;
    default: hipLaunchKernelGGL(up_project_mfma_kernel<4>, grid, dim3(256), 0, s, o_lat, o_scale, w_uv, num_items, H, R, Dv, out); break;
  }
  return hipGetLastError();
}

}  // namespace mla
