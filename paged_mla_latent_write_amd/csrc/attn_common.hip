// Kernels around the split-KV attention core:
//   plan_items        - per query item: request, visible key range, tile count,
//                       and the exclusive prefix sum of tile counts (the
//                       split plan; computed on the device from context_lens,
//                       so there is no host synchronisation)
//   combine_segments  - log-sum-exp merge of the partial results of items whose
//                       tiles were cut across workgroups
//   dense_combine     - the general LSE merge of [S][rows][dim] partials
//   absorb            - q_lat[i,h,:] = W_UK[h]^T q_nope[i,h,:]  (bf16 out)
//   up_project        - out[i,h,:] = W_UV[h] o_lat[i,h,:]        (bf16 out)
//
// Decode positions and context lengths follow "feat(serving): DeepSeek-V2/V3
// paged-attention shim (MLA)", Root causes items 2 and 4 (the newest token is
// written first and sits at position n - 1).  Prefill rows follow "[Attention]
// MLA with chunked prefill" (row i of an m-token chunk sits at n - m + i).  The
// window follows "[Models] Support MLA_SWA functionality", Motivation, with the
// boundary p - w < t <= p (the pages give none).  The weight-absorption
// reading of kv_b_proj (k_nope = W_UK c, v = W_UV c) is this library's.
#include <math.h>

#include "device_utils.h"
#include "mla_internal.h"
#include "plan_device.h"

namespace mla {
namespace {

constexpr int kPlanThreads = 1024;

__global__ __launch_bounds__(kPlanThreads) void plan_items_kernel(
    int mode, int32_t B, int32_t Nq, const int32_t* __restrict__ ctx,
    const int32_t* __restrict__ qsl, int32_t window, int32_t max_ctx, int32_t* __restrict__ item_b,
    int32_t* __restrict__ item_lo, int32_t* __restrict__ item_hi,
    int32_t* __restrict__ tile_start, int32_t G, int32_t* __restrict__ wg_tile,
    int32_t* __restrict__ wg_item, int32_t* __restrict__ item_wg) {
  __shared__ int32_t buf[kPlanThreads];
  __shared__ int32_t carry;
  __shared__ int32_t ts_lds[kPlanLds];
  __shared__ int32_t wt_lds[kPlanLds];
  plan_items_body<kPlanThreads>(buf, &carry, ts_lds, wt_lds, mode, B, Nq, ctx, qsl, window, max_ctx,
                                item_b, item_lo, item_hi, tile_start, G, wg_tile, wg_item, item_wg);
}
// One wave per (item, head).  Items whose tiles all fell to one workgroup were
// finished by the attention kernel; empty items get o = 0, lse = -inf; cut
// items are merged from the partial slots of the workgroups that cover them
// (slot 2g+1 for the first, which the item starts in, slot 2g after it), in
// one pass with a running maximum.  The merged row is written normalised (its
// o_scale set to 1).
__global__ __launch_bounds__(256) void combine_segments_kernel(AttnArgs a) {
  const int i = blockIdx.x;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int H = a.H, R = a.kv.R;
  if (h >= H) return;
  const int64_t row = static_cast<int64_t>(i) * H + h;
  float* dst = a.o_lat + row * R;
  const int g0 = a.item_wg[2 * i], g1 = a.item_wg[2 * i + 1];
  if (g0 < 0) {
    for (int r = lane; r < R; r += 64) dst[r] = 0.f;
    if (lane == 0) {
      a.lse[row] = -INFINITY;
      a.o_scale[row] = 1.f;
    }
    return;
  }
  if (g0 == g1) return;
  for (int r0 = lane * 8; r0 < R; r0 += 512) {
    float m = -INFINITY, tot = 0.f;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // segments in batches of kB: the batch's loads are issued together, then
    // merged against the running maximum
    constexpr int kB = 8;
    for (int gb = g0; gb <= g1; gb += kB) {
      float l[kB], sc[kB];
      float4 x0[kB], x1[kB];
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        const int g = gb + j;
        const bool live = g <= g1 && a.wg_tile[g] != a.wg_tile[g + 1];  // (no tiles: no slot)
        const int64_t slot = (g == g0) ? 2 * g + 1 : 2 * g;
        l[j] = live ? a.part_lse[slot * H + h] : -INFINITY;
        sc[j] = live ? a.part_scale[slot * H + h] : 0.f;
        if (live) {
          // 8 bf16 partial values (low half first in each word)
          const uint4 v = *reinterpret_cast<const uint4*>(a.part_o + (slot * H + h) * R + r0);
          x0[j] = make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                              __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u));
          x1[j] = make_float4(__uint_as_float(v.z << 16), __uint_as_float(v.z & 0xFFFF0000u),
                              __uint_as_float(v.w << 16), __uint_as_float(v.w & 0xFFFF0000u));
        } else {
          x0[j] = x1[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
      float mb = m;
#pragma unroll
      for (int j = 0; j < kB; ++j) mb = fmaxf(mb, l[j]);
      if (mb > m) {  // wave-uniform: rescale what was merged so far
        const float f = expf(m - mb);
        tot *= f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= f;
        m = mb;
      }
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        if (l[j] == -INFINITY) continue;
        const float e_l = expf(l[j] - m);
        tot += e_l;
        const float w = e_l * sc[j];
        acc[0] = fmaf(w, x0[j].x, acc[0]);
        acc[1] = fmaf(w, x0[j].y, acc[1]);
        acc[2] = fmaf(w, x0[j].z, acc[2]);
        acc[3] = fmaf(w, x0[j].w, acc[3]);
        acc[4] = fmaf(w, x1[j].x, acc[4]);
        acc[5] = fmaf(w, x1[j].y, acc[5]);
        acc[6] = fmaf(w, x1[j].z, acc[6]);
        acc[7] = fmaf(w, x1[j].w, acc[7]);
      }
    }
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
    float4* d4 = reinterpret_cast<float4*>(dst + r0);
    d4[0] = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    d4[1] = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
    if (lane == 0 && r0 == 0) {
      a.lse[row] = tot > 0.f ? m + logf(tot) : -INFINITY;
      a.o_scale[row] = 1.f;
    }
  }
}

__global__ __launch_bounds__(256) void dense_combine_kernel(const float* __restrict__ o_part,
                                                             const float* __restrict__ lse_part,
                                                             int32_t S, int32_t rows, int32_t dim,
                                                             float* __restrict__ o,
                                                             float* __restrict__ lse) {
  const int64_t row = blockIdx.x;
  float mx = -INFINITY;
  for (int s = 0; s < S; ++s) mx = fmaxf(mx, lse_part[static_cast<int64_t>(s) * rows + row]);
  float tot = 0.f;
  if (mx != -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const float l = lse_part[static_cast<int64_t>(s) * rows + row];
      tot += (l == -INFINITY) ? 0.f : expf(l - mx);
    }
  }
  for (int d = threadIdx.x; d < dim; d += blockDim.x) {
    float acc = 0.f;
    if (mx != -INFINITY) {
      for (int s = 0; s < S; ++s) {
        const float l = lse_part[static_cast<int64_t>(s) * rows + row];
        if (l == -INFINITY) continue;
        acc += expf(l - mx) * o_part[(static_cast<int64_t>(s) * rows + row) * dim + d];
      }
      acc /= tot;
    }
    o[row * dim + d] = acc;
  }
  if (threadIdx.x == 0) lse[row] = (mx == -INFINITY) ? -INFINITY : mx + logf(tot);
}

// q_lat[i,h,r] = sum_d q_nope[i,h,d] * W_UK[h,d,r]; fp32 accumulation, bf16 out.
// Block: one head, 16 items; thread t owns columns r = t + 256k.
constexpr int kGemmItems = 16;

__global__ __launch_bounds__(256) void absorb_kernel(const uint16_t* __restrict__ q_nope,
                                                      int64_t st, int64_t sh,
                                                      const uint16_t* __restrict__ w_uk,
                                                      int32_t Nq, int32_t H, int32_t Dn, int32_t R,
                                                      uint16_t* __restrict__ q_lat) {
  extern __shared__ float qs[];  // [kGemmItems][Dn]
  const int h = blockIdx.y;
  const int i0 = blockIdx.x * kGemmItems;
  const int ni = min(kGemmItems, Nq - i0);
  for (int idx = threadIdx.x; idx < kGemmItems * Dn; idx += blockDim.x) {
    const int it = idx / Dn, d = idx % Dn;
    qs[idx] = it < ni ? bf16_to_f32(q_nope[(i0 + it) * st + h * sh + d]) : 0.f;
  }
  __syncthreads();
  const uint16_t* w = w_uk + static_cast<int64_t>(h) * Dn * R;
  for (int r0 = 0; r0 < R; r0 += 256) {
    const int r = r0 + threadIdx.x;
    if (r >= R) break;
    float acc[kGemmItems];
#pragma unroll
    for (int it = 0; it < kGemmItems; ++it) acc[it] = 0.f;
    for (int d = 0; d < Dn; ++d) {
      const float wv = bf16_to_f32(w[static_cast<int64_t>(d) * R + r]);
#pragma unroll
      for (int it = 0; it < kGemmItems; ++it) acc[it] = fmaf(qs[it * Dn + d], wv, acc[it]);
    }
    for (int it = 0; it < ni; ++it)
      q_lat[(static_cast<int64_t>(i0 + it) * H + h) * R + r] = f32_to_bf16(acc[it]);
  }
}

// out[i,h,v] = sum_r W_UV[h,v,r] * o_lat[i,h,r]; fp32 accumulation, bf16 out.
// Block: one head, 16 items; a wave handles one output column v at a time,
// its lanes splitting r.
__global__ __launch_bounds__(256) void up_project_kernel(const float* __restrict__ o_lat,
                                                          const float* __restrict__ o_scale,
                                                          const uint16_t* __restrict__ w_uv,
                                                          int32_t Nq, int32_t H, int32_t R,
                                                          int32_t Dv, uint16_t* __restrict__ out) {
  extern __shared__ float os[];  // [kGemmItems][R]
  const int h = blockIdx.y;
  const int i0 = blockIdx.x * kGemmItems;
  const int ni = min(kGemmItems, Nq - i0);
  for (int idx = threadIdx.x; idx < kGemmItems * R; idx += blockDim.x) {
    const int it = idx / R, r = idx % R;
    const int64_t row = static_cast<int64_t>(i0 + it) * H + h;
    os[idx] = it < ni ? o_lat[row * R + r] * o_scale[row] : 0.f;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint16_t* w = w_uv + static_cast<int64_t>(h) * Dv * R;
  for (int v = wave; v < Dv; v += 4) {
    float acc[kGemmItems];
#pragma unroll
    for (int it = 0; it < kGemmItems; ++it) acc[it] = 0.f;
    for (int r = lane; r < R; r += 64) {
      const float wv = bf16_to_f32(w[static_cast<int64_t>(v) * R + r]);
#pragma unroll
      for (int it = 0; it < kGemmItems; ++it) acc[it] = fmaf(os[it * R + r], wv, acc[it]);
    }
#pragma unroll
    for (int it = 0; it < kGemmItems; ++it) acc[it] = wave_sum(acc[it]);
    if (lane < ni) {
      float mine = 0.f;
#pragma unroll
      for (int it = 0; it < kGemmItems; ++it) mine = (it == lane) ? acc[it] : mine;
      out[(static_cast<int64_t>(i0 + lane) * H + h) * Dv + v] = f32_to_bf16(mine);
    }
  }
}

__global__ __launch_bounds__(256) void latent_out_kernel(const float* __restrict__ o_lat,
                                                          const float* __restrict__ o_scale,
                                                          int64_t count, int32_t R,
                                                          uint16_t* __restrict__ out) {
  for (int64_t k = blockIdx.x * 256ll + threadIdx.x; k < count; k += 256ll * gridDim.x)
    out[k] = f32_to_bf16(o_lat[k] * o_scale[k / R]);
}

}  // namespace

hipError_t launch_plan(int mode, int32_t batch, int32_t num_items, const int32_t* context_lens,
                       const int32_t* query_start_loc, int32_t window, int32_t max_ctx,
                       const Plan& plan, hipStream_t s) {
  hipLaunchKernelGGL(plan_items_kernel, dim3(1), dim3(kPlanThreads), 0, s, mode, batch, num_items,
                     context_lens, query_start_loc, window, max_ctx, plan.item_b, plan.item_lo,
                     plan.item_hi, plan.tile_start, plan.G, plan.wg_tile, plan.wg_item,
                     plan.item_wg);
  return hipGetLastError();
}

hipError_t launch_combine_segments(const AttnArgs& a, hipStream_t s) {
  if (a.num_items == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_segments_kernel, dim3(a.num_items, (a.H + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dense_combine(const float* o_part, const float* lse_part, int32_t num_splits,
                                int32_t rows, int32_t dim, float* o, float* lse, hipStream_t s) {
  hipLaunchKernelGGL(dense_combine_kernel, dim3(rows), dim3(256), 0, s, o_part, lse_part,
                     num_splits, rows, dim, o, lse);
  return hipGetLastError();
}

hipError_t launch_absorb(const uint16_t* q_nope, int64_t st, int64_t sh, const uint16_t* w_uk,
                         int32_t num_items, int32_t H, int32_t Dn, int32_t R, uint16_t* q_lat,
                         hipStream_t s) {
  const dim3 grid((num_items + kGemmItems - 1) / kGemmItems, H);
  const size_t smem = sizeof(float) * kGemmItems * Dn;
  hipLaunchKernelGGL(absorb_kernel, grid, dim3(256), smem, s, q_nope, st, sh, w_uk, num_items, H,
                     Dn, R, q_lat);
  return hipGetLastError();
}

hipError_t launch_up_project(const float* o_lat, const float* o_scale, const uint16_t* w_uv,
                             int32_t num_items, int32_t H, int32_t R, int32_t Dv, uint16_t* out,
                             hipStream_t s) {
  const dim3 grid((num_items + kGemmItems - 1) / kGemmItems, H);
  const size_t smem = sizeof(float) * kGemmItems * R;
  hipLaunchKernelGGL(up_project_kernel, grid, dim3(256), smem, s, o_lat, o_scale, w_uv, num_items,
                     H, R, Dv, out);
  return hipGetLastError();
}

hipError_t launch_latent_out(const float* o_lat, const float* o_scale, int32_t num_items, int32_t H,
                             int32_t R, uint16_t* out, hipStream_t s) {
  const int64_t count = static_cast<int64_t>(num_items) * H * R;
  if (count == 0) return hipSuccess;
  const int64_t blocks = (count + 255) / 256;
  hipLaunchKernelGGL(latent_out_kernel, dim3(static_cast<unsigned>(blocks < 65536 ? blocks : 65536)),
                     dim3(256), 0, s, o_lat, o_scale, count, R, out);
  return hipGetLastError();
}

}  // namespace mla
