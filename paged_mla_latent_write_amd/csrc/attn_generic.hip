// Plain split-KV paged latent attention (no MFMA): the reference-shaped GPU
// path for any supported dimension (small MLA shapes, and a cross-check of the
// MFMA kernel).  Same work partition and outputs as the MFMA kernel.
//
// Per query item and head h (absorbed MLA; "[unified-memory] Let Kimi-Linear
// use the paged MLA attention backends", What this does and Validation: the
// kernels read the 512 + 64 latent cache through the block table):
//   s_t = scale * (q_lat[h] . c_t + q_pe[h] . r_t) over the visible keys,
//   o_lat[h] = softmax(s) . c, lse[h] = log sum exp(s),
// computed with an online softmax in base 2 over 16-token sub-tiles.
//
// Grid: (G workgroups of the tile stream) x (head blocks of hpb heads).
#include <math.h>

#include <atomic>

#include "device_utils.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kSub = 16;      // tokens per LDS sub-tile
constexpr int kMaxAcc = 16;   // accumulators per thread
constexpr int kMaxAttrDevices = 64;

__device__ __forceinline__ float load_latent(const CacheView& kv, int64_t row, int d) {
  if (kv.dtype == kKvBf16) {
    return bf16_to_f32(static_cast<const uint16_t*>(kv.data)[row * kv.D + d]);
  }
  const uint8_t c = static_cast<const uint8_t*>(kv.data)[row * kv.D + d];
  return e4m3_to_f32(c) * kv.scale[row];
}

__global__ __launch_bounds__(256) void attn_generic_kernel(AttnArgs a, int hpb) {
  extern __shared__ float smem[];
  const int D = a.kv.D, R = a.kv.R;
  const int Dp = D + 1;              // padded LDS row pitch (bank spread)
  const int tid = threadIdx.x;
  float* q_s = smem;                 // [hpb][D]
  float* kv_s = q_s + hpb * D;       // [kSub][Dp]
  float* p_s = kv_s + kSub * Dp;     // [hpb][kSub]
  float* m_s = p_s + hpb * kSub;     // [hpb]
  float* l_s = m_s + hpb;            // [hpb]
  float* al_s = l_s + hpb;           // [hpb]

  const int64_t g = blockIdx.x;
  const int64_t t0 = a.wg_tile[g], t1 = a.wg_tile[g + 1];
  if (t0 >= t1) return;
  // head blocks: one per grid row (the grid may also have fewer rows)
  for (int hb = blockIdx.y; hb * hpb < a.H; hb += gridDim.y) {
  const int h0 = hb * hpb;
  const int nh = min(hpb, a.H - h0);

  // item containing tile t0: largest i with tile_start[i] <= t0
  int lo = 0, hi = a.num_items;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.tile_start[mid] <= t0) lo = mid; else hi = mid;
  }
  int i = lo;
  const int ps = a.kv.page_size;
  const unsigned last_page = static_cast<unsigned>(a.kv.num_pages - 1);

  int64_t t = t0;
  while (t < t1) {
    while (a.tile_start[i + 1] <= t) ++i;  // skip items with no tiles
    const int64_t ts = a.tile_start[i], te = a.tile_start[i + 1];
    const int64_t seg_end = te < t1 ? te : t1;
    const int b = a.item_b[i];
    const int vlo = a.item_lo[i], vhi = a.item_hi[i];
    const int k_base = vlo / kTile;
    const int32_t* bt = a.block_tables + static_cast<int64_t>(b) * a.max_blocks;

    for (int idx = tid; idx < nh * D; idx += blockDim.x) {
      const int h = idx / D, d = idx % D;
      q_s[idx] = d < R ? bf16_to_f32(a.q_lat[i * a.q_lat_st + (h0 + h) * a.q_lat_sh + d])
                       : bf16_to_f32(a.q_pe[i * a.q_pe_st + (h0 + h) * a.q_pe_sh + (d - R)]);
    }
    if (tid < nh) {
      m_s[tid] = -INFINITY;
      l_s[tid] = 0.f;
    }
    float acc[kMaxAcc];
#pragma unroll
    for (int k = 0; k < kMaxAcc; ++k) acc[k] = 0.f;
    __syncthreads();

    for (int64_t tt = t; tt < seg_end; ++tt) {
      const int tok0 = (k_base + static_cast<int>(tt - ts)) * kTile;
      for (int half = 0; half < kTile / kSub; ++half) {
        const int s0 = tok0 + half * kSub;
        const int v0 = max(s0, vlo), v1 = min(s0 + kSub, vhi);
        if (v0 >= v1) continue;  // uniform over the block
        for (int idx = tid; idx < kSub * D; idx += blockDim.x) {
          const int j = idx / D, d = idx % D;
          const int pos = s0 + j;
          float v = 0.f;
          if (pos >= v0 && pos < v1) {
            const unsigned pg = min(static_cast<unsigned>(bt[pos / ps]), last_page);
            v = load_latent(a.kv, static_cast<int64_t>(pg) * ps + pos % ps, d);
          }
          kv_s[j * Dp + d] = v;
        }
        __syncthreads();
        if (tid < nh * kSub) {
          const int h = tid / kSub, j = tid % kSub;
          const int pos = s0 + j;
          float s = -INFINITY;
          if (pos >= v0 && pos < v1) {
            float dot = 0.f;
            for (int d = 0; d < D; ++d) dot = fmaf(q_s[h * D + d], kv_s[j * Dp + d], dot);
            s = dot * a.scale_log2;
          }
          p_s[tid] = s;
        }
        __syncthreads();
        if (tid < nh) {
          const int h = tid;
          float mx = m_s[h];
          for (int j = 0; j < kSub; ++j) mx = fmaxf(mx, p_s[h * kSub + j]);
          const float alpha = (mx == -INFINITY) ? 1.f : exp2f(m_s[h] - mx);
          float sum = 0.f;
          for (int j = 0; j < kSub; ++j) {
            const float s = p_s[h * kSub + j];
            const float e = (s == -INFINITY) ? 0.f : exp2f(s - mx);
            p_s[h * kSub + j] = e;
            sum += e;
          }
          l_s[h] = l_s[h] * alpha + sum;
          m_s[h] = mx;
          al_s[h] = alpha;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kMaxAcc; ++k) {
          const int idx = tid + 256 * k;
          if (idx < nh * R) {
            const int h = idx / R, r = idx % R;
            float v = acc[k] * al_s[h];
            for (int j = 0; j < kSub; ++j) v = fmaf(p_s[h * kSub + j], kv_s[j * Dp + r], v);
            acc[k] = v;
          }
        }
        __syncthreads();
      }
    }

    // (a complete item's row is fp32 o_lat; a split item's partial is bf16)
    const bool complete = (t == ts) && (seg_end == te);
    float* o_dst = nullptr;
    uint16_t* p_dst = nullptr;
    float* lse_dst;
    float* scl_dst;
    if (complete) {
      o_dst = a.o_lat + (static_cast<int64_t>(i) * a.H + h0) * R;
      lse_dst = a.lse + static_cast<int64_t>(i) * a.H + h0;
      scl_dst = a.o_scale + static_cast<int64_t>(i) * a.H + h0;
    } else {
      const int64_t slot = (ts < t0) ? 2 * g : 2 * g + 1;
      p_dst = a.part_o + (slot * a.H + h0) * R;
      lse_dst = a.part_lse + slot * a.H + h0;
      scl_dst = a.part_scale + slot * a.H + h0;
    }
#pragma unroll
    for (int k = 0; k < kMaxAcc; ++k) {
      const int idx = tid + 256 * k;
      if (idx < nh * R) {
        const float v = acc[k] / l_s[idx / R];
        if (complete) o_dst[idx] = v;
        else p_dst[idx] = f32_to_bf16(v);
      }
    }
    if (tid < nh) {
      lse_dst[tid] = (m_s[tid] + log2f(l_s[tid])) * kLn2;
      scl_dst[tid] = 1.0f;  // stored normalised
    }
    __syncthreads();
    t = seg_end;
  }
  __syncthreads();  // the next head block reuses the shared buffers
  }
}

int heads_per_block(int H, int R) {
  int hpb = (kMaxAcc * 256) / R;
  hpb = hpb < 1 ? 1 : hpb;
  hpb = hpb > 256 / kSub ? 256 / kSub : hpb;
  return hpb < H ? hpb : H;
}

}  // namespace

hipError_t launch_attn_generic(const AttnArgs& a, hipStream_t s) {
  const int hpb = heads_per_block(a.H, a.kv.R);
  const int nhb = (a.H + hpb - 1) / hpb;
  const size_t smem =
      sizeof(float) * (static_cast<size_t>(hpb) * a.kv.D + kSub * (a.kv.D + 1) + hpb * kSub + 3 * hpb);
  // The dynamic-LDS limit is raised once per device.  The flags are atomics:
  // threads that race on a first launch each set the same attribute.
  static std::atomic<bool> attr_set[kMaxAttrDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
  if (dev < 0 || dev >= kMaxAttrDevices || !attr_set[dev].load(std::memory_order_acquire)) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(attn_generic_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxAttrDevices) attr_set[dev].store(true, std::memory_order_release);
  }
  hipLaunchKernelGGL(attn_generic_kernel, dim3(a.G, nhb), dim3(256), smem, s, a, hpb);
  return hipGetLastError();
}

}  // namespace mla
