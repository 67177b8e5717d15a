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
//    the output dimension, the MFMA wants runs along K).  The block's query
//    rows and its output tile pass through LDS as well, so global memory sees
//    whole 256-byte rows (a lane's own fragment would take one cache line per
//    lane and instruction).  bf16 in, fp32 accumulate, bf16 out.
//  * up-project: W_UV rows already run along K, so B fragments come straight
//    from global memory.  o_lat is fp32; each A fragment is split into a bf16
//    high part and a bf16 remainder and both are multiplied (two MFMAs), which
//    keeps the product accurate to about 2^-16 relative.
#include <math.h>

#include <algorithm>

#include "device_utils.h"
#include "mla_internal.h"
#include "plan_device.h"
#include "write_device.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(T) __attribute__((address_space(3))) T*

constexpr int kAbsCols = 128;              // W_UK columns staged per chunk
constexpr int kAbsPitch = kAbsCols * 2 + 32;  // bytes per staged row (padded)
constexpr int kAbsMaxDn = 128;
constexpr int kAbsQPitch = kAbsMaxDn * 2 + 16;  // bytes per staged query / output row (padded)
static_assert(kAbsCols * 2 <= kAbsMaxDn * 2, "the output tile fits the query rows");

template <int MT>
__global__ __launch_bounds__(256) void absorb_mfma_kernel(const uint16_t* __restrict__ q_nope,
                                                          int64_t st, int64_t sh,
                                                          const uint16_t* __restrict__ w_uk,
                                                          int32_t Nq, int32_t H, int32_t Dn,
                                                          int32_t R, uint16_t* __restrict__ q_lat,
                                                          PlanArgs pa, TokenWrite tw) {
  __shared__ __attribute__((aligned(16))) char wt[kAbsMaxDn * kAbsPitch];
  __shared__ __attribute__((aligned(16))) char qs[32 * MT * kAbsQPitch];
  static_assert((256 + 1 + 2 * kPlanLds) * 4 <= kAbsMaxDn * kAbsPitch, "plan LDS fits the staging buffer");
  if (blockIdx.x * kAbsCols >= R) {
    // the extra columns of workgroups: the first computes the split plan, in
    // the staging buffer's LDS (pa.plan.G == 0: no plan asked for); the next
    // write the new tokens, one wavefront per token (tw.T == 0: none)
    const int planned = pa.plan.G > 0 ? 1 : 0;
    const int id = (blockIdx.x - R / kAbsCols) * gridDim.y * gridDim.z + blockIdx.y + gridDim.y * blockIdx.z;
    if (id < planned) {
      int32_t* l = reinterpret_cast<int32_t*>(wt);
      plan_items_body<256>(l, l + 256, l + 257, l + 257 + kPlanLds, pa.mode, pa.batch, pa.num_items,
                           pa.context_lens, pa.query_start_loc, pa.window, pa.max_ctx,
                           pa.plan.item_b, pa.plan.item_lo, pa.plan.item_hi, pa.plan.tile_start,
                           pa.plan.G, pa.plan.wg_tile, pa.plan.wg_item, pa.plan.item_wg);
    } else {
      const int64_t tok = static_cast<int64_t>(id - planned) * 4 + (threadIdx.x >> 6);
      if (tok < tw.T) write_token(tw, tok, threadIdx.x & 63);
    }
    return;
  }
  const int c0 = blockIdx.x * kAbsCols;  // this workgroup's 128 output columns
  const int h = blockIdx.y;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int g = lane >> 5, n32 = lane & 31;
  const int ksteps = Dn / 16;

  // transposed-read lane offsets (see the attention kernel for the layout)
  const int q = lane >> 4, jj = lane & 15, rr = jj >> 2, c4 = jj & 3;
  const int tr_off = (8 * g + rr) * kAbsPitch + (32 * wave + 16 * (q & 1) + 4 * c4) * 2;
  const uint16_t* wh = w_uk + static_cast<int64_t>(h) * Dn * R;

  // The block's query rows are staged in LDS (sixteen threads read one 256-byte
  // row), and so is its output tile (written back as 256-byte rows): a lane's
  // own MFMA fragments would touch one cache line per lane and instruction.
  constexpr int kQPer = 32 * MT * (kAbsMaxDn / 8) / 256;  // 16-byte chunks per thread
  i16x8 qv[kQPer];
  auto load_q = [&](int m0) {
#pragma unroll
    for (int j = 0; j < kQPer; ++j) {
      const int idx = t + 256 * j;
      const int r = idx / (kAbsMaxDn / 8), c = idx % (kAbsMaxDn / 8);
      const int item = m0 + r;
      i16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
      if (item < Nq && c < Dn / 8) v = *reinterpret_cast<const i16x8*>(q_nope + item * st + h * sh + 8 * c);
      qv[j] = v;
    }
  };
  auto store_q = [&]() {
#pragma unroll
    for (int j = 0; j < kQPer; ++j) {
      const int idx = t + 256 * j;
      const int r = idx / (kAbsMaxDn / 8), c = idx % (kAbsMaxDn / 8);
      *reinterpret_cast<i16x8*>(qs + r * kAbsQPitch + c * 16) = qv[j];
    }
  };
  const int m_first = blockIdx.z * 32 * MT, m_stride = gridDim.z * 32 * MT;
  if (m_first < Nq) load_q(m_first);
  {
    // stage W_UK[h][0:Dn][c0 : c0 + 128]: all loads first (16 B per thread
    // per step), then the LDS stores
    constexpr int kStage = kAbsMaxDn * (kAbsCols / 8) / 256;
    i16x8 wv[kStage];
#pragma unroll
    for (int j = 0; j < kStage; ++j) {
      const int idx = t + 256 * j;
      const int d = idx / (kAbsCols / 8), c = idx % (kAbsCols / 8);
      if (d < Dn) wv[j] = *reinterpret_cast<const i16x8*>(wh + static_cast<int64_t>(d) * R + c0 + 8 * c);
    }
#pragma unroll
    for (int j = 0; j < kStage; ++j) {
      const int idx = t + 256 * j;
      const int d = idx / (kAbsCols / 8), c = idx % (kAbsCols / 8);
      if (d < Dn) *reinterpret_cast<i16x8*>(wt + d * kAbsPitch + c * 16) = wv[j];
    }
  }
  store_q();
  __syncthreads();
  // item blocks of 32 MT: one per workgroup for decode-sized batches, several
  // for prefill-sized ones (the staged W_UK block is reused)
  for (int m0 = m_first; m0 < Nq; m0 += m_stride) {
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
        for (int mt = 0; mt < MT; ++mt) {
          const i16x8 af = *reinterpret_cast<const i16x8*>(qs + (32 * mt + n32) * kAbsQPitch + (16 * k + 8 * g) * 2);
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af),
                                                            __builtin_bit_cast(bf16x8, b), acc[mt],
                                                            0, 0, 0);
        }
      }
    }
    const int m1 = m0 + m_stride;
    if (m1 < Nq) load_q(m1);  // the next block's queries: in flight during the stores
    __syncthreads();          // every wave has read its query fragments
    // the output tile [32 MT items][128 columns] as bf16 rows in the query buffer
    const int col = 32 * wave + n32;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 32 * mt + 8 * (i >> 2) + 4 * g + (i & 3);
        *reinterpret_cast<uint16_t*>(qs + r * kAbsQPitch + col * 2) = f32_to_bf16(acc[mt][i]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 32 * MT * (kAbsCols / 8) / 256; ++j) {
      const int idx = t + 256 * j;
      const int r = idx / (kAbsCols / 8), c = idx % (kAbsCols / 8);
      const int item = m0 + r;
      if (item < Nq)
        *reinterpret_cast<i16x8*>(q_lat + (static_cast<int64_t>(item) * H + h) * R + c0 + 8 * c) =
            *reinterpret_cast<const i16x8*>(qs + r * kAbsQPitch + c * 16);
    }
    if (m1 < Nq) {
      __syncthreads();  // the output tile has been read
      store_q();
      __syncthreads();
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

// Combine + up-projection in one pass, for the split-KV decode/prefill path:
// a workgroup owns one head and 32 items.  Phase 1 merges each item's row of
// o_lat from the partial results of the workgroups its tiles were cut across
// (the same log-sum-exp merge as combine_segments, slots 2g+1 for the first
// workgroup and 2g after it) or takes the attention kernel's own row for an
// uncut item, normalises it and stages it in LDS as a bf16 high part and a
// bf16 remainder; phase 2 is the up-projection of up_project_mfma_kernel<1>
// with A fragments from LDS.  o_lat itself is never written.
constexpr int kCupMaxR = 512;
constexpr int kCupPitch = kCupMaxR + 8;  // bf16 per staged row (16 B pad: bank spread)

constexpr int kCupThreads = 512;

// SB: partial rows of one item loaded together.  SB = 1 is the low-register
// form for large item counts (prefill): phase 2 then loads its W_UV fragments
// eight k-steps at a time instead of all before the barrier, so that two
// workgroups fit on a compute unit.  Decode grids of at most one workgroup
// per compute unit take SB = 8, so that the partial rows of most items (a
// long context is cut across four to six workgroups) arrive in one round
// trip; larger decode grids take SB = 4 (on 512 workgroups of items cut
// across two or three workgroups each, SB = 8 measured 20 % slower).  IPW: items per workgroup, 32 or (grids
// smaller than the chip: few heads and requests) 4, merged by 128 threads each
// with up to SB = 16 segments per round trip; the up-projection's MFMA rows
// past those items are computed and discarded.
template <int SB, int IPW>
__global__ __launch_bounds__(kCupThreads) void combine_up_project_kernel(AttnArgs a,
                                                                         const uint16_t* __restrict__ w_uv,
                                                                         int32_t Dv, uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) __bf16 o_hi[32 * kCupPitch];
  __shared__ __attribute__((aligned(16))) __bf16 o_lo[32 * kCupPitch];
  const int h = blockIdx.y;
  const int m0 = blockIdx.x * IPW;
  const int H = a.H, R = a.kv.R, Nq = a.num_items;
  constexpr int kTpi = kCupThreads / IPW;  // threads per item
  const int t = threadIdx.x;

  // ---- phase 1: the kTpi threads (il, j) of item m0 + il merge its columns
  // 4 j + 4 kTpi e .. + 3: each load of the item's threads reads 16 kTpi
  // contiguous bytes.  The rows of up to SB segments are requested at once, as
  // soon as the item's workgroup range is known, so most items take one round
  // trip.
  {
    constexpr int kE = kCupMaxR / (4 * kTpi);  // float4 per thread per row
    const int il = t / kTpi, j = t % kTpi;
    const int item = m0 + il;
    float4 acc[kE];
#pragma unroll
    for (int e = 0; e < kE; ++e) acc[e] = make_float4(0.f, 0.f, 0.f, 0.f);
    float m = -INFINITY, tot = 0.f;
    if (item < Nq) {
      const int64_t row = static_cast<int64_t>(item) * H + h;
      const int g0 = a.item_wg[2 * item], g1 = a.item_wg[2 * item + 1];
      if (g0 >= 0 && g0 == g1) {
        // uncut: the attention kernel wrote the unnormalised row and 1 / l
        const float sc = a.o_scale[row];
        const float4* src = reinterpret_cast<const float4*>(a.o_lat + row * R);
#pragma unroll
        for (int e = 0; e < kE; ++e) {
          const int c = 4 * j + 4 * kTpi * e;
          if (c < R) {
            const float4 x = src[c >> 2];
            acc[e] = make_float4(x.x * sc, x.y * sc, x.z * sc, x.w * sc);
          }
        }
        m = 0.f;
        tot = 1.f;
      } else if (g0 >= 0) {
        for (int gb = g0; gb <= g1; gb += SB) {
          float l[SB], sc[SB];
          uint2 x[SB][kE];  // 4 bf16 partial values each (low half first)
#pragma unroll
          for (int p = 0; p < SB; ++p) {
            const int gg = gb + p;
            const bool in = gg <= g1;
            // A workgroup range of the item with no tiles wrote no slot: its
            // (stale) row is loaded with the others but gets no weight.
            const bool live = in && a.wg_tile[gg] != a.wg_tile[gg + 1];
            const int64_t slot = (gg == g0) ? 2 * gg + 1 : 2 * gg;
            const float lp = in ? a.part_lse[slot * H + h] : -INFINITY;
            sc[p] = in ? a.part_scale[slot * H + h] : 0.f;
            const uint2* src = reinterpret_cast<const uint2*>(a.part_o + (slot * H + h) * R);
#pragma unroll
            for (int e = 0; e < kE; ++e) {
              const int c = 4 * j + 4 * kTpi * e;
              x[p][e] = (in && c < R) ? src[c >> 2] : make_uint2(0u, 0u);
            }
            l[p] = live ? lp : -INFINITY;
          }
          float mb = m;
#pragma unroll
          for (int p = 0; p < SB; ++p) mb = fmaxf(mb, l[p]);
          if (mb > m) {  // uniform within the item's threads
            const float f = expf(m - mb);
            tot *= f;
#pragma unroll
            for (int e = 0; e < kE; ++e) acc[e] = make_float4(acc[e].x * f, acc[e].y * f, acc[e].z * f, acc[e].w * f);
            m = mb;
          }
#pragma unroll
          for (int p = 0; p < SB; ++p) {
            if (l[p] == -INFINITY) continue;
            const float e_l = expf(l[p] - m);
            tot += e_l;
            const float w = e_l * sc[p];
#pragma unroll
            for (int e = 0; e < kE; ++e) {
              acc[e].x = fmaf(w, __uint_as_float(x[p][e].x << 16), acc[e].x);
              acc[e].y = fmaf(w, __uint_as_float(x[p][e].x & 0xFFFF0000u), acc[e].y);
              acc[e].z = fmaf(w, __uint_as_float(x[p][e].y << 16), acc[e].z);
              acc[e].w = fmaf(w, __uint_as_float(x[p][e].y & 0xFFFF0000u), acc[e].w);
            }
          }
        }
        if (j == 0) a.lse[row] = tot > 0.f ? m + logf(tot) : -INFINITY;
      } else if (j == 0) {
        a.lse[row] = -INFINITY;  // no visible keys: out 0, lse -inf
      }
    }
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      const int c = 4 * j + 4 * kTpi * e;
      if (c < R) {
        const float xs[4] = {acc[e].x * inv, acc[e].y * inv, acc[e].z * inv, acc[e].w * inv};
        bf16x4 hi, lo;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          hi[q] = static_cast<__bf16>(xs[q]);
          lo[q] = static_cast<__bf16>(xs[q] - static_cast<float>(hi[q]));
        }
        *reinterpret_cast<bf16x4*>(o_hi + il * kCupPitch + c) = hi;
        *reinterpret_cast<bf16x4*>(o_lo + il * kCupPitch + c) = lo;
      }
    }
  }
  // ---- phase 2: out[item, h, v] = W_UV[h][v] . o[item], wave w < 4: v in [32 w, 32 w + 32).
  // Its W_UV fragments are requested before the barrier, so their latency
  // overlaps the other waves' merging.
  const int lane = t & 63, wave = t >> 6;
  const int g = lane >> 5, n32 = lane & 31;
  const int v = 32 * wave + n32;
  const bool up_wave = 32 * wave < Dv;
  const uint16_t* wrow = w_uv + (static_cast<int64_t>(h) * Dv + (up_wave ? v : 0)) * R;
  i16x8 b[SB > 1 ? kCupMaxR / 16 : 1];
  if constexpr (SB > 1) {
    if (up_wave) {
#pragma unroll
      for (int u = 0; u < kCupMaxR / 16; ++u)
        if (16 * u < R) b[u] = *reinterpret_cast<const i16x8*>(wrow + 16 * u + 8 * g);
    }
  }
  __syncthreads();
  if (!up_wave) return;
  f32x16 acc = f32x16{};
  if constexpr (SB > 1) {
#pragma unroll
    for (int u = 0; u < kCupMaxR / 16; ++u) {
      const int k = 16 * u;
      if (k >= R) break;
      const bf16x8 hi = *reinterpret_cast<const bf16x8*>(o_hi + n32 * kCupPitch + k + 8 * g);
      const bf16x8 lo = *reinterpret_cast<const bf16x8*>(o_lo + n32 * kCupPitch + k + 8 * g);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hi, __builtin_bit_cast(bf16x8, b[u]), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lo, __builtin_bit_cast(bf16x8, b[u]), acc, 0, 0, 0);
    }
  } else {
    // eight k-steps' fragments at a time
#pragma unroll
    for (int u0 = 0; u0 < kCupMaxR / 16; u0 += 8) {
      if (16 * u0 >= R) break;
      i16x8 bw[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (16 * (u0 + u) < R) bw[u] = *reinterpret_cast<const i16x8*>(wrow + 16 * (u0 + u) + 8 * g);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = 16 * (u0 + u);
        if (k >= R) break;
        const bf16x8 hi = *reinterpret_cast<const bf16x8*>(o_hi + n32 * kCupPitch + k + 8 * g);
        const bf16x8 lo = *reinterpret_cast<const bf16x8*>(o_lo + n32 * kCupPitch + k + 8 * g);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hi, __builtin_bit_cast(bf16x8, bw[u]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lo, __builtin_bit_cast(bf16x8, bw[u]), acc, 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = 8 * (i >> 2) + 4 * g + (i & 3);
    const int item = m0 + row;
    if (row < IPW && item < Nq) out[(static_cast<int64_t>(item) * H + h) * Dv + v] = f32_to_bf16(acc[i]);
  }
}

int pick_mt(int Nq) { return Nq <= 64 ? 1 : 4; }

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

bool combine_up_project_supported(int32_t R, int32_t Dv) {
  return up_project_mfma_supported(R, Dv) && R % 32 == 0 && R <= kCupMaxR;
}

hipError_t launch_combine_up_project(const AttnArgs& a, const uint16_t* w_uv, int32_t Dv, uint16_t* out,
                                     hipStream_t s) {
  const int blocks32 = (a.num_items + 31) / 32;
  const int cus = std::max(1, current_cu_count());
  if (a.num_items > cus) {  // prefill-sized: many workgroups, most items uncut
    hipLaunchKernelGGL((combine_up_project_kernel<1, 32>), dim3(blocks32, a.H), dim3(kCupThreads), 0, s, a, w_uv,
                       Dv, out);
  } else if (blocks32 * a.H < cus) {  // fewer workgroups than compute units
    hipLaunchKernelGGL((combine_up_project_kernel<16, 4>), dim3((a.num_items + 3) / 4, a.H), dim3(kCupThreads), 0,
                       s, a, w_uv, Dv, out);
  } else if (blocks32 * a.H <= cus) {  // one workgroup per compute unit: the register-heavy form
    hipLaunchKernelGGL((combine_up_project_kernel<8, 32>), dim3(blocks32, a.H), dim3(kCupThreads), 0, s, a, w_uv,
                       Dv, out);
  } else {
    hipLaunchKernelGGL((combine_up_project_kernel<4, 32>), dim3(blocks32, a.H), dim3(kCupThreads), 0, s, a, w_uv,
                       Dv, out);
  }
  return hipGetLastError();
}

hipError_t launch_absorb_mfma(const uint16_t* q_nope, int64_t st, int64_t sh, const uint16_t* w_uk,
                              int32_t num_items, int32_t H, int32_t Dn, int32_t R, uint16_t* q_lat,
                              const PlanArgs* plan, const TokenWrite* write, hipStream_t s) {
  PlanArgs pa{};
  if (plan) pa = *plan;  // else pa.plan.G == 0: no plan
  TokenWrite tw{};
  if (write) tw = *write;  // else tw.T == 0: nothing to write
  const int mt = pick_mt(num_items);
  // the W_UK block (Dn x 128 columns) is staged once per workgroup: at most
  // ~2048 workgroups in all, so large item counts loop over several blocks;
  // decode-sized batches (one or two blocks) take one workgroup per W_UK
  // block, which reads it from memory once (measured faster than two
  // workgroups each reading it for half the items)
  const int nblk = (num_items + 32 * mt - 1) / (32 * mt);
  const int gz = nblk <= 2 ? 1 : std::max(1, std::min(nblk, std::max(1, 2048 / std::max(1, (R / kAbsCols) * H))));
  // extra columns: the plan's workgroup, then one per four new tokens
  const int64_t extra = (plan ? 1 : 0) + (static_cast<int64_t>(tw.T) + 3) / 4;
  const int64_t per_col = static_cast<int64_t>(H) * gz;
  const dim3 grid(R / kAbsCols + static_cast<int>((extra + per_col - 1) / per_col), H, gz);
  switch (mt) {
    case 1: hipLaunchKernelGGL(absorb_mfma_kernel<1>, grid, dim3(256), 0, s, q_nope, st, sh, w_uk, num_items, H, Dn, R, q_lat, pa, tw); break;
    case 2: hipLaunchKernelGGL(absorb_mfma_kernel<2>, grid, dim3(256), 0, s, q_nope, st, sh, w_uk, num_items, H, Dn, R, q_lat, pa, tw); break;
    default: hipLaunchKernelGGL(absorb_mfma_kernel<4>, grid, dim3(256), 0, s, q_nope, st, sh, w_uk, num_items, H, Dn, R, q_lat, pa, tw); break;
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
