// Split-KV paged latent attention on CDNA4 matrix cores (gfx950), for the MLA
// latent shape kv_lora_rank 512 + qk_rope 64 with up to 128 query heads.
//
// What it computes (absorbed MLA; "[unified-memory] Let Kimi-Linear use the
// paged MLA attention backends", What this does and Validation: the kernels
// read the 512 + 64 latent cache through the block table, many heads share
// one latent KV): for each query item and head h,
//   s_t = scale * ([q_lat ; q_pe][h] . [c_t ; r_t])  over the visible keys t,
//   o_lat[h] = softmax(s) . c,   lse[h] = log sum exp(s).
// The work partition, the item plan and the outputs are the same as the plain
// kernel's (attn_generic.hip); only the inner loop differs.
//
// Design (one workgroup of four waves per compute unit):
//  * wave w owns heads [32w, 32w + 32).  Its query block Q[32 x 576] lives in
//    VGPRs as the B operand of S^T = K Q^T (36 fragments of 16 dims), and its
//    accumulator O^T[512 x 32] (fp32) as 16 MFMA 32x32 tiles in AGPRs.
//  * the key/value stream is cut into 32-token tiles (36 KB of bf16 latents).
//    Each tile is copied HBM -> LDS with global_load_lds (16 B per lane, no
//    VGPR staging) into one of 4 buffers, three tiles ahead of the compute, and
//    is shared by all waves (so every head reads each KV byte from HBM once).
//  * S^T (32 tokens x 32 heads) = 36 v_mfma_f32_32x32x16_bf16 with K rows read
//    by ds_read_b128; the softmax runs in the MFMA output layout (each lane
//    holds 16 tokens of one head; one cross-half exchange per reduction); the
//    probabilities are rounded to bf16 in registers and used directly as the B
//    operand of O^T += V^T P^T (32 MFMAs per tile), whose A operand is read
//    transposed from the same LDS tile by ds_read_b64_tr_b16.  The token order
//    inside each 16-token MFMA step is the one the MFMA output layout gives;
//    the V^T reads use the same order, so no shuffle of P is needed.
//  * online softmax in base 2 against a reference maximum fixed at each
//    segment's first tile, so the accumulators are never rescaled: only MFMAs
//    write them and only the final stores read them (any VALU work on them
//    would not fit the register file next to Q).  Later tiles may exceed the
//    reference by up to 2^64 in probability; a bigger jump flags the
//    workgroup, whose range the plain kernel then recomputes.  The kernel
//    writes the unnormalised O with lse and 1/l; consumers apply 1/l.
//  * LDS rows are 1152 B; 16-byte chunks are XOR-swizzled per token
//    (chunk ^ (2 (t mod 4) + (t div 4) mod 2) within groups of 8) so both the
//    row reads and the transposed reads hit distinct banks.
#include <math.h>

#include "device_utils.h"
#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kR = 512;
constexpr int kD = 576;
constexpr int kRowBytes = kD * 2;            // 1152
constexpr int kTileBytes = kTile * kRowBytes; // 36864
constexpr int kChunksPerTile = kTile * kD / 8; // 2304 16-byte chunks
constexpr int kKSteps = kD / 16;              // 36
constexpr int kMTiles = kR / 32;              // 16
constexpr float kRefSlack = 64.0f;

#define LDS_PTR(T) __attribute__((address_space(3))) T*

__device__ __forceinline__ int swz(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }

// s_waitcnt vmcnt(n) with lgkmcnt and expcnt left unconstrained (gfx9 encoding).
// Counts above the counter's range (63) clamp: memory operations retire in
// issue order, so "at most 63 outstanding" still implies the older ones are done.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  constexpr int n = N > 63 ? 63 : N;
  static_assert(n >= 0, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Read-only plan arrays, read through the constant address space: they do not
// change during the kernel, and this lets the compiler use scalar loads, so
// the vector-memory counter tracks only the tile copies.
#define CONST_PTR(T) const __attribute__((address_space(4))) T*
struct Meta {
  CONST_PTR(int32_t) item_b;
  CONST_PTR(int32_t) item_lo;
  CONST_PTR(int32_t) item_hi;
  CONST_PTR(int32_t) tile_start;
  CONST_PTR(int32_t) block_tables;
};

// 16-byte copy HBM -> LDS without VGPR staging: lane i's 16 bytes land at
// lds_base + 16 i (lds_base wave-uniform, in M0).  Issued as inline assembly
// so the compiler does not add its conservative "LDS DMA may alias this LDS
// read" waits (vmcnt(0) before LDS reads), which would drain the prefetch; the
// kernel orders the copies itself with explicit vmcnt waits and barriers.
__device__ __forceinline__ void lds_dma_16(const void* gptr, uint32_t lds_base) {
  // one wait state is required between writing M0 and an LDS-DMA load
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(gptr)
               : "memory", "m0");
}

struct TileInfo {
  int item;
  int b;
  int vlo, vhi;
  int tok0;  // absolute position of the tile's first token
};

__device__ __forceinline__ TileInfo tile_info(const Meta& m, int item, int64_t tile) {
  TileInfo ti;
  ti.item = item;
  ti.b = m.item_b[item];
  ti.vlo = m.item_lo[item];
  ti.vhi = m.item_hi[item];
  ti.tok0 = ((ti.vlo >> 5) + static_cast<int>(tile - m.tile_start[item])) * kTile;
  return ti;
}

// Next item owning `tile` (items with no tiles are skipped).
__device__ __forceinline__ int advance_item(const Meta& m, int num_items, int item, int64_t tile) {
  while (item + 1 < num_items && m.tile_start[item + 1] <= tile) ++item;
  return item;
}

// Copy one 32-token tile into an LDS buffer: 2304 chunks of 16 B, NW waves x
// (36 / NW) global_load_lds instructions of 64 lanes each.  Tokens outside the
// item's visible range load a clamped (valid, finite) token; their scores are
// masked later, so they contribute exactly zero.
template <int NW>
__device__ __forceinline__ void issue_tile(const AttnArgs& a, const Meta& m, const TileInfo& ti,
                                           LDS_PTR(char) buf, int wave, int lane) {
  constexpr int kPerWave = kChunksPerTile / 64 / NW;
  CONST_PTR(int32_t) bt = m.block_tables + static_cast<int64_t>(ti.b) * a.max_blocks;
  const int ps = a.kv.page_size;
  const int psh = a.kv.page_shift;
  const unsigned last_page = static_cast<unsigned>(a.kv.num_pages - 1);
  // The tile's page ids are wave-uniform (scalar loads, so the vector-memory
  // counter only tracks the tile copies).  A 32-token tile spans one page for
  // page sizes >= 32 and two pages of 16; the second is read only if it holds
  // a visible token (the block table is read up to ceil(n / ps) entries only).
  const int blk0 = ti.tok0 >> psh;
  const unsigned pg0 = min(static_cast<unsigned>(bt[blk0]), last_page);
  unsigned pg1 = pg0;
  if (ps < kTile && ti.tok0 + ps < ti.vhi) pg1 = min(static_cast<unsigned>(bt[blk0 + 1]), last_page);
  const char* base = static_cast<const char*>(a.kv.data);
#pragma unroll
  for (int k = 0; k < kPerWave; ++k) {
    const int blk = wave * kPerWave + k;
    const int s = blk * 64 + lane;
    const int t = s / 72;
    const int p = s - t * 72;
    const int c = (p & ~7) | ((p & 7) ^ swz(t));
    int pos = ti.tok0 + t;
    pos = pos < ti.vlo ? ti.vlo : pos;
    pos = pos >= ti.vhi ? ti.vhi - 1 : pos;
    const int in_page = pos - (blk0 << psh);  // 0 .. 2 * ps - 1
    const unsigned pg = in_page >= ps ? pg1 : pg0;
    const int off = in_page >= ps ? in_page - ps : in_page;
    const char* src = base + ((static_cast<int64_t>(pg) << psh) + off) * kRowBytes + c * 16;
    lds_dma_16(src, static_cast<uint32_t>(reinterpret_cast<uintptr_t>(buf)) + blk * 1024);
  }
}

template <int NW>
__global__ __launch_bounds__(NW * 64, 1) void attn_mfma_kernel(
    AttnArgs a, const int32_t* __restrict__ item_b, const int32_t* __restrict__ item_lo,
    const int32_t* __restrict__ item_hi, const int32_t* __restrict__ tile_start,
    const int32_t* __restrict__ block_tables) {
  const Meta m{(CONST_PTR(int32_t))item_b, (CONST_PTR(int32_t))item_lo, (CONST_PTR(int32_t))item_hi,
               (CONST_PTR(int32_t))tile_start, (CONST_PTR(int32_t))block_tables};
  __shared__ __attribute__((aligned(1024))) char lds_buf[4][kTileBytes];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 5;        // half of the wave
  const int n32 = lane & 31;      // head within the wave / token row for K reads
  const int head = wave * 32 + n32;
  const bool head_ok = head < a.H;
  // With fewer than 32 * NW heads the surplus waves still copy their share of
  // every tile (so the copy rate does not drop) but skip the arithmetic.
  const bool wave_active = wave * 32 < a.H;

  const int64_t W = m.tile_start[a.num_items];
  const int64_t wg = blockIdx.x;
  // redo[wg] is written once per launch by thread 0 (no separate memset, so
  // the call stays capturable): 1 if a score ran past the reference maximum.
  __shared__ int wg_overflow;
  if (threadIdx.x == 0) wg_overflow = 0;
  const int64_t t0 = wg_tile_begin(wg, W, a.G), t1 = wg_tile_begin(wg + 1, W, a.G);
  if (t0 >= t1) {
    if (threadIdx.x == 0) a.redo[wg] = 0;
    return;
  }
  const int ntiles = static_cast<int>(t1 - t0);
  bool overflow = false;

  int first_item;
  {
    int lo = 0, hi = a.num_items;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (m.tile_start[mid] <= t0) lo = mid; else hi = mid;
    }
    first_item = advance_item(m, a.num_items, lo, t0);
  }

  LDS_PTR(char) bufs[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) bufs[u] = (LDS_PTR(char))(&lds_buf[u][0]);

  // ---- lane-constant LDS offsets ----
  // K rows (A of S^T): token n32, chunk 2k + g.  (c & 7) ^ swz = (2k & 7) ^ (g ^ swz).
  const int y = g ^ swz(n32);
  int koff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) koff[j] = n32 * kRowBytes + (((2 * j) ^ y) << 4);
  // V^T (A of O^T) transposed reads: group q = lane / 16, jj = lane % 16.
  const int q = lane >> 4, jj = lane & 15, rr = jj >> 2, c4 = jj & 3;
  const int qs = (2 * (q & 1) + (c4 >> 1)) ^ (2 * rr + g);
  const int vbase = (4 * g + rr) * kRowBytes + 8 * (c4 & 1);
  const int voff_even = vbase + (qs << 4);
  const int voff_odd = vbase + ((4 ^ qs) << 4);

  // ---- load cursor: prologue issues the first three tiles ----
  int l_item = first_item;
  int64_t l_tile = t0;
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    if (p < ntiles) {
      l_item = advance_item(m, a.num_items, l_item, l_tile);
      issue_tile<NW>(a, m, tile_info(m, l_item, l_tile), bufs[p], wave, lane);
      ++l_tile;
    }
  }

  constexpr int kLoadsPerTile = kChunksPerTile / 64 / NW;
  bf16x8 qf[kKSteps];
  f32x16 acc[kMTiles];

  int tn = 0;               // tiles consumed so far (buffer tn % 4)
  int c_item = first_item;
  int64_t ctile = t0;
  while (ctile < t1) {
    // ---- a segment: the WG's tiles of one item ----
    c_item = advance_item(m, a.num_items, c_item, ctile);
    const int64_t item_ts = m.tile_start[c_item], item_te = m.tile_start[c_item + 1];
    const int64_t seg_begin = ctile;
    const int64_t seg_end = item_te < t1 ? item_te : t1;
    if (wave_active) {
      const uint16_t* ql = a.q_lat + c_item * a.q_lat_st + head * a.q_lat_sh;
      const uint16_t* qp = a.q_pe + c_item * a.q_pe_st + head * a.q_pe_sh;
#pragma unroll
      for (int k = 0; k < kKSteps; ++k) {
        i16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
        if (head_ok) {
          const uint16_t* src = k < kR / 16 ? ql + 16 * k + 8 * g : qp + 16 * (k - kR / 16) + 8 * g;
          v = *reinterpret_cast<const i16x8*>(src);
        }
        qf[k] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int mt = 0; mt < kMTiles; ++mt) acc[mt] = f32x16{};
      // consume the query loads here, so their completion wait sits outside
      // the tile loop (a wait inside would also drain the tile prefetch)
#pragma unroll
      for (int k = 0; k < kKSteps; ++k) asm volatile("" : "+v"(qf[k]));
    }
    float m_ref = 0.f, l_sum = 0.f;
    const int vlo = m.item_lo[c_item], vhi = m.item_hi[c_item];
    const int tok_first = ((vlo >> 5) + static_cast<int>(seg_begin - item_ts)) * kTile;

    for (int64_t tt = seg_begin; tt < seg_end; ++tt, ++tn) {
      const int rem = ntiles - tn - 1;
      if (rem >= 2) wait_vmcnt<2 * kLoadsPerTile>();
      else if (rem == 1) wait_vmcnt<kLoadsPerTile>();
      else wait_vmcnt<0>();
      __syncthreads();
      if (tn + 3 < ntiles) {
        l_item = advance_item(m, a.num_items, l_item, l_tile);
        issue_tile<NW>(a, m, tile_info(m, l_item, l_tile), bufs[(tn + 3) & 3], wave, lane);
        ++l_tile;
      }
      LDS_PTR(char) buf = bufs[tn & 3];
      const int tok0 = tok_first + static_cast<int>(tt - seg_begin) * kTile;

      if (wave_active) {
        // S^T = K Q^T  (32 tokens x 32 heads)
        f32x16 s = {};
#pragma unroll
        for (int k = 0; k < kKSteps; ++k) {
          const int off = koff[k & 3] + ((2 * k) & ~7) * 16;
          const i16x8 kv = *reinterpret_cast<LDS_PTR(const i16x8)>(buf + off);
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kv), qf[k], s, 0, 0, 0);
        }

        // mask + scale (log2 domain), tile max per head
        float tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int tok = tok0 + 8 * (i >> 2) + 4 * g + (i & 3);
          const float v = (tok >= vlo && tok < vhi) ? s[i] * a.scale_log2 : -INFINITY;
          s[i] = v;
          tmax = fmaxf(tmax, v);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        // The reference maximum is fixed by the segment's first tile; later
        // tiles may exceed it by up to kRefSlack (probabilities <= 2^kRefSlack,
        // far inside fp32 and bf16 range).  A larger jump marks this workgroup's
        // range for recomputation by the plain kernel (rare; never silently wrong).
        if (tt == seg_begin) m_ref = tmax;
        else if (tmax > m_ref + kRefSlack) overflow = true;
        bf16x8 pb[2];
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(s[i] - m_ref);
          psum += p;
          pb[i >> 3][i & 7] = static_cast<__bf16>(p);
        }
        l_sum += psum;

        // O^T += V^T P^T : 16 dim tiles x 2 token steps
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int mt = 0; mt < kMTiles; ++mt) {
            const int off = ((mt & 1) ? voff_odd : voff_even) + 128 * (mt >> 1) + kRowBytes * 16 * j;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                reinterpret_cast<LDS_PTR(i16x4)>(buf + off));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                reinterpret_cast<LDS_PTR(i16x4)>(buf + off + 8 * kRowBytes));
            const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v), pb[j],
                                                               acc[mt], 0, 0, 0);
          }
        }
      }
    }
    ctile = seg_end;

    // ---- segment done: write the unnormalised accumulator, lse and 1/l ----
    // (no arithmetic on the accumulator registers: consumers apply 1/l)
    const float l_tot = wave_active ? l_sum + __shfl_xor(l_sum, 32, 64) : 1.f;
    const bool complete = (seg_begin == item_ts) && (seg_end == item_te);
    float* o_dst;
    float* lse_dst;
    float* scl_dst;
    if (complete) {
      o_dst = a.o_lat + (static_cast<int64_t>(c_item) * a.H) * kR;
      lse_dst = a.lse + static_cast<int64_t>(c_item) * a.H;
      scl_dst = a.o_scale + static_cast<int64_t>(c_item) * a.H;
    } else {
      const int64_t slot = (item_ts < t0) ? 2 * wg : 2 * wg + 1;
      o_dst = a.part_o + (slot * a.H) * kR;
      lse_dst = a.part_lse + slot * a.H;
      scl_dst = a.part_scale + slot * a.H;
    }
    if (wave_active && head_ok) {
      float* orow = o_dst + static_cast<int64_t>(head) * kR;
#pragma unroll
      for (int mt = 0; mt < kMTiles; ++mt) {
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const f32x4 v = {acc[mt][4 * a4 + 0], acc[mt][4 * a4 + 1], acc[mt][4 * a4 + 2],
                           acc[mt][4 * a4 + 3]};
          *reinterpret_cast<f32x4*>(orow + 32 * mt + 8 * a4 + 4 * g) = v;
        }
      }
      if (g == 0) {
        lse_dst[head] = (m_ref + log2f(l_tot)) * kLn2;
        scl_dst[head] = 1.0f / l_tot;
      }
    }
  }
  if (__any(overflow) && lane == 0) wg_overflow = 1;
  __syncthreads();
  if (threadIdx.x == 0) a.redo[wg] = wg_overflow;
}

}  // namespace

bool mfma_attn_supported(const CacheView& kv, int32_t H) {
  return kv.dtype == kKvBf16 && kv.R == kR && kv.Dr == kD - kR && H >= 1 && H <= 128;
}

hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(attn_mfma_kernel<4>, dim3(a.G), dim3(256), 0, s, a, a.item_b, a.item_lo,
                     a.item_hi, a.tile_start, a.block_tables);
  return hipGetLastError();
}

}  // namespace mla
