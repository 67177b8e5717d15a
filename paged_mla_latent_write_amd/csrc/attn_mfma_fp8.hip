// Split-KV paged latent attention over an fp8 (E4M3) latent cache on CDNA4
// matrix cores (gfx950), for the MLA latent shape kv_lora_rank 512 +
// qk_rope 64 with up to 128 query heads.
//
// What it computes is the bf16 kernel's (attn_mfma.hip) with the cache read as
// dequantised values: token t holds E4M3 codes x_t[0..575] and one fp32 scale
// s_t ("[Models] Support MLA_SWA functionality", Modifications: a uint8 MLA
// cache; "[unified-memory] Let Kimi-Linear use the paged MLA attention
// backends", Validation: fp8_e4m3), value = e4m3(x_t) * s_t.  Every E4M3 value
// is exact in bf16, so the codes are converted to bf16 unscaled and the scale
// is applied where it is linear:
//   score_t = s_t * (q . e4m3(x_t)),   o += (P_t * s_t) e4m3(c_t).
//
// Design (one workgroup of four waves per compute unit, wave w owns heads
// [32w, 32w + 32), as in the bf16 kernel):
//  * a 32-token tile is 18 KiB of codes + 128 B of scales.  It is copied
//    HBM -> LDS with global_load_lds (no VGPR staging) into one of four
//    staging buffers, two tiles ahead of the compute: five copies per wave
//    (18 of codes, one of scales that waves 2 and 3 both issue).
//  * one step later the whole workgroup converts the staged codes once into a
//    bf16 tile (the layout and swizzle of the bf16 kernel's tiles), so the
//    four waves do not each convert the keys they all read.  Two bf16 tiles
//    alternate: tile t + 1 is converted during tile t's values step, between
//    its MFMAs (each lane its five 16-code chunks, destinations from a table
//    in LDS), and published by the barrier that starts step t + 1.
//  * S^T = K Q^T and O^T += V^T P^T run on v_mfma_f32_32x32x16_bf16 as two
//    hand-scheduled blocks per tile (attn_mfma_fp8_asm.inc, generated): K and
//    V^T fragments (ds_read_b128, ds_read_b64_tr_b16) stream through a ring of
//    registers a few MFMAs ahead, Q and the 512 x 32 accumulator sit in the
//    registers the bf16 kernel reserves for them (the compiler is limited to
//    the rest); the scales and the softmax run in C++ between the blocks.
//  * online softmax in base 2 against a reference maximum fixed by each
//    segment's first tile, so the accumulators are never rescaled (the blocks
//    hold no rescale step).  Probabilities up to 2^64 stay far inside fp32; a
//    score beyond that flags the workgroup, whose range the generic kernel
//    then recomputes exactly (redo).
#include <math.h>

#include "device_utils.h"
#include "mla_internal.h"

namespace mla {
namespace {

// Q (v62-v205), the accumulators (a0-a255) and the register ring: load_q,
// zero_q and store_acc from the bf16 kernel's blocks, and the fp8 kernel's own
// scores and values blocks
#include "attn_mfma_asm.inc"
#include "attn_mfma_fp8_asm.inc"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kR = 512;
constexpr int kD = 576;
constexpr int kRowBytes = kD * 2;              // 1152: one bf16 row in LDS
constexpr int kTileBytes = kTile * kRowBytes;  // 36864
constexpr int kCodeRow = kD;                   // 576: one fp8 row
constexpr int kCodeBytes = kTile * kCodeRow;   // 18432
constexpr int kStageBytes = kCodeBytes + 4 * kTile;  // codes + 32 fp32 scales
constexpr int kCodeChunks = kCodeBytes / 16;   // 1152 16-byte chunks
constexpr int kCopies = 5;                     // copy instructions per wave per tile
constexpr float kSlack = 64.0f;                // reference slack (log2 units)

#define LDS_PTR(T) __attribute__((address_space(3))) T*
#define CONST_PTR(T) const __attribute__((address_space(4))) T*

// the bf16 kernel's chunk swizzle (attn_mfma.hip): the tiles this kernel
// converts must have its layout, since the fragment reads are the same
__device__ __forceinline__ int swz(int t) {
  return (((t >> 1) & 1) << 2) ^ ((t >> 2) & 1) ^ (((t >> 3) & 1) << 1);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  constexpr int n = N > 63 ? 63 : N;
  __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// 16-byte copy HBM -> LDS: lane i's bytes land at lds_base + 16 i (inactive
// lanes copy nothing).  Inline assembly keeps the compiler from draining the
// copies with conservative waits; the kernel waits explicitly.
__device__ __forceinline__ void lds_dma_16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(gptr)
               : "memory", "m0");
}

struct Meta {
  CONST_PTR(int32_t) item_b;
  CONST_PTR(int32_t) item_lo;
  CONST_PTR(int32_t) item_hi;
  CONST_PTR(int32_t) tile_start;
  CONST_PTR(int32_t) block_tables;
};

__device__ __forceinline__ int advance_item(const Meta& m, int num_items, int item, int64_t tile) {
  while (item + 1 < num_items && m.tile_start[item + 1] <= tile) ++item;
  return item;
}

// Copy tile `tile` (owned by `item`) into a staging buffer: codes chunk c
// (token c / 36, bytes 16 (c % 36)) at byte 16 c, the 32 scales after them.
// Tokens outside the visible range load a clamped (valid) token's codes; their
// scores are masked and their scales zeroed before use.
__device__ __forceinline__ void copy_tile(const AttnArgs& a, const Meta& m, int item, int64_t tile,
                                          uint32_t stage, int wave, int lane_in) {
  // (an opaque copy of the lane index: the per-lane address arithmetic below is
  // then recomputed per tile rather than hoisted out of the tile loop, where it
  // would hold ~15 registers)
  int lane = lane_in;
  asm volatile("" : "+v"(lane));
  const int b = m.item_b[item];
  const int vlo = m.item_lo[item], vhi = m.item_hi[item];
  const int tok0 = ((vlo >> 5) + static_cast<int>(tile - m.tile_start[item])) * kTile;
  CONST_PTR(int32_t) bt = m.block_tables + static_cast<int64_t>(b) * a.max_blocks;
  const int ps = a.kv.page_size;
  const int psh = a.kv.page_shift;
  const unsigned last_page = static_cast<unsigned>(a.kv.num_pages - 1);
  // one page for page sizes >= 32, two of 16 (the second read only if it holds
  // a visible token: the block table is read up to ceil(n / ps) entries)
  const int blk0 = tok0 >> psh;
  const unsigned pg0 = min(static_cast<unsigned>(bt[blk0]), last_page);
  unsigned pg1 = pg0;
  if (ps < kTile && tok0 + ps < vhi) pg1 = min(static_cast<unsigned>(bt[blk0 + 1]), last_page);
  const char* codes = static_cast<const char*>(a.kv.data);
#pragma unroll
  for (int k = 0; k < kCopies - 1; ++k) {
    const int s = wave + 4 * k;  // slots 0..15
    const int c = 64 * s + lane;
    const int t = c / 36, p = c - 36 * (c / 36);
    int pos = tok0 + t;
    pos = pos < vlo ? vlo : pos;
    pos = pos >= vhi ? vhi - 1 : pos;
    const int in_page = pos - (blk0 << psh);
    const unsigned pg = in_page >= ps ? pg1 : pg0;
    const int off = in_page >= ps ? in_page - ps : in_page;
    lds_dma_16(codes + ((static_cast<int64_t>(pg) << psh) + off) * kCodeRow + 16 * p, stage + 1024 * s);
  }
  if (wave < 2) {  // slots 16, 17
    const int s = 16 + wave;
    const int c = 64 * s + lane;
    const int t = c / 36, p = c - 36 * (c / 36);
    int pos = tok0 + t;
    pos = pos < vlo ? vlo : pos;
    pos = pos >= vhi ? vhi - 1 : pos;
    const int in_page = pos - (blk0 << psh);
    const unsigned pg = in_page >= ps ? pg1 : pg0;
    const int off = in_page >= ps ? in_page - ps : in_page;
    lds_dma_16(codes + ((static_cast<int64_t>(pg) << psh) + off) * kCodeRow + 16 * p, stage + 1024 * s);
  } else if (lane < 8) {
    // scales of tokens 4 lane .. 4 lane + 3 (one page: 4 | ps), issued by waves
    // 2 and 3 alike so that every wave has five copies per tile
    const int in_page = tok0 + 4 * lane - (blk0 << psh);
    const unsigned pg = in_page >= ps ? pg1 : pg0;
    const int off = in_page >= ps ? in_page - ps : in_page;
    lds_dma_16(a.kv.scale + (static_cast<int64_t>(pg) << psh) + off, stage + kCodeBytes);
  }
}

// Convert a staged tile's codes into a bf16 tile (row t: 72 chunks of 8
// values, chunk j at slot (j & ~7) | ((j & 7) ^ swz(t))).  Thread i handles
// 16-code chunks i, i + 256, ...
__device__ __forceinline__ void convert_tile(LDS_PTR(const char) stage, LDS_PTR(char) tile) {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));  // (not hoisted out of the tile loop, as in copy_tile)
  for (int c = tid; c < kCodeChunks; c += 256) {
    const int t = c / 36, m2 = c - 36 * (c / 36);
    const i32x4 v = *reinterpret_cast<LDS_PTR(const i32x4)>(stage + 16 * c);
    bf16x8 lo, hi;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const bf16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[w], 1.0f, false);
      const bf16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[w], 1.0f, true);
      lo[4 * w] = a0[0]; lo[4 * w + 1] = a0[1]; lo[4 * w + 2] = a1[0]; lo[4 * w + 3] = a1[1];
      const bf16x2 b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[w + 2], 1.0f, false);
      const bf16x2 b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[w + 2], 1.0f, true);
      hi[4 * w] = b0[0]; hi[4 * w + 1] = b0[1]; hi[4 * w + 2] = b1[0]; hi[4 * w + 3] = b1[1];
    }
    const int j0 = 2 * m2, j1 = 2 * m2 + 1;
    const int p0 = (j0 & ~7) | ((j0 & 7) ^ swz(t)), p1 = (j1 & ~7) | ((j1 & 7) ^ swz(t));
    *reinterpret_cast<LDS_PTR(bf16x8)>(tile + t * kRowBytes + 16 * p0) = lo;
    *reinterpret_cast<LDS_PTR(bf16x8)>(tile + t * kRowBytes + 16 * p1) = hi;
  }
}

__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_num_vgpr(kCompilerVgprs))) void attn_mfma_fp8_kernel(
    AttnArgs a, const int32_t* __restrict__ item_b, const int32_t* __restrict__ item_lo,
    const int32_t* __restrict__ item_hi, const int32_t* __restrict__ tile_start,
    const int32_t* __restrict__ block_tables) {
  const Meta m{(CONST_PTR(int32_t))item_b, (CONST_PTR(int32_t))item_lo, (CONST_PTR(int32_t))item_hi,
               (CONST_PTR(int32_t))tile_start, (CONST_PTR(int32_t))block_tables};
  __shared__ __attribute__((aligned(1024))) char lds_tile[2][kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_stage[4][kStageBytes];
  // this thread's five conversion chunks (see convert_tile): entry j holds the
  // two 16-byte destinations of chunk tid + 256 j in a bf16 tile (low and high
  // 16 bits); a thread with no fifth chunk repeats its fourth
  __shared__ __attribute__((aligned(16))) uint32_t conv_tab[256][8];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5;
  const int n32 = lane & 31;
  const int head = wave * 32 + n32;
  const bool head_ok = head < a.H;
  const bool wave_active = wave * 32 < a.H;

  const int64_t wg = blockIdx.x;
  const int64_t t0 = a.wg_tile[wg], t1 = a.wg_tile[wg + 1];
  __shared__ int wg_overflow;
  if (threadIdx.x == 0) wg_overflow = 0;
  if (t0 >= t1) {
    if (threadIdx.x == 0) a.redo[wg] = 0;
    return;
  }
  bool overflow = false;
  const int ntiles = static_cast<int>(t1 - t0);
  const int first_item = advance_item(m, a.num_items, a.wg_item[wg], t0);

  LDS_PTR(char) tiles[2];
  LDS_PTR(char) stages[4];
  tiles[0] = (LDS_PTR(char))(&lds_tile[0][0]);
  tiles[1] = (LDS_PTR(char))(&lds_tile[1][0]);
#pragma unroll
  for (int u = 0; u < 4; ++u) stages[u] = (LDS_PTR(char))(&lds_stage[u][0]);
  auto stage_addr = [&](int u) { return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(stages[u & 3])); };

  // lane-constant LDS offsets (as in the bf16 kernel)
  const int y = g ^ swz(n32);
  int koff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) koff[j] = n32 * kRowBytes + (((2 * j) ^ y) << 4);
  const int q = lane >> 4, jj = lane & 15, rr = jj >> 2, c4 = jj & 3;
  const int xs = (2 * (q & 1) + (c4 >> 1)) ^ (4 * (rr >> 1)) ^ g;
  const int vbase = (4 * g + rr) * kRowBytes + 8 * (c4 & 1);
  const int voff_even = vbase + (xs << 4);
  const int voff_odd = vbase + ((4 ^ xs) << 4);
  const int voff_even_h = vbase + 8 * kRowBytes + ((2 ^ xs) << 4);
  const int voff_odd_h = vbase + 8 * kRowBytes + ((6 ^ xs) << 4);

  // ---- copy cursor: tiles 0, 1, 2 ahead of the loop ----
  int l_item = first_item;
  int64_t l_tile = t0;
  auto copy_next = [&](int slot) {
    l_item = advance_item(m, a.num_items, l_item, l_tile);
    copy_tile(a, m, l_item, l_tile, stage_addr(slot), wave, lane);
    ++l_tile;
  };
  for (int p = 0; p < 3; ++p)
    if (p < ntiles) copy_next(p);
  // tile 0 landed (the copies of tiles 1 and 2 may still be in flight)
  if (ntiles >= 3) wait_vmcnt<2 * kCopies>();
  else if (ntiles == 2) wait_vmcnt<kCopies>();
  else wait_vmcnt<0>();
  __syncthreads();
  convert_tile(stages[0], tiles[0]);
  {
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      int c = tid + 256 * j;
      if (c >= kCodeChunks) c -= 256;
      const int t = c / 36, m2 = c - 36 * (c / 36);
      const int j0 = 2 * m2, j1 = 2 * m2 + 1;
      const int p0 = (j0 & ~7) | ((j0 & 7) ^ swz(t)), p1 = (j1 & ~7) | ((j1 & 7) ^ swz(t));
      conv_tab[tid][j] = static_cast<uint32_t>(t * kRowBytes + 16 * p0) |
                         (static_cast<uint32_t>(t * kRowBytes + 16 * p1) << 16);
    }
  }

  zero_q();  // lanes of heads >= H keep zero queries

  int tn = 0;
  int c_item = first_item;
  int64_t ctile = t0;
  while (ctile < t1) {
    c_item = advance_item(m, a.num_items, c_item, ctile);
    const int64_t item_ts = m.tile_start[c_item], item_te = m.tile_start[c_item + 1];
    const int64_t seg_begin = ctile;
    const int64_t seg_end = item_te < t1 ? item_te : t1;
    // the item's queries (waits for every copy in flight too)
    if (wave_active && head_ok)
      load_q(a.q_lat + c_item * a.q_lat_st + head * a.q_lat_sh + 8 * g,
             a.q_pe + c_item * a.q_pe_st + head * a.q_pe_sh + 8 * g);
    float m_ref = 0.f, l_sum = 0.f;
    const int vlo = m.item_lo[c_item], vhi = m.item_hi[c_item];
    const int tok_first = ((vlo >> 5) + static_cast<int>(seg_begin - item_ts)) * kTile;

    for (int64_t tt = seg_begin; tt < seg_end; ++tt, ++tn) {
      // tile tn + 1 has landed once at most the copies of tile tn + 2 remain
      if (tn + 2 < ntiles) wait_vmcnt<kCopies>();
      else wait_vmcnt<0>();
      __syncthreads();  // tile tn + 1 staged; tile tn converted; buffers of tn - 1 free
      if (tn + 3 < ntiles) copy_next(tn + 3);
      // the next tile's conversion: inside this tile's values step (below)
      // in the waves that compute, here in the others
      const bool conv_next = tn + 1 < ntiles;
      if (conv_next && !wave_active) convert_tile(stages[(tn + 1) & 3], tiles[(tn + 1) & 1]);
      LDS_PTR(char) buf = tiles[tn & 1];
      LDS_PTR(const float) scl = (LDS_PTR(const float))(stages[tn & 3] + kCodeBytes);
      const int tok0 = tok_first + static_cast<int>(tt - seg_begin) * kTile;

      if (wave_active) {
        const uint32_t bbase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(buf));
        const uint32_t kcur[4] = {bbase + static_cast<uint32_t>(koff[0]), bbase + static_cast<uint32_t>(koff[1]),
                                  bbase + static_cast<uint32_t>(koff[2]), bbase + static_cast<uint32_t>(koff[3])};
        float s[16];
        fp8_scores(kcur, s);
        // per-token scale, mask, scale to log2 units; P * s_t as bf16 pairs
        // (element i of the lane's 16 is the low half of pair i / 2 when i is
        // even), the B operand of the values MFMAs.  The scales are read again
        // rather than held across the exponentials.  Tokens outside the
        // visible range (only in a tile that is not wholly inside it) get a
        // score of -inf and a scale of zero: their staged scale may be anything.
        const bool partial = !(tok0 >= vlo && tok0 + kTile <= vhi);  // uniform
        float tmax = -INFINITY;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x4 sv = *reinterpret_cast<LDS_PTR(const f32x4)>(scl + 8 * i4 + 4 * g);
#pragma unroll
          for (int e = 0; e < 4; ++e) s[4 * i4 + e] *= sv[e] * a.scale_log2;
        }
        if (partial) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int tok = tok0 + 8 * (i >> 2) + 4 * g + (i & 3);
            if (tok < vlo || tok >= vhi) s[i] = -INFINITY;
          }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[i]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        if (tt == seg_begin) m_ref = tmax;
        else if (tmax > m_ref + kSlack) overflow = true;
        uint32_t pb[8];
        float psum = 0.f;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          f32x4 sv = *reinterpret_cast<LDS_PTR(const f32x4)>(scl + 8 * i4 + 4 * g);
          if (partial) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int tok = tok0 + 8 * i4 + 4 * g + e;
              if (tok < vlo || tok >= vhi) sv[e] = 0.f;
            }
          }
#pragma unroll
          for (int e = 0; e < 4; e += 2) {
            const int i = 4 * i4 + e;
            const float p0 = __builtin_amdgcn_exp2f(s[i] - m_ref);
            const float p1 = __builtin_amdgcn_exp2f(s[i + 1] - m_ref);
            psum += p0 + p1;
            const bf16x2 pk = {static_cast<__bf16>(p0 * sv[e]), static_cast<__bf16>(p1 * sv[e + 1])};  // RNE
            pb[i >> 1] = __builtin_bit_cast(uint32_t, pk);
          }
        }
        l_sum += psum;
        const uint32_t vcur[4] = {bbase + static_cast<uint32_t>(voff_even), bbase + static_cast<uint32_t>(voff_odd),
                                  bbase + static_cast<uint32_t>(voff_even_h),
                                  bbase + static_cast<uint32_t>(voff_odd_h)};
        if (conv_next) {
          const uint32_t tid = threadIdx.x;
          const uint32_t cs = stage_addr(tn + 1) + 16 * tid;
          const uint32_t cs4 = cs + (tid < kCodeChunks - 1024 ? 16384u : 12288u);
          const uint32_t ct = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&conv_tab[0][0])) + 32 * tid;
          const uint32_t tb = __builtin_amdgcn_readfirstlane(
              static_cast<uint32_t>(reinterpret_cast<uintptr_t>(tiles[(tn + 1) & 1])));
          if (tt == seg_begin) fp8_values_conv_f1(vcur, pb, cs, cs4, ct, tb);
          else fp8_values_conv_f0(vcur, pb, cs, cs4, ct, tb);
        } else {
          if (tt == seg_begin) fp8_values_f1(vcur, pb);
          else fp8_values_f0(vcur, pb);
        }
      }
    }
    ctile = seg_end;

    // ---- segment done: the unnormalised accumulator, lse and 1/l ----
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
      store_acc(o_dst + static_cast<int64_t>(head) * kR + 4 * g);
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

bool mfma_fp8_attn_supported(const CacheView& kv, int32_t H) {
  return kv.dtype == kKvFp8 && kv.R == kR && kv.Dr == kD - kR && H >= 1 && H <= 128 && kv.page_size >= 16;
}

hipError_t launch_attn_mfma_fp8(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(attn_mfma_fp8_kernel, dim3(a.G), dim3(256), 0, s, a, a.item_b, a.item_lo, a.item_hi,
                     a.tile_start, a.block_tables);
  return hipGetLastError();
}

}  // namespace mla
