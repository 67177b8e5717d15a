// Split-KV paged latent attention over an fp8 (E4M3) latent cache on CDNA4
// matrix cores (gfx950), for the MLA latent shape kv_lora_rank 512 +
// qk_rope 64 with up to 128 query heads and pages of at least 16 tokens.
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
//  * a 32-token tile is 18 KiB of codes + 128 B of scales.  Lane i of the
//    workgroup copies the tile's 16-byte code chunks i, i + 256, ... HBM ->
//    LDS (global_load_lds, no VGPR staging) into one of two staging buffers,
//    three tiles ahead of the compute, so that wave w fills the 1 KiB spans
//    w, w + 4, ... of the buffer.  The wave alone converts its spans to bf16
//    (exact), lane l taking the span's 8-byte halves l and 64 + l, so a
//    staging buffer is refilled as soon as its owner wave has read it, with
//    no barrier, and the conversion's LDS reads and writes are free of bank
//    conflicts.  Waves 2 and 3 copy the scales into one of four 1 KiB scale
//    slots (lanes 8-63 repeat lanes 0-7 into the slot's pad).
//  * three bf16 tile buffers (the bf16 kernel's layout and swizzle): step n
//    reads the keys of tile n and the values of tile n - 1 and writes tile
//    n + 1, which the barrier ending the step publishes.
//  * each step is one generated block (attn_mfma_fp8_asm.inc): S^T = K Q^T of
//    tile n on v_mfma_f32_32x32x16_bf16 with the conversion of tile n + 1 and
//    the copies of tile n + 3 between its MFMAs, then O^T += V^T P^T of tile
//    n - 1 with the softmax of tile n (per-token scales, mask, reference
//    maximum, exp2, P * s_t rounded to bf16) between its MFMAs.  Q and the
//    512 x 32 accumulator sit in registers the compiler does not allocate.
//  * online softmax in base 2 against a reference maximum that moves up (with
//    a rescale of the accumulators) only when a tile's maximum passes it by
//    more than 16: the accumulators are rarely rescaled.
// With pages of 16 tokens a tile spans two pages, and the copies are issued
// by the C++ code after each block instead of inside it.
#include <math.h>

#include "device_utils.h"
#include "mla_internal.h"

namespace mla {
namespace {

// Operands of one tile step's block.
struct Fp8Step {
  uint32_t cs;      // tile n + 1's codes: staging buffer + 1024 wave + 8 lane (first span, half 0)
  uint32_t cs4;     // the same in the wave's fifth span (its fourth again when it has none)
  uint32_t ct;      // this lane's row of the conversion table
  uint32_t sc;      // tile n's scale slot + 16 g
  uint32_t cp;      // 1: the block issues the copies of tile n + 3
  uint32_t m0b;     // LDS destination of the first code copy (+ 4 KiB per copy)
  uint32_t m04;     // LDS destination of the fifth copy
  const char* sb;   // the copied tile's first code row
  const char* sb4;  // base of the fifth copy (codes, or the tile's 32 scales)
  uint32_t o0;      // this lane's byte offset from sb of its first chunk (16 tid)
  uint32_t o4;      // and of its fifth copy from sb4
};

// Q (v62-v205), the accumulators (a0-a255), the register ring: load_q,
// zero_q, store_acc, rescale_acc and tile_prefetch_k from the bf16 kernel's
// blocks, and the fp8 kernel's tile blocks
#include "attn_mfma_asm.inc"
#include "attn_mfma_fp8_asm.inc"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kR = 512;
constexpr int kD = 576;
constexpr int kRowBytes = kD * 2;              // 1152: one bf16 row in LDS
constexpr int kTileBytes = kTile * kRowBytes;  // 36864
constexpr int kCodeRow = kD;                   // 576: one fp8 row
constexpr int kCodeBytes = kTile * kCodeRow;   // 18432
constexpr int kCodeChunks = kCodeBytes / 16;   // 1152 16-byte chunks
constexpr int kCopies = 5;                     // copy instructions per wave per tile
constexpr int kScaleSlot = 1024;               // 64 lanes x 16 B (the first 128 B are the tile's)

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

// 16-byte copy HBM -> LDS: lane i's bytes land at lds_base + 16 i.  Inline
// assembly keeps the compiler from draining the copies with conservative
// waits; the kernel waits explicitly.
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

// Where a tile's rows are: its first token, the item's visible range, and
// the pages of its first and (pages of 16 tokens) second half.
struct TileLoc {
  int tok0, vlo, vhi;
  unsigned pg0, pg1;
};

__device__ __forceinline__ TileLoc locate(const AttnArgs& a, const Meta& m, int item, int64_t tile) {
  TileLoc L;
  const int b = m.item_b[item];
  L.vlo = m.item_lo[item];
  L.vhi = m.item_hi[item];
  L.tok0 = ((L.vlo >> 5) + static_cast<int>(tile - m.tile_start[item])) * kTile;
  CONST_PTR(int32_t) bt = m.block_tables + static_cast<int64_t>(b) * a.max_blocks;
  const unsigned last_page = static_cast<unsigned>(a.kv.num_pages - 1);
  const int blk0 = L.tok0 >> a.kv.page_shift;
  L.pg0 = min(static_cast<unsigned>(bt[blk0]), last_page);
  L.pg1 = L.pg0;
  // (the second entry is read only if it holds a visible token: the block
  // table is read up to ceil(n / page_size) entries)
  if (a.kv.page_size < kTile && L.tok0 + a.kv.page_size < L.vhi)
    L.pg1 = min(static_cast<unsigned>(bt[blk0 + 1]), last_page);
  return L;
}

// Token and byte of this lane's copy k: chunk c = tid + 256 k is token c / 36,
// bytes 16 (c % 36).  Tokens outside the visible range load a visible token's
// codes (clamped); their scores are masked and their P * s_t zeroed.
__device__ __forceinline__ int clamp_tok(const TileLoc& L, int t) {
  int pos = L.tok0 + t;
  pos = pos < L.vlo ? L.vlo : pos;
  return pos >= L.vhi ? L.vhi - 1 : pos;
}

// This lane's five copies of a tile (any page size): codes into its chunks of
// the staging buffer, or (waves 2 and 3, fifth copy) the 32 scales into the
// scale slot.
__device__ __forceinline__ void copy_tile(const AttnArgs& a, const TileLoc& L, uint32_t stage, uint32_t sslot,
                                          int wave, int tid_in) {
  // (an opaque copy of the thread index: the address arithmetic below is then
  // recomputed per tile rather than hoisted out of the tile loop)
  int tid = tid_in;
  asm volatile("" : "+v"(tid));
  const int ps = a.kv.page_size;
  const int psh = a.kv.page_shift;
  const int blk0 = L.tok0 >> psh;
  const char* codes = static_cast<const char*>(a.kv.data);
  // (one copy at a time: few registers live, the compiler has only v0-v53)
#pragma unroll 1
  for (int k = 0; k < kCopies; ++k) {
    if (k == kCopies - 1 && wave >= 2) break;
    const int c = tid + 256 * k;
    const int t = c / 36, p = c - 36 * (c / 36);
    const int in_page = clamp_tok(L, t) - (blk0 << psh);
    const unsigned pg = in_page >= ps ? L.pg1 : L.pg0;
    const int off = in_page >= ps ? in_page - ps : in_page;
    lds_dma_16(codes + ((static_cast<int64_t>(pg) << psh) + off) * kCodeRow + 16 * p,
               stage + 1024 * (k < 4 ? wave + 4 * k : 16 + wave));
  }
  if (wave >= 2) {
    // scales of tokens 4 (lane % 8) .. + 3 (one page: 4 | page size)
    const int in_page = L.tok0 + 4 * (tid & 7) - (blk0 << psh);
    const unsigned pg = in_page >= ps ? L.pg1 : L.pg0;
    const int off = in_page >= ps ? in_page - ps : in_page;
    lds_dma_16(a.kv.scale + (static_cast<int64_t>(pg) << psh) + off, sslot);
  }
}

// Wave-uniform values as the scalar operands of the blocks.
// (the builtin returns int: each half goes through uint32_t before it is
// widened, or a low half with bit 31 set would sign-extend over the high one)
__device__ __forceinline__ uint32_t uni(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(v));
}
__device__ __forceinline__ const char* uni(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = uni(static_cast<uint32_t>(v));
  const uint64_t hi = uni(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const char*>(lo | (hi << 32));
}

// The same copies as operands of a block, for a tile that lies in one page
// (pages of at least one tile) and wholly inside its item's visible range:
// this lane's chunk k is at sb + 16 (tid + 256 k).
__device__ __forceinline__ void copy_desc(Fp8Step& f, const AttnArgs& a, const TileLoc& L, uint32_t stage,
                                          uint32_t sslot, int wave) {
  const int64_t row0 = (static_cast<int64_t>(L.pg0) << a.kv.page_shift) + (L.tok0 & (a.kv.page_size - 1));
  f.sb = uni(static_cast<const char*>(a.kv.data) + row0 * kCodeRow);
  f.sb4 = wave < 2 ? f.sb : uni(a.kv.scale + row0);
  f.m0b = uni(stage + 1024 * wave);
  f.m04 = uni(wave < 2 ? stage + 1024 * (16 + wave) : sslot);
}

// Convert this lane's chunks of a staged tile (chunk c = tid + 256 j) into the
// bf16 tile: row t holds 72 chunks of 8 values, chunk j at slot
// (j & ~7) | ((j & 7) ^ swz(t)).
__device__ __forceinline__ void convert_own(uint32_t stage, uint32_t tile, int tid_in) {
  int tid = tid_in;
  asm volatile("" : "+v"(tid));
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
  __shared__ __attribute__((aligned(1024))) char lds_tile[3][kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_stage[2][kCodeBytes];
  __shared__ __attribute__((aligned(1024))) char lds_scale[4][kScaleSlot];
  // thread i's entry j: the 16-byte destinations in a bf16 tile (low and
  // high 16 bits) of the 8-byte halves lane and 64 + lane of its wave's span
  // j; the waves with no fifth span repeat their fourth
  __shared__ __attribute__((aligned(16))) uint32_t conv_tab[256 * 5];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int n32 = lane & 31;
  const int head = wave * 32 + n32;
  const bool head_ok = head < a.H;
  // with fewer than 128 heads the surplus waves still copy and convert their
  // chunks of every tile, but skip the arithmetic
  const bool wave_active = wave * 32 < a.H;

  // consecutive ranges (which mostly share an item, and so its queries) run
  // on the same XCD
  const int64_t wg = (gridDim.x & 7) == 0 ? (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3)
                                          : blockIdx.x;
  const int64_t t0 = a.wg_tile[wg], t1 = a.wg_tile[wg + 1];
  if (t0 >= t1) return;
  const int ntiles = static_cast<int>(t1 - t0);
  const int first_item = advance_item(m, a.num_items, a.wg_item[wg], t0);
  const bool direct = a.kv.page_size >= kTile;  // a tile lies in one page
  // this lane's offsets of its first chunk and of its fifth copy (codes, or
  // waves 2 and 3: the scales, lane % 8 repeating over the slot's pad)
  const uint32_t o0 = 16 * tid;
  const uint32_t o4 = wave < 2 ? 16 * (tid + 1024) : 16 * (tid & 7);
  // this lane's first code half in a staging buffer, for the conversion
  const uint32_t cofs = 1024 * wave + 8 * lane;

  const uint32_t tile_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&lds_tile[0][0]));
  const uint32_t stage_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&lds_stage[0][0]));
  const uint32_t scale_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&lds_scale[0][0]));
  auto tbuf = [&](int i) { return tile_base + static_cast<uint32_t>(i * kTileBytes); };
  auto stage = [&](int n) { return stage_base + static_cast<uint32_t>((n & 1) * kCodeBytes); };
  auto sslot = [&](int n) { return scale_base + static_cast<uint32_t>((n & 3) * kScaleSlot); };

  // lane-constant LDS offsets (as in the bf16 kernel)
  const int y = g ^ swz(n32);
  uint32_t koff[4], kcur[4], voff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) koff[j] = n32 * kRowBytes + (((2 * j) ^ y) << 4);
  {
    const int q = lane >> 4, jj = lane & 15, rr = jj >> 2, c4 = jj & 3;
    const int xs = (2 * (q & 1) + (c4 >> 1)) ^ (4 * (rr >> 1)) ^ g;
    const int vbase = (4 * g + rr) * kRowBytes + 8 * (c4 & 1);
    voff[0] = vbase + (xs << 4);
    voff[1] = vbase + ((4 ^ xs) << 4);
    voff[2] = vbase + 8 * kRowBytes + ((2 ^ xs) << 4);
    voff[3] = vbase + 8 * kRowBytes + ((6 ^ xs) << 4);
  }

  // ---- copy cursor: tile tn + 3 is copied in step tn; past the range's end
  // the last tile is copied again (so that every step has five copies per
  // wave, and the waits count the same) ----
  int l_item = first_item;
  int64_t l_tile = t0;
  auto next_loc = [&]() {
    const int64_t tile = l_tile < t1 ? l_tile : t1 - 1;
    l_item = advance_item(m, a.num_items, l_item, tile);
    ++l_tile;
    return locate(a, m, l_item, tile);
  };
  {
    const TileLoc L0 = next_loc();
    copy_tile(a, L0, stage(0), sslot(0), wave, tid);
    const TileLoc L1 = next_loc();
    copy_tile(a, L1, stage(1), sslot(1), wave, tid);
  }
  // (half u of the tile -- bytes 8u.. of the codes -- is bf16 chunk u % 72 of
  // row u / 72, at its swizzled slot)
  auto half_dest = [](int u) {
    const int t = u / 72, jc = u - 72 * (u / 72);
    const int p = (jc & ~7) | ((jc & 7) ^ swz(t));
    return static_cast<uint32_t>(t * kRowBytes + 16 * p);
  };
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    const int span = j < 4 ? wave + 4 * j : (wave < 2 ? 16 + wave : wave + 12);
    const int u = 128 * span + lane;
    conv_tab[tid * 5 + j] = half_dest(u) | (half_dest(u + 64) << 16);
  }
  wait_vmcnt<kCopies>();  // this lane's chunks of tile 0 (and the scales) have landed
  convert_own(stage(0), tbuf(0), tid);
  {
    const TileLoc L2 = next_loc();  // (after this lane's reads of tile 0's chunks)
    copy_tile(a, L2, stage(2), sslot(2), wave, tid);
  }
  __syncthreads();  // tile 0 converted, its scales in place
  zero_q();         // lanes of heads >= H keep zero queries
  if (wave_active) tile_prefetch_k(kcur, koff, tbuf(0));

  const uint32_t tab = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&conv_tab[0])) + 20 * tid;
  const float c = a.scale_log2;
  int tn = 0;
  int ib = 0;  // tile buffer of tile tn
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
      // The common case -- a tile inside the segment (not its first, second
      // or last) whose copy three tiles ahead is a wholly visible tile of the
      // same item, in one page -- runs as one statement that loops over those
      // tiles (fp8_hot_loop), reading the copies' block-table entries itself.
      if (wave_active && direct && tt - 1 > seg_begin) {
        const int64_t hot_end = min(min(seg_end - 1, item_te - 4), t1 - 3);
        if (tt < hot_end) {
          const int steps = static_cast<int>(hot_end - tt);
          l_item = advance_item(m, a.num_items, l_item, l_tile);  // the loop's first copy: tile tn + 3
          const TileLoc L = locate(a, m, l_item, l_tile);
          const int b = m.item_b[l_item];
          const int32_t* bt_row = block_tables + static_cast<int64_t>(b) * a.max_blocks;
          int tok = L.tok0;
          int32_t pg = static_cast<int32_t>(L.pg0);
          uint32_t n = uni(static_cast<uint32_t>(steps));
          uint32_t bs = uni(tbuf(ib)), bp = uni(tbuf(ib == 0 ? 2 : ib - 1)), bn = uni(tbuf(ib == 2 ? 0 : ib + 1));
          uint32_t cs = stage(tn + 1) + cofs;
          uint32_t cs4 = cs + (wave < 2 ? 16384u : 12288u);
          uint32_t ds = uni(stage(tn + 2) - stage(tn + 1));
          uint32_t scb = uni(sslot(tn));
          uint32_t sc = scb + 16 * g;
          uint32_t m0b = uni(stage(tn + 3) + 1024 * wave);
          fp8_hot_loop(kcur, koff, voff, c, m_ref, l_sum, bs, bp, bn, n, cs, cs4, tab, ds, sc, scb, 16 * g,
                       uni(scale_base), uni(scale_base + 4 * kScaleSlot), m0b, uni(wave >= 2 ? 1u : 0u), o0, o4,
                       tok, pg, uni(a.kv.data), reinterpret_cast<const float*>(uni(a.kv.scale)),
                       reinterpret_cast<const int32_t*>(uni(bt_row)), uni(static_cast<uint32_t>(a.kv.page_shift)),
                       uni(static_cast<uint32_t>(a.kv.page_size - 1)), uni(static_cast<uint32_t>(a.kv.num_pages - 1)));
          l_tile += steps;
          tt += steps;
          tn += steps;
          ib = (ib + steps) % 3;
        }
      }
      const int ibn = ib == 2 ? 0 : ib + 1;
      const int ibp = ib == 0 ? 2 : ib - 1;
      const uint32_t tail = tn + 1 < ntiles ? 1u : 0u;
      const TileLoc L = next_loc();           // tile tn + 3
      const uint32_t cstage = stage(tn + 1);  // tile tn + 1's codes, then tile tn + 3's
      const uint32_t cslot = sslot(tn + 3);
      if (!wave_active) {
        wait_vmcnt<kCopies>();
        convert_own(cstage, tbuf(ibn), tid);
        copy_tile(a, L, cstage, cslot, wave, tid);
        if (tail) __syncthreads();
        ib = ibn;
        continue;
      }
      Fp8Step f;
      f.cs = cstage + cofs;
      f.cs4 = f.cs + (wave < 2 ? 16384u : 12288u);
      f.ct = tab;
      f.sc = sslot(tn) + 16 * g;
      f.o0 = o0;
      f.o4 = o4;
      // copies inside the block for a tile in one page and wholly visible;
      // else (pages of 16 tokens, a tile at an item's edge) after it
      const bool in_block = direct && L.tok0 >= L.vlo && L.tok0 + kTile <= L.vhi;
      if (in_block) {
        f.cp = 1;
        copy_desc(f, a, L, cstage, cslot, wave);
      } else {
        f.cp = 0;
        f.m0b = f.m04 = 0;
        f.sb = f.sb4 = uni(a.kv.data);
      }
      const uint32_t tl = uni(tail);
      const int tok0 = tok_first + static_cast<int>(tt - seg_begin) * kTile;
      const bool masked = !(tok0 >= vlo && tok0 + kTile <= vhi);
      // masked tiles: element i of a lane is visible iff lo <= 8 (i / 4) + i % 4 < hi
      const int lo = vlo - tok0 - 4 * g, hi = vhi - tok0 - 4 * g;
      const uint32_t bs = uni(tbuf(ib)), bp = uni(tbuf(ibp)), bn = uni(tbuf(ibn));
      const bool first = tt == seg_begin, last = tt == seg_end - 1;
      uint32_t vn[4];  // the tile's own values addresses when it ends the segment
      if (first) {
        if (!last) {
          if (masked) fp8_first_tail_m1(kcur, koff, voff, bs, bp, bn, tl, c, m_ref, l_sum, f, lo, hi);
          else fp8_first_tail_m0(kcur, koff, voff, bs, bp, bn, tl, c, m_ref, l_sum, f);
          if (!in_block) copy_tile(a, L, cstage, cslot, wave, tid);
        } else {  // one-tile segment: its own values step follows
          if (masked) fp8_first_lastv_m1(kcur, koff, voff, bs, bs, bn, tl, c, m_ref, l_sum, f, vn, voff, lo, hi);
          else fp8_first_lastv_m0(kcur, koff, voff, bs, bs, bn, tl, c, m_ref, l_sum, f, vn, voff);
          if (!in_block) copy_tile(a, L, cstage, cslot, wave, tid);
          fp8_last_pv_f1(kcur, koff, vn, bn, tl);
        }
      } else {
        float fac;       // 2^(old - new) when the tile moved this lane's reference, else 1
        uint64_t moved;  // lanes whose reference moved
        const bool fpv = tt - 1 == seg_begin;  // first values step of the segment: O starts at 0
        if (!last) {
          if (fpv) {
            if (masked) fp8_step_tail_f1_m1(kcur, koff, voff, bs, bp, bn, tl, c, m_ref, l_sum, f, fac, moved, lo, hi);
            else fp8_step_tail_f1_m0(kcur, koff, voff, bs, bp, bn, tl, c, m_ref, l_sum, f, fac, moved);
          } else {
            if (masked) fp8_step_tail_f0_m1(kcur, koff, voff, bs, bp, bn, tl, c, m_ref, l_sum, f, fac, moved, lo, hi);
            else fp8_step_tail_f0_m0(kcur, koff, voff, bs, bp, bn, tl, c, m_ref, l_sum, f, fac, moved);
          }
          if (moved) rescale_acc(fac);  // rare: a score far above the reference
          if (!in_block) copy_tile(a, L, cstage, cslot, wave, tid);
        } else {
          if (fpv) {
            if (masked) fp8_step_lastv_f1_m1(kcur, koff, voff, bs, bp, bn, tl, c, m_ref, l_sum, f, fac, moved, vn, voff, lo, hi);
            else fp8_step_lastv_f1_m0(kcur, koff, voff, bs, bp, bn, tl, c, m_ref, l_sum, f, fac, moved, vn, voff);
          } else {
            if (masked) fp8_step_lastv_f0_m1(kcur, koff, voff, bs, bp, bn, tl, c, m_ref, l_sum, f, fac, moved, vn, voff, lo, hi);
            else fp8_step_lastv_f0_m0(kcur, koff, voff, bs, bp, bn, tl, c, m_ref, l_sum, f, fac, moved, vn, voff);
          }
          if (moved) rescale_acc(fac);  // before the tile's own values step
          if (!in_block) copy_tile(a, L, cstage, cslot, wave, tid);
          fp8_last_pv_f0(kcur, koff, vn, bn, tl);
        }
      }
      ib = ibn;
    }
    ctile = seg_end;

    // ---- segment done: the unnormalised accumulator, lse and 1/l ----
    const float l_tot = wave_active ? l_sum + __shfl_xor(l_sum, 32, 64) : 1.f;
    // (a complete item's row is fp32 o_lat; a split item's partial is bf16)
    const bool complete = (seg_begin == item_ts) && (seg_end == item_te);
    float* o_dst = nullptr;
    uint16_t* p_dst = nullptr;
    float* lse_dst;
    float* scl_dst;
    if (complete) {
      o_dst = a.o_lat + (static_cast<int64_t>(c_item) * a.H) * kR;
      lse_dst = a.lse + static_cast<int64_t>(c_item) * a.H;
      scl_dst = a.o_scale + static_cast<int64_t>(c_item) * a.H;
    } else {
      const int64_t slot = (item_ts < t0) ? 2 * wg : 2 * wg + 1;
      p_dst = a.part_o + (slot * a.H) * kR;
      lse_dst = a.part_lse + slot * a.H;
      scl_dst = a.part_scale + slot * a.H;
    }
    if (wave_active && head_ok) {
      if (complete) store_acc(o_dst + static_cast<int64_t>(head) * kR + 4 * g);
      else store_acc_bf16(p_dst + static_cast<int64_t>(head) * kR + 4 * g);
      if (g == 0) {
        lse_dst[head] = (m_ref + log2f(l_tot)) * kLn2;
        scl_dst[head] = 1.0f / l_tot;
      }
    }
  }
  // the copies issued past the range's end land before the workgroup's LDS
  // is released
  wait_vmcnt<0>();
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
