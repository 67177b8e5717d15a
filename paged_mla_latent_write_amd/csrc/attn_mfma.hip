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
//    accumulator O^T[512 x 32] (fp32) as 16 MFMA 32x32 tiles in AGPRs.  Both
//    sit in registers the compiler is not given (see attn_mfma_asm.inc).
//  * the key/value stream is cut into 32-token tiles (36 KB of bf16 latents).
//    Each tile is copied HBM -> LDS with global_load_lds (16 B per lane, no
//    VGPR staging) into one of 4 buffers, two tiles ahead of the compute, and
//    is shared by all waves (so every head reads each KV byte from HBM once).
//  * tile step t (one inline-assembly block per wave): S^T(t) = 36
//    v_mfma_f32_32x32x16_bf16 with K rows read by ds_read_b128 and the copies
//    of tile t + 2 issued between them; then O^T += V^T P^T for tile t - 1 (32
//    MFMAs, V^T read transposed from that tile's buffer by ds_read_b64_tr_b16)
//    with the softmax of tile t interleaved.  The softmax runs in the MFMA
//    output layout (each lane holds 16 tokens of one head; one cross-half
//    exchange per reduction); P is rounded to bf16 in registers and used
//    directly as the B operand.  The token order inside each 16-token MFMA step
//    is the one the MFMA output layout gives; the V^T reads use the same order,
//    so no shuffle of P is needed.
//  * softmax in base 2 against a reference maximum set at each segment's first
//    tile, so the accumulators are normally never rescaled.  A tile whose max
//    passes the reference by more than 16 moves the reference up: the row sum
//    is scaled in the block and the accumulators right after it (rare; the
//    probabilities stay <= 2^16).  The kernel writes the unnormalised O with
//    lse and 1/l; consumers apply 1/l.
//  * LDS rows are 1152 B; 16-byte chunks are XOR-swizzled per token within
//    groups of 8 (swz below, from bits 1-3 of the token index) so both the row
//    reads and the transposed reads hit distinct banks.
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
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kR = 512;
constexpr int kD = 576;
constexpr int kRowBytes = kD * 2;            // 1152
constexpr int kTileBytes = kTile * kRowBytes; // 36864
constexpr int kChunksPerTile = kTile * kD / 8; // 2304 16-byte chunks
constexpr int kKSteps = kD / 16;              // 36
constexpr int kMTiles = kR / 32;              // 16

#define LDS_PTR(T) __attribute__((address_space(3))) T*

// XOR swizzle of a token row's 16-byte chunks within aligned groups of 8.  With
// 64 LDS banks the 1152-byte row pitch already separates odd and even rows by
// half the banks; bits 1..3 of the token index then spread the 16 rows of a
// ds_read_b128 cycle and the 4 rows x 64 B of a transposed-read cycle over all
// banks (a bank-conflict model of both access patterns finds none).
__device__ __forceinline__ int swz(int t) {
  return (((t >> 1) & 1) << 2) ^ ((t >> 2) & 1) ^ (((t >> 3) & 1) << 1);
}

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
  CONST_PTR(int32_t) wg_tile;
  CONST_PTR(int32_t) wg_item;
};

// ---- the per-tile blocks (generated; see gen_attn_mfma_asm.py) ----
#include "attn_mfma_asm.inc"

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

// 16-byte copies HBM -> LDS addressed as a wave-uniform 64-bit base (SGPRs)
// plus this lane's 32-bit offset: lane i's 16 bytes land at lds_base + 16 i.
__device__ __forceinline__ void lds_dma_16_sbase(const char* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 offset:0"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

// The copy cursor: which tile a workgroup copies next, and where it lives.
// Every field is wave-uniform (scalar registers).  The page ids of the next
// tile are loaded one tile ahead, when the cursor advances, so the copy issue
// itself never waits for a block-table read; item metadata is read once per
// item.
struct LoadCursor {
  int tile;       // next tile to copy (index in the workgroup's tile stream)
  int end;        // one past the workgroup's last tile
  int item;       // item owning `tile`
  int item_end;   // first tile of the next item
  int tok;        // absolute position of `tile`'s first token
  int vlo, vhi;   // the item's visible key range
  CONST_PTR(int32_t) bt_row;  // block-table row of the item's request
  int32_t pg0, pg1;           // block-table entries of `tile` (pg1: second page when ps < 32),
                              // clamped to the cache only when used, so their loads are
                              // waited for at the next copy, not here
};

// Enter the item that owns c.tile (items with no tiles are skipped).
__device__ __forceinline__ void cursor_enter_item(LoadCursor& c, const AttnArgs& a, const Meta& m) {
  while (c.item + 1 < a.num_items && m.tile_start[c.item + 1] <= c.tile) ++c.item;
  c.item_end = m.tile_start[c.item + 1];
  c.vlo = m.item_lo[c.item];
  c.vhi = m.item_hi[c.item];
  c.tok = ((c.vlo >> 5) + (c.tile - m.tile_start[c.item])) * kTile;
  c.bt_row = m.block_tables + static_cast<int64_t>(m.item_b[c.item]) * a.max_blocks;
}

// Read the page ids of c.tile.  Only block-table entries below ceil(vhi / ps)
// are read: the tile's first token is < vhi, and the second page is read only
// if it holds a visible token.
__device__ __forceinline__ void cursor_fetch_pages(LoadCursor& c, const AttnArgs& a) {
  const int blk = c.tok >> a.kv.page_shift;
  const bool two = a.kv.page_size < kTile && c.tok + a.kv.page_size < c.vhi;
  c.pg0 = c.bt_row[blk];
  c.pg1 = c.bt_row[blk + (two ? 1 : 0)];  // (no dependence on pg0's value: not waited for here)
}

// True when c.tile is wholly visible and inside one page: its 36 KB are then
// contiguous in HBM and every lane's source is a fixed offset from one base.
__device__ __forceinline__ bool cursor_contiguous(const LoadCursor& c, const AttnArgs& a) {
  return a.kv.page_size >= kTile && c.tok >= c.vlo && c.tok + kTile <= c.vhi;
}

// HBM address of c.tile's first row (contiguous tiles).
__device__ __forceinline__ const char* cursor_src(const LoadCursor& c, const AttnArgs& a) {
  const int psh = a.kv.page_shift;
  const unsigned pg0 = min(static_cast<unsigned>(c.pg0), static_cast<unsigned>(a.kv.num_pages - 1));
  const int blk0 = c.tok >> psh;
  return static_cast<const char*>(a.kv.data) +
         ((static_cast<int64_t>(pg0) << psh) + (c.tok - (blk0 << psh))) * kRowBytes;
}

// Copy tile c.tile into an LDS buffer (2304 chunks of 16 B: kLoads copies of
// 64 lanes per wave).  Tokens outside the visible range load a clamped (valid,
// finite) token; their scores are masked, so they contribute exactly zero.
template <int NW>
__device__ __forceinline__ void cursor_copy(const LoadCursor& c, const AttnArgs& a, uint32_t lds0,
                                            const uint32_t (&lofs_in)[(kChunksPerTile / 64 / NW + 1) / 2]) {
  constexpr int kPerWave = kChunksPerTile / 64 / NW;
  // Opaque copies: keeps the compiler from hoisting the per-copy address
  // arithmetic out of the tile loop (it would hold ~30 registers for it).
  uint32_t lofs[(kPerWave + 1) / 2];
#pragma unroll
  for (int i = 0; i < (kPerWave + 1) / 2; ++i) {
    lofs[i] = lofs_in[i];
    asm volatile("" : "+v"(lofs[i]));
  }
  const int ps = a.kv.page_size;
  const int psh = a.kv.page_shift;
  if (cursor_contiguous(c, a)) {
    const char* src = cursor_src(c, a);
#pragma unroll
    for (int k = 0; k < kPerWave; ++k)
      lds_dma_16_sbase(src, (lofs[k >> 1] >> (16 * (k & 1))) & 0xFFFF, lds0 + k * 1024);
    return;
  }
  const char* base = static_cast<const char*>(a.kv.data);
  const int blk0 = c.tok >> psh;
  const unsigned last_page = static_cast<unsigned>(a.kv.num_pages - 1);
  const unsigned pg0 = min(static_cast<unsigned>(c.pg0), last_page);
  const unsigned pg1 = min(static_cast<unsigned>(c.pg1), last_page);
#pragma unroll
  for (int k = 0; k < kPerWave; ++k) {
    const int lo = static_cast<int>((lofs[k >> 1] >> (16 * (k & 1))) & 0xFFFF);
    const int t = lo / kRowBytes;           // token row of this lane's chunk
    const int cbyte = lo - t * kRowBytes;   // its (swizzled-source) byte offset in the row
    int pos = c.tok + t;
    pos = pos < c.vlo ? c.vlo : pos;
    pos = pos >= c.vhi ? c.vhi - 1 : pos;
    const int in_page = pos - (blk0 << psh);  // 0 .. 2 * ps - 1
    const unsigned pg = in_page >= ps ? pg1 : pg0;
    const int off = in_page >= ps ? in_page - ps : in_page;
    const char* src = base + ((static_cast<int64_t>(pg) << psh) + off) * kRowBytes + cbyte;
    lds_dma_16(src, lds0 + k * 1024);
  }
}

// Move the cursor to the next tile and start reading its page ids (they are
// waited for only when that tile is copied).
__device__ __forceinline__ void cursor_advance(LoadCursor& c, const AttnArgs& a, const Meta& m) {
  ++c.tile;
  c.tok += kTile;
  if (c.tile < c.end) {
    if (c.tile >= c.item_end) {
      ++c.item;
      cursor_enter_item(c, a, m);
    }
    cursor_fetch_pages(c, a);
  }
}

// Next item owning `tile` (items with no tiles are skipped).
__device__ __forceinline__ int advance_item(const Meta& m, int num_items, int item, int tile) {
  while (item + 1 < num_items && m.tile_start[item + 1] <= tile) ++item;
  return item;
}

template <int NW>
__global__ __launch_bounds__(NW * 64, 1) __attribute__((amdgpu_num_vgpr(kCompilerVgprs))) void attn_mfma_kernel(
    AttnArgs a, const int32_t* __restrict__ item_b, const int32_t* __restrict__ item_lo,
    const int32_t* __restrict__ item_hi, const int32_t* __restrict__ tile_start,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ wg_tile,
    const int32_t* __restrict__ wg_item) {
  const Meta m{(CONST_PTR(int32_t))item_b, (CONST_PTR(int32_t))item_lo, (CONST_PTR(int32_t))item_hi,
               (CONST_PTR(int32_t))tile_start, (CONST_PTR(int32_t))block_tables,
               (CONST_PTR(int32_t))wg_tile, (CONST_PTR(int32_t))wg_item};
  __shared__ __attribute__((aligned(1024))) char lds_buf[4][kTileBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int g = lane >> 5;        // half of the wave
  const int n32 = lane & 31;      // head within the wave / token row for K reads
  const int head = wave * 32 + n32;
  const bool head_ok = head < a.H;
  // With fewer than 32 * NW heads the surplus waves still copy their share of
  // every tile (so the copy rate does not drop) but skip the arithmetic.
  const bool wave_active = wave * 32 < a.H;

  // Workgroups are dispatched round-robin over the 8 XCDs (each with its own
  // L2); ranges are numbered so that consecutive ranges -- which mostly share
  // an item, and so its queries -- run on the same XCD.
  const int64_t wg = (gridDim.x & 7) == 0 ? (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3)
                                          : blockIdx.x;
  const int t0 = m.wg_tile[wg], t1 = m.wg_tile[wg + 1];
  if (t0 >= t1) return;
  const int ntiles = t1 - t0;
  const int first_item = m.wg_item[wg];

  LDS_PTR(char) bufs[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) bufs[u] = (LDS_PTR(char))(&lds_buf[u][0]);

  // ---- lane-constant LDS offsets ----
  // K rows (A of S^T): token n32, chunk 2k + g.  (c & 7) ^ swz = (2k & 7) ^ (g ^ swz).
  const int y = g ^ swz(n32);
  // V^T (A of O^T) transposed reads: group q = lane / 16, jj = lane % 16 reads
  // token 16 j + 8 h + 4 g + rr, dims 32 mt + 16 (q & 1) + 4 c4 .. + 3; the
  // swizzle of that token is 4 (rr >> 1) ^ g ^ 2 h.
  const int q = lane >> 4, jj = lane & 15, rr = jj >> 2, c4 = jj & 3;
  const int xs = (2 * (q & 1) + (c4 >> 1)) ^ (4 * (rr >> 1)) ^ g;
  const int vbase = (4 * g + rr) * kRowBytes + 8 * (c4 & 1);
  const int voff_even = vbase + (xs << 4);
  const int voff_odd = vbase + ((4 ^ xs) << 4);
  const int voff_even_h = vbase + 8 * kRowBytes + ((2 ^ xs) << 4);
  const int voff_odd_h = vbase + 8 * kRowBytes + ((6 ^ xs) << 4);

  // ---- per-lane source offsets of this wave's tile copies ----
  // Copy k of wave w fills LDS slots s = 64 (w * kLoads + k) + lane of the tile
  // (16 B each, row-major with 72 slots per token); slot (t, p) holds source
  // chunk c = p ^ swizzle(t) of token t, i.e. byte t * 1152 + 16 c of the tile.
  constexpr int kLoads = kChunksPerTile / 64 / NW;
  uint32_t lofs[(kLoads + 1) / 2] = {};  // two 16-bit offsets per register
#pragma unroll
  for (int k = 0; k < kLoads; ++k) {
    const int sl = (wave * kLoads + k) * 64 + lane;
    const int t = sl / 72;
    const int p = sl - t * 72;
    const uint32_t o = t * kRowBytes + (((p & ~7) | ((p & 7) ^ swz(t))) << 4);
    lofs[k >> 1] |= o << (16 * (k & 1));
  }

  // ---- copy cursor ----
  // Tile n is copied while tile n - 2 is computed (buffer n % 4): step n reads
  // buffers n % 4 (scores) and (n - 1) % 4 (values of the previous tile).
  // Barrier n + 1 sits at the end of step n, after its values step and its
  // wait for tile n + 1, so buffer (n + 2) % 4 -- last read in step n - 1 --
  // is free for the copy that step n + 1 issues... i.e. step n copies tile
  // n + 2 into the buffer freed before barrier n.  After barrier n + 1 the
  // step reads the first K fragments of tile n + 1, so the next step starts
  // on data already in registers.
  LoadCursor cur;
  cur.tile = t0;
  cur.end = t1;
  cur.item = first_item;
  cursor_enter_item(cur, a, m);
  cursor_fetch_pages(cur, a);
  const uint32_t lds_wave = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(bufs[0])) + wave * kLoads * 1024);
  // tile 0, then the first item's queries, then tile 1: the first step needs
  // only the first two (the wait below leaves tile 1's copies in flight)
  cursor_copy<NW>(cur, a, lds_wave, lofs);
  cursor_advance(cur, a, m);

  uint32_t koff[4], kcur[4], voff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) koff[j] = n32 * kRowBytes + (((2 * j) ^ y) << 4);
  voff[0] = voff_even;
  voff[1] = voff_odd;
  voff[2] = voff_even_h;
  voff[3] = voff_odd_h;
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(bufs[0]));
  const float c = a.scale_log2;

  // Q (v62-v205) and the O^T accumulators (a0-a255) live in registers the
  // compiler does not allocate; only the blocks of attn_mfma_asm.inc touch them.
  zero_q();
  int c_item = advance_item(m, a.num_items, first_item, t0);
  // the first item's queries (lanes of heads >= H keep zeros)
  if (wave_active && head_ok)
    load_q_nowait(a.q_lat + c_item * a.q_lat_st + head * a.q_lat_sh + 8 * g,
                  a.q_pe + c_item * a.q_pe_st + head * a.q_pe_sh + 8 * g);
  if (ntiles > 1) {
    cursor_copy<NW>(cur, a, lds_wave + kTileBytes, lofs);
    cursor_advance(cur, a, m);
    wait_vmcnt<kLoads>();  // tile 0 and the queries have landed
  } else {
    wait_vmcnt<0>();
  }
  __syncthreads();  // barrier 0: tile 0 is in LDS
  if (wave_active) tile_prefetch_k(kcur, koff, lds_base);

  int tn = 0;               // tiles consumed so far (buffer tn % 4)
  int ctile = t0;
  while (ctile < t1) {
    // ---- a segment: the WG's tiles of one item ----
    c_item = advance_item(m, a.num_items, c_item, ctile);
    const int item_ts = m.tile_start[c_item], item_te = m.tile_start[c_item + 1];
    const int seg_begin = ctile;
    const int seg_end = item_te < t1 ? item_te : t1;
    float m_ref = 0.f, l_sum = 0.f;
    const int vlo = m.item_lo[c_item], vhi = m.item_hi[c_item];
    const int tok_first = ((vlo >> 5) + (seg_begin - item_ts)) * kTile;

    for (int tt = seg_begin; tt < seg_end; ++tt, ++tn) {
      // The common case -- a tile inside the segment (not its first, second
      // or last) whose copy two tiles ahead lies inside the same item, not at
      // its edges, and in one page -- runs as one statement that loops over
      // those tiles (tile_hot_loop).  Those tiles are wholly visible, and so
      // is each copy; the loop reads the next copy's page id itself (in
      // bounds: a tile of the same item).  The cursor's second page id is not
      // kept up to date there; with pages of at least one tile it is never
      // used.
      if (wave_active && tt - 1 > seg_begin && a.kv.page_size >= kTile) {
        const int hot_end = min(min(seg_end - 1, t1 - 2), item_te - 3);
        if (tt < hot_end) {
          const int steps = hot_end - tt;
          uint32_t n = steps;
          uint32_t xs = lds_base + (tn & 3) * kTileBytes, xp = lds_base + ((tn - 1) & 3) * kTileBytes;
          uint32_t xn = lds_base + ((tn + 1) & 3) * kTileBytes, xc = lds_base + ((tn + 2) & 3) * kTileBytes;
          int tok = cur.tok;
          int32_t pg = cur.pg0;
          tile_hot_loop(kcur, koff, voff, c, m_ref, l_sum, xs, xp, xn, xc, lds_wave - lds_base, n, tok, pg,
                        static_cast<const char*>(a.kv.data), (const int32_t*)cur.bt_row,
                        static_cast<uint32_t>(a.kv.page_shift), static_cast<uint32_t>(a.kv.page_size - 1),
                        static_cast<uint32_t>(a.kv.num_pages - 1), lofs);
          cur.tile += steps;
          cur.tok = tok;
          cur.pg0 = pg;
          tt += steps;
          tn += steps;
        }
      }
      // copies of tile tn + 2: inside the step block when the tile is
      // contiguous, else issued here
      const bool copy = tn + 2 < ntiles;
      const uint32_t lds_copy = __builtin_amdgcn_readfirstlane(lds_wave + ((tn + 2) & 3) * kTileBytes);
      const int tok0 = tok_first + (tt - seg_begin) * kTile;
      const bool masked = !(tok0 >= vlo && tok0 + kTile <= vhi);
      const bool fused_copy = copy && wave_active && !masked && cursor_contiguous(cur, a);
      const char* sb = nullptr;
      if (copy) {
        if (fused_copy) sb = cursor_src(cur, a);
        else cursor_copy<NW>(cur, a, lds_copy, lofs);
        cursor_advance(cur, a, m);
      }
      // the end of step tn waits for tile tn + 1 (with the copy of tile tn + 2
      // still in flight) and passes barrier tn + 1; the last tile has neither
      const uint32_t tail = tn + 1 < ntiles ? (copy ? 2u : 1u) : 0u;
      if (!wave_active) {
        if (tail == 2) wait_vmcnt<kLoads>();
        if (tail == 1) wait_vmcnt<0>();
        if (tail != 0) __syncthreads();
        continue;
      }
      const uint32_t bs = lds_base + (tn & 3) * kTileBytes;
      const uint32_t bp = lds_base + ((tn - 1) & 3) * kTileBytes;
      const uint32_t bn = lds_base + ((tn + 1) & 3) * kTileBytes;
      // masked tiles: element i of a lane is visible iff lo <= 8 (i / 4) + i % 4 < hi
      const int lo = vlo - tok0 - 4 * g, hi = vhi - tok0 - 4 * g;
      const bool first = tt == seg_begin, last = tt == seg_end - 1;
      uint32_t vn[4];  // the tile's own values addresses when it ends the segment
      if (first) {
        if (!last) {
          if (masked) tile_first_tail_d0_m1(kcur, koff, voff, bs, bp, bn, tail, c, m_ref, l_sum, lo, hi);
          else if (fused_copy) tile_first_tail_d1_m0(kcur, koff, voff, bs, bp, bn, tail, c, m_ref, l_sum, sb, lds_copy, lofs);
          else tile_first_tail_d0_m0(kcur, koff, voff, bs, bp, bn, tail, c, m_ref, l_sum);
        } else {  // one-tile segment: its own values step follows
          if (masked) tile_first_lastv_d0_m1(kcur, koff, voff, bs, bs, bn, tail, c, m_ref, l_sum, vn, voff, lo, hi);
          else if (fused_copy) tile_first_lastv_d1_m0(kcur, koff, voff, bs, bs, bn, tail, c, m_ref, l_sum, vn, voff, sb, lds_copy, lofs);
          else tile_first_lastv_d0_m0(kcur, koff, voff, bs, bs, bn, tail, c, m_ref, l_sum, vn, voff);
          tile_last_pv_f1(kcur, koff, vn, bn, tail);
        }
      } else {
        float fac;       // 2^(old - new) when the tile moved this lane's reference, else 1
        uint64_t moved;  // lanes whose reference moved
        const bool fpv = tt - 1 == seg_begin;  // first values step of the segment: O starts at 0
        if (!last) {
          if (fpv) {
            if (masked) tile_step_tail_d0_f1_m1(kcur, koff, voff, bs, bp, bn, tail, c, m_ref, l_sum, fac, moved, lo, hi);
            else if (fused_copy) tile_step_tail_d1_f1_m0(kcur, koff, voff, bs, bp, bn, tail, c, m_ref, l_sum, fac, moved, sb, lds_copy, lofs);
            else tile_step_tail_d0_f1_m0(kcur, koff, voff, bs, bp, bn, tail, c, m_ref, l_sum, fac, moved);
          } else {
            if (masked) tile_step_tail_d0_f0_m1(kcur, koff, voff, bs, bp, bn, tail, c, m_ref, l_sum, fac, moved, lo, hi);
            else if (fused_copy) tile_step_tail_d1_f0_m0(kcur, koff, voff, bs, bp, bn, tail, c, m_ref, l_sum, fac, moved, sb, lds_copy, lofs);
            else tile_step_tail_d0_f0_m0(kcur, koff, voff, bs, bp, bn, tail, c, m_ref, l_sum, fac, moved);
          }
          if (moved) rescale_acc(fac);  // rare: a score far above the reference
        } else {
          if (fpv) {
            if (masked) tile_step_lastv_d0_f1_m1(kcur, koff, voff, bs, bp, bn, tail, c, m_ref, l_sum, fac, moved, vn, voff, lo, hi);
            else if (fused_copy) tile_step_lastv_d1_f1_m0(kcur, koff, voff, bs, bp, bn, tail, c, m_ref, l_sum, fac, moved, vn, voff, sb, lds_copy, lofs);
            else tile_step_lastv_d0_f1_m0(kcur, koff, voff, bs, bp, bn, tail, c, m_ref, l_sum, fac, moved, vn, voff);
          } else {
            if (masked) tile_step_lastv_d0_f0_m1(kcur, koff, voff, bs, bp, bn, tail, c, m_ref, l_sum, fac, moved, vn, voff, lo, hi);
            else if (fused_copy) tile_step_lastv_d1_f0_m0(kcur, koff, voff, bs, bp, bn, tail, c, m_ref, l_sum, fac, moved, vn, voff, sb, lds_copy, lofs);
            else tile_step_lastv_d0_f0_m0(kcur, koff, voff, bs, bp, bn, tail, c, m_ref, l_sum, fac, moved, vn, voff);
          }
          if (moved) rescale_acc(fac);  // before the tile's own values step
          tile_last_pv_f0(kcur, koff, vn, bn, tail);
        }
      }
    }
    ctile = seg_end;

    // ---- segment done: the unnormalised accumulator, lse and 1/l
    // (no arithmetic on the accumulator registers: consumers apply 1/l)
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
    // A wave whose 32 heads all exist stores through LDS (coalesced rows),
    // using its own 9 KB copy region of the buffers of the segment's last two
    // tiles: every wave has finished with those once it passed the last
    // tile's barrier, and the WG's last segment (no such barrier) gets one
    // here.  Its next copy into either region is issued by this wave itself,
    // after these reads.
    const bool lds_store = (wave + 1) * 32 <= a.H;
    if (ctile >= t1) __syncthreads();
    if (wave_active && lds_store) {
      const uint32_t reg_a = lds_base + ((tn - 2) & 3) * kTileBytes + wave * kLoads * 1024;
      const uint32_t reg_b = lds_base + ((tn - 1) & 3) * kTileBytes + wave * kLoads * 1024;
      const uint32_t w_off = n32 * 272 + 16 * g;
      if (complete) {
        const uint32_t r_off = (lane >> 4) * 272 + (lane & 15) * 16;
        store_acc_lds(reinterpret_cast<char*>(o_dst + static_cast<int64_t>(wave * 32) * kR),
                      (lane >> 4) * 2048 + (lane & 15) * 16, reg_a + w_off, reg_b + w_off, reg_a + r_off,
                      reg_b + r_off);
      } else {
        const uint32_t r_off = (lane >> 3) * 272 + (lane & 7) * 32;
        store_acc_lds_bf16(p_dst + static_cast<int64_t>(wave * 32) * kR, (lane >> 3) * 1024 + (lane & 7) * 16,
                           reg_a + w_off, reg_b + w_off, reg_a + r_off, reg_b + r_off);
      }
    } else if (wave_active && head_ok) {
      if (complete) store_acc(o_dst + static_cast<int64_t>(head) * kR + 4 * g);
      else store_acc_bf16(p_dst + static_cast<int64_t>(head) * kR + 4 * g);
    }
    if (wave_active && head_ok && g == 0) {
      lse_dst[head] = (m_ref + log2f(l_tot)) * kLn2;
      scl_dst[head] = 1.0f / l_tot;
    }
    // the next segment's queries (its first K fragments are already read)
    if (ctile < t1 && wave_active && head_ok) {
      const int n_item = advance_item(m, a.num_items, c_item, ctile);
      load_q(a.q_lat + n_item * a.q_lat_st + head * a.q_lat_sh + 8 * g,
             a.q_pe + n_item * a.q_pe_st + head * a.q_pe_sh + 8 * g);
    }
  }
}

}  // namespace

bool mfma_attn_supported(const CacheView& kv, int32_t H) {
  return kv.dtype == kKvBf16 && kv.R == kR && kv.Dr == kD - kR && H >= 1 && H <= 128;
}

hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(attn_mfma_kernel<4>, dim3(a.G), dim3(256), 0, s, a, a.item_b, a.item_lo,
                     a.item_hi, a.tile_start, a.block_tables, a.wg_tile, a.wg_item);
  return hipGetLastError();
}

}  // namespace mla
