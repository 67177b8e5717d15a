// Split-KV paged latent attention over an fp8 E4M3 cache on the fp8 matrix
// cores of gfx950 (v_mfma_f32_32x32x64_f8f6f4): the cache codes are the MFMA
// operands as stored, the queries and the probabilities are quantised to E4M3
// ("[unified-memory] Let Kimi-Linear use the paged MLA attention backends",
// Validation: the fp8_e4m3 cache rows; "Support dsv4 model", Model
// Architecture and Inference: the packed FP8 KV layout).  The result is an
// approximation of the exact softmax over the dequantised cache; its error
// against that definition is what the tests bound.
//
// What it computes, per query item and head h over the visible keys t with
// codes k_t (576 per token: 512 latent + 64 rope) and scale s_t:
//   q = [q_lat ; q_pe][h],  sq = max|q| / 448,  q ~ sq (hi + lo) with
//   hi = e4m3(q / sq) and lo = e4m3(q / sq - hi)    (a two-term expansion: a
//       single e4m3 term loses too much for sharply peaked scores),
//   a_t = scale log2(e) * sq * s_t * ((hi + lo) . k_t)     (base-2 score),
//   p_t = 2^(a_t - m),  l = sum p_t,  lse = (m + log2 l) ln 2,
//   o = sum_t e4m3(p_t s_t 2^E) 2^-E c_t      (c_t: the latent codes),
// with m a reference maximum (as in the bf16 kernel: set by a segment's
// first step, moved when a step's maximum passes it by more than 16) and E a
// per-head, per-step power of two that puts the step's largest p_t s_t in
// [128, 256); the matrix cores apply 2^-E through the instruction's E8M0
// operand scale.  The outputs are those of the other kernels: unnormalised o
// with lse and 1/l per head, for complete items or the split slots.
//
// Design (one workgroup of four waves per compute unit, wave w owning heads
// [32w, 32w + 32)):
//  * a step is 64 tokens (the K of one values MFMA).  Its 36 KB of codes and
//    256 B of scales are copied HBM -> LDS with global_load_lds into one of
//    two buffers, one step ahead; the 16-byte chunks of token t are placed at
//    chunk ^ ((t >> 2) & 3), which keeps both the row reads of the scores and
//    the transposed reads of the values free of bank conflicts.
//  * scores: S^T[64 x 32 heads] = K Q^T as 2 x 9 k-steps, each two MFMAs
//    (hi, lo).  hi lives in VGPRs (the B operand, 72 registers), lo in LDS
//    (128 rows of 576 codes, 592-byte pitch).
//  * the softmax runs in the MFMA output layout (a lane holds 32 of the 64
//    tokens of one head); the lane's E4M3 probabilities are, in that order,
//    its B operand of the values MFMA, and the transposed reads of V
//    (ds_read_b64_tr_b8) fetch the tokens in the same order.
//  * O^T[512 x 32] accumulates in 16 MFMA tiles (accumulation registers).
#include <math.h>

#include "device_utils.h"
#include "mla_internal.h"

namespace mla {
namespace {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kR = 512;
constexpr int kD = 576;
constexpr int kStepTok = 64;                    // tokens per step (two plan tiles)
constexpr int kRow = kD;                        // bytes per cached token (codes)
constexpr int kBufBytes = kStepTok * kRow;      // 36864
constexpr int kChunks = kBufBytes / 16;         // 2304
constexpr int kCopies = kChunks / 256;          // 9 per thread
constexpr int kKSteps = kD / 64;                // 9
constexpr int kRBlocks = kR / 32;               // 16
constexpr int kQPitch = kD + 16;                // 592: rows of 16 lanes hit distinct banks
constexpr int kE8M0One = 127;                   // E8M0 code of 1.0
constexpr float kLn2 = 0.69314718055994531f;
static_assert(kCopies * 256 == kChunks, "a step is 9 copies of 16 B per thread");
static_assert(kStepTok == 2 * kTile, "a step is two plan tiles");

#define LDS_PTR(T) __attribute__((address_space(3))) T*
#define CONST_PTR(T) const __attribute__((address_space(4))) T*

// Slot of 16-byte chunk c of token row t in a staged step.
__device__ __forceinline__ int chunk_slot(int c, int t) { return c ^ ((t >> 2) & 3); }

// s_waitcnt vmcnt(0) with lgkmcnt and expcnt unconstrained.
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8)); }

// 16-byte copy HBM -> LDS, lane i's bytes at lds_base + 16 i (lds_base wave
// uniform).  Inline assembly: the kernel orders the copies itself (a vmcnt(0)
// wait and a barrier before a buffer is read or refilled).
__device__ __forceinline__ void lds_dma_16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(gptr)
               : "memory", "m0");
}

// 4-byte copy HBM -> LDS (lane i's dword at lds_base + 4 i).
__device__ __forceinline__ void lds_dma_4(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(gptr)
               : "memory", "m0");
}

// The same copy addressed as a wave-uniform 64-bit base (SGPRs) plus this
// lane's 32-bit offset.
__device__ __forceinline__ void lds_dma_16_sbase(const char* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 offset:0"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(sbase)
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

// A step: its first plan tile, the item, the item's visible range and the
// token of the step's first row.
struct Step {
  int item, b;           // the item and its request
  int64_t ts, te, tile;  // the item's plan tiles and the step's first
  int vlo, vhi, tok0;
};

// (item metadata is read when the cursor enters an item, not per step)
__device__ __forceinline__ Step make_step(const Meta& m, int item, int64_t tile) {
  Step s;
  s.item = item;
  s.b = m.item_b[item];
  s.ts = m.tile_start[item];
  s.te = m.tile_start[item + 1];
  s.tile = tile;
  s.vlo = m.item_lo[item];
  s.vhi = m.item_hi[item];
  s.tok0 = ((s.vlo >> 5) + static_cast<int>(tile - s.ts)) * kTile;
  return s;
}

// The cache rows of this thread's copies of a step: codes chunk p = tid +
// 256 j is token p / 36 (slot p % 36); lanes 0-15 of wave 0 also copy the
// scales of tokens 4 lane .. + 3 (a group of 4 lies in one page).  Rows
// outside the item's visible range copy the nearest visible row (their
// scores are masked and their weights zeroed).  The block-table entries are
// read one step before the copies, so their latency is hidden by a step of
// compute instead of serialising the copies.
struct StepRows {
  int32_t pg[kCopies + 1];  // page of each copy's row (the last: the scales)
};

__device__ __forceinline__ int step_pos(const Step& st, int t) {
  const int pos = st.tok0 + t;
  return pos < st.vlo ? st.vlo : (pos >= st.vhi ? st.vhi - 1 : pos);
}

__device__ __forceinline__ int scale_pos(const Step& st, int lane) {
  const int pos = st.tok0 + 4 * lane;
  const int lo4 = st.vlo & ~3, hi4 = (st.vhi - 1) & ~3;
  return pos < lo4 ? lo4 : (pos > hi4 ? hi4 : pos);
}

__device__ __forceinline__ void load_rows(const AttnArgs& a, const Meta& m, const Step& st, StepRows& r,
                                          int wave, int tid_in) {
  // (an opaque copy of the thread index: the per-copy arithmetic is
  // recomputed per step instead of being hoisted out of the loops, where it
  // would hold registers for the whole kernel)
  int tid = tid_in;
  asm volatile("" : "+v"(tid));
  const int psh = a.kv.page_shift;
  const int32_t* bt = a.block_tables + static_cast<int64_t>(st.b) * a.max_blocks;
#pragma unroll
  for (int j = 0; j < kCopies; ++j) {
    const int p = tid + 256 * j;
    r.pg[j] = bt[step_pos(st, p / 36) >> psh];
  }
  const int lane = tid & 63;
  r.pg[kCopies] = (wave == 0 && lane < 16) ? bt[scale_pos(st, lane) >> psh] : 0;
}

__device__ __forceinline__ void copy_step(const AttnArgs& a, const Step& st, const StepRows& r, uint32_t dst,
                                          uint32_t sdst, int wave, int tid_in) {
  int tid = tid_in;
  asm volatile("" : "+v"(tid));
  const int psh = a.kv.page_shift, pmask = a.kv.page_size - 1;
  const unsigned last_page = static_cast<unsigned>(a.kv.num_pages - 1);
  const char* codes = static_cast<const char*>(a.kv.data);
#pragma unroll
  for (int j = 0; j < kCopies; ++j) {
    const int p = tid + 256 * j;
    const int t = p / 36, s = p - 36 * (p / 36);
    const int c = chunk_slot(s, t);  // the slot map is its own inverse
    const unsigned pg = min(static_cast<unsigned>(r.pg[j]), last_page);
    const int64_t row = (static_cast<int64_t>(pg) << psh) + (step_pos(st, t) & pmask);
    lds_dma_16(codes + row * kRow + 16 * c, dst + 4096 * j + 1024 * wave);
  }
  const int lane = tid & 63;
  if (wave == 0 && lane < 16) {
    const unsigned pg = min(static_cast<unsigned>(r.pg[kCopies]), last_page);
    const int64_t row = (static_cast<int64_t>(pg) << psh) + (scale_pos(st, lane) & pmask);
    lds_dma_16(a.kv.scale + row, sdst);
  }
}

// A step whose 64 rows are all visible and lie in at most two pages, split
// at row 32 (pages of 32 tokens or more; a step starts at a multiple of 32):
// its rows are two runs of contiguous cache rows, copied with wave-uniform
// bases and per-lane offsets that do not change from step to step.  Rows
// 32..63 are addressed from base_hi, which points 32 rows before their page's
// first row (the same offsets serve both runs).  The pages are read with
// scalar loads one step ahead of the copies.
struct FastStep {
  bool on, two;
};

// Whether a step takes the fast copies; if so, lanes 0 and 1 of wave 0 copy
// its two block-table entries into pg_slot (an LDS pair), one step before
// its copies read them.  (In registers, the entries would be merged across
// the loop's paths with moves that wait for the loads inside the step.)
__device__ __forceinline__ FastStep fast_step(const AttnArgs& a, const Step& st, uint32_t pg_slot, int wave,
                                              int lane) {
  FastStep f;
  f.on = a.kv.page_size >= 32 && st.vlo <= st.tok0 && st.tok0 + kStepTok <= st.vhi;
  f.two = false;
  if (!f.on) return f;
  const int psh = a.kv.page_shift;
  const int blk_lo = st.tok0 >> psh, blk_hi = (st.tok0 + 32) >> psh;
  f.two = blk_hi != blk_lo;
  if (wave == 0 && lane < 2)
    lds_dma_4(a.block_tables + static_cast<int64_t>(st.b) * a.max_blocks + (lane == 0 ? blk_lo : blk_hi),
              pg_slot);
  return f;
}

// voff[j]: this lane's byte offset of copy j inside a step's rows (token t,
// chunk s ^ f(t)); t4_lo: copy 4's token is below 32.
// The fast copies of a step in pieces: part 0 forms the bases (from the
// block-table pair in LDS) and issues the scales' copy; part j + 1 issues
// copy j.  Spread over the first matrix instructions of a step, their issue
// overlaps the matrix cores' work.
struct FastBases {
  const char* lo;
  const char* hi;
};

__device__ __forceinline__ FastBases fast_bases(const AttnArgs& a, const Step& st, const FastStep& f,
                                                uint32_t pg_slot, uint32_t sdst, int wave, int lane) {
  const int psh = a.kv.page_shift, pmask = a.kv.page_size - 1;
  const unsigned last_page = static_cast<unsigned>(a.kv.num_pages - 1);
  const i32x2 pp = *reinterpret_cast<LDS_PTR(const i32x2)>(pg_slot);
  const unsigned pl = min(static_cast<unsigned>(__builtin_amdgcn_readfirstlane(pp[0])), last_page);
  const unsigned ph = min(static_cast<unsigned>(__builtin_amdgcn_readfirstlane(pp[1])), last_page);
  const int64_t row_lo = (static_cast<int64_t>(pl) << psh) + (st.tok0 & pmask);
  const int64_t row_hi = f.two ? (static_cast<int64_t>(ph) << psh) - 32 : row_lo;
  if (wave == 0 && lane < 16) lds_dma_16(a.kv.scale + (lane < 8 ? row_lo : row_hi) + 4 * lane, sdst);
  FastBases b;
  b.lo = static_cast<const char*>(a.kv.data) + row_lo * kRow;
  b.hi = static_cast<const char*>(a.kv.data) + row_hi * kRow;
  return b;
}

// voff[j]: this lane's byte offset of copy j inside a step's rows (token t,
// chunk s ^ f(t)); t4_lo: copy 4's token is below 32.
__device__ __forceinline__ void copy_fast_one(int j, const FastStep& f, const FastBases& b, const uint32_t* voff,
                                              bool t4_lo, uint32_t dst, int wave) {
  const uint32_t lds = dst + 4096 * j + 1024 * wave;
  if (j < 4 || !f.two) {
    lds_dma_16_sbase(b.lo, voff[j], lds);
  } else if (j > 4) {
    lds_dma_16_sbase(b.hi, voff[j], lds);
  } else {  // copy 4 straddles row 32: two exec-masked halves
    if (t4_lo) lds_dma_16_sbase(b.lo, voff[j], lds);
    else lds_dma_16_sbase(b.hi, voff[j], lds);
  }
}

// max over the two lanes of a head (lanes l and l ^ 32), by a lane-half
// swap (no LDS round trip).
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Two floats as packed bf16 (round to nearest even), the first in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_bits_f32(uint32_t bits) { return __uint_as_float(bits << 16); }

// One k-step of one 32-token block's scores: s += K hi, then s += K lo (two
// 32x32x64 E4M3 MFMAs).  Written as assembly so that the score accumulators
// stay in VGPRs (the compiler otherwise places them in the accumulation
// registers the values' accumulators need, and spills).  The compiler does not
// see these as matrix instructions, so the blocks carry their own wait states:
// FIRST: after the VALU writes of the zeroed accumulator; LAST: 24 states
// before VALU instructions may read the result (16-pass XDL writes).
#define MLA_KSTEP_MFMAS                              \
  "v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0\n\t"  \
  "v_mfma_f32_32x32x64_f8f6f4 %0, %1, %3, %0\n\t"
template <bool FIRST, bool LAST>
__device__ __forceinline__ void mfma_kstep(f32x16& s, const i32x8& ka, const i32x8& qh, const i32x8& ql) {
  if constexpr (FIRST)
    asm volatile("s_nop 4\n\t" MLA_KSTEP_MFMAS : "+v"(s) : "v"(ka), "v"(qh), "v"(ql));
  else if constexpr (LAST)
    asm volatile(MLA_KSTEP_MFMAS "s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s) : "v"(ka), "v"(qh), "v"(ql));
  else
    asm volatile(MLA_KSTEP_MFMAS : "+v"(s) : "v"(ka), "v"(qh), "v"(ql));
}
#undef MLA_KSTEP_MFMAS



__global__ __launch_bounds__(256, 1) void attn_f8mfma_kernel(AttnArgs a, const int32_t* __restrict__ item_b,
                                                             const int32_t* __restrict__ item_lo,
                                                             const int32_t* __restrict__ item_hi,
                                                             const int32_t* __restrict__ tile_start,
                                                             const int32_t* __restrict__ block_tables) {
  const Meta m{(CONST_PTR(int32_t))item_b, (CONST_PTR(int32_t))item_lo, (CONST_PTR(int32_t))item_hi,
               (CONST_PTR(int32_t))tile_start, (CONST_PTR(int32_t))block_tables};
  __shared__ __attribute__((aligned(1024))) char lds_kv[2][kBufBytes];
  __shared__ __attribute__((aligned(16))) float lds_sc[2][kStepTok];
  __shared__ __attribute__((aligned(16))) char lds_qlo[128 * kQPitch];
  __shared__ __attribute__((aligned(16))) int32_t lds_pg[2][4];  // block-table pairs of the fast copies

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int n32 = lane & 31;
  const int head = 32 * wave + n32;
  const bool head_ok = head < a.H;
  const bool wave_active = 32 * wave < a.H;

  // consecutive ranges (which mostly share an item) on the same XCD
  const int64_t wg = (gridDim.x & 7) == 0 ? (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3)
                                          : blockIdx.x;
  const int64_t t0 = a.wg_tile[wg], t1 = a.wg_tile[wg + 1];
  if (t0 >= t1) return;

  const uint32_t kv_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&lds_kv[0][0]));
  const uint32_t sc_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&lds_sc[0][0]));
  auto kvbuf = [&](int n) { return kv_base + static_cast<uint32_t>((n & 1) * kBufBytes); };
  auto scbuf = [&](int n) { return sc_base + static_cast<uint32_t>((n & 1) * kStepTok * 4); };

  // ---- lane-constant LDS offsets ----
  // scores: token row n32 of block blk, chunk 4 ks + 2 g + u at slot
  // 4 ks + ((2 g + u) ^ f), f = (n32 >> 2) & 3
  const int fk = (n32 >> 2) & 3;
  const uint32_t k_off0 = n32 * kRow + 16 * ((2 * g) ^ fk);
  const uint32_t k_off1 = n32 * kRow + 16 * ((2 * g + 1) ^ fk);
  // values: lane (G = lane / 16, i = lane % 16, b = i / 2, h = i % 2) reads
  // for read q the row of token 32 (q >> 1) + 16 (q & 1) + 8 (b >> 2) + 4 g
  // + (b & 3), columns 32 rb + 16 (G & 1) + 8 h .. + 7, so that the lane's
  // byte 8 q + b' of the A operand is the token whose probability is byte
  // 8 q + b' of the B operand
  uint32_t v_even[4], v_odd[4];
  {
    const int G = lane >> 4, i16 = lane & 15, b = i16 >> 1, h = i16 & 1;
    const int fv = (2 * (b >> 2) + g) & 3;  // (token >> 2) & 3 of every read's row
    const int x = (G & 1) ^ fv;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int T = 32 * (q >> 1) + 16 * (q & 1) + 8 * (b >> 2) + 4 * g + (b & 3);
      v_even[q] = T * kRow + 16 * x + 8 * h;
      v_odd[q] = T * kRow + 16 * (x ^ 2) + 8 * h;
    }
  }
  const uint32_t qlo_off = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_qlo)) + head * kQPitch + 32 * g;

  // ---- step cursor: the step being copied ----
  int c_item = advance_item(m, a.num_items, a.wg_item[wg], t0);
  Step nxt = make_step(m, c_item, t0);
  bool have_next = true;
  auto advance = [&](const Step& s) {
    // the step after s in this workgroup's range, if any
    const int64_t seg_end = s.te < t1 ? s.te : t1;
    if (s.tile + 2 < seg_end) {
      Step r = s;
      r.tile += 2;
      r.tok0 += kStepTok;
      return r;
    }
    have_next = seg_end < t1;
    if (!have_next) return s;
    return make_step(m, advance_item(m, a.num_items, s.item, seg_end), seg_end);
  };
  // lane-constant offsets of the fast copies
  uint32_t voff[kCopies];
#pragma unroll
  for (int j = 0; j < kCopies; ++j) {
    const int p = tid + 256 * j;
    const int t = p / 36, sl = p - 36 * (p / 36);
    voff[j] = t * kRow + 16 * chunk_slot(sl, t);
  }
  const bool t4_lo = (tid + 1024) / 36 < 32;
  // The step `nxt` (step n + 1 while step n runs) was prepared during step
  // n - 1: for fast copies its block-table pair sits in LDS slot (n + 1) & 1;
  // other steps read their rows' pages when they are copied.
  const uint32_t pg_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&lds_pg[0][0]));
  auto pgslot = [&](int step) { return pg_base + static_cast<uint32_t>((step & 1) * 16); };
  FastStep fs;
  auto prep = [&](int step) { fs = fast_step(a, nxt, pgslot(step), wave, lane); };
  // copies of step `nxt` into buffer `step`: part 0 alone for general
  // copies, parts 0..kCopies for fast ones
  FastBases fb;
  auto copy_part = [&](int step, int part) {
    if (fs.on) {
      if (part == 0) fb = fast_bases(a, nxt, fs, pgslot(step), scbuf(step), wave, lane);
      else copy_fast_one(part - 1, fs, fb, voff, t4_lo, kvbuf(step), wave);
    } else if (part == 0) {
      StepRows rows;
      load_rows(a, m, nxt, rows, wave, tid);
      copy_step(a, nxt, rows, kvbuf(step), scbuf(step), wave, tid);
    }
  };
  auto copy_nxt = [&](int step) {
#pragma unroll
    for (int part = 0; part <= kCopies; ++part) copy_part(step, part);
  };
  prep(0);
  wait_vmcnt0();
  __syncthreads();  // step 0's block-table pair is in LDS
  copy_nxt(0);
  nxt = advance(nxt);
  if (have_next) prep(1);

  i32x8 qhi[kKSteps];
  f32x16 acc[kRBlocks];
  const float c_log2 = a.scale_log2;
  int n = 0;  // steps done
  int64_t ctile = t0;
  while (ctile < t1) {
    c_item = advance_item(m, a.num_items, c_item, ctile);
    const int64_t item_ts = m.tile_start[c_item], item_te = m.tile_start[c_item + 1];
    const int64_t seg_begin = ctile;
    const int64_t seg_end = item_te < t1 ? item_te : t1;
    const int vlo = m.item_lo[c_item], vhi = m.item_hi[c_item];
    const int tok_item0 = (vlo >> 5) * kTile;
    const int vis_hi = min(vhi, tok_item0 + static_cast<int>(seg_end - item_ts) * kTile);

    // ---- the item's queries: hi codes in registers, lo codes in LDS ----
    __syncthreads();  // every wave is done with the previous segment's lo codes
    float qscale = 0.f;
    if (wave_active) {
      const uint16_t* ql = a.q_lat + c_item * a.q_lat_st + head * a.q_lat_sh + 32 * g;
      const uint16_t* qp = a.q_pe + c_item * a.q_pe_st + head * a.q_pe_sh + 32 * g;
      auto qrow = [&](int ks) { return ks < kKSteps - 1 ? ql + 64 * ks : qp; };
      float amax = 0.f;
      if (head_ok) {
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
          const i32x4* src = reinterpret_cast<const i32x4*>(qrow(ks));
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const i32x4 w = src[u];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t x = static_cast<uint32_t>(w[e]);
              amax = fmaxf(amax, fmaxf(fabsf(bf16_bits_f32(x & 0xFFFF)), fabsf(bf16_bits_f32(x >> 16))));
            }
          }
        }
      }
      amax = half_max(amax);
      const float sq = amax > 0.f ? amax / 448.f : 1.f;
      const float inv = amax > 0.f ? 448.f / amax : 1.f;
      qscale = sq * c_log2;
      // (the rows are re-read three k-steps ahead of their conversion, so the
      // loads' latency overlaps the conversions)
      constexpr int kQAhead = 3;
      i32x4 ring[kQAhead][4];
      auto qload = [&](int ks) {
        const i32x4* src = reinterpret_cast<const i32x4*>(qrow(ks));
#pragma unroll
        for (int u = 0; u < 4; ++u) ring[ks % kQAhead][u] = head_ok ? src[u] : i32x4{0, 0, 0, 0};
      };
#pragma unroll
      for (int ks = 0; ks < kQAhead; ++ks) qload(ks);
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        i32x4 raw[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) raw[u] = ring[ks % kQAhead][u];
        if (ks + kQAhead < kKSteps) qload(ks + kQAhead);
        i32x8 hi, lo;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          // values 4 w .. 4 w + 3 of this lane's 32
          const i32x4 r = raw[w >> 1];
          const uint32_t p0 = static_cast<uint32_t>(r[2 * (w & 1)]), p1 = static_cast<uint32_t>(r[2 * (w & 1) + 1]);
          const float x0 = bf16_bits_f32(p0 & 0xFFFF) * inv, x1 = bf16_bits_f32(p0 >> 16) * inv;
          const float x2 = bf16_bits_f32(p1 & 0xFFFF) * inv, x3 = bf16_bits_f32(p1 >> 16) * inv;
          int h = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
          h = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, h, true);
          const f32x2 d01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(h, 1.0f, false);
          const f32x2 d23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(h, 1.0f, true);
          int l = __builtin_amdgcn_cvt_pk_fp8_f32(x0 - d01[0], x1 - d01[1], 0, false);
          l = __builtin_amdgcn_cvt_pk_fp8_f32(x2 - d23[0], x3 - d23[1], l, true);
          hi[w] = h;
          lo[w] = l;
        }
        qhi[ks] = hi;
        *reinterpret_cast<LDS_PTR(i32x4)>(qlo_off + 64 * ks) = i32x4{lo[0], lo[1], lo[2], lo[3]};
        *reinterpret_cast<LDS_PTR(i32x4)>(qlo_off + 64 * ks + 16) = i32x4{lo[4], lo[5], lo[6], lo[7]};
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int rb = 0; rb < kRBlocks; ++rb) acc[rb] = f32x16{};
    float m_ref = 0.f, m_base = 0.f, l_sum = 0.f;
    int k_sh = 0;  // m_ref - m_base, whole octaves

    for (int64_t tt = seg_begin; tt < seg_end; tt += 2, ++n) {
      wait_vmcnt0();     // this wave's copies of the step have landed
      __syncthreads();   // everyone's have; the other buffer is free
      // copy step n + 1 (its pages were read during step n - 1), then read
      // the pages of step n + 2; the working waves do this between their
      // first matrix instructions
      const bool copy_next = have_next;
      auto issue_copies = [&](int part) {
        if (copy_next) copy_part(n + 1, part);
      };
      auto next_rows = [&]() {
        if (copy_next) {
          nxt = advance(nxt);
          if (have_next) prep(n + 2);
        }
      };
      if (!wave_active) {
#pragma unroll
        for (int part = 0; part <= kCopies; ++part) issue_copies(part);
        next_rows();
        continue;
      }
      const uint32_t B = kvbuf(n);
      const uint32_t SB = scbuf(n);
      const int tok0 = tok_item0 + static_cast<int>(tt - item_ts) * kTile;
      // visible rows of the step: this lane's element (blk, jj, i) is row
      // 32 blk + 8 jj + 4 g + i, visible iff 32 blk + 8 jj + i lies in
      // [lo_g, hi_g) (constants against two per-lane bounds); most steps
      // are wholly visible (wave-uniform)
      const int lo_g = vlo - tok0 - 4 * g, hi_g = vis_hi - tok0 - 4 * g;
      const bool edge = !(vlo <= tok0 && vis_hi >= tok0 + kStepTok);
      const bool first = tt == seg_begin;

      struct KOp { i32x8 ka, ql; };
      auto kop = [&](int blk, int ks) {
        const uint32_t kb = B + blk * 32 * kRow + 64 * ks;
        const i32x4 a0 = *reinterpret_cast<LDS_PTR(const i32x4)>(kb + k_off0);
        const i32x4 a1 = *reinterpret_cast<LDS_PTR(const i32x4)>(kb + k_off1);
        const i32x4 l0 = *reinterpret_cast<LDS_PTR(const i32x4)>(qlo_off + 64 * ks);
        const i32x4 l1 = *reinterpret_cast<LDS_PTR(const i32x4)>(qlo_off + 64 * ks + 16);
        KOp o;
        o.ka = i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        o.ql = i32x8{l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
        return o;
      };
      // Softmax of one block, in stages: this lane's 16 elements j are rows
      // 32 blk + 8 (j >> 2) + 4 g + (j & 3).  s holds the raw scores, then
      // the base-2 logits, then the weights p_t s_t 2^E.
      struct Blk { float sc[16]; float mx, smax, madj, psum; int E; };
      auto stage_scales = [&](Blk& z, int blk) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x4 s4 = *reinterpret_cast<LDS_PTR(const f32x4)>(SB + 4 * (32 * blk + 8 * jj + 4 * g));
#pragma unroll
          for (int i = 0; i < 4; ++i) z.sc[4 * jj + i] = s4[i];
        }
      };
      auto stage_logits = [&](Blk& z, f32x16& sv, int blk) {
        float mx = -INFINITY, smax = 0.f;
        if (edge) {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int T = 32 * blk + 8 * (j >> 2) + (j & 3);
            const bool vis = T >= lo_g && T < hi_g;
            z.sc[j] = vis ? z.sc[j] : 0.f;  // (a masked row's scale may be NaN)
            sv[j] = vis ? sv[j] * qscale * z.sc[j] : -INFINITY;
            mx = fmaxf(mx, sv[j]);
            smax = fmaxf(smax, z.sc[j]);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            sv[j] = sv[j] * qscale * z.sc[j];
            mx = fmaxf(mx, sv[j]);
            smax = fmaxf(smax, z.sc[j]);
          }
        }
        z.mx = mx;
        z.smax = smax;
      };
      // (rare) a maximum past the reference by more than 16 moves it by whole
      // octaves; the accumulator keeps the units of m_base and later weights
      // are scaled up by 2^k_sh through the E8M0 operand scale; past 64
      // octaves the old contributions (below 2^-48 of the new ones) are
      // dropped and the units restart.  Returns true on a restart.
      auto move_ref = [&](float mxb) {
        bool restart = false;
        int kn = static_cast<int>(ceilf(mxb - m_base));
        if (kn > 64) {
#pragma unroll
          for (int rb = 0; rb < kRBlocks; ++rb) acc[rb] = f32x16{};
          l_sum = 0.f;
          m_base = mxb;
          kn = 0;
          restart = true;
        }
        k_sh = kn;
        m_ref = m_base + static_cast<float>(kn);
        return restart;
      };
      // the head's block maximum and largest scale; E from the bound
      // 2^(mx - m_ref) smax on the block's weights puts them below 2^8
      auto stage_ref = [&](Blk& z, bool set_ref) {
        z.mx = half_max(z.mx);
        z.smax = half_max(z.smax);
        bool restart = false;
        if (set_ref) {
          m_base = m_ref = z.mx;
          k_sh = 0;
        } else if (z.mx > m_ref + 16.f) {
          restart = move_ref(z.mx);
        }
        const float ub = exp2f(z.mx - m_ref) * z.smax;
        int E = ub > 0.f ? 8 - __builtin_amdgcn_frexp_expf(ub) : 0;
        E = E > 100 ? 100 : (E < -100 ? -100 : E);
        z.E = E;
        z.madj = m_ref - static_cast<float>(E);
        z.psum = 0.f;
        return restart;
      };
      auto stage_weights = [&](Blk& z, f32x16& sv, int j0, int cnt) {
#pragma unroll
        for (int j = j0; j < j0 + cnt; ++j) {
          const float pe = __builtin_amdgcn_exp2f(sv[j] - z.madj);  // p 2^E; 0 for masked rows
          z.psum += pe;
          sv[j] = pe * z.sc[j];
        }
      };
      auto stage_pack = [&](Blk& z, const f32x16& sv, i32x8& pb, int w0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          int v = __builtin_amdgcn_cvt_pk_fp8_f32(sv[4 * q], sv[4 * q + 1], 0, false);
          v = __builtin_amdgcn_cvt_pk_fp8_f32(sv[4 * q + 2], sv[4 * q + 3], v, true);
          pb[w0 + q] = v;
        }
        l_sum += __builtin_amdgcn_ldexpf(z.psum, k_sh - z.E);
        int sbv = kE8M0One - z.E + k_sh;  // 2^(k_sh - E)
        return sbv < 1 ? 1 : (sbv > 254 ? 254 : sbv);
      };

      // ---- block 0 scores; the next step's copies go out between them ----
      f32x16 s0 = f32x16{}, s1 = f32x16{};
      KOp nk = kop(0, 0);
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        const KOp ck = nk;
        nk = ks + 1 < kKSteps ? kop(0, ks + 1) : kop(1, 0);
        if (ks == 0) mfma_kstep<true, false>(s0, ck.ka, qhi[ks], ck.ql);
        else if (ks == kKSteps - 1) mfma_kstep<false, true>(s0, ck.ka, qhi[ks], ck.ql);
        else mfma_kstep<false, false>(s0, ck.ka, qhi[ks], ck.ql);
        // the next step's copies: the bases and scales, then copies 0-8 two
        // at a time, then the pair after that
        if (ks == 0) issue_copies(0);
        if (ks >= 1 && ks <= 5) {
          issue_copies(2 * ks - 1);
          if (2 * ks <= kCopies) issue_copies(2 * ks);
        }
        if (ks == 6) next_rows();
        __builtin_amdgcn_sched_barrier(0);
      }
      // ---- block 1 scores, block 0's softmax between them ----
      Blk z0, z1;
      i32x8 pb;
      int sb0 = kE8M0One;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        const KOp ck = nk;
        if (ks + 1 < kKSteps) nk = kop(1, ks + 1);
        if (ks == 0) mfma_kstep<true, false>(s1, ck.ka, qhi[ks], ck.ql);
        else if (ks == kKSteps - 1) mfma_kstep<false, true>(s1, ck.ka, qhi[ks], ck.ql);
        else mfma_kstep<false, false>(s1, ck.ka, qhi[ks], ck.ql);
        if (ks == 0) stage_scales(z0, 0);
        if (ks == 1) stage_logits(z0, s0, 0);
        if (ks == 2) stage_ref(z0, first);
        if (ks >= 3 && ks <= 6) stage_weights(z0, s0, 4 * (ks - 3), 4);
        if (ks == 7) sb0 = stage_pack(z0, s0, pb, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      // ---- block 1's softmax ----
      stage_scales(z1, 1);
      stage_logits(z1, s1, 1);
      if (stage_ref(z1, false)) {
        // block 1 restarted the units: block 0's weights (in the old units)
        // are dropped
        pb[0] = pb[1] = pb[2] = pb[3] = 0;
      }
      stage_weights(z1, s1, 0, 16);
      const int sb1 = stage_pack(z1, s1, pb, 4);
      // lane n supplies the E8M0 scale of the K bytes 0-15 of lanes n and
      // n + 32 (block 0's tokens), lane n + 32 that of bytes 16-31 (block 1's)
      const int sb = g == 0 ? sb0 : sb1;

      // ---- values: O^T[r][h] += sum_t V[t][r] P[t][h] 2^(k_sh - E), the
      // reads of block rb + 1 in flight during block rb's MFMA ----
      auto v_ops = [&](int rb) {
        const uint32_t* vo = (rb & 1) ? v_odd : v_even;
        const uint32_t cb = B + 64 * (rb >> 1);
        const i32x2 r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_PTR(i32x2))(cb + vo[0]));
        const i32x2 r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_PTR(i32x2))(cb + vo[1]));
        const i32x2 r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_PTR(i32x2))(cb + vo[2]));
        const i32x2 r3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_PTR(i32x2))(cb + vo[3]));
        return i32x8{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
      };
      i32x8 nv = v_ops(0);
#pragma unroll
      for (int rb = 0; rb < kRBlocks; ++rb) {
        const i32x8 cv = nv;
        if (rb + 1 < kRBlocks) nv = v_ops(rb + 1);
        __builtin_amdgcn_sched_barrier(0);  // (the next reads go out before this MFMA)
        acc[rb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cv, pb, acc[rb], 0, 0, 0, kE8M0One, 0, sb);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    ctile = seg_end;

    // ---- segment done: the unnormalised accumulator, lse and 1/l ----
    const float l_tot = wave_active ? l_sum + __shfl_xor(l_sum, 32, 64) : 1.f;
    // (a complete item's row is fp32 o_lat; a split item's partial is bf16)
    const bool complete = (seg_begin == item_ts) && (seg_end == item_te);
    // A partial goes to bf16 through LDS: each lane's accumulators are
    // written to a private 64-byte slot of the lo-code region and read back
    // for the conversion (read directly, the compiler stages all 256
    // accumulation registers through VGPRs and moves them around the step
    // loop).  Every wave is past its last reads of the lo codes here.
    if (!complete) __syncthreads();
    if (wave_active && head_ok) {
      float* lse_dst;
      float* scl_dst;
      if (complete) {
        float* orow = a.o_lat + (static_cast<int64_t>(c_item) * a.H + head) * kR + 4 * g;
        lse_dst = a.lse + static_cast<int64_t>(c_item) * a.H;
        scl_dst = a.o_scale + static_cast<int64_t>(c_item) * a.H;
#pragma unroll
        for (int rb = 0; rb < kRBlocks; ++rb) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            *reinterpret_cast<f32x4*>(orow + 32 * rb + 8 * jj) =
                f32x4{acc[rb][4 * jj], acc[rb][4 * jj + 1], acc[rb][4 * jj + 2], acc[rb][4 * jj + 3]};
        }
      } else {
        const int64_t slot = (item_ts < t0) ? 2 * wg : 2 * wg + 1;
        uint16_t* prow = a.part_o + (slot * a.H + head) * kR + 4 * g;
        lse_dst = a.part_lse + slot * a.H;
        scl_dst = a.part_scale + slot * a.H;
        const uint32_t stg = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_qlo)) + 64 * tid;
#pragma unroll
        for (int rb = 0; rb < kRBlocks; ++rb) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            *reinterpret_cast<LDS_PTR(f32x4)>(stg + 16 * jj) =
                f32x4{acc[rb][4 * jj], acc[rb][4 * jj + 1], acc[rb][4 * jj + 2], acc[rb][4 * jj + 3]};
          asm volatile("" ::: "memory");  // (a real round trip: no forwarding of the stored registers)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const f32x4 v = *reinterpret_cast<LDS_PTR(const f32x4)>(stg + 16 * jj);
            *reinterpret_cast<i32x2*>(prow + 32 * rb + 8 * jj) =
                i32x2{static_cast<int>(pack_bf16(v[0], v[1])), static_cast<int>(pack_bf16(v[2], v[3]))};
          }
        }
      }
      if (g == 0) {
        lse_dst[head] = (m_base + log2f(l_tot)) * kLn2;
        scl_dst[head] = 1.0f / l_tot;
      }
    }
  }
  // copies issued past the last step land before the workgroup's LDS is released
  wait_vmcnt0();
}

}  // namespace

bool f8mfma_attn_supported(const CacheView& kv, int32_t H) {
  return kv.dtype == kKvFp8 && kv.R == kR && kv.Dr == kD - kR && H >= 1 && H <= 128 && kv.page_size >= 4;
}

hipError_t launch_attn_f8mfma(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(attn_f8mfma_kernel, dim3(a.G), dim3(256), 0, s, a, a.item_b, a.item_lo, a.item_hi,
                     a.tile_start, a.block_tables);
  return hipGetLastError();
}

}  // namespace mla
