// Chunked prefill in the expanded (non-absorbed) form.
//
// "[Attention] MLA with chunked prefill", Future work: the cached latents are
// up-projected with kv_b_proj into a workspace and prefill attends in the
// per-head form; "feat(serving): DeepSeek-V2/V3 paged-attention shim (MLA)",
// Changes: prefill attention with keys qk_nope + qk_rope and values
// v_head_dim.  Per head h and key t of a request:
//   k_t = [W_UK[h] c_t ; r_t]  (128 + 64),   v_t = W_UV[h] c_t  (128),
// and query row i (position p = n - m + i) attends to its causal / window
// range with scores scale * ([q_nope ; q_pe] . k_t).  The result equals the
// absorbed form's; this form does 2 H (Dn + Dr + Dv) flops per (row, key)
// pair instead of 2 H (2R + Dr), plus 2 H R (Dn + Dv) per key for the
// up-projection.
//
// The keys a request's rows can see, [lo, n), are up-projected into a
// workspace bounded by 1.25 GiB: when the longest such range fits, a launch
// pair covers whole ranges of as many requests as fit (one pass, no running
// state); otherwise requests go one at a time in passes of ck keys, merged:
//   kv_expand_kernel   K_exp[h][j][0:128] = W_UK[h] c_{k0+j},
//                      V_expT[h][0:128][j] = W_UV[h] c_{k0+j},
//                      kpe[j][0:64] = r_{k0+j}, all bf16 (fp8 caches: the
//                      codes are multiplied exactly and the per-token scale
//                      is applied to the fp32 result);
//   attn_expanded_kernel  one workgroup per (128 query rows, head): S^T =
//                      K Q^T and O^T += V^T P^T on matrix cores over
//                      32-key tiles, online softmax against a reference
//                      maximum, and a log-sum-exp merge with the previous
//                      passes' running state; the last pass writes out and
//                      lse.
// Request, context length and row range are read on the device, so the host
// launches a fixed number of passes per request (from max_blocks * page_size)
// and passes past a request's context return at once.
#include <math.h>

#include <type_traits>

#include "device_utils.h"
#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kXDn = 128, kXDr = 64, kXDv = 128, kXDq = kXDn + kXDr;

__device__ __forceinline__ f32x16 mfma(const i16x8& a, const i16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// The pass's key range of request b: [k0, k0 + ntok); false when the pass lies
// past the request's context.  Also returns n, m (rows), P = n - m.
__device__ __forceinline__ bool pass_range(const XPassArgs& a, int b, int64_t* n_out, int64_t* m_out,
                                           int64_t* k0_out, int64_t* ntok_out) {
  const int64_t n = min(max(static_cast<int64_t>(a.context_lens[b]), int64_t{0}), a.max_ctx);
  const int64_t m = a.query_start_loc[b + 1] - a.query_start_loc[b];
  if (m <= 0 || m > n) return false;
  const int64_t P = n - m;
  const int64_t lo = a.window > 0 ? max(int64_t{0}, P - a.window + 1) : 0;
  const int64_t k0 = lo + static_cast<int64_t>(a.pass) * a.ck;
  if (k0 >= n) return false;
  *n_out = n;
  *m_out = m;
  *k0_out = k0;
  *ntok_out = min(static_cast<int64_t>(a.ck), n - k0);
  return true;
}

// ---------------------------------------------------------------------------
// Up-projection of one pass's keys (a gathered GEMM: tokens x R times R x 128)
// ---------------------------------------------------------------------------

constexpr int kGTok = 256;                 // tokens per workgroup tile
constexpr int kGThreads = 512;             // 8 waves: 4 token quarters x (K, V)
constexpr int kGN = 256;                   // output columns per tile: one head's K (128) and V (128)
// bf16 caches: R in 32-wide stages, three LDS buffers (copies of stage s + 2
// issued during stage s's MFMAs); fp8 caches: 64-wide stages, one buffer
constexpr int kGK = 32, kGPitch = kGK * 2 + 16, kGBufs = 3;
constexpr int kGK8 = 64, kGPitch8 = kGK8 * 2 + 16;

// V_expT keeps each 16-key group with its second and third quads swapped
// (keys 4..7 after 8..11): the attention kernel's MFMA reads the eight keys
// of a lane's P fragment (keys 4g..4g+3 and 8+4g..8+4g+3 of the group, lane
// half g) as one contiguous 16-byte run.
__device__ __forceinline__ int vperm(int j) {
  const int q = (j >> 2) & 3;
  return (q == 1 || q == 2) ? (j ^ 12) : j;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Two fp32 values as a bf16 pair (hardware conversion, nearest even).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

constexpr int kGRowSlots = kGPitch / 16;   // 16-byte LDS slots per row (4 of data, one of pad)
constexpr int kGSlots = (kGTok + kGN) * kGRowSlots;  // slots of one stage (A then B rows)
constexpr int kGDma = kGSlots / kGThreads;            // copies per thread per stage (5)
constexpr int kGStageBytes = (kGTok + kGN) * kGPitch;
static_assert(kGSlots % kGThreads == 0, "stage copies");

// 16-byte copy HBM -> LDS: lane i's bytes land at lds_base + 16 i.  Inline
// assembly keeps the compiler from draining the copies with conservative
// waits; the kernel waits explicitly.
__device__ __forceinline__ void lds_dma_16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(gptr)
               : "memory", "m0");
}

// s_waitcnt vmcnt(n) with lgkmcnt and expcnt left unconstrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <bool kFp8>
__global__ __launch_bounds__(kGThreads, 1) void kv_expand_kernel(XPassArgs a) {
  // A (tokens) and B (weight rows) of the stages
  constexpr int kSmem = kFp8 ? (kGTok + kGN) * kGPitch8 : kGBufs * kGStageBytes;
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  __shared__ float tok_scale[kFp8 ? kGTok : 1];
  const int tile = blockIdx.x, h = blockIdx.y, bz = blockIdx.z;
  const int b = a.b0 + bz;
  int64_t n, m, k0, ntok;
  if (!pass_range(a, b, &n, &m, &k0, &ntok)) return;
  const int j0 = tile * kGTok;
  if (j0 >= ntok) return;
  const int ck = a.ck;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int g = lane >> 5, n32 = lane & 31;
  const CacheView& kv = a.kv;
  const int R = kv.R;
  const int32_t* bt = a.block_tables + static_cast<int64_t>(b) * a.max_blocks;
  const unsigned last_page = static_cast<unsigned>(kv.num_pages - 1);
  // B rows 0..127: W_UK[h] rows, 128..255: W_UV[h] rows
  const uint16_t* Wk = a.w_uk + static_cast<int64_t>(h) * kXDn * R;
  const uint16_t* Wv = a.w_uv + static_cast<int64_t>(h) * kXDv * R;
  uint16_t* k_exp = a.k_exp + static_cast<int64_t>(bz) * a.H * ck * kXDn;
  uint16_t* v_expT = a.v_expT + static_cast<int64_t>(bz) * a.H * kXDv * ck;
  uint16_t* kpe = a.kpe + static_cast<int64_t>(bz) * ck * kXDr;

  auto cache_row = [&](int j) -> int64_t {
    const int64_t tok = k0 + min(j, static_cast<int>(ntok) - 1);
    const unsigned pg = min(static_cast<unsigned>(bt[tok >> kv.page_shift]), last_page);
    return static_cast<int64_t>(pg) * kv.page_size + (tok & (kv.page_size - 1));
  };
  const char* cache = static_cast<const char*>(kv.data);
  // wave tile: 64 tokens x 128 columns (all K or all V)
  const int tm = wave >> 1, tn = wave & 1;  // tm 0..3
  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) acc[i][jj] = f32x16{};
  // The MFMAs of k-step ks of a stage on the LDS rows at as / bs (rows of
  // kP bytes).  V waves compute tokens x dims (a lane ends with four
  // consecutive tokens of one dim: a piece of a V^T row); K waves compute
  // dims x tokens (four consecutive dims of one token: a piece of a K row).
  auto kstep_mfma = [&](auto kt, auto pitch_c, int ks, const char* as, const char* bs) {
    constexpr bool kK = decltype(kt)::value;
    constexpr int kP = decltype(pitch_c)::value;
    i16x8 af[2], bf[4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      af[i] = *reinterpret_cast<const i16x8*>(as + (64 * tm + 32 * i + n32) * kP + (16 * ks + 8 * g) * 2);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      bf[jj] = *reinterpret_cast<const i16x8*>(bs + (128 * tn + 32 * jj + n32) * kP + (16 * ks + 8 * g) * 2);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        acc[i][jj] = kK ? mfma(bf[jj], af[i], acc[i][jj]) : mfma(af[i], bf[jj], acc[i][jj]);
  };

  if constexpr (!kFp8) {
    // Stage slot z (16 bytes; 5 per 80-byte row: 4 of data, one of pad) of
    // the A rows then the B rows is filled by thread z % 512, copy z / 512
    // (each wave's copy covers 64 consecutive slots, so lane i's bytes land
    // at the copy's base + 16 i).  Pad slots repeat the row's last chunk;
    // token rows past the pass's keys repeat its last row (finite values,
    // never attended).  The block-table loads go out together (each lane
    // loads for every token copy, whatever its slot holds).
    constexpr int kACopies = (kGTok * kGRowSlots + kGThreads - 1) / kGThreads;  // copies with token rows (3)
    int64_t tok[kACopies];
    unsigned pg[kACopies];
#pragma unroll
    for (int k = 0; k < kACopies; ++k) {
      const int z = kGThreads * k + t;
      const int r = (z < kGTok * kGRowSlots ? z : z - kGTok * kGRowSlots) / kGRowSlots;
      tok[k] = k0 + min(j0 + r, static_cast<int>(ntok) - 1);
      pg[k] = static_cast<unsigned>(bt[tok[k] >> kv.page_shift]);
    }
    // (opaque: the compiler may not sink a load into the branch that uses it)
#pragma unroll
    for (int k = 0; k < kACopies; ++k) asm volatile("" : "+v"(pg[k]));
    const char* dsrc[kGDma];
#pragma unroll
    for (int k = 0; k < kGDma; ++k) {
      const int z = kGThreads * k + t;
      const bool is_a = z < kGTok * kGRowSlots;
      const int zr = is_a ? z : z - kGTok * kGRowSlots;
      const int r = zr / kGRowSlots, cc = min(zr - kGRowSlots * r, kGRowSlots - 2);
      const char* wp = reinterpret_cast<const char*>(r < kXDn ? Wk + static_cast<int64_t>(r) * R
                                                             : Wv + static_cast<int64_t>(r - kXDn) * R) + 16 * cc;
      if (k < kACopies) {
        const int64_t row = static_cast<int64_t>(min(pg[k], last_page)) * kv.page_size +
                            (tok[k] & (kv.page_size - 1));
        dsrc[k] = is_a ? cache + row * kv.D * 2 + 16 * cc : wp;
      } else {
        dsrc[k] = wp;
      }
    }
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem)) + 1024 * wave;
    // copies [k_lo, k_hi) of stage st into its buffer
    auto issue = [&](int st, int k_lo, int k_hi) {
#pragma unroll
      for (int k = 0; k < kGDma; ++k)
        if (k >= k_lo && k < k_hi)
          lds_dma_16(dsrc[k] + 2 * kGK * st, lds0 + (st % kGBufs) * kGStageBytes + 16 * kGThreads * k);
    };
    const int nst = R / kGK;
    issue(0, 0, kGDma);
    if (nst > 1) issue(1, 0, kGDma);
    auto stages = [&](auto kt) {
      for (int st = 0; st < nst; ++st) {
        // this thread's copies of stage st have landed (stage st + 1's may not)
        if (st + 1 < nst) wait_vmcnt<kGDma>();
        else wait_vmcnt<0>();
        // every thread's have, and every wave is done with stage st - 1's
        // buffer, which stage st + 2's copies (issued between this stage's
        // MFMAs) refill
        __syncthreads();
        const char* base = smem + (st % kGBufs) * kGStageBytes;
        const bool more = st + 2 < nst;
        if (more) issue(st + 2, 0, 3);
        kstep_mfma(kt, std::integral_constant<int, kGPitch>{}, 0, base, base + kGTok * kGPitch);
        if (more) issue(st + 2, 3, kGDma);
        kstep_mfma(kt, std::integral_constant<int, kGPitch>{}, 1, base, base + kGTok * kGPitch);
      }
    };
    if (tn == 1) stages(std::false_type{});
    else stages(std::true_type{});
  } else {
    // fp8 caches: the next stage's loads land in registers during this
    // stage's MFMAs; the codes are converted on their way to LDS.  This
    // thread's A chunks (16 codes of a token row per stage; rows past the
    // pass's keys load zeros) and B chunks, as pointers fixed over the stages.
    char* const As = smem;
    char* const Bs = smem + kGTok * kGPitch8;
    constexpr int kAq = kGTok * 4 / kGThreads;  // 16-code A chunks per thread (2)
    constexpr int kBq = kGN * 8 / kGThreads;    // 8-value B chunks per thread (4)
    const char* asrc[kAq];
    bool aok[kAq];
#pragma unroll
    for (int q = 0; q < kAq; ++q) {
      const int idx = t + kGThreads * q;
      const int r = idx >> 2, c = idx & 3;
      asrc[q] = cache + cache_row(j0 + r) * kv.D + 16 * c;
      aok[q] = j0 + r < ntok;
    }
    const uint16_t* bsrc[kBq];
#pragma unroll
    for (int q = 0; q < kBq; ++q) {
      const int idx = t + kGThreads * q;
      const int r = idx >> 3, c = idx & 7;
      bsrc[q] = (r < kXDn ? Wk + static_cast<int64_t>(r) * R : Wv + static_cast<int64_t>(r - kXDn) * R) + 8 * c;
    }
    if (t < kGTok) {
      const int j = j0 + t;
      tok_scale[t] = j < ntok ? kv.scale[cache_row(j)] : 0.0f;
    }
    i32x4 ra[kAq];
    i16x8 rb[kBq];
    auto load_stage = [&](int kc) {
#pragma unroll
      for (int q = 0; q < kAq; ++q) {
        i32x4 v = {0, 0, 0, 0};
        if (aok[q]) v = *reinterpret_cast<const i32x4*>(asrc[q] + kc);
        ra[q] = v;
      }
#pragma unroll
      for (int q = 0; q < kBq; ++q) rb[q] = *reinterpret_cast<const i16x8*>(bsrc[q] + kc);
    };
    auto store_stage = [&]() {
#pragma unroll
      for (int q = 0; q < kAq; ++q) {
        // 16 E4M3 codes -> 16 bf16 values (exact: every E4M3 value is a bf16 value)
        const int idx = t + kGThreads * q;
        const int r = idx >> 2, c = idx & 3;
        i32x4 lo, hi;
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          lo[2 * w] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ra[q][w], 1.0f, false));
          lo[2 * w + 1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ra[q][w], 1.0f, true));
          hi[2 * w] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ra[q][w + 2], 1.0f, false));
          hi[2 * w + 1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ra[q][w + 2], 1.0f, true));
        }
        *reinterpret_cast<i32x4*>(As + r * kGPitch8 + c * 32) = lo;
        *reinterpret_cast<i32x4*>(As + r * kGPitch8 + c * 32 + 16) = hi;
      }
#pragma unroll
      for (int q = 0; q < kBq; ++q) {
        const int idx = t + kGThreads * q;
        *reinterpret_cast<i16x8*>(Bs + (idx >> 3) * kGPitch8 + (idx & 7) * 16) = rb[q];
      }
    };
    load_stage(0);
    for (int kc = 0; kc < R; kc += kGK8) {
      store_stage();
      __syncthreads();
      if (kc + kGK8 < R) load_stage(kc + kGK8);  // in flight during this stage's MFMAs
      if (tn == 1) {
#pragma unroll
        for (int ks = 0; ks < kGK8 / 16; ++ks)
          kstep_mfma(std::false_type{}, std::integral_constant<int, kGPitch8>{}, ks, As, Bs);
      } else {
#pragma unroll
        for (int ks = 0; ks < kGK8 / 16; ++ks)
          kstep_mfma(std::true_type{}, std::integral_constant<int, kGPitch8>{}, ks, As, Bs);
      }
      __syncthreads();
    }
  }

  // epilogue: 16-byte stores, 16 per lane.  V waves: element e of
  // acc[i][jj] is token 64 tm + 32 i + 8 (e / 4) + 4 g + e % 4 of dim
  // 32 jj + n32.  With V^T's quad order a lane's quads e4 = 2p and 2p + 1
  // (tokens 16 p + 4 g + 0..3 and + 8..11) are adjacent in memory.  K waves:
  // element e is dim 32 jj + 8 (e / 4) + 4 g + e % 4 of token 64 tm + 32 i +
  // n32; a swap of lanes l + 32 and l (dims 4..7 for 8..11) gives lane half 0
  // dims 16 p + 0..7 and half 1 dims 16 p + 8..15.
  auto quad = [&](int i, int jj, int e4, float sc0, float sc1, float sc2, float sc3) -> uint2 {
    return make_uint2(pack_bf16(acc[i][jj][4 * e4] * sc0, acc[i][jj][4 * e4 + 1] * sc1),
                      pack_bf16(acc[i][jj][4 * e4 + 2] * sc2, acc[i][jj][4 * e4 + 3] * sc3));
  };
  if (tn == 1) {
    uint16_t* vrow = v_expT + static_cast<int64_t>(h) * kXDv * ck + j0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d = 32 * jj + n32;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const int r = 64 * tm + 32 * i + 16 * p + 4 * g;  // tile-local token of quad e4 = 2 p
          float sc[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) sc[e] = kFp8 ? tok_scale[r + (e < 4 ? e : e + 4)] : 1.0f;
          const uint2 q0 = quad(i, jj, 2 * p, sc[0], sc[1], sc[2], sc[3]);
          const uint2 q1 = quad(i, jj, 2 * p + 1, sc[4], sc[5], sc[6], sc[7]);
          *reinterpret_cast<uint4*>(vrow + static_cast<int64_t>(d) * ck + vperm(r)) =
              make_uint4(q0.x, q0.y, q1.x, q1.y);
        }
      }
    }
  } else {
    uint16_t* krow = k_exp + (static_cast<int64_t>(h) * ck + j0) * kXDn;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 64 * tm + 32 * i + n32;  // tile-local token
      const float sc = kFp8 ? tok_scale[r] : 1.0f;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const uint2 qa = quad(i, jj, 2 * p, sc, sc, sc, sc);      // dims 16 p + 4 g + 0..3
          const uint2 qb = quad(i, jj, 2 * p + 1, sc, sc, sc, sc);  // dims 16 p + 8 + 4 g + 0..3
          const auto sx = __builtin_amdgcn_permlane32_swap(qa.x, qb.x, false, false);
          const auto sy = __builtin_amdgcn_permlane32_swap(qa.y, qb.y, false, false);
          // half 0: [own qa, partner's qa] = dims 16 p + 0..7; half 1:
          // [partner's qb, own qb] = dims 16 p + 8..15
          *reinterpret_cast<uint4*>(krow + static_cast<int64_t>(r) * kXDn + 32 * jj + 16 * p + 8 * g) =
              make_uint4(sx[0], sy[0], sx[1], sy[1]);
        }
      }
    }
  }
  // the rope part of the keys, shared by every head (written once): 8-value
  // chunks, four per thread; tokens past the pass's keys get zeros
  if (h == 0) {
    constexpr int kQ = kGTok * (kXDr / 8) / kGThreads;
    int64_t row[kQ];
#pragma unroll
    for (int q = 0; q < kQ; ++q) row[q] = cache_row(j0 + ((t + kGThreads * q) >> 3));
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int c = t + kGThreads * q, r = c >> 3, part = c & 7;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (j0 + r < ntok) {
        if constexpr (!kFp8) {
          v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(kv.data) + row[q] * kv.D + R + 8 * part);
        } else {
          const uint2 codes =
              *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(kv.data) + row[q] * kv.D + R + 8 * part);
          const float sc = kv.scale[row[q]];
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t word = e < 2 ? codes.x : codes.y;
            const int sh = 16 * (e & 1);
            w[e] = static_cast<uint32_t>(f32_to_bf16(e4m3_to_f32((word >> sh) & 0xFF) * sc)) |
                   (static_cast<uint32_t>(f32_to_bf16(e4m3_to_f32((word >> (sh + 8)) & 0xFF) * sc)) << 16);
          }
          v = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
      *reinterpret_cast<uint4*>(kpe + static_cast<int64_t>(j0 + r) * kXDr + 8 * part) = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Attention of 128 query rows of one head over one pass's keys
// ---------------------------------------------------------------------------

constexpr int kAT = 32;                        // keys per tile
constexpr int kAKPitch = kXDq * 2 + 16;        // bytes per LDS key row (400)
constexpr int kAVPitch = kAT * 2 + 16;         // bytes per LDS V^T row (80)
constexpr float kRescaleSlack = 8.0f;          // log2 units

__global__ __launch_bounds__(256, 2) void attn_expanded_kernel(XPassArgs a) {
  __shared__ __attribute__((aligned(16))) char Ks[3][kAT * kAKPitch];
  __shared__ __attribute__((aligned(16))) char Vs[3][kXDv * kAVPitch];
  // XCD-aware numbering: workgroups are dispatched round-robin over the 8
  // XCDs (each with its own L2).  The row blocks of one (request, head) read
  // the same key and value tiles, so they are made the consecutive
  // workgroups of one XCD (k-th workgroup on XCD x: group (k / nrb) * 8 + x,
  // row block k % nrb), while consecutive groups still go to different XCDs.
  const int nrb = gridDim.x;
  const int groups = gridDim.y * gridDim.z;
  const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  int rb = blockIdx.x, grp = blockIdx.y + gridDim.y * blockIdx.z;
  if (groups % 8 == 0) {
    const int x = lin % 8, k = lin / 8;
    grp = (k / nrb) * 8 + x;
    rb = k % nrb;
  }
  const int h = grp % gridDim.y, bz = grp / gridDim.y, b = a.b0 + bz;
  int64_t n, m, k0, ntok;
  if (!pass_range(a, b, &n, &m, &k0, &ntok)) return;
  if (static_cast<int64_t>(rb) * 128 >= m) return;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int g = lane >> 5, n32 = lane & 31;
  const int64_t P = n - m;
  const bool first = a.pass == 0;
  const bool last = k0 + ntok >= n;
  const int64_t row_base = a.query_start_loc[b];
  const int ck = a.ck;
  // this workgroup's rows [r_lo, r_hi) (request-local) and the keys they see
  const int64_t r_lo = static_cast<int64_t>(rb) * 128, r_hi = min(r_lo + 128, m);
  const int64_t key_hi = min(k0 + ntok, P + r_hi);  // last row sees keys <= P + r_hi - 1
  int64_t key_lo = k0;
  if (a.window > 0) key_lo = max(key_lo, P + r_lo - a.window + 1);
  const int tile_lo = key_lo < key_hi ? static_cast<int>((key_lo - k0) / kAT) : 0;
  const int tile_hi = key_lo < key_hi ? static_cast<int>((key_hi - k0 + kAT - 1) / kAT) : 0;

  // this lane's query row (request-local) and its position
  const int64_t ri = r_lo + 32 * wave + n32;
  const bool row_ok = ri < m && row_base + ri >= 0 && row_base + ri < a.total_q;
  const int64_t q_row = row_ok ? row_base + ri : 0;
  const int64_t pos = P + ri;
  // Q^T fragments: k-step s covers query dims 16 s .. 16 s + 15 (nope, then rope)
  i16x8 qf[kXDq / 16];
#pragma unroll
  for (int s = 0; s < kXDq / 16; ++s) {
    const int d = 16 * s + 8 * g;
    const uint16_t* src = d < kXDn ? a.q_nope + q_row * a.qn_st + h * a.qn_sh + d
                                   : a.q_pe + q_row * a.qp_st + h * a.qp_sh + (d - kXDn);
    qf[s] = *reinterpret_cast<const i16x8*>(src);
  }

  // tile loads: 5 chunks of 16 B per thread (K_exp 512, kpe 256, V^T 512);
  // chunk q of tile `tile` is at src[q] + j0 * stride(q) elements, j0 = 32 tile
  const uint16_t* kexp_h = a.k_exp + (static_cast<int64_t>(bz) * a.H + h) * ck * kXDn;
  const uint16_t* vexp_h = a.v_expT + (static_cast<int64_t>(bz) * a.H + h) * kXDv * ck;
  const uint16_t* kpe_b = a.kpe + static_cast<int64_t>(bz) * ck * kXDr;
  const uint16_t* src[5];
  uint32_t dst[5];  // byte offsets in a K / V buffer
#pragma unroll
  for (int q = 0; q < 5; ++q) {
    const int idx = t + 256 * q;
    if (q < 2) {  // K_exp: key idx / 16, chunk idx % 16
      src[q] = kexp_h + (idx >> 4) * kXDn + 8 * (idx & 15);
      dst[q] = (idx >> 4) * kAKPitch + 16 * (idx & 15);
    } else if (q == 2) {  // kpe: key (idx - 512) / 8, chunk % 8
      const int k = idx - 512;
      src[q] = kpe_b + (k >> 3) * kXDr + 8 * (k & 7);
      dst[q] = (k >> 3) * kAKPitch + kXDn * 2 + 16 * (k & 7);
    } else {  // V^T: row (idx - 768) / 4, chunk % 4
      const int k = idx - 768;
      src[q] = vexp_h + static_cast<int64_t>(k >> 2) * ck + 8 * (k & 3);
      dst[q] = (k >> 2) * kAVPitch + 16 * (k & 3);
    }
  }
  i16x8 ld[5];
  auto load_tile = [&](int tile) {
    const int64_t j0 = static_cast<int64_t>(tile) * kAT;
#pragma unroll
    for (int q = 0; q < 5; ++q) {
      const int64_t stride = q < 2 ? kXDn : (q == 2 ? kXDr : 1);
      ld[q] = *reinterpret_cast<const i16x8*>(src[q] + j0 * stride);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 5; ++q) {
      char* base = q < 3 ? Ks[buf] : Vs[buf];
      *reinterpret_cast<i16x8*>(base + dst[q]) = ld[q];
    }
  };

  f32x16 o[kXDv / 32];
#pragma unroll
  for (int db = 0; db < kXDv / 32; ++db) o[db] = f32x16{};
  float m_ref = -INFINITY, l_sum = 0.f;
  const float c = a.scale_log2;  // > 0 (the host routes other scales to the absorbed form)

  // S^T = K Q^T (keys x rows) of the tile in buffer `buf`
  // (the key fragments are read six at a time, so that the MFMAs do not
  // each wait for their own LDS read)
  auto scores = [&](int buf) {
    f32x16 sc = f32x16{};
    const char* kb = Ks[buf] + n32 * kAKPitch + 16 * g;
#pragma unroll
    for (int s0 = 0; s0 < kXDq / 16; s0 += 6) {
      i16x8 kf[6];
#pragma unroll
      for (int u = 0; u < 6; ++u) kf[u] = *reinterpret_cast<const i16x8*>(kb + 32 * (s0 + u));
#pragma unroll
      for (int u = 0; u < 6; ++u) sc = mfma(kf[u], qf[s0 + u], sc);
    }
    // (the order above, kept by the scheduler: six LDS reads, six MFMAs)
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
    return sc;
  };
  // the keys of this lane's row inside [k0, k0 + ntok): key <= pos, and with a
  // window key > pos - window; as tile-relative bounds lo <= key - tile_key < hi
  const int64_t vis_hi = row_ok ? min(pos + 1, k0 + ntok) : k0;
  const int64_t vis_lo = a.window > 0 ? pos - a.window + 1 : INT64_MIN / 2;
  auto clamp32 = [](int64_t x) { return static_cast<int>(min(max(x, int64_t{0}), int64_t{kAT})); };

  // Software pipeline over three LDS buffers (tile t in buffer t mod 3): the
  // scores of tile t + 1 are issued on the matrix cores before the softmax of
  // tile t runs on the vector ALUs, and tile t + 2 is loaded meanwhile.
  if (tile_lo < tile_hi) {
    load_tile(tile_lo);
    store_tile(0);
  }
  if (tile_lo + 1 < tile_hi) {
    load_tile(tile_lo + 1);
    store_tile(1);
  }
  __syncthreads();
  f32x16 s_cur = tile_lo < tile_hi ? scores(0) : f32x16{};
  int cur = 0, nxt = 1, far = 2;
  for (int tile = tile_lo; tile < tile_hi; ++tile) {
    const bool has_next = tile + 1 < tile_hi, has_far = tile + 2 < tile_hi;
    if (has_far) load_tile(tile + 2);  // in flight during this tile's math
    f32x16 s_next = f32x16{};
    if (has_next) s_next = scores(nxt);
    f32x16 s = s_cur;
    // this tile's V^T fragments, read before the softmax so that they land
    // during it
    i16x8 vf[kXDv / 32][2];
    {
      const char* vb = Vs[cur] + n32 * kAVPitch + 16 * g;
#pragma unroll
      for (int db = 0; db < kXDv / 32; ++db)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) vf[db][kk] = *reinterpret_cast<const i16x8*>(vb + 32 * db * kAVPitch + 32 * kk);
    }
    // mask (tiles the lane's row does not wholly see), tile maximum of the
    // raw scores (a row's 32 keys sit in lanes n32 and n32 + 32; the scale
    // is positive, so it is applied to the maximum)
    const int64_t tile_key = k0 + static_cast<int64_t>(tile) * kAT;
    const int lo = clamp32(vis_lo - tile_key), hi = clamp32(vis_hi - tile_key);
    if (__ballot(lo != 0 || hi != kAT) != 0) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int off = 8 * (e >> 2) + 4 * g + (e & 3);
        s[e] = (off >= lo && off < hi) ? s[e] : -INFINITY;
      }
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
    for (int e = 3; e < 16; ++e) mx = fmaxf(mx, s[e]);
    {
      // (the other half of the row's keys sits in lane l ^ 32: a lane swap,
      // no LDS round trip)
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c;
    }
    // move the reference when this tile's maximum passes it by the slack
    // (always on a row's first visible tile: the reference starts at -inf)
    const bool move = mx > m_ref + kRescaleSlack;
    if (__ballot(move) != 0) {
      const float alpha = move ? exp2f(m_ref - mx) : 1.0f;  // 0 when the reference was -inf
      if (move) {
        m_ref = mx;
        l_sum *= alpha;
      }
#pragma unroll
      for (int db = 0; db < kXDv / 32; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
    }
    // p = 2^(s c - m_ref) <= 2^8 (v_exp_f32; masked keys give exp2(-inf) = 0),
    // rounded to bf16 pairs by the hardware conversion (nearest even)
    const float m_use = m_ref == -INFINITY ? 0.f : m_ref;  // a row with nothing visible yet
    uint32_t pk[8];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s[e], c, -m_use));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s[e + 1], c, -m_use));
      psum += p0 + p1;
      pk[e >> 1] = pack_bf16(p0, p1);
    }
    l_sum += psum;
    // O^T += V^T P^T; MFMA k-slot 8 g + j of key half kk is key 16 kk + 4 g + j
    // (j < 4) or 16 kk + 8 + 4 g + (j - 4): the keys this lane's P registers
    // hold, which the quad-swapped V^T columns 16 kk + 8 g .. + 7 hold in order
#pragma unroll
    for (int db = 0; db < kXDv / 32; ++db) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const i32x4 pv = {static_cast<int>(pk[4 * kk]), static_cast<int>(pk[4 * kk + 1]),
                          static_cast<int>(pk[4 * kk + 2]), static_cast<int>(pk[4 * kk + 3])};
        o[db] = mfma(vf[db][kk], __builtin_bit_cast(i16x8, pv), o[db]);
      }
    }
    // buffer `far` last held tile t - 1, whose values were read before the
    // barrier that ended the previous step
    if (has_far) store_tile(far);
    __syncthreads();
    s_cur = s_next;
    const int tmp = cur;
    cur = nxt;
    nxt = far;
    far = tmp;
  }

  // merge with the previous passes and store
  l_sum += __shfl_xor(l_sum, 32, 64);
  if (!row_ok) return;
  const int64_t st_row = (row_base + ri) * a.H + h;  // state / output row
  float* o_st = a.o_acc + st_row * kXDv;
  float scale_new = 1.0f, scale_old = 0.0f;
  float m_tot = m_ref, l_tot = l_sum;
  if (!first) {
    const float m_prev = a.m_acc[st_row], l_prev = a.l_acc[st_row];
    m_tot = fmaxf(m_prev, m_ref);
    scale_old = m_prev == -INFINITY ? 0.f : exp2f(m_prev - m_tot);
    scale_new = m_ref == -INFINITY ? 0.f : exp2f(m_ref - m_tot);
    l_tot = l_prev * scale_old + l_sum * scale_new;
  }
#pragma unroll
  for (int db = 0; db < kXDv / 32; ++db) {
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const int d = 32 * db + 8 * e4 + 4 * g;  // this lane's dims d .. d + 3
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = o[db][4 * e4 + e] * scale_new;
      if (!first) {
        const float4 prev = *reinterpret_cast<const float4*>(o_st + d);
        v[0] += prev.x * scale_old;
        v[1] += prev.y * scale_old;
        v[2] += prev.z * scale_old;
        v[3] += prev.w * scale_old;
      }
      if (last) {
        const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
        uint16_t* dst = a.out + st_row * kXDv + d;
        *reinterpret_cast<uint2*>(dst) =
            make_uint2(f32_to_bf16(v[0] * inv) | (static_cast<uint32_t>(f32_to_bf16(v[1] * inv)) << 16),
                       f32_to_bf16(v[2] * inv) | (static_cast<uint32_t>(f32_to_bf16(v[3] * inv)) << 16));
      } else {
        *reinterpret_cast<float4*>(o_st + d) = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
  }
  if (g == 0) {
    if (last) {
      if (a.lse) a.lse[st_row] = l_tot > 0.f ? (m_tot + log2f(l_tot)) * kLn2 : -INFINITY;
    } else {
      a.m_acc[st_row] = m_tot;
      a.l_acc[st_row] = l_tot;
    }
  }
}

}  // namespace

bool prefill_expanded_supported(const CacheView& kv, int32_t H, int32_t Dn, int32_t Dv) {
  // (the pass length is a multiple of the up-projection's token tile)
  static_assert(kGTok == 256, "pass lengths are rounded to 256 keys");
  return kv.Dr == kXDr && kv.R % kGK8 == 0 && Dn == kXDn && Dv == kXDv && H >= 1 && H <= 1024;
}

hipError_t launch_prefill_expanded_pass(const XPassArgs& a, int32_t max_q_len, hipStream_t s) {
  const dim3 grid(a.ck / kGTok, a.H, a.batch);
  if (a.kv.dtype == kKvFp8)
    hipLaunchKernelGGL(kv_expand_kernel<true>, grid, dim3(kGThreads), 0, s, a);
  else
    hipLaunchKernelGGL(kv_expand_kernel<false>, grid, dim3(kGThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_expanded_kernel, dim3((max_q_len + 127) / 128, a.H, a.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
