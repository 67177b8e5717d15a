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
constexpr int kGK = 64;                    // R per LDS stage
constexpr int kGPitch = kGK * 2 + 16;      // bytes per LDS row

// V_expT keeps each 16-key group with its second and third quads swapped
// (keys 4..7 after 8..11): the attention kernel's MFMA reads the eight keys
// of a lane's P fragment (keys 4g..4g+3 and 8+4g..8+4g+3 of the group, lane
// half g) as one contiguous 16-byte run.
__device__ __forceinline__ int vperm(int j) {
  const int q = (j >> 2) & 3;
  return (q == 1 || q == 2) ? (j ^ 12) : j;
}

__global__ __launch_bounds__(kGThreads, 1) void kv_expand_kernel(XPassArgs a) {
  __shared__ __attribute__((aligned(16))) char As[kGTok * kGPitch];
  __shared__ __attribute__((aligned(16))) char Bs[kGN * kGPitch];
  __shared__ float tok_scale[kGTok];
  const int bz = blockIdx.z, b = a.b0 + bz;
  int64_t n, m, k0, ntok;
  if (!pass_range(a, b, &n, &m, &k0, &ntok)) return;
  const int j0 = blockIdx.x * kGTok;
  if (j0 >= ntok) return;
  const int h = blockIdx.y;
  const int ck = a.ck;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int g = lane >> 5, n32 = lane & 31;
  const CacheView& kv = a.kv;
  const int R = kv.R;
  const bool fp8 = kv.dtype == kKvFp8;
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
  // cache rows of this thread's A chunks (fixed over the stages)
  int64_t arow[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = fp8 ? ((t + kGThreads * q) >> 2) : ((t + kGThreads * q) >> 3);
    arow[q] = (fp8 && q >= 2) ? 0 : cache_row(j0 + r);
  }
  if (t < kGTok) {
    const int j = j0 + t;
    tok_scale[t] = (fp8 && j < ntok) ? kv.scale[cache_row(j)] : 1.0f;
  }

  // wave tile: 64 tokens x 128 columns (all K or all V)
  const int tm = wave >> 1, tn = wave & 1;  // tm 0..3
  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) acc[i][jj] = f32x16{};

  // The next stage's global loads are issued before this stage's MFMAs and
  // land in registers; they are stored to LDS after the stage.
  i16x8 ra[4], rb[4];
  uint4 rc[2];
  auto load_stage = [&](int kc) {
    if (!fp8) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int idx = t + kGThreads * q;
        const int r = idx >> 3, c = idx & 7;
        i16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
        if (j0 + r < ntok)
          v = *reinterpret_cast<const i16x8*>(static_cast<const uint16_t*>(kv.data) + arow[q] * kv.D + kc + 8 * c);
        ra[q] = v;
      }
    } else {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int idx = t + kGThreads * q;
        const int r = idx >> 2, c = idx & 3;
        uint4 codes = make_uint4(0, 0, 0, 0);
        if (j0 + r < ntok)
          codes = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(kv.data) + arow[q] * kv.D + kc + 16 * c);
        rc[q] = codes;
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = t + kGThreads * q;
      const int r = idx >> 3, c = idx & 7;
      const uint16_t* W = r < kXDn ? Wk + static_cast<int64_t>(r) * R : Wv + static_cast<int64_t>(r - kXDn) * R;
      rb[q] = *reinterpret_cast<const i16x8*>(W + kc + 8 * c);
    }
  };
  auto store_stage = [&]() {
    if (!fp8) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int idx = t + kGThreads * q;
        *reinterpret_cast<i16x8*>(As + (idx >> 3) * kGPitch + (idx & 7) * 16) = ra[q];
      }
    } else {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int idx = t + kGThreads * q;
        const int r = idx >> 2, c = idx & 3;
        const uint32_t w4[4] = {rc[q].x, rc[q].y, rc[q].z, rc[q].w};
        i16x8 lo, hi;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // E4M3 -> bf16 is exact (3 mantissa bits, exponent range inside bf16's)
          lo[e] = static_cast<short>(__float_as_uint(e4m3_to_f32((w4[e >> 2] >> (8 * (e & 3))) & 0xFF)) >> 16);
          hi[e] = static_cast<short>(__float_as_uint(e4m3_to_f32((w4[2 + (e >> 2)] >> (8 * (e & 3))) & 0xFF)) >> 16);
        }
        *reinterpret_cast<i16x8*>(As + r * kGPitch + c * 32) = lo;
        *reinterpret_cast<i16x8*>(As + r * kGPitch + c * 32 + 16) = hi;
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = t + kGThreads * q;
      *reinterpret_cast<i16x8*>(Bs + (idx >> 3) * kGPitch + (idx & 7) * 16) = rb[q];
    }
  };
  load_stage(0);
  for (int kc = 0; kc < R; kc += kGK) {
    store_stage();
    __syncthreads();
    if (kc + kGK < R) load_stage(kc + kGK);  // in flight during this stage's MFMAs
#pragma unroll
    for (int ks = 0; ks < kGK / 16; ++ks) {
      i16x8 af[2], bf[4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const i16x8*>(As + (64 * tm + 32 * i + n32) * kGPitch + (16 * ks + 8 * g) * 2);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        bf[jj] = *reinterpret_cast<const i16x8*>(Bs + (128 * tn + 32 * jj + n32) * kGPitch + (16 * ks + 8 * g) * 2);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[i][jj] = mfma(af[i], bf[jj], acc[i][jj]);
    }
    __syncthreads();
  }

  // epilogue: element e of acc[i][jj] is token 64 tm + 32 i + 8 (e / 4) + 4 g + e % 4,
  // column d = 32 jj + n32 of the wave's K (tn = 0) or V (tn = 1) block
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int d = 32 * jj + n32;
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int r = 64 * tm + 32 * i + 8 * e4 + 4 * g;  // tile-local token of element 4 e4
        uint16_t v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = f32_to_bf16(acc[i][jj][4 * e4 + e] * tok_scale[r + e]);
        if (tn == 1) {
          // V_expT[h][d][vperm(j)]: four consecutive tokens (a quad), one 8-byte store
          uint16_t* dst = v_expT + (static_cast<int64_t>(h) * kXDv + d) * ck + vperm(j0 + r);
          *reinterpret_cast<uint2*>(dst) = make_uint2(v[0] | (static_cast<uint32_t>(v[1]) << 16),
                                                      v[2] | (static_cast<uint32_t>(v[3]) << 16));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            k_exp[(static_cast<int64_t>(h) * ck + j0 + r + e) * kXDn + d] = v[e];
        }
      }
    }
  }
  // the rope part of the keys, shared by every head (written once)
  if (h == 0) {
    for (int idx = t; idx < kGTok * kXDr; idx += kGThreads) {
      const int r = idx / kXDr, c = idx % kXDr;
      const int j = j0 + r;
      uint16_t v = 0;
      if (j < ntok) {
        const int64_t row = cache_row(j);
        if (!fp8) {
          v = static_cast<const uint16_t*>(kv.data)[row * kv.D + R + c];
        } else {
          const uint8_t code = static_cast<const uint8_t*>(kv.data)[row * kv.D + R + c];
          v = f32_to_bf16(e4m3_to_f32(code) * kv.scale[row]);
        }
      }
      kpe[static_cast<int64_t>(j) * kXDr + c] = v;
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

  // tile loads: 5 chunks of 16 B per thread (K_exp 512, kpe 256, V^T 512)
  const uint16_t* kexp_h = a.k_exp + (static_cast<int64_t>(bz) * a.H + h) * ck * kXDn;
  const uint16_t* vexp_h = a.v_expT + (static_cast<int64_t>(bz) * a.H + h) * kXDv * ck;
  const uint16_t* kpe_b = a.kpe + static_cast<int64_t>(bz) * ck * kXDr;
  i16x8 ld[5];
  auto load_tile = [&](int tile) {
    const int j0 = tile * kAT;
#pragma unroll
    for (int q = 0; q < 5; ++q) {
      const int idx = t + 256 * q;
      if (idx < 512) {  // K_exp: key idx / 16, chunk idx % 16
        ld[q] = *reinterpret_cast<const i16x8*>(kexp_h + static_cast<int64_t>(j0 + (idx >> 4)) * kXDn + 8 * (idx & 15));
      } else if (idx < 768) {  // kpe: key (idx - 512) / 8, chunk % 8
        const int k = idx - 512;
        ld[q] = *reinterpret_cast<const i16x8*>(kpe_b + static_cast<int64_t>(j0 + (k >> 3)) * kXDr + 8 * (k & 7));
      } else {  // V^T: row (idx - 768) / 4, chunk % 4
        const int k = idx - 768;
        ld[q] = *reinterpret_cast<const i16x8*>(vexp_h + static_cast<int64_t>(k >> 2) * ck + j0 + 8 * (k & 3));
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 5; ++q) {
      const int idx = t + 256 * q;
      if (idx < 512) {
        *reinterpret_cast<i16x8*>(Ks[buf] + (idx >> 4) * kAKPitch + 16 * (idx & 15)) = ld[q];
      } else if (idx < 768) {
        const int k = idx - 512;
        *reinterpret_cast<i16x8*>(Ks[buf] + (k >> 3) * kAKPitch + kXDn * 2 + 16 * (k & 7)) = ld[q];
      } else {
        const int k = idx - 768;
        *reinterpret_cast<i16x8*>(Vs[buf] + (k >> 2) * kAVPitch + 16 * (k & 3)) = ld[q];
      }
    }
  };

  f32x16 o[kXDv / 32];
#pragma unroll
  for (int db = 0; db < kXDv / 32; ++db) o[db] = f32x16{};
  float m_ref = -INFINITY, l_sum = 0.f;
  const float c = a.scale_log2;

  // S^T = K Q^T (keys x rows) of the tile in buffer `buf`
  auto scores = [&](int buf) {
    f32x16 sc = f32x16{};
    const char* kb = Ks[buf] + n32 * kAKPitch + 16 * g;
#pragma unroll
    for (int st = 0; st < kXDq / 16; ++st) sc = mfma(*reinterpret_cast<const i16x8*>(kb + 32 * st), qf[st], sc);
    return sc;
  };

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
  for (int tile = tile_lo; tile < tile_hi; ++tile) {
    const int i = tile - tile_lo;
    const int cur = i % 3, nxt = (i + 1) % 3, far = (i + 2) % 3;
    const bool has_next = tile + 1 < tile_hi, has_far = tile + 2 < tile_hi;
    if (has_far) load_tile(tile + 2);  // in flight during this tile's math
    f32x16 s_next = f32x16{};
    if (has_next) s_next = scores(nxt);
    f32x16 s = s_cur;
    // scale, mask, tile maximum (a row's 32 keys sit in lanes n32 and n32 + 32)
    const int64_t tile_key = k0 + static_cast<int64_t>(tile) * kAT;
    const bool full = row_ok && tile_key + kAT - 1 <= P + r_lo + 32 * wave &&  // every row of the wave sees the whole tile
                      tile_key + kAT <= k0 + ntok &&
                      (a.window <= 0 || tile_key > P + r_lo + 32 * wave + 31 - a.window);
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float x = s[e] * c;
      if (!full) {
        const int64_t key = tile_key + 8 * (e >> 2) + 4 * g + (e & 3);
        const bool vis = row_ok && key <= pos && key < k0 + ntok && (a.window <= 0 || key > pos - a.window);
        x = vis ? x : -INFINITY;
      }
      s[e] = x;
      mx = fmaxf(mx, x);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
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
    // p = 2^(s - m_ref) <= 2^8 (v_exp_f32; masked keys give exp2(-inf) = 0),
    // rounded to bf16 by the hardware conversion (nearest even)
    bf16x8 pb[2];
    const float m_use = m_ref == -INFINITY ? 0.f : m_ref;  // a row with nothing visible yet
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = __builtin_amdgcn_exp2f(s[e] - m_use);
      l_sum += p;
      pb[e >> 3][e & 7] = static_cast<__bf16>(p);
    }
    // O^T += V^T P^T; MFMA k-slot 8 g + j of key half kk is key 16 kk + 4 g + j
    // (j < 4) or 16 kk + 8 + 4 g + (j - 4): the keys this lane's P registers
    // hold, which the quad-swapped V^T columns 16 kk + 8 g .. + 7 hold in order
    const char* vb = Vs[cur] + n32 * kAVPitch + 16 * g;
#pragma unroll
    for (int db = 0; db < kXDv / 32; ++db) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        o[db] = mfma(*reinterpret_cast<const i16x8*>(vb + 32 * db * kAVPitch + 32 * kk),
                     __builtin_bit_cast(i16x8, pb[kk]), o[db]);
    }
    // buffer `far` last held tile t - 1, whose values were read before the
    // barrier that ended the previous step
    if (has_far) store_tile(far);
    __syncthreads();
    s_cur = s_next;
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
  return kv.Dr == kXDr && kv.R % kGK == 0 && Dn == kXDn && Dv == kXDv && H >= 1 && H <= 1024;
}

hipError_t launch_prefill_expanded_pass(const XPassArgs& a, int32_t max_q_len, hipStream_t s) {
  hipLaunchKernelGGL(kv_expand_kernel, dim3(a.ck / kGTok, a.H, a.batch), dim3(kGThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_expanded_kernel, dim3((max_q_len + 127) / 128, a.H, a.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
