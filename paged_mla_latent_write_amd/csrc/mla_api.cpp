// Host side of the C ABI: argument validation, workspace carving and launch
// sequencing.  No device memory is allocated here and nothing synchronises
// with the host; every launch goes to the caller's stream.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <vector>

#include "../../include/mla.h"
#include "mla_internal.h"

namespace {

using mla::AttnArgs;
using mla::CacheView;

constexpr size_t kAlign = 256;
constexpr int kMaxDevices = 64;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Compute units of the current device, cached per device id.  The cache is
// an array of atomics: concurrent first calls from several threads each
// query the device and store the same value.
std::atomic<int> g_cu_count[kMaxDevices];

}  // namespace

int mla::current_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev < kMaxDevices) {
    const int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return -1;
  if (dev < kMaxDevices) g_cu_count[dev].store(n, std::memory_order_relaxed);
  return n;
}

namespace {

bool page_size_ok(int ps) { return ps == 16 || ps == 32 || ps == 64 || ps == 128; }

mla_status check_cache(const mla_cache* c) {
  if (!c || !c->data) return MLA_ERR_INVALID_ARGUMENT;
  if (c->num_layers <= 0 || c->num_pages <= 0 || c->page_size <= 0 || c->kv_lora_rank <= 0 ||
      c->qk_rope_dim < 0)
    return MLA_ERR_INVALID_ARGUMENT;
  if (c->dtype != MLA_KV_BF16 && c->dtype != MLA_KV_FP8_E4M3) return MLA_ERR_INVALID_ARGUMENT;
  if (c->dtype == MLA_KV_FP8_E4M3 && !c->scale) return MLA_ERR_INVALID_ARGUMENT;
  if (!page_size_ok(c->page_size)) return MLA_ERR_UNSUPPORTED;
  const int D = c->kv_lora_rank + c->qk_rope_dim;
  if (c->kv_lora_rank % 8 != 0 || c->qk_rope_dim % 8 != 0 || D < 8 || D > 1024)
    return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

mla_status check_attn(const mla_attn* a) {
  if (!a) return MLA_ERR_INVALID_ARGUMENT;
  if (a->num_heads <= 0 || a->num_heads > 1024) return MLA_ERR_INVALID_ARGUMENT;
  if (a->w_uk && (a->qk_nope_dim <= 0 || a->qk_nope_dim > 1024)) return MLA_ERR_INVALID_ARGUMENT;
  if (a->w_uv && (a->v_head_dim <= 0 || a->v_head_dim > 1024)) return MLA_ERR_INVALID_ARGUMENT;
  if (!isfinite(a->scale)) return MLA_ERR_INVALID_ARGUMENT;
  if (a->num_workgroups < 0) return MLA_ERR_INVALID_ARGUMENT;
  return MLA_OK;
}

size_t elem_bytes(int dtype) { return dtype == MLA_KV_BF16 ? 2 : 1; }

// Workspace regions (byte offsets from the workspace base).
struct Layout {
  int G = 0;
  size_t q_lat = 0, o_lat = 0, lse = 0, o_scale = 0, item_b = 0, item_lo = 0, item_hi = 0,
         tile_start = 0, wg_tile = 0, wg_item = 0, item_wg = 0, part_o = 0, part_lse = 0,
         part_scale = 0, total = 0;
};

// Returns false when the number of workgroups cannot be determined.
bool make_layout(const mla_cache* c, const mla_attn* a, int64_t num_items, Layout* L) {
  int G = a->num_workgroups;
  if (G <= 0) {
    G = mla::current_cu_count();
    if (G <= 0) return false;
  }
  const int64_t H = a->num_heads, R = c->kv_lora_rank;
  size_t off = 0;
  L->G = G;
  L->q_lat = off;
  if (a->w_uk) off = align_up(off + sizeof(uint16_t) * num_items * H * R);
  L->o_lat = off;
  off = align_up(off + sizeof(float) * num_items * H * R);
  L->lse = off;
  off = align_up(off + sizeof(float) * num_items * H);
  L->o_scale = off;
  off = align_up(off + sizeof(float) * num_items * H);
  L->item_b = off;
  off = align_up(off + sizeof(int32_t) * num_items);
  L->item_lo = off;
  off = align_up(off + sizeof(int32_t) * num_items);
  L->item_hi = off;
  off = align_up(off + sizeof(int32_t) * num_items);
  L->tile_start = off;
  off = align_up(off + sizeof(int32_t) * (num_items + 1));
  L->wg_tile = off;
  off = align_up(off + sizeof(int32_t) * (G + 1));
  L->wg_item = off;
  off = align_up(off + sizeof(int32_t) * G);
  L->item_wg = off;
  off = align_up(off + sizeof(int32_t) * 2 * num_items);
  L->part_o = off;
  off = align_up(off + sizeof(uint16_t) * 2 * G * H * R);  // bf16 partials
  L->part_lse = off;
  off = align_up(off + sizeof(float) * 2 * G * H);
  L->part_scale = off;
  off = align_up(off + sizeof(float) * 2 * G * H);
  L->total = off;
  return true;
}

// Index-list attention workspace: per chunk of query rows, the compacted
// rows (and fp8 scales), kept counts and identity block tables, then the
// dense decode workspace for one chunk.
constexpr size_t kSparseCompactBudget = size_t{512} << 20;

struct SparseLayout {
  int64_t chunk = 0;
  int32_t rows_per_item = 0, nblk = 0;
  size_t data = 0, scale = 0, ctx = 0, bt = 0, dense = 0, total = 0;
  Layout dense_layout;
};

mla_cache compact_cache_desc(const mla_cache* c, void* data, float* scale, int64_t items, int32_t nblk) {
  mla_cache cc = *c;
  cc.data = data;
  cc.scale = scale;
  cc.num_layers = 1;
  cc.num_pages = static_cast<int32_t>(items * nblk);
  cc.page_size = mla::kCompactPage;
  return cc;
}

bool make_sparse_layout(const mla_cache* c, const mla_attn* a, int64_t num_q, int32_t topk,
                        SparseLayout* S) {
  const int64_t rows = std::max<int64_t>(mla::kCompactPage,
                                         (static_cast<int64_t>(topk) + mla::kCompactPage - 1) /
                                             mla::kCompactPage * mla::kCompactPage);
  if (rows > (1 << 24)) return false;
  S->rows_per_item = static_cast<int32_t>(rows);
  S->nblk = static_cast<int32_t>(rows / mla::kCompactPage);
  const bool fp8 = c->dtype == MLA_KV_FP8_E4M3;
  const size_t row_bytes = static_cast<size_t>(c->kv_lora_rank + c->qk_rope_dim) * elem_bytes(c->dtype);
  const size_t per_item = rows * row_bytes + (fp8 ? rows * 4 : 0);
  S->chunk = std::max<int64_t>(1, std::min<int64_t>(num_q, kSparseCompactBudget / per_item));
  if (S->chunk * S->nblk >= (1ll << 31)) return false;
  size_t off = 0;
  S->data = off;
  off = align_up(off + S->chunk * rows * row_bytes);
  S->scale = off;
  if (fp8) off = align_up(off + S->chunk * rows * sizeof(float));
  S->ctx = off;
  off = align_up(off + S->chunk * sizeof(int32_t));
  S->bt = off;
  off = align_up(off + S->chunk * S->nblk * sizeof(int32_t));
  S->dense = off;
  const mla_cache cc = compact_cache_desc(c, nullptr, nullptr, S->chunk, S->nblk);
  if (!make_layout(&cc, a, S->chunk, &S->dense_layout)) return false;
  S->total = off + S->dense_layout.total;
  return true;
}

// One layer of the cache as the kernels see it.
CacheView layer_view(const mla_cache* cache, int32_t layer_idx) {
  const int R = cache->kv_lora_rank;
  const int64_t layer_elems =
      static_cast<int64_t>(cache->num_pages) * cache->page_size * (R + cache->qk_rope_dim);
  CacheView kv;
  kv.data = static_cast<const char*>(cache->data) + layer_idx * layer_elems * elem_bytes(cache->dtype);
  kv.scale = cache->dtype == MLA_KV_FP8_E4M3
                 ? cache->scale + static_cast<int64_t>(layer_idx) * cache->num_pages * cache->page_size
                 : nullptr;
  kv.dtype = cache->dtype == MLA_KV_BF16 ? mla::kKvBf16 : mla::kKvFp8;
  kv.num_pages = cache->num_pages;
  kv.page_size = cache->page_size;
  kv.page_shift = __builtin_ctz(static_cast<unsigned>(cache->page_size));
  kv.R = R;
  kv.Dr = cache->qk_rope_dim;
  kv.D = R + cache->qk_rope_dim;
  return kv;
}

// Expanded-form prefill workspace: the up-projected keys and values of one
// launch pair (a group of requests, or one request's pass), and, when a
// request's visible range needs several passes, the running per-(row, head)
// output state.  The keys' and values' share is bounded by kXBudget.
struct XLayout {
  int32_t ck = 0;     // keys per pass (a multiple of 256)
  int32_t group = 0;  // requests per launch pair
  int32_t npass = 0;  // passes per request
  size_t k_exp = 0, v_exp = 0, kpe = 0, o_acc = 0, m_acc = 0, l_acc = 0, total = 0;
};

constexpr size_t kXBudget = size_t{1280} << 20;

// `need` bounds the keys one request's rows can see: the context, or, with a
// window, the chunk (at most q_bound rows) plus the window.  The size query
// has no max_q_len and bounds the chunk by total_q; the call uses max_q_len
// when that layout fits the workspace it is given.
XLayout make_xlayout(const mla_attn* a, int64_t batch, int64_t total_q, int64_t max_ctx,
                     int64_t q_bound) {
  XLayout X;
  const int64_t H = a->num_heads;
  const int64_t B = std::max<int64_t>(batch, 1);
  const int64_t need = std::max<int64_t>(
      1, a->window > 0 ? std::min<int64_t>(max_ctx, q_bound + a->window - 1) : max_ctx);
  const size_t per_key = sizeof(uint16_t) * (H * 256 + 64);  // K and V of every head, and the rope part
  const int64_t ck_full = (need + 255) / 256 * 256;
  if (static_cast<size_t>(ck_full) * per_key <= kXBudget) {
    X.ck = static_cast<int32_t>(ck_full);
    X.group = static_cast<int32_t>(std::min<int64_t>(B, kXBudget / (ck_full * per_key)));
    X.npass = 1;
  } else {
    X.ck = static_cast<int32_t>(std::max<int64_t>(256, static_cast<int64_t>(kXBudget / per_key) / 256 * 256));
    X.group = 1;
    X.npass = static_cast<int32_t>((need + X.ck - 1) / X.ck);
  }
  size_t off = 0;
  X.k_exp = off;
  off = align_up(off + sizeof(uint16_t) * X.group * H * X.ck * 128);
  X.v_exp = off;
  off = align_up(off + sizeof(uint16_t) * X.group * H * 128 * X.ck);
  X.kpe = off;
  off = align_up(off + sizeof(uint16_t) * X.group * X.ck * 64);
  const int64_t st_rows = X.npass > 1 ? total_q : 0;
  X.o_acc = off;
  off = align_up(off + sizeof(float) * st_rows * H * 128);
  X.m_acc = off;
  off = align_up(off + sizeof(float) * st_rows * H);
  X.l_acc = off;
  off = align_up(off + sizeof(float) * st_rows * H);
  X.total = off;
  return X;
}

// Which form mla_prefill_chunk runs.  The expanded one needs both weights and
// a shape its kernels take; it runs when asked for, or, without a flag, for
// windowed calls whose chunks average at least 64 rows: there it does a small
// up-projection (chunk + window keys) instead of per-row latent outputs
// (measured on the mixed step's window-128 layer: 0.61 ms against 1.15 ms).
// Full-attention prefill stays absorbed unless asked for (9.6 ms against
// 9.1 ms on the mixed step's full layers).
bool prefill_route_expanded(const mla_cache* c, const mla_attn* a, int32_t batch, int32_t total_q) {
  if (a->flags & (MLA_FLAG_GENERIC_KERNELS | MLA_FLAG_PREFILL_ABSORBED)) return false;
  if (!a->w_uk || !a->w_uv) return false;
  if (!(a->scale > 0.f)) return false;  // (the kernel scales the tile maximum of the raw scores)
  const CacheView kv = layer_view(c, 0);
  if (!mla::prefill_expanded_supported(kv, a->num_heads, a->qk_nope_dim, a->v_head_dim)) return false;
  if (a->flags & MLA_FLAG_PREFILL_EXPANDED) return true;
  return static_cast<int64_t>(total_q) >= 64 * static_cast<int64_t>(batch);
}

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

mla_status to_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

// ---- MLA_DEBUG_CHECK: host-side validation of device-array contents ----
//
// With the environment variable MLA_DEBUG_CHECK set to anything but "" or
// "0", each call first copies its index arrays (context lengths, the used
// prefix of the block tables, query_start_loc, slot mappings) to the host,
// waits for them, and checks the caller contract the kernels otherwise only
// clamp against.  A violation returns MLA_ERR_INVALID_ARGUMENT and enqueues
// nothing.  The check synchronises the stream, so it is refused
// (MLA_ERR_UNSUPPORTED) while the stream is being captured into a graph.
// The contract is the one whose violation the pages report as a crash
// ("[unified-memory] Let Kimi-Linear use the paged MLA attention backends",
// Two pre-existing issues, item 1: a query count that disagrees with the
// last query_start_loc entry).

bool debug_check_enabled() {
  const char* v = getenv("MLA_DEBUG_CHECK");
  return v != nullptr && v[0] != 0 && !(v[0] == '0' && v[1] == 0);
}

mla_status debug_prepare(hipStream_t s) {
  if (s == nullptr) return MLA_OK;  // the null stream cannot be captured
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess) return MLA_ERR_HIP;
  return cs == hipStreamCaptureStatusNone ? MLA_OK : MLA_ERR_UNSUPPORTED;
}

template <typename T>
mla_status fetch(std::vector<T>* dst, const T* src, size_t n, hipStream_t s) {
  dst->assign(n, T{});
  if (n == 0) return MLA_OK;
  if (hipMemcpyAsync(dst->data(), src, n * sizeof(T), hipMemcpyDeviceToHost, s) != hipSuccess)
    return MLA_ERR_HIP;
  return hipStreamSynchronize(s) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

// Attention calls: 0 <= n_b <= max_blocks * page_size; the first
// ceil(n_b / page_size) block-table entries of each request name a page of
// the cache; for prefill, query_start_loc starts at 0, does not decrease,
// ends at total_q_tokens, and each request's chunk fits its context and
// max_q_len.
mla_status debug_check_attention(int mode, const mla_cache* c, const int32_t* block_tables,
                                 int32_t max_blocks, const int32_t* context_lens, int32_t batch,
                                 const int32_t* qsl, int32_t total_q, int32_t max_q_len,
                                 hipStream_t s) {
  mla_status st = debug_prepare(s);
  if (st != MLA_OK) return st;
  std::vector<int32_t> ctx, bt, q;
  if ((st = fetch(&ctx, context_lens, batch, s)) != MLA_OK) return st;
  if ((st = fetch(&bt, block_tables, static_cast<size_t>(batch) * max_blocks, s)) != MLA_OK)
    return st;
  const int64_t ps = c->page_size;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t n = ctx[b];
    if (n < 0 || n > static_cast<int64_t>(max_blocks) * ps) return MLA_ERR_INVALID_ARGUMENT;
    for (int64_t j = 0; j < (n + ps - 1) / ps; ++j) {
      const int32_t pg = bt[static_cast<size_t>(b) * max_blocks + j];
      if (pg < 0 || pg >= c->num_pages) return MLA_ERR_INVALID_ARGUMENT;
    }
  }
  if (mode == mla::kPlanPrefill) {
    if ((st = fetch(&q, qsl, static_cast<size_t>(batch) + 1, s)) != MLA_OK) return st;
    if (q[0] != 0 || q[batch] != total_q) return MLA_ERR_INVALID_ARGUMENT;
    for (int32_t b = 0; b < batch; ++b) {
      const int64_t m = static_cast<int64_t>(q[b + 1]) - q[b];
      if (m < 0 || m > ctx[b] || m > max_q_len) return MLA_ERR_INVALID_ARGUMENT;
    }
  }
  return MLA_OK;
}

// Cache writes: every slot is negative (a pad row) or names a slot of the
// cache, and the non-negative slots of one call are distinct.
mla_status debug_check_slots(const mla_cache* c, const int64_t* slot_mapping, int32_t num_tokens,
                             hipStream_t s) {
  mla_status st = debug_prepare(s);
  if (st != MLA_OK) return st;
  std::vector<int64_t> sl;
  if ((st = fetch(&sl, slot_mapping, num_tokens, s)) != MLA_OK) return st;
  const int64_t slots = static_cast<int64_t>(c->num_pages) * c->page_size;
  std::vector<uint8_t> seen(static_cast<size_t>(slots), 0);
  for (const int64_t v : sl) {
    if (v < 0) continue;
    if (v >= slots || seen[static_cast<size_t>(v)]) return MLA_ERR_INVALID_ARGUMENT;
    seen[static_cast<size_t>(v)] = 1;
  }
  return MLA_OK;
}

// Shared by decode (one item per request) and prefill (one item per query row).
mla_status run_attention(int mode, const mla_cache* cache, int32_t layer_idx, const mla_attn* attn,
                         const void* q_nope, int64_t qn_st, int64_t qn_sh, const void* q_pe,
                         int64_t qp_st, int64_t qp_sh, const int32_t* qsl, int32_t num_items,
                         const int32_t* block_tables, int32_t max_blocks,
                         const int32_t* context_lens, int32_t batch, int32_t max_q_len,
                         void* out, float* lse_or_null, void* workspace, size_t workspace_bytes,
                         void* stream, const mla::TokenWrite* tw = nullptr) {
  mla_status st = check_cache(cache);
  if (st != MLA_OK) return st;
  if ((st = check_attn(attn)) != MLA_OK) return st;
  if (layer_idx < 0 || layer_idx >= cache->num_layers) return MLA_ERR_INVALID_ARGUMENT;
  if (batch < 0 || num_items < 0 || max_blocks <= 0) return MLA_ERR_INVALID_ARGUMENT;
  if (batch == 0 || num_items == 0) return MLA_OK;
  if (!q_nope || !q_pe || !block_tables || !context_lens || !out) return MLA_ERR_INVALID_ARGUMENT;
  if (mode == mla::kPlanPrefill && !qsl) return MLA_ERR_INVALID_ARGUMENT;
  const int64_t max_ctx64 = static_cast<int64_t>(max_blocks) * cache->page_size;
  if (max_ctx64 > (1ll << 30)) return MLA_ERR_UNSUPPORTED;
  // the tile counts are int32 on the device
  if (static_cast<int64_t>(num_items) * (max_ctx64 / mla::kTile + 1) >= (1ll << 31))
    return MLA_ERR_UNSUPPORTED;

  Layout L;
  if (!make_layout(cache, attn, num_items, &L)) return MLA_ERR_HIP;
  if (!workspace || workspace_bytes < L.total) return MLA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return MLA_ERR_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (debug_check_enabled()) {
    st = debug_check_attention(mode, cache, block_tables, max_blocks, context_lens, batch, qsl,
                               num_items, max_q_len, s);
    if (st != MLA_OK) return st;
  }
  const int H = attn->num_heads, R = cache->kv_lora_rank;

  const int64_t layer_elems =
      static_cast<int64_t>(cache->num_pages) * cache->page_size * (R + cache->qk_rope_dim);
  CacheView kv;
  kv.data = static_cast<const char*>(cache->data) + layer_idx * layer_elems * elem_bytes(cache->dtype);
  kv.scale = cache->dtype == MLA_KV_FP8_E4M3
                 ? cache->scale + static_cast<int64_t>(layer_idx) * cache->num_pages * cache->page_size
                 : nullptr;
  kv.dtype = cache->dtype == MLA_KV_BF16 ? mla::kKvBf16 : mla::kKvFp8;
  kv.num_pages = cache->num_pages;
  kv.page_size = cache->page_size;
  kv.page_shift = __builtin_ctz(static_cast<unsigned>(cache->page_size));
  kv.R = R;
  kv.Dr = cache->qk_rope_dim;
  kv.D = R + cache->qk_rope_dim;

  hipError_t e;
  const uint16_t* q_lat = static_cast<const uint16_t*>(q_nope);
  int64_t ql_st = qn_st, ql_sh = qn_sh;
  const bool generic = (attn->flags & MLA_FLAG_GENERIC_KERNELS) != 0;
  const auto aligned16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  mla::Plan plan;
  plan.item_b = at<int32_t>(workspace, L.item_b);
  plan.item_lo = at<int32_t>(workspace, L.item_lo);
  plan.item_hi = at<int32_t>(workspace, L.item_hi);
  plan.tile_start = at<int32_t>(workspace, L.tile_start);
  plan.wg_tile = at<int32_t>(workspace, L.wg_tile);
  plan.wg_item = at<int32_t>(workspace, L.wg_item);
  plan.item_wg = at<int32_t>(workspace, L.item_wg);
  plan.G = L.G;
  const mla::PlanArgs pa{mode, batch, num_items, context_lens, qsl, attn->window,
                         static_cast<int32_t>(max_ctx64), plan};
  bool planned = false;  // the MFMA absorb launch computes the plan too

  const bool absorb_mfma = attn->w_uk && !generic && mla::absorb_mfma_supported(attn->qk_nope_dim, R) &&
                           aligned16(q_nope) && aligned16(attn->w_uk) && qn_st % 8 == 0 && qn_sh % 8 == 0;
  if (tw && tw->T > 0 && !absorb_mfma) {
    // new tokens to write, and no absorb launch to carry them: a write launch first
    e = mla::launch_write_kv(tw->cache, tw->scale, tw->dtype, tw->num_slots, tw->R, tw->Dr, tw->c_kv,
                             tw->c_stride, tw->k_pe, tw->k_stride, tw->slots, tw->T, s);
    if (e != hipSuccess) return MLA_ERR_HIP;
  }
  if (attn->w_uk) {
    uint16_t* ql = at<uint16_t>(workspace, L.q_lat);
    const bool mfma = absorb_mfma;
    e = mfma ? mla::launch_absorb_mfma(static_cast<const uint16_t*>(q_nope), qn_st, qn_sh,
                                       static_cast<const uint16_t*>(attn->w_uk), num_items, H,
                                       attn->qk_nope_dim, R, ql, &pa, tw, s)
             : mla::launch_absorb(static_cast<const uint16_t*>(q_nope), qn_st, qn_sh,
                                  static_cast<const uint16_t*>(attn->w_uk), num_items, H,
                                  attn->qk_nope_dim, R, ql, s);
    if (e != hipSuccess) return MLA_ERR_HIP;
    planned = mfma;
    q_lat = ql;
    ql_st = static_cast<int64_t>(H) * R;
    ql_sh = R;
  }
  if (!planned) {
    e = mla::launch_plan(mode, batch, num_items, context_lens, qsl, attn->window,
                         static_cast<int32_t>(max_ctx64), plan, s);
    if (e != hipSuccess) return MLA_ERR_HIP;
  }

  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.kv = kv;
  a.q_lat = q_lat;
  a.q_lat_st = ql_st;
  a.q_lat_sh = ql_sh;
  a.q_pe = static_cast<const uint16_t*>(q_pe);
  a.q_pe_st = qp_st;
  a.q_pe_sh = qp_sh;
  a.block_tables = block_tables;
  a.max_blocks = max_blocks;
  a.item_b = plan.item_b;
  a.item_lo = plan.item_lo;
  a.item_hi = plan.item_hi;
  a.tile_start = plan.tile_start;
  a.wg_tile = plan.wg_tile;
  a.wg_item = plan.wg_item;
  a.item_wg = plan.item_wg;
  a.num_items = num_items;
  a.H = H;
  a.G = L.G;
  a.scale_log2 = attn->scale * 1.4426950408889634f;
  a.o_lat = at<float>(workspace, L.o_lat);
  a.lse = lse_or_null ? lse_or_null : at<float>(workspace, L.lse);
  a.o_scale = at<float>(workspace, L.o_scale);
  a.part_o = at<uint16_t>(workspace, L.part_o);
  a.part_lse = at<float>(workspace, L.part_lse);
  a.part_scale = at<float>(workspace, L.part_scale);

  // (the MFMA kernel takes the tile maximum on unscaled scores: scale > 0)
  const bool use_mfma = !generic && mla::mfma_attn_supported(kv, H) && attn->scale > 0.f &&
                        (ql_st % 8 == 0) && (ql_sh % 8 == 0) && (qp_st % 8 == 0) &&
                        (qp_sh % 8 == 0) && aligned16(q_lat) && aligned16(q_pe);
  if (attn->kernel_events[0] &&
      hipEventRecord(static_cast<hipEvent_t>(attn->kernel_events[0]), s) != hipSuccess)
    return MLA_ERR_HIP;
  // (the fp8 kernel copies 16-byte runs of scales: 4 per run, 16-byte aligned)
  const bool use_mfma_fp8 = !generic && mla::mfma_fp8_attn_supported(kv, H) && attn->scale > 0.f &&
                            (ql_st % 8 == 0) && (ql_sh % 8 == 0) && (qp_st % 8 == 0) &&
                            (qp_sh % 8 == 0) && aligned16(q_lat) && aligned16(q_pe) &&
                            aligned16(kv.scale);
  const bool use_f8mfma = (attn->flags & MLA_FLAG_FP8_MFMA) != 0 && !generic &&
                         mla::f8mfma_attn_supported(kv, H) && (ql_st % 8 == 0) && (ql_sh % 8 == 0) &&
                         (qp_st % 8 == 0) && (qp_sh % 8 == 0) && aligned16(q_lat) && aligned16(q_pe) &&
                         aligned16(kv.scale);
  if (use_f8mfma) {
    e = mla::launch_attn_f8mfma(a, s);
  } else if (use_mfma_fp8) {
    e = mla::launch_attn_mfma_fp8(a, s);
  } else {
    e = use_mfma ? mla::launch_attn_mfma(a, s) : mla::launch_attn_generic(a, s);
  }
  if (e != hipSuccess) return MLA_ERR_HIP;
  if (attn->kernel_events[1] &&
      hipEventRecord(static_cast<hipEvent_t>(attn->kernel_events[1]), s) != hipSuccess)
    return MLA_ERR_HIP;
  if (attn->w_uv && !generic && mla::combine_up_project_supported(R, attn->v_head_dim) &&
      aligned16(attn->w_uv))
    return to_status(mla::launch_combine_up_project(a, static_cast<const uint16_t*>(attn->w_uv),
                                                    attn->v_head_dim, static_cast<uint16_t*>(out), s));
  e = mla::launch_combine_segments(a, s);
  if (e != hipSuccess) return MLA_ERR_HIP;

  if (attn->w_uv) {
    const bool mfma = !generic && mla::up_project_mfma_supported(R, attn->v_head_dim) &&
                      aligned16(attn->w_uv);
    e = mfma ? mla::launch_up_project_mfma(a.o_lat, a.o_scale,
                                           static_cast<const uint16_t*>(attn->w_uv), num_items, H,
                                           R, attn->v_head_dim, static_cast<uint16_t*>(out), s)
             : mla::launch_up_project(a.o_lat, a.o_scale, static_cast<const uint16_t*>(attn->w_uv),
                                      num_items, H, R, attn->v_head_dim,
                                      static_cast<uint16_t*>(out), s);
  } else {
    e = mla::launch_latent_out(a.o_lat, a.o_scale, num_items, H, R, static_cast<uint16_t*>(out), s);
  }
  return to_status(e);
}

// Expanded-form prefill: per group of requests (or per request, in passes),
// an up-projection launch and an attention launch that merges into the
// running state (no host sync: the device reads lengths and row ranges).
mla_status run_prefill_expanded(const mla_cache* cache, int32_t layer_idx, const mla_attn* attn,
                                const void* q_nope, int64_t qn_st, int64_t qn_sh, const void* q_pe,
                                int64_t qp_st, int64_t qp_sh, const int32_t* qsl, int32_t total_q,
                                int32_t max_q_len, const int32_t* block_tables, int32_t max_blocks,
                                const int32_t* context_lens, int32_t batch, void* out,
                                float* lse_or_null, void* workspace, size_t workspace_bytes,
                                void* stream) {
  if (layer_idx < 0 || layer_idx >= cache->num_layers) return MLA_ERR_INVALID_ARGUMENT;
  if (batch < 0 || max_blocks <= 0) return MLA_ERR_INVALID_ARGUMENT;
  if (batch == 0 || total_q == 0) return MLA_OK;
  if (!q_nope || !q_pe || !qsl || !block_tables || !context_lens || !out)
    return MLA_ERR_INVALID_ARGUMENT;
  const int64_t max_ctx64 = static_cast<int64_t>(max_blocks) * cache->page_size;
  if (max_ctx64 > (1ll << 30)) return MLA_ERR_UNSUPPORTED;
  const auto aligned16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  const CacheView kv = layer_view(cache, layer_idx);
  if (!aligned16(q_nope) || !aligned16(q_pe) || qn_st % 8 || qn_sh % 8 || qp_st % 8 || qp_sh % 8 ||
      !aligned16(attn->w_uk) || !aligned16(attn->w_uv) || !aligned16(kv.data) || !aligned16(out))
    return MLA_ERR_UNSUPPORTED;
  XLayout X = make_xlayout(attn, batch, total_q, max_ctx64, max_q_len);
  if (X.total > workspace_bytes) X = make_xlayout(attn, batch, total_q, max_ctx64, total_q);
  if (!workspace || workspace_bytes < X.total) return MLA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return MLA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (debug_check_enabled()) {
    const mla_status st = debug_check_attention(mla::kPlanPrefill, cache, block_tables, max_blocks,
                                                context_lens, batch, qsl, total_q, max_q_len, s);
    if (st != MLA_OK) return st;
  }
  if (max_q_len == 0) return MLA_OK;
  mla::XPassArgs a;
  memset(&a, 0, sizeof(a));
  a.kv = kv;
  a.block_tables = block_tables;
  a.max_blocks = max_blocks;
  a.max_ctx = max_ctx64;
  a.context_lens = context_lens;
  a.query_start_loc = qsl;
  a.window = attn->window;
  a.H = attn->num_heads;
  a.total_q = total_q;
  a.w_uk = static_cast<const uint16_t*>(attn->w_uk);
  a.w_uv = static_cast<const uint16_t*>(attn->w_uv);
  a.q_nope = static_cast<const uint16_t*>(q_nope);
  a.qn_st = qn_st;
  a.qn_sh = qn_sh;
  a.q_pe = static_cast<const uint16_t*>(q_pe);
  a.qp_st = qp_st;
  a.qp_sh = qp_sh;
  a.scale_log2 = attn->scale * 1.4426950408889634f;
  a.k_exp = at<uint16_t>(workspace, X.k_exp);
  a.v_expT = at<uint16_t>(workspace, X.v_exp);
  a.kpe = at<uint16_t>(workspace, X.kpe);
  a.o_acc = at<float>(workspace, X.o_acc);
  a.m_acc = at<float>(workspace, X.m_acc);
  a.l_acc = at<float>(workspace, X.l_acc);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse_or_null;
  a.ck = X.ck;
  if (attn->kernel_events[0] &&
      hipEventRecord(static_cast<hipEvent_t>(attn->kernel_events[0]), s) != hipSuccess)
    return MLA_ERR_HIP;
  for (int32_t b0 = 0; b0 < batch; b0 += X.group) {
    a.b0 = b0;
    a.batch = std::min(X.group, batch - b0);
    for (int j = 0; j < X.npass; ++j) {
      a.pass = j;
      if (mla::launch_prefill_expanded_pass(a, max_q_len, s) != hipSuccess) return MLA_ERR_HIP;
    }
  }
  if (attn->kernel_events[1] &&
      hipEventRecord(static_cast<hipEvent_t>(attn->kernel_events[1]), s) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

}  // namespace

extern "C" {

const char* mla_status_string(mla_status status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARGUMENT: return "MLA_ERR_INVALID_ARGUMENT";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
  }
  return "MLA_ERR_UNKNOWN";
}

const char* mla_version(void) { return "paged-mla-gfx950 0.1"; }

// mla_write_kv's argument checks (and, with MLA_DEBUG_CHECK, its slot check);
// on success *w describes the write (w->T == 0: nothing to write).
static mla_status prepare_write(const mla_cache* cache, int32_t layer_idx, const void* c_kv, int64_t c_kv_row_stride,
                         const void* k_pe, int64_t k_pe_row_stride, const int64_t* slot_mapping,
                         int32_t num_tokens, hipStream_t s, mla::TokenWrite* w) {
  mla_status st = check_cache(cache);
  if (st != MLA_OK) return st;
  if (layer_idx < 0 || layer_idx >= cache->num_layers || num_tokens < 0)
    return MLA_ERR_INVALID_ARGUMENT;
  memset(w, 0, sizeof(*w));
  if (num_tokens == 0) return MLA_OK;
  if (!c_kv || !slot_mapping || (cache->qk_rope_dim > 0 && !k_pe)) return MLA_ERR_INVALID_ARGUMENT;
  if (c_kv_row_stride < cache->kv_lora_rank || k_pe_row_stride < cache->qk_rope_dim)
    return MLA_ERR_INVALID_ARGUMENT;
  if (debug_check_enabled()) {
    st = debug_check_slots(cache, slot_mapping, num_tokens, s);
    if (st != MLA_OK) return st;
  }
  const int64_t slots = static_cast<int64_t>(cache->num_pages) * cache->page_size;
  const int64_t D = cache->kv_lora_rank + cache->qk_rope_dim;
  void* layer = static_cast<char*>(cache->data) + layer_idx * slots * D * elem_bytes(cache->dtype);
  float* scale = cache->dtype == MLA_KV_FP8_E4M3 ? cache->scale + layer_idx * slots : nullptr;
  *w = mla::make_token_write(layer, scale, cache->dtype == MLA_KV_BF16 ? mla::kKvBf16 : mla::kKvFp8, slots,
                             cache->kv_lora_rank, cache->qk_rope_dim, static_cast<const uint16_t*>(c_kv),
                             c_kv_row_stride, static_cast<const uint16_t*>(k_pe), k_pe_row_stride,
                             slot_mapping, num_tokens);
  return MLA_OK;
}

mla_status mla_write_kv(const mla_cache* cache, int32_t layer_idx, const void* c_kv,
                        int64_t c_kv_row_stride, const void* k_pe, int64_t k_pe_row_stride,
                        const int64_t* slot_mapping, int32_t num_tokens, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  mla::TokenWrite w;
  const mla_status st =
      prepare_write(cache, layer_idx, c_kv, c_kv_row_stride, k_pe, k_pe_row_stride, slot_mapping, num_tokens, s, &w);
  if (st != MLA_OK || w.T == 0) return st;
  return to_status(mla::launch_write_kv(w.cache, w.scale, w.dtype, w.num_slots, w.R, w.Dr, w.c_kv, w.c_stride,
                                        w.k_pe, w.k_stride, w.slots, w.T, s));
}

mla_status mla_write_kv_fused(const mla_cache* cache, int32_t layer_idx, const void* c_kv,
                              int64_t c_kv_row_stride, const void* k_pe, int64_t k_pe_row_stride,
                              const mla_kv_transform* tf, const int64_t* slot_mapping,
                              int32_t num_tokens, void* stream) {
  mla_status st = check_cache(cache);
  if (st != MLA_OK) return st;
  if (layer_idx < 0 || layer_idx >= cache->num_layers || num_tokens < 0 || !tf)
    return MLA_ERR_INVALID_ARGUMENT;
  if (!isfinite(tf->norm_eps) || tf->norm_eps < 0.f) return MLA_ERR_INVALID_ARGUMENT;
  if (tf->cos_sin && (!tf->positions || tf->max_position <= 0 || cache->qk_rope_dim % 2 != 0))
    return MLA_ERR_INVALID_ARGUMENT;
  if (num_tokens == 0) return MLA_OK;
  if (!c_kv || !slot_mapping || (cache->qk_rope_dim > 0 && !k_pe)) return MLA_ERR_INVALID_ARGUMENT;
  if (c_kv_row_stride < cache->kv_lora_rank || k_pe_row_stride < cache->qk_rope_dim)
    return MLA_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (debug_check_enabled()) {
    if ((st = debug_check_slots(cache, slot_mapping, num_tokens, s)) != MLA_OK) return st;
    if (tf->cos_sin) {
      std::vector<int64_t> pos;
      if ((st = fetch(&pos, tf->positions, num_tokens, s)) != MLA_OK) return st;
      for (const int64_t p : pos)
        if (p < 0 || p >= tf->max_position) return MLA_ERR_INVALID_ARGUMENT;
    }
  }
  const int64_t slots = static_cast<int64_t>(cache->num_pages) * cache->page_size;
  const int64_t D = cache->kv_lora_rank + cache->qk_rope_dim;
  void* layer = static_cast<char*>(cache->data) + layer_idx * slots * D * elem_bytes(cache->dtype);
  float* scale = cache->dtype == MLA_KV_FP8_E4M3 ? cache->scale + layer_idx * slots : nullptr;
  mla::KvTransform k;
  k.norm_weight = static_cast<const uint16_t*>(tf->norm_weight);
  k.eps = tf->norm_eps;
  k.cos_sin = tf->cos_sin;
  k.positions = tf->positions;
  k.max_position = tf->max_position;
  k.interleaved = tf->rope_interleaved != 0;
  return to_status(mla::launch_write_kv_fused(
      layer, scale, cache->dtype == MLA_KV_BF16 ? mla::kKvBf16 : mla::kKvFp8, slots,
      cache->kv_lora_rank, cache->qk_rope_dim, static_cast<const uint16_t*>(c_kv), c_kv_row_stride,
      static_cast<const uint16_t*>(k_pe), k_pe_row_stride, slot_mapping, num_tokens, k, s));
}

size_t mla_sparse_workspace_size(const mla_cache* cache, const mla_attn* attn, int32_t batch,
                                 int32_t num_q, int32_t topk, int32_t max_blocks_per_seq) {
  if (check_cache(cache) != MLA_OK || check_attn(attn) != MLA_OK || batch < 0 || num_q < 0 ||
      topk <= 0 || max_blocks_per_seq <= 0)
    return 0;
  SparseLayout S;
  if (!make_sparse_layout(cache, attn, std::max<int64_t>(num_q, 1), topk, &S)) return 0;
  return S.total;
}

mla_status mla_sparse_attention(const mla_cache* cache, int32_t layer_idx, const mla_attn* attn,
                                const void* q_nope, int64_t q_nope_stride_t,
                                int64_t q_nope_stride_h, const void* q_pe, int64_t q_pe_stride_t,
                                int64_t q_pe_stride_h, const int32_t* key_indices, int32_t topk,
                                const int32_t* query_start_loc, int32_t num_q, int32_t max_q_len,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t batch, void* out,
                                float* lse_or_null, void* workspace, size_t workspace_bytes,
                                void* stream) {
  mla_status st = check_cache(cache);
  if (st != MLA_OK) return st;
  if ((st = check_attn(attn)) != MLA_OK) return st;
  if (layer_idx < 0 || layer_idx >= cache->num_layers) return MLA_ERR_INVALID_ARGUMENT;
  if (batch < 0 || num_q < 0 || topk <= 0 || max_blocks_per_seq <= 0 || max_q_len < 0)
    return MLA_ERR_INVALID_ARGUMENT;
  if (!query_start_loc && num_q != batch) return MLA_ERR_INVALID_ARGUMENT;
  if (batch == 0 || num_q == 0) return MLA_OK;
  if (!q_nope || !q_pe || !key_indices || !block_tables || !context_lens || !out)
    return MLA_ERR_INVALID_ARGUMENT;
  const int64_t max_ctx64 = static_cast<int64_t>(max_blocks_per_seq) * cache->page_size;
  if (max_ctx64 > (1ll << 30)) return MLA_ERR_UNSUPPORTED;
  SparseLayout S;
  if (!make_sparse_layout(cache, attn, num_q, topk, &S)) return MLA_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < S.total) return MLA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return MLA_ERR_WORKSPACE;
  const int64_t slots = static_cast<int64_t>(cache->num_pages) * cache->page_size;
  const int64_t D = cache->kv_lora_rank + cache->qk_rope_dim;
  const char* layer = static_cast<const char*>(cache->data) + layer_idx * slots * D * elem_bytes(cache->dtype);
  const uintptr_t need_align = cache->dtype == MLA_KV_BF16 ? 16 : 8;
  if ((reinterpret_cast<uintptr_t>(layer) & (need_align - 1)) != 0) return MLA_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (debug_check_enabled()) {
    st = debug_check_attention(query_start_loc ? mla::kPlanPrefill : mla::kPlanDecode, cache,
                               block_tables, max_blocks_per_seq, context_lens, batch,
                               query_start_loc, num_q, query_start_loc ? max_q_len : 1, s);
    if (st != MLA_OK) return st;
  }
  const int H = attn->num_heads;
  const int dv = attn->w_uv ? attn->v_head_dim : cache->kv_lora_rank;
  mla_attn dense = *attn;
  dense.window = 0;  // applied by the compaction
  for (int64_t r0 = 0; r0 < num_q; r0 += S.chunk) {
    const int32_t n = static_cast<int32_t>(std::min<int64_t>(S.chunk, num_q - r0));
    mla::CompactArgs ca;
    ca.cache = layer;
    ca.scale = cache->dtype == MLA_KV_FP8_E4M3 ? cache->scale + layer_idx * slots : nullptr;
    ca.num_pages = cache->num_pages;
    ca.page_size = cache->page_size;
    ca.page_shift = __builtin_ctz(static_cast<unsigned>(cache->page_size));
    ca.D = static_cast<int32_t>(D);
    ca.elem_bytes = static_cast<int32_t>(elem_bytes(cache->dtype));
    ca.key_indices = key_indices;
    ca.topk = topk;
    ca.query_start_loc = query_start_loc;
    ca.batch = batch;
    ca.context_lens = context_lens;
    ca.block_tables = block_tables;
    ca.max_blocks = max_blocks_per_seq;
    ca.max_ctx = max_ctx64;
    ca.window = attn->window;
    ca.row0 = r0;
    ca.rows_per_item = S.rows_per_item;
    ca.out_data = at<char>(workspace, S.data);
    ca.out_scale = cache->dtype == MLA_KV_FP8_E4M3 ? at<float>(workspace, S.scale) : nullptr;
    ca.out_ctx = at<int32_t>(workspace, S.ctx);
    ca.out_bt = at<int32_t>(workspace, S.bt);
    if (mla::launch_compact_keys(ca, n, s) != hipSuccess) return MLA_ERR_HIP;
    const mla_cache cc = compact_cache_desc(cache, ca.out_data, ca.out_scale, n, S.nblk);
    st = run_attention(mla::kPlanDecode, &cc, 0, &dense,
                       static_cast<const uint16_t*>(q_nope) + r0 * q_nope_stride_t, q_nope_stride_t,
                       q_nope_stride_h, static_cast<const uint16_t*>(q_pe) + r0 * q_pe_stride_t,
                       q_pe_stride_t, q_pe_stride_h, nullptr, n, ca.out_bt, S.nblk, ca.out_ctx, n, 1,
                       static_cast<uint16_t*>(out) + r0 * H * dv,
                       lse_or_null ? lse_or_null + r0 * H : nullptr, at<char>(workspace, S.dense),
                       S.dense_layout.total, stream);
    if (st != MLA_OK) return st;
  }
  return MLA_OK;
}

size_t mla_decode_workspace_size(const mla_cache* cache, const mla_attn* attn, int32_t batch,
                                 int32_t max_blocks_per_seq) {
  if (check_cache(cache) != MLA_OK || check_attn(attn) != MLA_OK || batch < 0 ||
      max_blocks_per_seq <= 0)
    return 0;
  Layout L;
  if (!make_layout(cache, attn, batch, &L)) return 0;
  return L.total;
}

size_t mla_prefill_workspace_size(const mla_cache* cache, const mla_attn* attn, int32_t batch,
                                  int32_t total_q_tokens, int32_t max_blocks_per_seq) {
  if (check_cache(cache) != MLA_OK || check_attn(attn) != MLA_OK || batch < 0 ||
      total_q_tokens < 0 || max_blocks_per_seq <= 0)
    return 0;
  if (prefill_route_expanded(cache, attn, batch, total_q_tokens))
    return make_xlayout(attn, batch, total_q_tokens,
                        static_cast<int64_t>(max_blocks_per_seq) * cache->page_size, total_q_tokens)
        .total;
  Layout L;
  if (!make_layout(cache, attn, total_q_tokens, &L)) return 0;
  return L.total;
}

mla_status mla_decode(const mla_cache* cache, int32_t layer_idx, const mla_attn* attn,
                      const void* q_nope, int64_t q_nope_stride_b, int64_t q_nope_stride_h,
                      const void* q_pe, int64_t q_pe_stride_b, int64_t q_pe_stride_h,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t batch, void* out, float* lse_or_null,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return run_attention(mla::kPlanDecode, cache, layer_idx, attn, q_nope, q_nope_stride_b,
                       q_nope_stride_h, q_pe, q_pe_stride_b, q_pe_stride_h, nullptr, batch,
                       block_tables, max_blocks_per_seq, context_lens, batch, 1, out, lse_or_null,
                       workspace, workspace_bytes, stream);
}

mla_status mla_decode_write(const mla_cache* cache, int32_t layer_idx, const mla_attn* attn,
                            const void* c_kv, int64_t c_kv_row_stride, const void* k_pe,
                            int64_t k_pe_row_stride, const int64_t* slot_mapping, int32_t num_tokens,
                            const void* q_nope, int64_t q_nope_stride_b, int64_t q_nope_stride_h,
                            const void* q_pe, int64_t q_pe_stride_b, int64_t q_pe_stride_h,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t batch, void* out, float* lse_or_null,
                            void* workspace, size_t workspace_bytes, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  mla::TokenWrite w;
  mla_status st =
      prepare_write(cache, layer_idx, c_kv, c_kv_row_stride, k_pe, k_pe_row_stride, slot_mapping, num_tokens, s, &w);
  if (st != MLA_OK) return st;
  if (batch < 0) return MLA_ERR_INVALID_ARGUMENT;
  if ((st = check_attn(attn)) != MLA_OK) return st;
  // nothing to decode: the write alone
  if (batch == 0 && w.T > 0)
    return to_status(mla::launch_write_kv(w.cache, w.scale, w.dtype, w.num_slots, w.R, w.Dr, w.c_kv, w.c_stride,
                                          w.k_pe, w.k_stride, w.slots, w.T, s));
  return run_attention(mla::kPlanDecode, cache, layer_idx, attn, q_nope, q_nope_stride_b,
                       q_nope_stride_h, q_pe, q_pe_stride_b, q_pe_stride_h, nullptr, batch,
                       block_tables, max_blocks_per_seq, context_lens, batch, 1, out, lse_or_null,
                       workspace, workspace_bytes, stream, &w);
}

mla_status mla_prefill_chunk(const mla_cache* cache, int32_t layer_idx, const mla_attn* attn,
                             const void* q_nope, int64_t q_nope_stride_t, int64_t q_nope_stride_h,
                             const void* q_pe, int64_t q_pe_stride_t, int64_t q_pe_stride_h,
                             const int32_t* query_start_loc, int32_t total_q_tokens,
                             int32_t max_q_len, const int32_t* block_tables,
                             int32_t max_blocks_per_seq, const int32_t* context_lens,
                             int32_t batch, void* out, float* lse_or_null, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (total_q_tokens < 0 || max_q_len < 0) return MLA_ERR_INVALID_ARGUMENT;
  if (check_cache(cache) == MLA_OK && check_attn(attn) == MLA_OK &&
      prefill_route_expanded(cache, attn, batch, total_q_tokens))
    return run_prefill_expanded(cache, layer_idx, attn, q_nope, q_nope_stride_t, q_nope_stride_h,
                                q_pe, q_pe_stride_t, q_pe_stride_h, query_start_loc, total_q_tokens,
                                max_q_len, block_tables, max_blocks_per_seq, context_lens, batch,
                                out, lse_or_null, workspace, workspace_bytes, stream);
  return run_attention(mla::kPlanPrefill, cache, layer_idx, attn, q_nope, q_nope_stride_t,
                       q_nope_stride_h, q_pe, q_pe_stride_t, q_pe_stride_h, query_start_loc,
                       total_q_tokens, block_tables, max_blocks_per_seq, context_lens, batch,
                       max_q_len, out, lse_or_null, workspace, workspace_bytes, stream);
}

mla_status mla_decode_combine(const float* o_part, const float* lse_part, int32_t num_splits,
                              int32_t batch, int32_t num_heads, int32_t dim, float* o, float* lse,
                              void* stream) {
  if (num_splits < 0 || batch < 0 || num_heads < 0 || dim < 0) return MLA_ERR_INVALID_ARGUMENT;
  const int64_t rows = static_cast<int64_t>(batch) * num_heads;
  if (rows == 0) return MLA_OK;
  if (!o || !lse || (num_splits > 0 && (!o_part || !lse_part))) return MLA_ERR_INVALID_ARGUMENT;
  if (rows > (1ll << 31) - 1) return MLA_ERR_UNSUPPORTED;
  return to_status(mla::launch_dense_combine(o_part, lse_part, num_splits,
                                             static_cast<int32_t>(rows), dim, o, lse,
                                             static_cast<hipStream_t>(stream)));
}

}  // extern "C"
