// Internal declarations shared by the host layer (mla_api.cpp) and the HIP
// kernel files.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Split-KV work unit: 32 consecutive token positions of one query item's
// visible key range, aligned to absolute token position (tile k covers
// positions [32k, 32k + 32)).
constexpr int kTile = 32;
// Estimated cost of one segment (an item's run of tiles inside one
// workgroup's range) beyond its tiles, in tile steps: storing the partial
// result and loading the next queries, and the slower first, second and last
// steps.  The split plan balances tiles plus this per item across workgroups.
constexpr int kSegmentCostTiles = 12;

enum PlanMode { kPlanDecode = 0, kPlanPrefill = 1 };
enum KvDtype { kKvBf16 = 0, kKvFp8 = 1 };

// One layer of the latent cache.
struct CacheView {
  const void* data;      // layer base: [num_pages][page_size][D]
  const float* scale;    // layer base: [num_pages][page_size] (fp8), else null
  int32_t dtype;         // KvDtype
  int32_t num_pages;
  int32_t page_size;
  int32_t page_shift;    // log2(page_size)
  int32_t R;             // kv_lora_rank
  int32_t Dr;            // qk_rope_dim
  int32_t D;             // R + Dr
};

// Per-item plan produced on the device (see plan_items in attn_common.hip).
// An item is one query token: a decode request, or one prefill row.
struct Plan {
  int32_t* item_b;       // [Nq] request of the item
  int32_t* item_lo;      // [Nq] first visible key position
  int32_t* item_hi;      // [Nq] one past the last visible key position
  int32_t* tile_start;   // [Nq + 1] exclusive prefix sum of the items' tile counts
  int32_t* wg_tile;      // [G + 1] first tile of each workgroup's range (non-decreasing; may be empty)
  int32_t* wg_item;      // [G] item owning each workgroup's first tile
  int32_t* item_wg;      // [2 Nq] first and last workgroup covering each item's tiles
  int32_t G;             // workgroups the tile stream is divided over
};

struct AttnArgs {
  CacheView kv;
  const uint16_t* q_lat;  // bf16 latent query rows [.., H, R]
  int64_t q_lat_st, q_lat_sh;
  const uint16_t* q_pe;   // bf16 rope query rows [.., H, Dr]
  int64_t q_pe_st, q_pe_sh;
  const int32_t* block_tables;
  int32_t max_blocks;
  const int32_t* item_b;
  const int32_t* item_lo;
  const int32_t* item_hi;
  const int32_t* tile_start;
  const int32_t* wg_tile;  // [G + 1] (see Plan)
  const int32_t* wg_item;  // [G]
  const int32_t* item_wg;  // [2 Nq] (see Plan)
  int32_t num_items;
  int32_t H;
  int32_t G;              // workgroups the tile stream is divided over
  float scale_log2;       // softmax scale * log2(e)
  // Results.  o values are stored unnormalised together with a per-head
  // factor (o_scale / part_scale = 1/l); the normalised row is o * factor.
  float* o_lat;           // [Nq][H][R] fp32 (complete items)
  float* lse;             // [Nq][H] fp32 natural log (complete items)
  float* o_scale;         // [Nq][H]
  uint16_t* part_o;       // [2G][H][R] bf16 partials (cut items; unnormalised, RNE)
  float* part_lse;        // [2G][H]
  float* part_scale;      // [2G][H]
};

// Compute units of the current device (cached per device; -1 on error).
int current_cu_count();

// Device-side view of mla_kv_transform (the fused write's norm and rotation).
struct KvTransform {
  const uint16_t* norm_weight;  // bf16 [R], or null: no RMSNorm
  float eps;
  const float* cos_sin;         // fp32 [max_position][Dr], or null: no rotation
  const int64_t* positions;     // [T]
  int32_t max_position;
  int32_t interleaved;          // 1: pairs (2i, 2i+1); 0: pairs (i, i + Dr/2)
};

// Index-list attention: the compaction of each query item's kept keys into
// its own run of kCompactPage-token pages (sparse.hip).
constexpr int kCompactPage = 64;
struct CompactArgs {
  const void* cache;             // layer base, [num_pages][page_size][D]
  const float* scale;            // layer base [num_pages][page_size] (fp8), else null
  int32_t num_pages, page_size, page_shift, D, elem_bytes;
  const int32_t* key_indices;    // [rows][topk]
  int32_t topk;
  const int32_t* query_start_loc;  // [batch + 1] (prefill) or null (decode)
  int32_t batch;
  const int32_t* context_lens;
  const int32_t* block_tables;
  int32_t max_blocks;
  int64_t max_ctx;               // max_blocks * page_size
  int32_t window;
  int64_t row0;                  // first query row of this launch
  int32_t rows_per_item;         // pages per item * kCompactPage
  void* out_data;                // [items][rows_per_item][D]
  float* out_scale;              // [items][rows_per_item] (fp8), else null
  int32_t* out_ctx;              // [items] kept keys
  int32_t* out_bt;               // [items][rows_per_item / kCompactPage] identity block table
};

// Expanded-form chunked prefill (prefill_expanded.hip): one launch pair
// covers up to `ck` keys (a multiple of 256) of requests b0 .. b0 + batch - 1;
// the launch's last grid dimension runs over those requests.
struct XPassArgs {
  CacheView kv;
  const int32_t* block_tables;
  int32_t max_blocks;
  int64_t max_ctx;
  const int32_t* context_lens;
  const int32_t* query_start_loc;
  int32_t b0, batch, pass, ck, window, H;
  int32_t total_q;         // rows of q / out / state (a row past it is never touched)
  const uint16_t* w_uk;    // [H][128][R]
  const uint16_t* w_uv;    // [H][128][R]
  const uint16_t* q_nope;  // [Tq][H][128] (strides)
  int64_t qn_st, qn_sh;
  const uint16_t* q_pe;    // [Tq][H][64] (strides)
  int64_t qp_st, qp_sh;
  float scale_log2;
  uint16_t* k_exp;         // [batch][H][ck][128]
  uint16_t* v_expT;        // [batch][H][128][ck]
  uint16_t* kpe;           // [batch][ck][64]
  float* o_acc;            // [Tq][H][128] running (unnormalised) output (several passes only)
  float* m_acc;            // [Tq][H] running maximum (log2 units)
  float* l_acc;            // [Tq][H] running sum
  uint16_t* out;           // [Tq][H][128]
  float* lse;              // [Tq][H] or null
};
bool prefill_expanded_supported(const CacheView& kv, int32_t H, int32_t Dn, int32_t Dv);
hipError_t launch_prefill_expanded_pass(const XPassArgs& a, int32_t max_q_len, hipStream_t s);

// ---- launchers (each returns the launch's hipGetLastError) ----
hipError_t launch_write_kv(void* cache_layer, float* scale_layer, int32_t dtype, int64_t num_slots,
                           int32_t R, int32_t Dr, const uint16_t* c_kv, int64_t c_stride,
                           const uint16_t* k_pe, int64_t k_stride, const int64_t* slots,
                           int32_t num_tokens, hipStream_t s);

hipError_t launch_write_kv_fused(void* cache_layer, float* scale_layer, int32_t dtype,
                                 int64_t num_slots, int32_t R, int32_t Dr, const uint16_t* c_kv,
                                 int64_t c_stride, const uint16_t* k_pe, int64_t k_stride,
                                 const int64_t* slots, int32_t num_tokens, const KvTransform& tf,
                                 hipStream_t s);

hipError_t launch_compact_keys(const CompactArgs& a, int32_t items, hipStream_t s);

hipError_t launch_plan(int mode, int32_t batch, int32_t num_items, const int32_t* context_lens,
                       const int32_t* query_start_loc, int32_t window, int32_t max_ctx,
                       const Plan& plan, hipStream_t s);

// The split plan's inputs and outputs, for a launch that runs it beside other
// work (launch_absorb_mfma).
struct PlanArgs {
  int mode;
  int32_t batch, num_items;
  const int32_t* context_lens;
  const int32_t* query_start_loc;
  int32_t window, max_ctx;
  Plan plan;
};

hipError_t launch_attn_generic(const AttnArgs& a, hipStream_t s);

// True when the MFMA split-KV kernel handles this shape (R 512, Dr 64, H <= 128).
bool mfma_attn_supported(const CacheView& kv, int32_t H);
hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t s);

// True when the fp8 MFMA split-KV kernel handles this shape (E4M3 cache,
// R 512, Dr 64, H <= 128).
bool mfma_fp8_attn_supported(const CacheView& kv, int32_t H);
hipError_t launch_attn_mfma_fp8(const AttnArgs& a, hipStream_t s);
// fp8 caches on the fp8 matrix cores (queries and probabilities quantised).
bool f8mfma_attn_supported(const CacheView& kv, int32_t H);
hipError_t launch_attn_f8mfma(const AttnArgs& a, hipStream_t s);

hipError_t launch_combine_segments(const AttnArgs& a, hipStream_t s);

hipError_t launch_absorb(const uint16_t* q_nope, int64_t st, int64_t sh, const uint16_t* w_uk,
                         int32_t num_items, int32_t H, int32_t Dn, int32_t R, uint16_t* q_lat,
                         hipStream_t s);

hipError_t launch_up_project(const float* o_lat, const float* o_scale, const uint16_t* w_uv,
                             int32_t num_items, int32_t H, int32_t R, int32_t Dv, uint16_t* out,
                             hipStream_t s);

hipError_t launch_latent_out(const float* o_lat, const float* o_scale, int32_t num_items, int32_t H,
                             int32_t R, uint16_t* out, hipStream_t s);

// New tokens of one layer for mla_write_kv's per-token write (write_device.h).
struct TokenWrite {
  void* cache;          // the layer's rows [num_slots][R + Dr] (bf16 or E4M3 codes)
  float* scale;         // the layer's fp32 scales [num_slots] (fp8), else null
  int64_t num_slots;
  const uint16_t* c_kv;
  int64_t c_stride;
  const uint16_t* k_pe;
  int64_t k_stride;
  const int64_t* slots;
  int32_t dtype;        // kKvBf16 / kKvFp8
  int32_t R, Dr;
  int32_t T;            // tokens (0: nothing to write)
  int32_t vec;          // 16-byte row chunks (R, Dr, strides multiples of 8, rows 16-byte aligned; fp8: R + Dr <= 1024)
};
TokenWrite make_token_write(void* cache_layer, float* scale_layer, int32_t dtype, int64_t num_slots, int32_t R,
                            int32_t Dr, const uint16_t* c_kv, int64_t c_stride, const uint16_t* k_pe,
                            int64_t k_stride, const int64_t* slots, int32_t num_tokens);

// Matrix-core versions of the two per-head projections (head_gemm.hip).
bool absorb_mfma_supported(int32_t Dn, int32_t R);
bool up_project_mfma_supported(int32_t R, int32_t Dv);
// With `plan` non-null the same launch also computes the split plan, in one
// extra workgroup; with `write` non-null (and write->T > 0) further extra
// workgroups write those tokens into the cache, one wavefront per token.
hipError_t launch_absorb_mfma(const uint16_t* q_nope, int64_t st, int64_t sh, const uint16_t* w_uk,
                              int32_t num_items, int32_t H, int32_t Dn, int32_t R, uint16_t* q_lat,
                              const PlanArgs* plan, const TokenWrite* write, hipStream_t s);
hipError_t launch_up_project_mfma(const float* o_lat, const float* o_scale, const uint16_t* w_uv,
                                  int32_t num_items, int32_t H, int32_t R, int32_t Dv, uint16_t* out,
                                  hipStream_t s);

// Combine of cut items fused with the up-projection (head_gemm.hip): reads
// the partial slots (or an uncut item's o_lat row) and writes out and the lse
// of cut and empty items; o_lat is not written.
bool combine_up_project_supported(int32_t R, int32_t Dv);
hipError_t launch_combine_up_project(const AttnArgs& a, const uint16_t* w_uv, int32_t Dv, uint16_t* out,
                                     hipStream_t s);

hipError_t launch_dense_combine(const float* o_part, const float* lse_part, int32_t num_splits,
                                int32_t rows, int32_t dim, float* o, float* lse, hipStream_t s);

}  // namespace mla
