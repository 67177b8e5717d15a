/*
 * mla.h - C ABI of libmla.so: paged multi-head latent attention (MLA,
 * DeepSeek-V2/V3 style) over a block-table-indexed latent KV cache, for AMD
 * MI355X (gfx950).
 *
 * Sources (web pages, cited by title and section):
 *   [SHIM]    "feat(serving): DeepSeek-V2/V3 paged-attention shim (MLA)"
 *   [SWA]     "[Models] Support MLA_SWA functionality"
 *   [CHUNK]   "[Attention] MLA with chunked prefill"
 *   [UNIFIED] "[unified-memory] Let Kimi-Linear use the paged MLA attention
 *             backends"
 *   [DSV4]    "Support dsv4 model"
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked (host).  Descriptor structs
 *     (mla_cache, mla_attn) are passed by host pointer and read during the
 *     call only.
 *   - The caller owns every buffer, the workspace included.  The library
 *     allocates no device memory and keeps no pointer after it returns; it
 *     reads exactly the buffers passed (no copies made at plan time), so the
 *     calls can be captured in a HIP graph.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     null stream).  Nothing synchronises with the host.
 *   - Errors: argument problems found on the host return a status and enqueue
 *     nothing.  The contents of device arrays (block tables, lengths, slots)
 *     are a caller contract; out-of-range entries are clamped or skipped by
 *     the kernels so that they never read or write outside the buffers, and
 *     the results for the affected rows are then unspecified.  A failed
 *     kernel launch returns MLA_ERR_HIP.  The library never aborts.
 *   - Debug check: with the environment variable MLA_DEBUG_CHECK set (to
 *     anything but "" or "0"), every call first copies its index arrays to
 *     the host, waits for the stream, and verifies the caller contract:
 *     0 <= context_lens[b] <= max_blocks_per_seq * page_size; the first
 *     ceil(context_lens[b] / page_size) block-table entries name pages of the
 *     cache; query_start_loc starts at 0, never decreases, ends at
 *     total_q_tokens ("[unified-memory] ...", Two pre-existing issues, item 1:
 *     a query count disagreeing with the last query_start_loc entry crashed
 *     the kernel there) and each chunk fits its context and max_q_len; write
 *     slots are negative or name distinct slots of the cache.  A violation
 *     returns MLA_ERR_INVALID_ARGUMENT with nothing enqueued.  The check
 *     synchronises, so under stream capture it returns MLA_ERR_UNSUPPORTED.
 *   - Thread safety: the library keeps no per-call state between calls; its
 *     only process-wide state (a per-device compute-unit count and a kernel
 *     attribute flag) is held in atomics.  Calls that share a workspace or
 *     write the same outputs must not overlap.
 *   - bf16 values are IEEE binary32 truncated to the top 16 bits (bfloat16).
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, layer out of range, ... */
  MLA_ERR_UNSUPPORTED = 2,      /* dimensions or page size the kernels do not handle */
  MLA_ERR_WORKSPACE = 3,        /* workspace missing or smaller than the *_workspace_size */
  MLA_ERR_HIP = 4               /* a HIP call or kernel launch failed */
} mla_status;

typedef enum {
  MLA_KV_BF16 = 0,     /* latent vectors stored as bf16 */
  MLA_KV_FP8_E4M3 = 1  /* OCP E4M3 codes (uint8) plus one fp32 scale per token */
} mla_kv_dtype;

/*
 * Latent KV cache, caller-owned ([SHIM] "Root causes" item 5 and "Changes":
 * one cache with a leading layer dimension, addressed by layer_idx;
 * [UNIFIED] "Validation": kv_lora_rank 512 + qk_rope_head_dim 64).
 *
 *   data : [num_layers][num_pages][page_size][kv_lora_rank + qk_rope_dim],
 *          contiguous.  Each token's row is [c_kv | k_pe].  Element type is
 *          bf16 (MLA_KV_BF16) or uint8 E4M3 codes (MLA_KV_FP8_E4M3).
 *   scale: [num_layers][num_pages][page_size] fp32, one per token (fp8 only;
 *          NULL for bf16).  Dequantised value = e4m3(code) * scale.
 * Supported by the GPU kernels: page_size in {16, 32, 64, 128};
 * kv_lora_rank a multiple of 8 and 8 <= kv_lora_rank + qk_rope_dim <= 1024.
 */
typedef struct {
  void* data;
  float* scale;
  int32_t dtype;        /* mla_kv_dtype */
  int32_t num_layers;
  int32_t num_pages;
  int32_t page_size;
  int32_t kv_lora_rank; /* R  */
  int32_t qk_rope_dim;  /* Dr */
} mla_cache;

/* Flags for mla_attn.flags (testing and comparison only). */
#define MLA_FLAG_GENERIC_KERNELS 1u /* use the plain (non-MFMA) kernels for every shape */
/* mla_prefill_chunk form: absorbed (latent-space attention, as decode) or
 * expanded (keys and values up-projected per head through W_UK / W_UV into
 * the workspace, [CHUNK] "Future work"); without either flag the library
 * picks one (see mla_prefill_chunk). */
#define MLA_FLAG_PREFILL_ABSORBED 2u
#define MLA_FLAG_PREFILL_EXPANDED 4u
/* fp8 E4M3 caches (kv_lora_rank 512, qk_rope_dim 64, up to 128 heads): run
 * the scores and the values on the fp8 matrix cores, reading the cache codes
 * as stored ([UNIFIED] "Validation": the fp8_e4m3 cache rows; [DSV4] "Model
 * Architecture and Inference": packed FP8 KV).  The queries enter as a
 * two-term E4M3 expansion (hi + lo, one scale per head) and the
 * probabilities as E4M3 with a power-of-two scale per head and step, so the
 * result approximates the exact softmax over the dequantised cache (errors
 * against the exact result: well inside max-abs 0.1 and rel-L2 3e-2 on the
 * tested inputs, against ~2e-3 for the default path, which is exact up to
 * rounding).  Absorbed-form decode and prefill; ignored for bf16 caches and
 * other shapes. */
#define MLA_FLAG_FP8_MFMA 8u

/*
 * Per-call attention parameters.
 *   w_uk : bf16 [num_heads][qk_nope_dim][kv_lora_rank].  q_lat[h] =
 *          W_UK[h]^T q_nope[h] (weight absorption; the up-projection kv_b_proj
 *          of [CHUNK] "Future work" read as k_nope = W_UK[h] c_kv).  NULL means
 *          q_nope is already latent: [.., num_heads][kv_lora_rank].
 *   w_uv : bf16 [num_heads][v_head_dim][kv_lora_rank]; out[h] = W_UV[h] o_lat[h]
 *          ([SHIM] "Changes": output sliced to v_head_dim).  NULL means the
 *          output is the latent o_lat: [.., num_heads][kv_lora_rank].
 *   scale: softmax scale, e.g. 1/sqrt(qk_nope + qk_rope); used as given
 *          ([SHIM] "Root causes" item 3: never derived from a padded dim).
 *   window: <= 0 full attention; w > 0 a query at position p sees keys t with
 *          p - w < t <= p ([SWA] "Motivation"; the pages give no boundary
 *          convention, this one keeps exactly min(w, p + 1) keys).
 *   num_workgroups: 0 = one workgroup per compute unit for the split-KV work
 *          partition; > 0 forces that many (testing).
 *   kernel_events: optional pair of hipEvent_t (either may be NULL).  When
 *          set, [0] is recorded on the call's stream just before the split-KV
 *          attention kernel and [1] just after it, so a caller can time that
 *          kernel alone (profiling).
 */
typedef struct {
  int32_t num_heads;
  int32_t qk_nope_dim;
  int32_t v_head_dim;
  const void* w_uk;
  const void* w_uv;
  float scale;
  int32_t window;
  int32_t num_workgroups;
  uint32_t flags;
  void* kernel_events[2];
} mla_attn;

/*
 * mla_write_kv - scatter new tokens into the cache ([SHIM] "Root causes"
 * item 2 and "Changes": KV is written whenever a slot mapping is present, for
 * decode tokens as well as prefill tokens).
 *   c_kv : bf16 [num_tokens][kv_lora_rank], row stride c_kv_row_stride elements
 *   k_pe : bf16 [num_tokens][qk_rope_dim], row stride k_pe_row_stride elements
 *          (already rotated: RoPE is applied by the caller)
 *   slot_mapping : int64 [num_tokens]; token i goes to page s / page_size,
 *          offset s % page_size of layer layer_idx.  s < 0 is a pad row and
 *          writes nothing ([UNIFIED] "Cuda-graph safety": stale pad-row
 *          locations must not scatter into live pages).  s >= num_pages *
 *          page_size is skipped.  Two tokens of one call must not share a
 *          slot (which one lands is then unspecified); a later call
 *          overwrites an earlier one.
 * bf16 cache: bit copy.  fp8 cache: per token amax over all R + Dr values,
 * scale = amax / 448 (fp32, correctly rounded; 1.0 when amax is 0), code =
 * E4M3 round-to-nearest-even of x / scale saturated to +-448, scale stored
 * beside the codes.  num_tokens == 0 is a no-op.
 */
mla_status mla_write_kv(const mla_cache* cache, int32_t layer_idx,
                        const void* c_kv, int64_t c_kv_row_stride,
                        const void* k_pe, int64_t k_pe_row_stride,
                        const int64_t* slot_mapping, int32_t num_tokens, void* stream);

/*
 * Normalisation and rotation folded into the cache write ("Support dsv4
 * model", Model Architecture and Inference: fused normalization/RoPE and
 * packed KV writers; [CHUNK] "Future work": the cache holds kv_c_normed, the
 * latent after its RMSNorm).  Read by host pointer during the call.
 *   norm_weight : bf16 [kv_lora_rank]; NULL writes the latent as given
 *   norm_eps    : RMSNorm epsilon, finite and >= 0
 *   cos_sin     : fp32 [max_position][qk_rope_dim], the caller's RoPE table:
 *                 for position p the cosines of its qk_rope_dim/2 angles, then
 *                 their sines; NULL writes k_pe as given
 *   positions   : int64 [num_tokens] (device), each token's position; needed
 *                 with cos_sin.  Positions outside [0, max_position) are a
 *                 caller error (clamped on the device)
 *   rope_interleaved : 1 rotates pairs (2i, 2i+1), 0 pairs (i, i + Dr/2)
 */
typedef struct {
  const void* norm_weight;
  float norm_eps;
  const float* cos_sin;
  const int64_t* positions;
  int32_t max_position;
  int32_t rope_interleaved;
} mla_kv_transform;

/*
 * mla_write_kv_fused - mla_write_kv of the transformed rows: for each token,
 *   latent  c' = bf16( c / sqrt(mean(c^2) + eps) * norm_weight )   (RMSNorm)
 *   rope    r' = bf16( (a cos - b sin, b cos + a sin) on each pair (a, b) )
 * (arithmetic in fp32 on the device, each value rounded to bf16 to nearest
 * even), then written exactly as mla_write_kv writes [c' | r'] (bit copy, or
 * the fp8 quantisation).  Arguments and errors as mla_write_kv; c_kv and k_pe
 * are the un-normalised latent and the un-rotated rope part.
 */
mla_status mla_write_kv_fused(const mla_cache* cache, int32_t layer_idx,
                              const void* c_kv, int64_t c_kv_row_stride,
                              const void* k_pe, int64_t k_pe_row_stride,
                              const mla_kv_transform* transform,
                              const int64_t* slot_mapping, int32_t num_tokens, void* stream);

/*
 * Workspace bytes mla_decode needs for these arguments (0 if the arguments
 * are invalid).  Depends on batch, heads, dims, w_uk/w_uv presence and the
 * number of workgroups (the device's compute-unit count unless forced).
 */
size_t mla_decode_workspace_size(const mla_cache* cache, const mla_attn* attn, int32_t batch,
                                 int32_t max_blocks_per_seq);

/*
 * mla_decode - absorbed-form split-KV decode: one query token per request.
 * Request b attends to its context_lens[b] cached tokens (the newest one, at
 * position n - 1, included: the caller writes it with mla_write_kv first;
 * [SHIM] "Root causes" items 2 and 4), through block_tables[b][t / page_size]
 * ([UNIFIED] "What this does": kernels read the block table directly).
 *   q_nope : bf16 [batch][num_heads][qk_nope_dim] (or [..][kv_lora_rank] when
 *            w_uk is NULL), strides q_nope_stride_b / _h in elements, last dim
 *            contiguous
 *   q_pe   : bf16 [batch][num_heads][qk_rope_dim], strides q_pe_stride_b / _h
 *   block_tables : int32 [batch][max_blocks_per_seq]; only the first
 *            ceil(n / page_size) entries of a row are read
 *   context_lens : int32 [batch]; n = 0 gives out 0 and lse -inf
 *   out    : bf16 [batch][num_heads][v_head_dim] (or [..][kv_lora_rank] when
 *            w_uv is NULL), contiguous
 *   lse_or_null : fp32 [batch][num_heads], natural-log log-sum-exp of the
 *            scaled scores, or NULL
 *   workspace : device memory of at least mla_decode_workspace_size bytes,
 *            256-byte aligned; its contents need not be initialised
 */
mla_status mla_decode(const mla_cache* cache, int32_t layer_idx, const mla_attn* attn,
                      const void* q_nope, int64_t q_nope_stride_b, int64_t q_nope_stride_h,
                      const void* q_pe, int64_t q_pe_stride_b, int64_t q_pe_stride_h,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t batch,
                      void* out, float* lse_or_null,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_decode_write - mla_write_kv of the step's new tokens followed by
 * mla_decode, as one call ([SHIM] "Root causes" item 2: a decode step writes
 * its tokens before attending over them).  The write arguments are
 * mla_write_kv's (c_kv, c_kv_row_stride, k_pe, k_pe_row_stride,
 * slot_mapping, num_tokens: same meaning, layout, checks and errors), the
 * rest are mla_decode's; the results (cache contents, out, lse) are those of
 * the two calls in order on the same stream.  When the decode runs the
 * matrix-core absorb (w_uk given, the MFMA shapes), the tokens are written by
 * extra workgroups of that first launch, beside the absorb and the split
 * plan, which saves the write's own launch; otherwise a write launch runs
 * first.  Workspace: mla_decode_workspace_size.  A call whose arguments are
 * invalid enqueues nothing (neither the write nor the decode).  batch 0 writes
 * only.
 */
mla_status mla_decode_write(const mla_cache* cache, int32_t layer_idx, const mla_attn* attn,
                            const void* c_kv, int64_t c_kv_row_stride,
                            const void* k_pe, int64_t k_pe_row_stride,
                            const int64_t* slot_mapping, int32_t num_tokens,
                            const void* q_nope, int64_t q_nope_stride_b, int64_t q_nope_stride_h,
                            const void* q_pe, int64_t q_pe_stride_b, int64_t q_pe_stride_h,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t batch,
                            void* out, float* lse_or_null,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_decode_noalloc - mla_decode without a caller workspace, for callers that
 * cannot allocate device memory (code under graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments, results and
 * errors as mla_decode, minus workspace / workspace_bytes.
 *
 * The workspace is a device array inside the library, MLA_NOALLOC_SCRATCH_BYTES
 * bytes on every GPU the library runs on, held until the process ends.  Its
 * device address is looked up on the first call made with a device current.
 * A call whose mla_decode_workspace_size exceeds MLA_NOALLOC_SCRATCH_BYTES
 * returns MLA_ERR_WORKSPACE and enqueues nothing (192 MiB covers one GPU's
 * full 128-head set at 128 requests with one workgroup per compute unit).
 * The call allocates nothing.  All calls on one GPU share the array: calls
 * that overlap in time on one GPU (two streams, two threads) race and must
 * not be issued.
 */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)192 << 20)
mla_status mla_decode_noalloc(const mla_cache* cache, int32_t layer_idx, const mla_attn* attn,
                              const void* q_nope, int64_t q_nope_stride_b, int64_t q_nope_stride_h,
                              const void* q_pe, int64_t q_pe_stride_b, int64_t q_pe_stride_h,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, int32_t batch,
                              void* out, float* lse_or_null, void* stream);

/*
 * mla_decode_combine - log-sum-exp merge of split-KV partial results
 * (the identity lse = log sum_s exp(lse_s), o = sum_s exp(lse_s - lse) o_s;
 * the pages do not state it).
 *   o_part   : fp32 [num_splits][batch][num_heads][dim], each normalised
 *   lse_part : fp32 [num_splits][batch][num_heads], natural log; -inf marks
 *              an empty partial (weight 0, its o_part is not read)
 *   o        : fp32 [batch][num_heads][dim]; lse : fp32 [batch][num_heads]
 * If every partial of a row is empty the row gets o = 0, lse = -inf.
 */
mla_status mla_decode_combine(const float* o_part, const float* lse_part, int32_t num_splits,
                              int32_t batch, int32_t num_heads, int32_t dim,
                              float* o, float* lse, void* stream);

/* Workspace bytes mla_prefill_chunk needs (0 if the arguments are invalid). */
size_t mla_prefill_workspace_size(const mla_cache* cache, const mla_attn* attn, int32_t batch,
                                  int32_t total_q_tokens, int32_t max_blocks_per_seq);

/*
 * mla_prefill_chunk - causal chunked prefill over the paged context
 * ([CHUNK]: new query tokens attend causally to the existing context plus
 * the chunk; chunking must not change results).  Request b owns query rows
 * query_start_loc[b] .. query_start_loc[b+1]-1 (m_b rows).  Its chunk
 * tokens are already in the cache (written with mla_write_kv) at positions
 * n_b - m_b .. n_b - 1, n_b = context_lens[b]; row i sees keys
 * t <= n_b - m_b + i, and the window.
 *   q_nope : bf16 [total_q_tokens][num_heads][qk_nope_dim] (latent when w_uk
 *            is NULL), strides q_nope_stride_t / _h
 *   q_pe   : bf16 [total_q_tokens][num_heads][qk_rope_dim]
 *   query_start_loc : int32 [batch + 1] (device), query_start_loc[batch] ==
 *            total_q_tokens (caller contract)
 *   total_q_tokens, max_q_len : host values
 *   out    : bf16 [total_q_tokens][num_heads][v_head_dim or kv_lora_rank]
 *   lse_or_null : fp32 [total_q_tokens][num_heads] or NULL
 * Two forms compute the same result.  Absorbed: each query row is a decode
 * item of the latent-space kernels.  Expanded ([CHUNK] "Future work"): the
 * keys the chunk's rows can see are up-projected per head through W_UK and
 * W_UV (kv_b_proj) into the workspace and attended with q_nope (128) + q_pe
 * (64) against [W_UK c ; k_pe], values W_UV c (128).  The up-projected keys
 * take at most 1.25 GiB of workspace: requests go in groups whose visible
 * ranges all fit, or, for a range longer than that, one at a time in passes
 * whose results are merged by log-sum-exp.  The expanded form needs w_uk and w_uv, qk_rope_dim
 * 64, qk_nope_dim = v_head_dim = 128, kv_lora_rank a multiple of 64 and scale > 0
 * (otherwise the absorbed form runs, flag or not).
 * MLA_FLAG_PREFILL_ABSORBED / _EXPANDED choose; without a flag the expanded
 * form runs for calls whose chunks average at least 64 rows, the absorbed one
 * otherwise.  mla_prefill_workspace_size returns the
 * chosen form's size (the same attn flags must be passed to both calls).
 */
mla_status mla_prefill_chunk(const mla_cache* cache, int32_t layer_idx, const mla_attn* attn,
                             const void* q_nope, int64_t q_nope_stride_t, int64_t q_nope_stride_h,
                             const void* q_pe, int64_t q_pe_stride_t, int64_t q_pe_stride_h,
                             const int32_t* query_start_loc, int32_t total_q_tokens,
                             int32_t max_q_len,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t batch,
                             void* out, float* lse_or_null,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Index-list (top-k / sparse) attention ("[Models] Support MLA_SWA
 * functionality", Modifications: a top-k indexer builds each query's key
 * list, the sliding window is expressed as such a list; "Support dsv4 model",
 * Model Architecture and Inference: sparse index construction).
 *
 * Query row r attends to the positions key_indices[r][0 .. topk-1] of its
 * request's sequence that its ordinary visible range holds: t <= p, and
 * p - w < t with a window w > 0 (attn->window), where p is the row's position
 * (decode: n_b - 1; prefill: n_b - m_b + i as in mla_prefill_chunk).
 * Negative entries are unused slots; entries outside the range are ignored;
 * a position listed twice in one row is a caller error.  A row with no kept
 * key gets out 0 and lse -inf.  The softmax does not depend on list order.
 *   key_indices     : int32 [num_q][topk] (device), row r's list
 *   query_start_loc : int32 [batch + 1] (device) for prefill rows, or NULL
 *                     for decode (then num_q == batch, row b = request b)
 *   max_q_len       : host; the longest chunk (prefill), ignored for decode
 *   other arguments : as mla_decode / mla_prefill_chunk (q rows [num_q][H][..],
 *                     out [num_q][H][Dv or R], lse [num_q][H] or NULL)
 * The kept rows of each query are first gathered, in list order, into pages
 * of the workspace; the rows are then attended by the decode kernels.  Query
 * rows are processed in chunks that bound that gather to 512 MiB.
 */
size_t mla_sparse_workspace_size(const mla_cache* cache, const mla_attn* attn, int32_t batch,
                                 int32_t num_q, int32_t topk, int32_t max_blocks_per_seq);
mla_status mla_sparse_attention(const mla_cache* cache, int32_t layer_idx, const mla_attn* attn,
                                const void* q_nope, int64_t q_nope_stride_t,
                                int64_t q_nope_stride_h, const void* q_pe, int64_t q_pe_stride_t,
                                int64_t q_pe_stride_h, const int32_t* key_indices, int32_t topk,
                                const int32_t* query_start_loc, int32_t num_q, int32_t max_q_len,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t batch,
                                void* out, float* lse_or_null,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Human-readable name of a status code (static string). */
const char* mla_status_string(mla_status status);

/* Library version string (static). */
const char* mla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
