// Index-list (top-k) attention, first half: compaction.
//
// "[Models] Support MLA_SWA functionality", Modifications: a top-k indexer
// builds each query's key list, and the sliding window is expressed as such a
// list; "Support dsv4 model", Model Architecture and Inference: sparse index
// construction.  A query at position p attends to the positions of its list
// that its ordinary visible range holds (p - w < t <= p with a window w > 0,
// t <= p otherwise); negative entries are unused slots and other entries are
// ignored.
//
// Workgroup (item, s) handles entries [256 s, 256 s + 256) of an item's list:
// it counts the item's kept entries before its segment (a block reduction over
// the list prefix, a few KB of int32), scans its own segment, and copies the
// rows of its kept entries, in list order, from the paged cache into the
// item's private run of 64-token pages in the workspace.  The last segment
// writes the item's kept count, the first its identity block table.
// The dense decode pipeline (absorb, split plan, matrix-core attention,
// combine + up-projection) then runs over those pages as if each item were a
// decode request with a context of its kept count: softmax attention does not
// depend on the order of its keys, so the result is the list's attention.
#include "device_utils.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kThreads = 256;

template <typename Chunk>
__global__ __launch_bounds__(kThreads) void compact_keys_kernel(CompactArgs a) {
  __shared__ int32_t scan[kThreads];
  __shared__ int64_t src_row[kThreads];
  __shared__ int32_t dst_row[kThreads];
  __shared__ int32_t carry;
  const int tid = threadIdx.x;
  const int item = blockIdx.x;          // local index within this chunk
  const int seg = blockIdx.y;           // 256-entry segment of the item's list
  const int64_t g = a.row0 + item;      // query row (decode: request)
  // the item's request and query position (as the split plan derives them)
  int b;
  int64_t p;
  if (a.query_start_loc == nullptr) {
    b = static_cast<int>(g);
    const int64_t n = min(max(static_cast<int64_t>(a.context_lens[b]), int64_t{0}), a.max_ctx);
    p = n - 1;
  } else {
    int lo = 0, hi = a.batch;  // largest b < batch with qsl[b] <= g
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.query_start_loc[mid] <= g) lo = mid; else hi = mid;
    }
    b = lo;
    const int64_t n = min(max(static_cast<int64_t>(a.context_lens[b]), int64_t{0}), a.max_ctx);
    const int64_t m = a.query_start_loc[b + 1] - a.query_start_loc[b];
    p = min(n - m + (g - a.query_start_loc[b]), n - 1);
  }
  const int64_t vis_hi = p + 1;
  const int64_t vis_lo = a.window > 0 ? max(int64_t{0}, p - a.window + 1) : 0;
  const int32_t* list = a.key_indices + g * a.topk;
  const int32_t* bt = a.block_tables + static_cast<int64_t>(b) * a.max_blocks;
  const int64_t row_bytes = static_cast<int64_t>(a.D) * a.elem_bytes;
  const int chunks_per_row = static_cast<int>(row_bytes / sizeof(Chunk));
  const char* src_base = static_cast<const char*>(a.cache);
  char* dst_base = static_cast<char*>(a.out_data) + static_cast<int64_t>(item) * a.rows_per_item * row_bytes;
  const unsigned last_page = static_cast<unsigned>(a.num_pages - 1);
  // kept entries of the list before this segment
  int32_t before = 0;
  for (int k = tid; k < seg * kThreads; k += kThreads) {
    const int64_t t = list[k];
    before += (t >= vis_lo && t < vis_hi) ? 1 : 0;
  }
  scan[tid] = before;
  __syncthreads();
  for (int off = kThreads / 2; off > 0; off >>= 1) {
    if (tid < off) scan[tid] += scan[tid + off];
    __syncthreads();
  }
  if (tid == 0) carry = scan[0];
  __syncthreads();
  {
    const int k0 = seg * kThreads;
    const int k = k0 + tid;
    int64_t t = -1;
    bool keep = false;
    if (k < a.topk) {
      t = list[k];
      keep = t >= vis_lo && t < vis_hi;
    }
    // exclusive position of this entry among the kept ones (block scan)
    scan[tid] = keep ? 1 : 0;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
      const int32_t add = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    const int32_t total = scan[kThreads - 1];
    const int32_t local = scan[tid] - (keep ? 1 : 0);
    if (keep) {
      const unsigned pg = min(static_cast<unsigned>(bt[t >> a.page_shift]), last_page);
      src_row[local] = static_cast<int64_t>(pg) * a.page_size + (t & (a.page_size - 1));
      dst_row[local] = carry + local;
    }
    __syncthreads();
    // copy the kept rows: chunk c of the batch is row c / chunks_per_row
    for (int c = tid; c < total * chunks_per_row; c += kThreads) {
      const int e = c / chunks_per_row, part = c - e * chunks_per_row;
      const Chunk* src = reinterpret_cast<const Chunk*>(src_base + src_row[e] * row_bytes) + part;
      Chunk* dst = reinterpret_cast<Chunk*>(dst_base + static_cast<int64_t>(dst_row[e]) * row_bytes) + part;
      *dst = *src;
    }
    if (a.scale != nullptr && tid < total)
      a.out_scale[static_cast<int64_t>(item) * a.rows_per_item + dst_row[tid]] = a.scale[src_row[tid]];
    if (tid == 0 && seg == static_cast<int>(gridDim.y) - 1) a.out_ctx[item] = carry + total;
  }
  if (seg == 0) {
    const int nblk = a.rows_per_item / kCompactPage;
    for (int j = tid; j < nblk; j += kThreads)
      a.out_bt[static_cast<int64_t>(item) * nblk + j] = item * nblk + j;
  }
}

}  // namespace

hipError_t launch_compact_keys(const CompactArgs& a, int32_t items, hipStream_t s) {
  const dim3 grid(items, (a.topk + kThreads - 1) / kThreads);
  if (a.elem_bytes == 2) {
    hipLaunchKernelGGL(compact_keys_kernel<uint4>, grid, dim3(kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL(compact_keys_kernel<uint2>, grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace mla
