// C-ABI entry points: host-side argument checks, launch geometry, status codes.
// Declarations and the full argument contract are in include/pmqa.h.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include "pmqa.h"
#include "pmqa_internal.h"

namespace {

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
// tokens per page: powers of two from 1 (token-level tables) to 256
bool valid_page_size(int32_t ps) { return is_pow2(ps) && ps <= 256; }

int log2_exact(int64_t x) {
  int l = 0;
  while ((int64_t{1} << l) < x) ++l;
  return l;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// The launch geometry of a logits call, from its sizes alone: the launch and
// the name query both take it from here.
struct LogitsPlan {
  pmqa::LogitsShape sh;
  int64_t max_tokens;  // the grid covers every token a request could have
  int64_t max_iters;   // 64-token iterations the contexts could hold
  int64_t n_rgroups;   // waves sharing a request's next_n rows
  bool flat;           // one single-wave workgroup per iteration
};

LogitsPlan plan_logits(int32_t batch, int32_t next_n, int32_t page_size, int64_t out_row_stride,
                       int32_t num_heads, int64_t block_table_stride) {
  LogitsPlan pl;
  // the table row's capacity and the output row's width bound a context
  int64_t max_tokens = block_table_stride * (int64_t)page_size;
  if (out_row_stride < max_tokens) max_tokens = out_row_stride;
  if (max_tokens > INT32_MAX) max_tokens = INT32_MAX;
  pl.max_tokens = max_tokens;
  pl.sh = pmqa::logits_shape(num_heads, next_n);
  pl.n_rgroups = (next_n + pl.sh.rows_per_wave - 1) / pl.sh.rows_per_wave;
  pl.max_iters = (int64_t)batch * ((max_tokens + pl.sh.iter_tokens - 1) / pl.sh.iter_tokens);
  pl.flat = pl.n_rgroups == 1 && pl.max_iters <= pl.sh.flat_max_items;
  return pl;
}

// The host-checkable preconditions of a logits call's sizes (pointers aside).
pmqa_status check_logits_sizes(int32_t batch, int32_t next_n, int32_t page_size,
                               int64_t out_row_stride, int32_t num_heads, int32_t head_dim,
                               int64_t block_table_stride) {
  if (batch < 0 || next_n < 1 || out_row_stride < 1 || block_table_stride < 1)
    return PMQA_ERR_SHAPE;
  if (!valid_page_size(page_size)) return PMQA_ERR_SHAPE;
  if (head_dim != pmqa::kHeadDim) return PMQA_ERR_UNSUPPORTED;
  if (!(num_heads == 16 || num_heads == 32 || num_heads == 64 || num_heads == 128))
    return PMQA_ERR_UNSUPPORTED;
  if ((int64_t)batch * next_n > INT32_MAX) return PMQA_ERR_SHAPE;
  return PMQA_OK;
}

}  // namespace

namespace pmqa {

int64_t topk_segment_grid(int64_t rows, int32_t k, int64_t max_row_len, uint64_t workspace_bytes) {
  if (rows < 1 || k < 1) return 1;
  if (max_row_len > INT32_MAX) max_row_len = INT32_MAX;
  // rows one workgroup holds in registers are never split; longer ones are
  // cut into segments of at most kTopkSplitKeys scores while the merge has
  // room for their candidates
  if (max_row_len <= kTopkSegmentKeys) return 1;
  int64_t g = (max_row_len + kTopkSplitKeys - 1) / kTopkSplitKeys;  // segments a row needs
  const int64_t merge_cap = kTopkMergeKeys / k;  // the merge holds segments * k candidates
  if (g > merge_cap) g = merge_cap;
  const uint64_t per_segment = (uint64_t)rows * (uint64_t)k * 8u;  // candidates of every row
  if ((uint64_t)g > workspace_bytes / per_segment) g = (int64_t)(workspace_bytes / per_segment);
  return g > 1 ? g : 1;
}

}  // namespace pmqa

extern "C" {

const char* pmqa_status_string(pmqa_status status) {
  switch (status) {
    case PMQA_OK: return "ok";
    case PMQA_ERR_NULL: return "null pointer argument";
    case PMQA_ERR_SHAPE: return "size or stride out of range";
    case PMQA_ERR_UNSUPPORTED: return "unsupported shape or dtype (num_heads 16/32/64/128, head_dim 128, k fp32 or bf16)";
    case PMQA_ERR_WORKSPACE: return "workspace missing (NULL with a nonzero size)";
    case PMQA_ERR_HIP: return "HIP runtime error at launch";
    case PMQA_ERR_ALIGNMENT: return "pointer not aligned as required";
  }
  return "unknown status";
}

int32_t pmqa_version(void) { return 100; }

pmqa_status pmqa_logits_kernel(int32_t batch, int32_t next_n, int32_t page_size,
                               int64_t out_row_stride, int32_t num_heads, int32_t head_dim,
                               int64_t block_table_stride, char* name, int32_t name_len) {
  if (!name || name_len < 1) return PMQA_ERR_NULL;
  const pmqa_status sizes = check_logits_sizes(batch, next_n, page_size, out_row_stride, num_heads,
                                               head_dim, block_table_stride);
  if (sizes != PMQA_OK) return sizes;
  const LogitsPlan pl = plan_logits(batch, next_n, page_size, out_row_stride, num_heads,
                                    block_table_stride);
  const int jw = pl.sh.rows_per_wave;
  int n;
  if (pl.flat) {
    n = snprintf(name, (size_t)name_len, "logits_flat_kernel<%d,%d>", num_heads, jw);
  } else if (const int sring = pmqa::shared_ring_depth(num_heads, jw, (int)pl.n_rgroups)) {
    n = snprintf(name, (size_t)name_len, "logits_shared_kernel<%d,%d,%d>", num_heads,
                 (int)pl.n_rgroups, sring);
  } else {
    int waves = 0, ring = 0;
    pmqa::persistent_geometry(num_heads, jw, &waves, &ring);
    n = snprintf(name, (size_t)name_len, "logits_kernel<%d,%d,%d,%d>", num_heads, jw, waves, ring);
  }
  return n >= 0 && n < name_len ? PMQA_OK : PMQA_ERR_SHAPE;
}

}  // extern "C"

namespace {

pmqa_status logits_impl(const void* q, const void* kv_cache, const float* weights,
                        const int32_t* context_lens, const int64_t* block_tables,
                        int32_t page_size, int32_t next_n, float* out, int64_t out_row_stride,
                        int32_t batch, int32_t num_heads, int32_t head_dim,
                        int64_t block_table_stride, void* stream, const pmqa::LaunchTiming& tm,
                        int kv_layout = pmqa::kLayoutRecords) {
  const pmqa_status sizes = check_logits_sizes(batch, next_n, page_size, out_row_stride, num_heads,
                                               head_dim, block_table_stride);
  if (sizes != PMQA_OK) return sizes;
  // the preshuffled layout's tiles hold min(page_size, 16) tokens; pages of
  // 1, 2 or 4 tokens would cut its 16-byte pieces across pages
  if (kv_layout == pmqa::kLayoutPreshuffled && page_size < 8) return PMQA_ERR_UNSUPPORTED;
  if (batch == 0) return PMQA_OK;
  if (!q || !kv_cache || !weights || !context_lens || !block_tables || !out)
    return PMQA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(weights, 16) || !aligned(kv_cache, 4) || !aligned(out, 4) ||
      !aligned(context_lens, 4) || !aligned(block_tables, 8))
    return PMQA_ERR_ALIGNMENT;

  pmqa::LogitsParams p{};
  p.q = static_cast<const uint8_t*>(q);
  p.kv = static_cast<const uint8_t*>(kv_cache);
  p.w = weights;
  p.ctx = context_lens;
  p.tables = block_tables;
  p.out = out;
  p.out_stride = out_row_stride;
  p.table_stride = block_table_stride;
  p.page_bytes = (int64_t)page_size * pmqa::kRecordBytes;
  p.batch = batch;
  p.next_n = next_n;
  p.page_size = page_size;
  p.log2_page = log2_exact(page_size);
  p.kv_layout = kv_layout;
  // chunks of a preshuffled 8-32-token page: 33 * page_size / 4; the gather
  // divides by it as a multiply by ceil(2^20 / it) (exact below 576)
  p.pre_magic = kv_layout == pmqa::kLayoutPreshuffled && page_size < 64
                    ? (uint32_t)(((1u << 20) + (33u * page_size / 4u) - 1u) / (33u * page_size / 4u))
                    : 0u;
  const LogitsPlan pl = plan_logits(batch, next_n, page_size, out_row_stride, num_heads,
                                    block_table_stride);
  p.max_tokens = (int32_t)pl.max_tokens;
  const pmqa::LogitsShape& sh = pl.sh;
  const int64_t n_rgroups = pl.n_rgroups;
  // the grid's work units: enough to fill the chip, and at least 4 per request
  // so that the device-side split (runs never cross requests) stays balanced
  // when requests are long and few units are resident at once; never more
  // than the iterations the contexts could hold, never fewer than the batch
  const int64_t max_iters = pl.max_iters;
  int64_t n_slices = sh.target_waves / n_rgroups;
  if (n_slices < 4 * (int64_t)batch) n_slices = 4 * (int64_t)batch;
  if (n_slices > max_iters) n_slices = max_iters;
  if (n_slices > INT32_MAX / n_rgroups) n_slices = INT32_MAX / n_rgroups;  // still >= batch
  p.n_slices = (int32_t)n_slices;
  p.n_rgroups = (int32_t)n_rgroups;
  p.flat_items = pl.flat ? max_iters : 0;
  // small block tables and q rows are pulled into L2 at kernel start, while
  // the context lengths are read, so that the page-id and q loads that depend
  // on them hit L2
  const int64_t kWarmMax = int64_t{4} << 20;
  const int64_t kWarmTableMax = int64_t{1} << 20;  // per XCD L2 (4 MB each): a quarter at most
  const int64_t table_bytes = (int64_t)batch * block_table_stride * 8;
  const int64_t q_bytes = (int64_t)batch * next_n * num_heads * head_dim;
  p.warm_table_lines = table_bytes <= kWarmTableMax ? (table_bytes + 127) / 128 : 0;
  p.warm_q_lines = q_bytes <= kWarmMax ? q_bytes / 128 : 0;
  if (!is_pow2(page_size)) return PMQA_ERR_SHAPE;

  hipError_t e = pmqa::launch_logits(p, sh, num_heads, tm, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PMQA_OK : PMQA_ERR_HIP;
}

pmqa_status topk_impl(const float* logits, const int32_t* context_lens, int32_t k,
                      int32_t* out_idx, int32_t batch, int32_t next_n, int64_t logits_row_stride,
                      void* workspace, size_t workspace_bytes, void* stream,
                      const pmqa::LaunchTiming& tm) {
  if (batch < 0 || next_n < 1 || logits_row_stride < 1) return PMQA_ERR_SHAPE;
  if (k < 1 || k > pmqa::kTopkMaxK) return PMQA_ERR_SHAPE;
  if ((int64_t)batch * next_n > INT32_MAX) return PMQA_ERR_SHAPE;
  if (workspace_bytes > 0 && !workspace) return PMQA_ERR_WORKSPACE;
  if (batch == 0) return PMQA_OK;
  if (!logits || !context_lens || !out_idx) return PMQA_ERR_NULL;
  if (!aligned(logits, 4) || !aligned(context_lens, 4) || !aligned(out_idx, 4) ||
      (workspace_bytes > 0 && !aligned(workspace, 16)))
    return PMQA_ERR_ALIGNMENT;
  const int64_t rows = (int64_t)batch * next_n;
  pmqa::TopkParams p{};
  p.logits = logits;
  p.ctx = context_lens;
  p.out_idx = out_idx;
  p.row_stride = logits_row_stride;
  p.batch = batch;
  p.next_n = next_n;
  p.k = k;
  p.seg_grid = (int32_t)pmqa::topk_segment_grid(rows, k, logits_row_stride, workspace_bytes);
  if (p.seg_grid > 1) {
    const int64_t slots = rows * p.seg_grid * k;
    p.cand_val = static_cast<float*>(workspace);
    p.cand_idx = reinterpret_cast<int32_t*>(p.cand_val + slots);
  }
  hipError_t e = pmqa::launch_topk(p, tm, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PMQA_OK : PMQA_ERR_HIP;
}

pmqa_status kcache_impl(const void* k, int32_t k_dtype, const int64_t* slot_mapping,
                        int32_t num_tokens, int32_t head_dim, void* kv_cache, int64_t num_slots,
                        void* stream, const pmqa::LaunchTiming& tm,
                        int layout = pmqa::kLayoutRecords, int32_t page_size = 0) {
  if (num_tokens < 0 || num_slots < 0) return PMQA_ERR_SHAPE;
  if (layout == pmqa::kLayoutPreshuffled) {
    if (!valid_page_size(page_size)) return PMQA_ERR_SHAPE;
    if (page_size < 8) return PMQA_ERR_UNSUPPORTED;
    if (num_slots % page_size != 0) return PMQA_ERR_SHAPE;  // whole pages only
  }
  if (k_dtype != PMQA_DTYPE_F32 && k_dtype != PMQA_DTYPE_BF16) return PMQA_ERR_UNSUPPORTED;
  if (head_dim != pmqa::kHeadDim) return PMQA_ERR_UNSUPPORTED;
  if (num_tokens > 0 && (!k || !slot_mapping || (num_slots > 0 && !kv_cache)))
    return PMQA_ERR_NULL;
  if (!aligned(k, 16) || !aligned(slot_mapping, 8) || !aligned(kv_cache, 4))
    return PMQA_ERR_ALIGNMENT;
  if (num_tokens == 0) return PMQA_OK;
  pmqa::KCacheParams p{};
  p.k = k;
  p.slots = slot_mapping;
  p.cache = static_cast<uint8_t*>(kv_cache);
  p.num_slots = num_slots;
  p.num_tokens = num_tokens;
  p.bf16 = k_dtype == PMQA_DTYPE_BF16 ? 1 : 0;
  p.layout = layout;
  p.log2_page = layout == pmqa::kLayoutPreshuffled ? log2_exact(page_size) : 0;
  const hipError_t e = pmqa::launch_kcache(p, tm, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PMQA_OK : PMQA_ERR_HIP;
}

pmqa::LaunchTiming timing(void* start_event, void* stop_event) {
  pmqa::LaunchTiming tm;
  tm.start = static_cast<hipEvent_t>(start_event);
  tm.stop = static_cast<hipEvent_t>(stop_event);
  return tm;
}

}  // namespace

extern "C" {

pmqa_status paged_mqa_logits(const void* q, const void* kv_cache, const float* weights,
                             const int32_t* context_lens, const int64_t* block_tables,
                             int32_t page_size, int32_t next_n, float* out,
                             int64_t out_row_stride, int32_t batch, int32_t num_heads,
                             int32_t head_dim, int64_t block_table_stride, void* stream) {
  return logits_impl(q, kv_cache, weights, context_lens, block_tables, page_size, next_n, out,
                     out_row_stride, batch, num_heads, head_dim, block_table_stride, stream,
                     pmqa::LaunchTiming{});
}

pmqa_status paged_mqa_logits_timed(const void* q, const void* kv_cache, const float* weights,
                                   const int32_t* context_lens, const int64_t* block_tables,
                                   int32_t page_size, int32_t next_n, float* out,
                                   int64_t out_row_stride, int32_t batch, int32_t num_heads,
                                   int32_t head_dim, int64_t block_table_stride, void* stream,
                                   void* start_event, void* stop_event) {
  return logits_impl(q, kv_cache, weights, context_lens, block_tables, page_size, next_n, out,
                     out_row_stride, batch, num_heads, head_dim, block_table_stride, stream,
                     timing(start_event, stop_event));
}

pmqa_status paged_mqa_logits_preshuffled(const void* q, const void* kv_cache,
                                         const float* weights, const int32_t* context_lens,
                                         const int64_t* block_tables, int32_t page_size,
                                         int32_t next_n, float* out, int64_t out_row_stride,
                                         int32_t batch, int32_t num_heads, int32_t head_dim,
                                         int64_t block_table_stride, void* stream) {
  return logits_impl(q, kv_cache, weights, context_lens, block_tables, page_size, next_n, out,
                     out_row_stride, batch, num_heads, head_dim, block_table_stride, stream,
                     pmqa::LaunchTiming{}, pmqa::kLayoutPreshuffled);
}

pmqa_status paged_mqa_logits_preshuffled_timed(const void* q, const void* kv_cache,
                                               const float* weights, const int32_t* context_lens,
                                               const int64_t* block_tables, int32_t page_size,
                                               int32_t next_n, float* out, int64_t out_row_stride,
                                               int32_t batch, int32_t num_heads, int32_t head_dim,
                                               int64_t block_table_stride, void* stream,
                                               void* start_event, void* stop_event) {
  return logits_impl(q, kv_cache, weights, context_lens, block_tables, page_size, next_n, out,
                     out_row_stride, batch, num_heads, head_dim, block_table_stride, stream,
                     timing(start_event, stop_event), pmqa::kLayoutPreshuffled);
}

pmqa_status quantize_k_cache_preshuffled(const void* k, int32_t k_dtype,
                                         const int64_t* slot_mapping, int32_t num_tokens,
                                         int32_t head_dim, void* kv_cache, int64_t num_slots,
                                         int32_t page_size, void* stream) {
  return kcache_impl(k, k_dtype, slot_mapping, num_tokens, head_dim, kv_cache, num_slots, stream,
                     pmqa::LaunchTiming{}, pmqa::kLayoutPreshuffled, page_size);
}

pmqa_status topk_per_row(const float* logits, const int32_t* context_lens, int32_t k,
                         int32_t* out_idx, int32_t batch, int32_t next_n,
                         int64_t logits_row_stride, void* workspace, size_t workspace_bytes,
                         void* stream) {
  return topk_impl(logits, context_lens, k, out_idx, batch, next_n, logits_row_stride, workspace,
                   workspace_bytes, stream, pmqa::LaunchTiming{});
}

pmqa_status topk_per_row_timed(const float* logits, const int32_t* context_lens, int32_t k,
                               int32_t* out_idx, int32_t batch, int32_t next_n,
                               int64_t logits_row_stride, void* workspace, size_t workspace_bytes,
                               void* stream, void* start_event, void* stop_event) {
  return topk_impl(logits, context_lens, k, out_idx, batch, next_n, logits_row_stride, workspace,
                   workspace_bytes, stream, timing(start_event, stop_event));
}

static_assert(PMQA_NOALLOC_SCRATCH_BYTES == pmqa::kTopkScratchBytes,
              "the header states the scratch size the library holds");

pmqa_status topk_per_row_noalloc(const float* logits, const int32_t* context_lens, int32_t k,
                                 int32_t* out_idx, int32_t batch, int32_t next_n,
                                 int64_t logits_row_stride, void* stream) {
  // the split topk_per_row makes for rows as long as the stride, in the
  // library's fixed scratch; larger is refused before anything else happens
  if (batch < 0 || next_n < 1 || logits_row_stride < 1) return PMQA_ERR_SHAPE;
  if (k < 1 || k > pmqa::kTopkMaxK) return PMQA_ERR_SHAPE;
  if ((int64_t)batch * next_n > INT32_MAX) return PMQA_ERR_SHAPE;
  const size_t need = topk_per_row_workspace_size(batch * next_n, k, logits_row_stride);
  if (need > pmqa::kTopkScratchBytes) return PMQA_ERR_WORKSPACE;
  if (batch == 0) return PMQA_OK;
  if (!logits || !context_lens || !out_idx) return PMQA_ERR_NULL;
  void* scratch = nullptr;
  if (need > 0 && pmqa::topk_scratch(&scratch) != hipSuccess) return PMQA_ERR_HIP;
  return topk_impl(logits, context_lens, k, out_idx, batch, next_n, logits_row_stride, scratch,
                   need, stream, pmqa::LaunchTiming{});
}

size_t topk_per_row_workspace_size(int32_t rows, int32_t k, int64_t max_row_len) {
  if (rows < 0 || k < 1 || k > pmqa::kTopkMaxK || max_row_len < 0) return 0;
  const int64_t g = pmqa::topk_segment_grid(rows, k, max_row_len, UINT64_MAX);
  return g > 1 ? (size_t)rows * (size_t)g * (size_t)k * 8u : 0u;
}

pmqa_status quantize_k_cache(const void* k, int32_t k_dtype, const int64_t* slot_mapping,
                             int32_t num_tokens, int32_t head_dim, void* kv_cache,
                             int64_t num_slots, void* stream) {
  return kcache_impl(k, k_dtype, slot_mapping, num_tokens, head_dim, kv_cache, num_slots, stream,
                     pmqa::LaunchTiming{});
}

pmqa_status quantize_k_cache_timed(const void* k, int32_t k_dtype, const int64_t* slot_mapping,
                                   int32_t num_tokens, int32_t head_dim, void* kv_cache,
                                   int64_t num_slots, void* stream, void* start_event,
                                   void* stop_event) {
  return kcache_impl(k, k_dtype, slot_mapping, num_tokens, head_dim, kv_cache, num_slots, stream,
                     timing(start_event, stop_event));
}

pmqa_status pmqa_check_inputs(const int32_t* context_lens, const int64_t* block_tables,
                              int32_t batch, int32_t page_size, int64_t block_table_stride,
                              int64_t out_row_stride, int64_t num_pages, int32_t* result,
                              void* stream) {
  if (batch < 0 || block_table_stride < 1 || out_row_stride < 1 || num_pages < 1)
    return PMQA_ERR_SHAPE;
  if (!valid_page_size(page_size)) return PMQA_ERR_SHAPE;
  if (!result || (batch > 0 && (!context_lens || !block_tables))) return PMQA_ERR_NULL;
  if (!aligned(result, 4) || !aligned(context_lens, 4) || !aligned(block_tables, 8))
    return PMQA_ERR_ALIGNMENT;
  pmqa::CheckParams p{};
  p.ctx = context_lens;
  p.tables = block_tables;
  p.result = result;
  p.table_stride = block_table_stride;
  p.out_stride = out_row_stride;
  p.num_pages = num_pages;
  p.page_size = page_size;
  p.batch = batch;
  const hipError_t e = pmqa::launch_check(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PMQA_OK : PMQA_ERR_HIP;
}

}  // extern "C"
