// Internal launch interface between the C-ABI host layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pmqa {

// Head dimension of q and of every K record (the matrix-core K depth).
constexpr int kHeadDim = 128;
// Bytes of one K-cache token record: kHeadDim e4m3fn codes + one fp32 scale.
constexpr int kRecordBytes = kHeadDim + 4;

struct LogitsParams {
  const uint8_t* q;        // [rows, H, 128] e4m3fn
  const uint8_t* kv;       // page pool
  const float* w;          // [rows, H]
  const int32_t* ctx;      // [batch]
  const int64_t* tables;   // [batch, table_stride]
  float* out;              // rows at r*out_stride
  int64_t out_stride;      // elements
  int64_t table_stride;    // entries
  int64_t page_bytes;      // page_size * kRecordBytes
  int32_t batch;
  int32_t next_n;
  int32_t page_size;
  int32_t log2_page;
  int32_t max_tokens;      // min(table_stride*page_size, out_stride), clamped to int32
  int32_t n_slices;        // work units of the grid (>= batch); each takes one run
  int32_t n_rgroups;       // waves per run splitting the next_n rows
  int64_t warm_table_lines;  // 128-byte lines of the block table to pull into every XCD's L2
  int64_t warm_q_lines;      // 128-byte lines of q to pull into L2 once (0: none)
  int64_t flat_items;        // > 0: flat geometry over this many possible iterations
  int32_t kv_layout;         // 0: per-token records; 1: preshuffled pages (8..256 tokens)
  uint32_t pre_magic;        // preshuffled pages of 8..32 tokens: ceil(2^20 / chunks per page)
};

// Byte layouts of the page pool (see paged_mqa_logits_preshuffled).
constexpr int kLayoutRecords = 0;
constexpr int kLayoutPreshuffled = 1;

// Optional events recorded by the kernel dispatch itself at its start and end.
struct LaunchTiming {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// Launch geometry chosen on the host for a head count and next_n.
struct LogitsShape {
  int rows_per_wave;  // next_n rows one wave holds (JW)
  int iter_tokens;    // tokens per iteration of a wave
  int target_waves;   // waves of the persistent grid when there is enough work
  int flat_max_items; // flat geometry when every row of a request fits one wave and
                      // the possible iterations are at most this many (0: never)
};
LogitsShape logits_shape(int heads, int next_n);
// Ring depth of the shared-ring geometry, or 0 where it does not apply: one
// next_n row per wave of 128 heads, with 2 or 4 rows per request (a
// workgroup of 4 or 2 waves' units then holds 8 or 4 slots).
inline constexpr int shared_ring_depth(int heads, int rows_per_wave, int n_rgroups) {
  return heads == 128 && rows_per_wave == 1 ? (n_rgroups == 4 ? 8 : (n_rgroups == 2 ? 4 : 0)) : 0;
}
// Workgroup waves and iterations in flight of the persistent geometry.
void persistent_geometry(int heads, int rows_per_wave, int* waves, int* ring);
hipError_t launch_logits(const LogitsParams& p, const LogitsShape& sh, int heads,
                         const LaunchTiming& tm, hipStream_t stream);

// Largest k the top-k accepts (the indexer keeps at most 2048 tokens per row).
constexpr int kTopkMaxK = 2048;
// Scores one top-k workgroup selects from registers: a row longer than this is
// split into segments of at most this many scores (while the workspace has
// room for their candidates), and a row's merge takes at most this many
// candidates (segments * k).
constexpr int kTopkSegmentKeys = 16384;
constexpr int kTopkMergeKeys = 16384;
// Scores a segment of a split row holds when the grid has room: 8 a thread,
// the layout the value-bucket select keeps within the register budget of two
// workgroups per CU.
constexpr int kTopkSplitKeys = 8192;

// Segments of a row of n visible scores (n > k) in a stage-1 grid of `grid`
// segments per row.  1: the grid does not split rows (grid 1), or the row
// fits one split segment.  Otherwise as many segments of at most
// kTopkSplitKeys scores as the grid holds; when that is not enough, `grid`
// segments of at most kTopkSegmentKeys; 0 for a longer row (the merge launch
// selects it whole).  Every segment of a split row holds more than 4096
// scores, so more than k <= 2048.
__host__ __device__ inline int topk_row_segments(int n, int grid) {
  if (grid <= 1) return 1;
  const int n_small = (n + kTopkSplitKeys - 1) / kTopkSplitKeys;
  if (n_small <= grid) return n_small;
  const int n_large = (n + kTopkSegmentKeys - 1) / kTopkSegmentKeys;
  return n_large <= grid ? grid : 0;
}

struct TopkParams {
  const float* logits;
  const int32_t* ctx;
  int32_t* out_idx;
  float* cand_val;         // workspace: [rows, seg_grid, k] candidate scores
  int32_t* cand_idx;       // workspace: [rows, seg_grid, k] candidate indices
  int64_t row_stride;
  int32_t batch;
  int32_t next_n;
  int32_t k;
  int32_t seg_grid;        // most segments a row is split into (1: no split)
};

// Bytes of the fixed scratch array the allocation-free top-k uses as its
// workspace (one copy per GPU).
constexpr uint64_t kTopkScratchBytes = uint64_t{64} << 20;
// This device's copy of that array (looked up once per device).
hipError_t topk_scratch(void** ptr);

// Most segments a row of up to max_row_len scores is split into, given the
// workspace bytes for its candidates (0 bytes: 1, no split).
int64_t topk_segment_grid(int64_t rows, int32_t k, int64_t max_row_len, uint64_t workspace_bytes);

hipError_t launch_topk(const TopkParams& p, const LaunchTiming& tm, hipStream_t stream);

struct CheckParams {
  const int32_t* ctx;
  const int64_t* tables;
  int32_t* result;         // [2]: requests that violate, lowest such request (batch: none)
  int64_t table_stride;
  int64_t out_stride;
  int64_t num_pages;
  int32_t page_size;
  int32_t batch;
};

hipError_t launch_check(const CheckParams& p, hipStream_t stream);

struct KCacheParams {
  const void* k;           // [num_tokens, kHeadDim] fp32 or bf16
  const int64_t* slots;    // [num_tokens] cache rows
  uint8_t* cache;          // page pool of num_slots records
  int64_t num_slots;
  int32_t num_tokens;
  int32_t bf16;            // 1: k holds bf16, 0: fp32
  int32_t layout;          // kLayoutRecords or kLayoutPreshuffled
  int32_t log2_page;       // preshuffled: log2(page_size)
};

hipError_t launch_kcache(const KCacheParams& p, const LaunchTiming& tm, hipStream_t stream);

}  // namespace pmqa
