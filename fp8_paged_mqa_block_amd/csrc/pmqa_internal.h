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
  int32_t n_chunks;        // token chunks per request covered by the grid
  int32_t n_rgroups;       // waves per chunk splitting the next_n rows
  uint32_t n_units;        // batch * n_chunks * n_rgroups wave units
};

hipError_t launch_logits(const LogitsParams& p, int heads, int rows_per_wave_j,
                         hipStream_t stream);
// Number of MTP rows one wave holds for a given head count (the host uses it
// to size the grid; the kernel is instantiated for exactly these).
int logits_rows_per_wave(int heads, int next_n);
// Tokens one wave unit covers.
int logits_wave_tokens();

struct TopkParams {
  const float* logits;
  const int32_t* ctx;
  int32_t* out_idx;
  int64_t row_stride;
  int32_t batch;
  int32_t next_n;
  int32_t k;
};

hipError_t launch_topk(const TopkParams& p, hipStream_t stream);

}  // namespace pmqa
