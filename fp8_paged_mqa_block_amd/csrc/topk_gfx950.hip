// Per-row top-k of the logits rows for gfx950 (MI355X).
//
// The selection that follows the logits (top_k_per_row_decode in aiter PR
// #4244, first paragraph): for each row r, the indices of the k largest scores
// among its visible tokens [0, visible(r)), -1 in the slots left over.
//
// One 1024-thread workgroup per row runs an exact radix select on
// order-preserving 32-bit keys (4 passes of 8 bits, histograms per wavefront in
// LDS so that clustered keys do not pile onto one counter), which yields the
// exact key of the k-th largest score.  A collection pass then writes every
// index whose key is larger (wavefront-aggregated slot reservation) and, among
// keys equal to the threshold, the lowest indices first (an ordered block scan
// runs only when equal keys outnumber the free slots).  Rows short enough to
// fit are staged once into LDS so the passes do not re-read global memory.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pmqa_internal.h"

namespace pmqa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 256;
constexpr int kStageCap = 16384;  // keys staged in LDS (64 KiB)

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u << 1) == 0u) u = 0u;  // -0 and +0 are the same score
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t ballot(bool pred) { return __ballot(pred); }

__device__ __forceinline__ int lane_rank(uint64_t mask) {
  // number of set bits of mask below this lane
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

template <bool STAGED>
__device__ __forceinline__ uint32_t key_at(const float* __restrict__ row,
                                           const uint32_t* __restrict__ staged, int i) {
  if constexpr (STAGED) return staged[i];
  else return order_key(row[i]);
}

template <bool STAGED>
__device__ void select_row(const float* __restrict__ row, uint32_t* staged, int n, int k,
                           int32_t* __restrict__ out, uint32_t (*hist)[kBins],
                           uint32_t* shared) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  uint32_t prefix = 0, prefix_mask = 0;
  int remaining = k;  // rank of the threshold among keys sharing the prefix
  uint32_t eq_count = 0;

  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < kWaves * kBins; i += kThreads) (&hist[0][0])[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += kThreads) {
      const uint32_t key = key_at<STAGED>(row, staged, i);
      if ((key & prefix_mask) == prefix) atomicAdd(&hist[wave][(key >> shift) & 0xFFu], 1u);
    }
    __syncthreads();
    // bin totals, then the digit holding the remaining-th largest key
    if (tid < kBins) {
      uint32_t s = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) s += hist[w][tid];
      hist[0][tid] = s;
    }
    __syncthreads();
    if (wave == 0) {
      // lane l owns bins 4l..4l+3; suffix sums from the top bin down
      uint32_t c[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) c[q] = hist[0][4 * lane + q];
      const uint32_t mine = c[0] + c[1] + c[2] + c[3];
      // inclusive suffix scan over lanes (lane 63 = highest bins)
      uint32_t suf = mine;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_down(suf, off);
        if (lane + off < 64) suf += o;
      }
      const uint32_t above_lane = suf - mine;  // keys in bins of higher lanes
      uint32_t acc = above_lane;
      int found = -1;
      uint32_t above = 0, cnt = 0;
#pragma unroll
      for (int q = 3; q >= 0; --q) {
        if (found < 0 && acc + c[q] >= (uint32_t)remaining && acc < (uint32_t)remaining) {
          found = 4 * lane + q;
          above = acc;
          cnt = c[q];
        }
        acc += c[q];
      }
      if (found >= 0) {
        shared[0] = (uint32_t)found;
        shared[1] = above;
        shared[2] = cnt;
      }
    }
    __syncthreads();
    const uint32_t digit = shared[0];
    remaining -= (int)shared[1];
    eq_count = shared[2];
    prefix |= digit << shift;
    prefix_mask |= 0xFFu << shift;
    __syncthreads();
  }

  // prefix is now the exact key of the k-th largest score; `remaining` keys
  // equal to it are taken, `k - remaining` keys are strictly larger.
  const uint32_t thr = prefix;
  const bool take_all_equal = eq_count == (uint32_t)remaining;
  if (tid == 0) shared[3] = 0u;
  __syncthreads();
  for (int base = 0; base < n; base += kThreads) {
    const int i = base + tid;
    const uint32_t key = i < n ? key_at<STAGED>(row, staged, i) : 0u;
    const bool sel = i < n && (key > thr || (take_all_equal && key == thr));
    const uint64_t mask = ballot(sel);
    if (mask) {
      uint32_t slot0 = 0;
      if (lane == 0) slot0 = atomicAdd(&shared[3], (uint32_t)__popcll(mask));
      slot0 = __shfl(slot0, 0);
      const uint32_t slot = slot0 + (uint32_t)lane_rank(mask);
      if (sel && slot < (uint32_t)k) out[slot] = i;
    }
  }
  if (take_all_equal) return;
  // ties at the threshold outnumber the free slots: lowest indices first
  __syncthreads();
  uint32_t* wave_cnt = shared + 8;
  int taken = 0;
  const int first_slot = k - remaining;
  for (int base = 0; base < n && taken < remaining; base += kThreads) {
    const int i = base + tid;
    const bool eq = i < n && key_at<STAGED>(row, staged, i) == thr;
    const uint64_t mask = ballot(eq);
    if (lane == 0) wave_cnt[wave] = (uint32_t)__popcll(mask);
    __syncthreads();
    int before = 0, total = 0;
    for (int w = 0; w < kWaves; ++w) {
      const int cw = (int)wave_cnt[w];
      if (w < wave) before += cw;
      total += cw;
    }
    const int rank = taken + before + lane_rank(mask);
    if (eq && rank < remaining) out[first_slot + rank] = i;
    taken += total;
    __syncthreads();
  }
}

__global__ __launch_bounds__(kThreads) void topk_kernel(TopkParams p) {
  __shared__ uint32_t hist[kWaves][kBins];
  __shared__ uint32_t shared[32];
  __shared__ uint32_t staged[kStageCap];

  const int r = blockIdx.x;
  const int b = r / p.next_n;
  const int j = r - b * p.next_n;
  const int ctx = max(p.ctx[b], 0);
  int n = min(max(ctx - p.next_n + j + 1, 0), ctx);
  if ((int64_t)n > p.row_stride) n = (int)p.row_stride;
  const int k = p.k;
  int32_t* out = p.out_idx + (int64_t)r * k;
  const float* row = p.logits + (int64_t)r * p.row_stride;

  if (n <= k) {
    for (int i = threadIdx.x; i < k; i += kThreads) out[i] = i < n ? i : -1;
    return;
  }
  if (n <= kStageCap) {
    for (int i = threadIdx.x; i < n; i += kThreads) staged[i] = order_key(row[i]);
    __syncthreads();
    select_row<true>(row, staged, n, k, out, hist, shared);
  } else {
    select_row<false>(row, staged, n, k, out, hist, shared);
  }
}

}  // namespace

hipError_t launch_topk(const TopkParams& p, const LaunchTiming& tm, hipStream_t stream) {
  const uint32_t rows = (uint32_t)p.batch * (uint32_t)p.next_n;
  if (tm.start || tm.stop)
    hipExtLaunchKernelGGL(topk_kernel, dim3(rows), dim3(kThreads), 0, stream, tm.start, tm.stop,
                          0, p);
  else
    hipLaunchKernelGGL(topk_kernel, dim3(rows), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pmqa
