// Debug check of the preconditions that live in device memory, which the
// scoring and selection calls cannot check without a synchronisation: every
// context length fits the request's table row and output row, and every page
// id the context uses lies inside the pool (the failure classes the pages
// report are stores silently dropped at large output strides, aiter PR #4244,
// and wrong pages from wrapped ids, ATOM PR #2533).  The check reads the
// context lengths and the used table entries only and never dereferences an
// id.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pmqa_internal.h"

namespace pmqa {
namespace {

constexpr int kCheckThreads = 256;

__global__ void check_init(int32_t* result, int32_t batch) {
  if (threadIdx.x == 0) {
    result[0] = 0;
    result[1] = batch;
  }
}

// One workgroup per request.
__global__ __launch_bounds__(kCheckThreads) void check_request(CheckParams p) {
  __shared__ int bad;
  const int b = blockIdx.x;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  const int64_t ctx = max(p.ctx[b], 0);
  const int64_t capacity = p.table_stride * p.page_size;
  if (threadIdx.x == 0 && (ctx > capacity || ctx > p.out_stride)) bad = 1;
  // used entries, never past the row
  const int64_t used = (min(ctx, capacity) + p.page_size - 1) / p.page_size;
  const int64_t* row = p.tables + (int64_t)b * p.table_stride;
  int mine = 0;
  for (int64_t i = threadIdx.x; i < used; i += kCheckThreads) {
    const int64_t id = row[i];
    mine |= (id < 0 || id >= p.num_pages) ? 1 : 0;
  }
  if (mine) atomicOr(&bad, 1);
  __syncthreads();
  if (threadIdx.x == 0 && bad) {
    atomicAdd(&p.result[0], 1);
    atomicMin(&p.result[1], b);
  }
}

}  // namespace

hipError_t launch_check(const CheckParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(check_init, dim3(1), dim3(64), 0, stream, p.result, p.batch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.batch == 0) return e;
  hipLaunchKernelGGL(check_request, dim3((uint32_t)p.batch), dim3(kCheckThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pmqa
