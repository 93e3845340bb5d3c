// K-cache producer for gfx950 (MI355X): quantises new K rows into the paged
// fp8 cache records that the logits kernel reads.
//
// For token i with cache slot s (the pool's flat token row, page * page_size +
// offset in page):
//   scale = max_d |k[i, d]| / 448 in fp32 (1 when that quotient is 0),
//   code[d] = e4m3fn(clamp(k[i, d] / scale, -448, 448)), round to nearest even,
// written as the record at byte s * (D + 4): the D codes, then the scale as a
// little-endian fp32 (the record layout of the paged cache: the last 4 bytes
// of a token row hold its scale, aiter PR #4244 reproducer).  Slots are int64
// and the byte offset is formed in 64-bit (ATOM PR #2533: the cache writers
// address rows by int64 slots).  Slots outside [0, num_slots) are skipped.
// The same producer can instead write the preshuffled page layout (the same
// 132 bytes per token, regrouped inside each page into tiles of up to 16
// tokens: all tokens' first 16 code bytes, then their next 16, ..., then
// their scales), so that a gather of one token's 16-byte piece across the
// tile's tokens is one contiguous run.
//
// One 16-lane row of a wave per token, 8 elements per lane: the row's amax is
// a DPP max inside the row (no LDS), the quotient is the IEEE fp32 division,
// and v_cvt_pk_fp8_f32 (OCP e4m3 on gfx950, round to nearest even) encodes the
// clamped quotients.  Records sit at a 132-byte stride, so they are 4-byte
// aligned only: each lane stores its 8 codes as two dwords and the row's
// first lane the scale.  The kernel is bound by HBM: per token it reads 4*D
// (fp32) or 2*D (bf16) bytes of k and 8 bytes of slot and writes D + 4 bytes.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pmqa_internal.h"
#include "wave_ops.h"

namespace pmqa {
namespace {

constexpr int kLanesPerToken = 16;
constexpr int kElemsPerLane = kHeadDim / kLanesPerToken;  // 8
constexpr int kTokensPerWave = 64 / kLanesPerToken;       // 4
constexpr int kWavesPerBlock = 4;
constexpr int kTokensPerBlock = kTokensPerWave * kWavesPerBlock;
constexpr float kE4m3Max = 448.0f;

static_assert(kElemsPerLane == 8, "loads and stores below assume 8 elements per lane");

// This lane's 8 consecutive elements of row `tok` (elements 8m .. 8m+7), widened to fp32.
template <bool BF16>
__device__ __forceinline__ void load_elems(const void* k, int64_t tok, int m,
                                           float (&x)[kElemsPerLane]) {
  if constexpr (BF16) {
    const uint4 v = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(k) +
                                                    tok * kHeadDim + m * kElemsPerLane);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);  // bf16 bits are the high half of fp32
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(k) +
                                                      tok * kHeadDim + m * kElemsPerLane);
    const float4 a = p[0], b = p[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

template <bool BF16>
__global__ __launch_bounds__(64 * kWavesPerBlock) void kcache_kernel(KCacheParams p) {
  const int lane = threadIdx.x & 63;
  const int m = lane & (kLanesPerToken - 1);
  const int64_t tok = (int64_t)blockIdx.x * kTokensPerBlock +
                      (threadIdx.x >> 6) * kTokensPerWave + (lane >> 4);
  const bool live = tok < p.num_tokens;
  float x[kElemsPerLane];
#pragma unroll
  for (int i = 0; i < kElemsPerLane; ++i) x[i] = 0.f;
  int64_t slot = -1;
  if (live) {
    load_elems<BF16>(p.k, tok, m, x);
    slot = p.slots[tok];
  }
  // |x| bit patterns order like the magnitudes they encode; every lane of the
  // row takes part in the DPP max (rows past the last token hold zeros)
  uint32_t a = 0u;
#pragma unroll
  for (int i = 0; i < kElemsPerLane; ++i) a = max(a, __float_as_uint(x[i]) & 0x7FFFFFFFu);
  a = row_max(a);
  if (!live || slot < 0 || slot >= p.num_slots) return;

  float scale = __uint_as_float(a) / kE4m3Max;
  if (scale == 0.f) scale = 1.f;
  uint32_t w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float y[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      y[j] = __builtin_fminf(__builtin_fmaxf(x[4 * h + j] / scale, -kE4m3Max), kE4m3Max);
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);  // bytes 0, 1
    v = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], v, true);       // bytes 2, 3
    w[h] = (uint32_t)v;
  }
  if (p.layout == kLayoutPreshuffled) {
    // the preshuffled page layout: token u of page g sits in tile u / R
    // (R = min(page_size, 16) tokens) as its place mm = u % R; the tile holds
    // piece c (row bytes [16c, 16c+16)) of its R tokens at (c * R + mm) * 16,
    // then their scales at 128 * R + 4 * mm.  Lane m's 8 codes are half of
    // piece m / 2.
    const int lp = p.log2_page;
    const int64_t page = slot >> lp;
    const int u = (int)(slot & ((int64_t{1} << lp) - 1));
    const int lr = lp < 4 ? lp : 4;  // log2 R
    const int mm = u & ((1 << lr) - 1);
    uint8_t* tile = p.cache + (page << lp) * (int64_t)kRecordBytes +
                    (int64_t)((u >> lr) << lr) * kRecordBytes;
    uint32_t* dst =
        reinterpret_cast<uint32_t*>(tile + ((((m >> 1) << lr) + mm) * 16) + (m & 1) * 8);
    dst[0] = w[0];
    dst[1] = w[1];
    if (m == 0)
      *reinterpret_cast<uint32_t*>(tile + (kHeadDim << lr) + 4 * mm) = __float_as_uint(scale);
    return;
  }
  uint32_t* rec = reinterpret_cast<uint32_t*>(p.cache + slot * (int64_t)kRecordBytes);
  rec[2 * m] = w[0];
  rec[2 * m + 1] = w[1];
  if (m == 0) rec[kHeadDim / 4] = __float_as_uint(scale);
}

}  // namespace

hipError_t launch_kcache(const KCacheParams& p, const LaunchTiming& tm, hipStream_t stream) {
  const int64_t blocks = ((int64_t)p.num_tokens + kTokensPerBlock - 1) / kTokensPerBlock;
  auto kern = p.bf16 ? kcache_kernel<true> : kcache_kernel<false>;
  if (tm.start || tm.stop)
    hipExtLaunchKernelGGL(kern, dim3((uint32_t)blocks), dim3(64 * kWavesPerBlock), 0, stream,
                          tm.start, tm.stop, 0, p);
  else
    hipLaunchKernelGGL(kern, dim3((uint32_t)blocks), dim3(64 * kWavesPerBlock), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pmqa
