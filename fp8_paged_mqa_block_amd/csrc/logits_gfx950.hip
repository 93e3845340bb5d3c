// FP8 paged MQA logits for gfx950 (MI355X).
//
// Computes, for every output row r = b*next_n + j of request b and token t of
// its context,
//     logit[r, t] = sum_h w[r, h] * relu(scale_t * (q[r, h, :] . k_t))
// with q and k in e4m3fn, the dot on the fp8 matrix cores
// (v_mfma_f32_16x16x128_f8f6f4, fp32 accumulate), the scale/relu/head-weighted
// sum fused in registers, -inf on the masked tail [visible, ctx) and no write
// past the context.  The op is the one the pages call
// deepgemm_fp8_paged_mqa_logits (aiter PR #4244, bug description and fix);
// the score formula is the DSA indexer score, adopted where the pages are
// silent.
//
// Mapping onto CDNA4:
//  * one wavefront owns a "wave unit": request b, a 256-token chunk of its
//    context, and a group of up to JW of its next_n rows.  The unit's rows of
//    q (JW*H x 128 e4m3fn) stay in VGPRs as MFMA A operands, heads on the M
//    dimension, so each lane ends up holding 4 heads of one token and the head
//    reduction is in-lane FMAs plus two cross-lane adds;
//  * K is gathered straight from the paged pool into B-operand registers: lane
//    l reads 32 bytes of token (l % 16).  Each lane forms its own token's
//    address from the block table, so a 16-token tile may draw on several
//    pages smaller than the tile (aiter PR #6626 section 1 builds one tile from
//    several 8-token pages); the unit's page ids are read once, before its
//    tiles, one id per lane, and passed to the token lanes by a lane shuffle;
//  * page byte offsets are int64 (id * page_size * 132) and the output row
//    base is int64 (row * out_row_stride) with int32 columns, so pools and
//    outputs beyond 2^31 bytes are addressed correctly (aiter PR #4244 "Fix";
//    ATOM PR #2533 "Address Triton decode KV rows with int64 ids");
//  * workgroups are dealt round-robin over the 8 XCDs, so the grid is
//    re-indexed to give each XCD a contiguous run of units: a request's
//    chunks share one L2, which keeps its q and table warm.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pmqa_internal.h"

namespace pmqa {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// K records are 132 bytes, so a token's bytes are only 4-byte aligned.
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4))) __attribute__((aligned(4)));

constexpr int kTile = 16;                 // tokens per MFMA tile (N)
constexpr int kTilesPerIter = 4;          // 64 tokens: one per lane at store time
constexpr int kIterTokens = kTile * kTilesPerIter;
constexpr int kWaveTokens = 256;          // tokens per wave unit
constexpr int kWavesPerGroup = 4;         // waves per workgroup
constexpr int kThreads = 64 * kWavesPerGroup;

__device__ __forceinline__ v8i load_q32(const uint8_t* p) {
  const u32x4* v = reinterpret_cast<const u32x4*>(p);  // 32-byte aligned
  u32x4 a = v[0], b = v[1];
  v8i r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

__device__ __forceinline__ v8i load_k32(const uint8_t* p) {
  const u32x4_a4* v = reinterpret_cast<const u32x4_a4*>(p);  // 4-byte aligned
  u32x4 a = v[0], b = v[1];
  v8i r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

__device__ __forceinline__ v4f mfma_fp8(v8i a, v8i b) {
  v4f zero = {0.f, 0.f, 0.f, 0.f};
  // cbsz = blgp = 0 selects e4m3 for both operands; zero scale operands select
  // the unscaled instruction.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// e4m3 -> f16 is exact (every e4m3 value is an f16 value).  Eight bytes of a
// lane's 32-byte operand become one f16 MFMA operand.
__device__ __forceinline__ v8h fp8x8_to_f16(int lo, int hi) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)lo, 1.0f, false);
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)lo, 1.0f, true);
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)hi, 1.0f, false);
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)hi, 1.0f, true);
  v8h r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// The same 16x16x128 product with exact products and fp32 sums: four chained
// 16x16x32 f16 MFMAs over the operands' four 8-byte slices.  A and B are sliced
// identically, so every K index meets its partner exactly once.
__device__ __forceinline__ v4f mfma_exact(v8i a, const v8h (&b)[4]) {
  v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    // convert the q slice at its use: the empty asm keeps the compiler from
    // hoisting all converted q tiles out of the token loop, which would double
    // the registers q occupies
    int lo = a[2 * c], hi = a[2 * c + 1];
    asm volatile("" : "+v"(lo), "+v"(hi));
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(fp8x8_to_f16(lo, hi), b[c], acc, 0, 0, 0);
  }
  return acc;
}

// Rows that see fewer tokens than this are scored on the exact-sum path.  The
// fp8 matrix core sums each run of 8 consecutive products after aligning them
// to the largest, keeping about 14 bits below it; on a row of a few tokens
// whose head-weighted sum cancels, that rounding can reach a few 1e-4 of the
// row's largest score, while rows of 32 tokens or more stay near 4e-5.
constexpr int kExactRows = 128;

struct UnitCtx {
  const uint8_t* kv;
  float* out;
  int64_t out_stride;
  int64_t page_base;  // lane i: byte offset of the unit's i-th page
  int b, ctx, ctx_eff, t_begin, t_end, j0, next_n, p_first, lp, in_page_mask, lane, m, kq;
};

template <int H, int JW, bool EXACT>
__device__ __forceinline__ void run_unit(const UnitCtx& u, const v8i (&qa)[JW][H / 16],
                                         const v4f (&wv)[JW][H / 16]) {
  constexpr int HT = H / 16;
  const float neg_inf = -__builtin_inff();
  for (int it0 = u.t_begin; it0 < u.t_end; it0 += kIterTokens) {
    // addresses first (lanes past the unit's end read the pool's first record,
    // and their results are never stored), then every load of the iteration
    int64_t off[kTilesPerIter];
#pragma unroll
    for (int tile = 0; tile < kTilesPerIter; ++tile) {
      const int t = it0 + tile * kTile + u.m;
      const bool valid = t < u.t_end;
      const int slot = valid ? (t >> u.lp) - u.p_first : 0;
      const int64_t base = __shfl(u.page_base, slot);
      const int64_t o = base + (int32_t)((t & u.in_page_mask) * kRecordBytes);
      off[tile] = valid ? o : int64_t{0};
    }
    v8i kb[kTilesPerIter];
    float ks[kTilesPerIter];
#pragma unroll
    for (int tile = 0; tile < kTilesPerIter; ++tile) {
      const uint8_t* rec = u.kv + off[tile];
      kb[tile] = load_k32(rec + u.kq * 32);
      ks[tile] = *reinterpret_cast<const float*>(rec + kHeadDim);
    }

    float keep[JW];
#pragma unroll
    for (int jj = 0; jj < JW; ++jj) keep[jj] = 0.f;
#pragma unroll
    for (int tile = 0; tile < kTilesPerIter; ++tile) {
      const float s = ks[tile];
      v8h kh[4];
      if constexpr (EXACT) {
#pragma unroll
        for (int c = 0; c < 4; ++c) kh[c] = fp8x8_to_f16(kb[tile][2 * c], kb[tile][2 * c + 1]);
      }
#pragma unroll
      for (int jj = 0; jj < JW; ++jj) {
        float sum = 0.f;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
          v4f acc;
          if constexpr (EXACT) acc = mfma_exact(qa[jj][ht], kh);
          else acc = mfma_fp8(qa[jj][ht], kb[tile]);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sum = __builtin_fmaf(wv[jj][ht][i], __builtin_fmaxf(acc[i] * s, 0.f), sum);
        }
        sum += __shfl_xor(sum, 16);
        sum += __shfl_xor(sum, 32);
        if (u.kq == tile) keep[jj] = sum;
      }
    }

    const int t = it0 + u.lane;
#pragma unroll
    for (int jj = 0; jj < JW; ++jj) {
      const int j = u.j0 + jj;
      if (j >= u.next_n) break;
      const int vis = min(max(u.ctx - u.next_n + j + 1, 0), u.ctx_eff);
      float* orow = u.out + ((int64_t)u.b * u.next_n + j) * u.out_stride;
      if (t < vis)
        orow[t] = keep[jj];
      else if (t < u.ctx_eff)
        orow[t] = neg_inf;
    }
  }
}

// H heads; JW next_n rows per wave.
template <int H, int JW>
__global__ __launch_bounds__(kThreads) void logits_kernel(LogitsParams p) {
  constexpr int HT = H / 16;  // 16-head A tiles per row
  UnitCtx u;
  u.lane = threadIdx.x & 63;
  u.m = u.lane & 15;   // token within a tile (B column / A row)
  u.kq = u.lane >> 4;  // 32-byte quarter of the head dimension
  const uint32_t nwg = gridDim.x;  // a multiple of 8
  const uint32_t wg = (blockIdx.x & 7u) * (nwg >> 3) + (blockIdx.x >> 3);
  const uint32_t unit = wg * kWavesPerGroup + (threadIdx.x >> 6);
  if (unit >= p.n_units) return;

  const int g = (int)(unit % (uint32_t)p.n_rgroups);
  const uint32_t bc = unit / (uint32_t)p.n_rgroups;
  const int c = (int)(bc % (uint32_t)p.n_chunks);
  u.b = (int)(bc / (uint32_t)p.n_chunks);
  u.ctx = max(p.ctx[u.b], 0);
  u.ctx_eff = min(u.ctx, p.max_tokens);
  u.t_begin = c * kWaveTokens;
  if (u.t_begin >= u.ctx_eff) return;
  u.t_end = min(u.t_begin + kWaveTokens, u.ctx_eff);
  u.j0 = g * JW;
  u.next_n = p.next_n;
  u.kv = p.kv;
  u.out = p.out;
  u.out_stride = p.out_stride;

  // q rows and weights of this unit, in MFMA A-operand order
  v8i qa[JW][HT];
  v4f wv[JW][HT];
#pragma unroll
  for (int jj = 0; jj < JW; ++jj) {
    const int j = min(u.j0 + jj, u.next_n - 1);  // rows past next_n are never stored
    const int64_t row = (int64_t)u.b * u.next_n + j;
    const uint8_t* qrow = p.q + row * (int64_t)(H * kHeadDim);
    const float* wrow = p.w + row * H;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      qa[jj][ht] = load_q32(qrow + (ht * 16 + u.m) * kHeadDim + u.kq * 32);
      wv[jj][ht] = *reinterpret_cast<const v4f*>(wrow + ht * 16 + u.kq * 4);
    }
  }

  // page ids of the unit, one per lane (at most 32 for 8-token pages)
  u.lp = p.log2_page;
  u.p_first = u.t_begin >> u.lp;
  const int n_pg = ((u.t_end - 1) >> u.lp) - u.p_first + 1;
  u.page_base = 0;
  if (u.lane < n_pg)
    u.page_base = p.tables[(int64_t)u.b * p.table_stride + u.p_first + u.lane] * p.page_bytes;
  u.in_page_mask = p.page_size - 1;

  // the unit's first row sees the fewest tokens
  const int min_vis = min(max(u.ctx - u.next_n + u.j0 + 1, 0), u.ctx);
  if (min_vis < kExactRows)
    run_unit<H, JW, true>(u, qa, wv);
  else
    run_unit<H, JW, false>(u, qa, wv);
}

template <int H, int JW>
hipError_t launch_one(const LogitsParams& p, hipStream_t stream) {
  uint32_t n_wg = (p.n_units + kWavesPerGroup - 1) / kWavesPerGroup;
  n_wg = (n_wg + 7u) & ~7u;
  hipLaunchKernelGGL((logits_kernel<H, JW>), dim3(n_wg), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int H>
hipError_t launch_heads(const LogitsParams& p, int jw, hipStream_t stream) {
  if constexpr (H <= 64) {
    switch (jw) {
      case 1: return launch_one<H, 1>(p, stream);
      case 2: return launch_one<H, 2>(p, stream);
      case 3: return launch_one<H, 3>(p, stream);
      case 4: return launch_one<H, 4>(p, stream);
    }
  } else {
    switch (jw) {
      case 1: return launch_one<H, 1>(p, stream);
      case 2: return launch_one<H, 2>(p, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace

int logits_wave_tokens() { return kWaveTokens; }

int logits_rows_per_wave(int heads, int next_n) {
  // at most 256 q rows (128 VGPRs of A operands) per wave
  const int cap = heads >= 128 ? 1 : (heads >= 64 ? 3 : 4);
  return next_n < cap ? next_n : cap;
}

hipError_t launch_logits(const LogitsParams& p, int heads, int jw, hipStream_t stream) {
  switch (heads) {
    case 16: return launch_heads<16>(p, jw, stream);
    case 32: return launch_heads<32>(p, jw, stream);
    case 64: return launch_heads<64>(p, jw, stream);
    case 128: return launch_heads<128>(p, jw, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pmqa
