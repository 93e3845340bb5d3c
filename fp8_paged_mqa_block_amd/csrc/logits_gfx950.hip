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
//  * decode shapes (every next_n row of a request within one wave of 64 q
//    rows, and a grid bound of at most two residencies) take the flat
//    geometry of logits_flat_kernel: one single-wave workgroup per 64-token
//    iteration, the whole grid resident at once.  Other shapes take the
//    persistent logits_kernel below;
//  * the work is each request's list of 64-token iterations.  Every wave
//    reads the context lengths and computes the split itself (the host never
//    reads them): a request is cut into runs of at most P iterations, P the
//    smallest length for which every run gets a wave unit, and a wave takes
//    one run.  A run never leaves its request, so the wave loads its q rows
//    once, and a long context is spread over many waves;
//  * a wave also owns a group of up to JW of the next_n rows.  Their q (JW*H x
//    128 e4m3fn) stays in VGPRs as MFMA A operands, heads on the M dimension,
//    so each lane ends up holding 4 heads of one token and the head reduction
//    is in-lane FMAs plus two cross-lane adds;
//  * K is staged through LDS by the memory pipeline itself
//    (global_load_lds_dwordx4): an iteration's 64 token records are copied
//    whole, 16 bytes per lane per instruction, each record as its 8 value
//    chunks plus the 16 bytes that end with its scale (144 bytes in LDS), so
//    every instruction reads consecutive cache lines, no VGPR holds data in
//    flight and the MFMA B operands come back as aligned 16-byte LDS reads;
//  * pages hold whole records, a power of two from 1 to 256 of them.  Pages
//    smaller than the 16-token matrix tile are assembled into one tile (aiter
//    PR #6626 section 1 builds a tile from several 8-token pages): every
//    16-byte chunk takes its own record's page id, so token-level tables
//    (1-token pages: the dense row-id tables of ATOM PR #2533) take the same
//    path.  Pages of 64 tokens or more hold a whole iteration, whose gather is
//    then a wave-uniform page base plus fixed per-lane offsets.  Page ids are
//    read ahead of the gather;
//  * page byte offsets are int64 (id * page_size * 132) and the output row
//    base is int64 (row * out_row_stride) with int32 columns, so pools and
//    outputs beyond 2^31 bytes are addressed correctly (aiter PR #4244 "Fix";
//    ATOM PR #2533 "Address Triton decode KV rows with int64 ids");
//  * workgroups are dealt round-robin over the 8 XCDs; the grid is re-indexed
//    so that each XCD gets a contiguous run of workgroups, and the wave units
//    are dealt wave-major over those workgroups so that every CU gets a share
//    when the runs are fewer than the waves.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pmqa_internal.h"
#include "wave_ops.h"

namespace pmqa {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 16;                 // tokens per MFMA tile (N)
constexpr int kTilesPerIter = 4;          // 64 tokens: one per lane at store time
constexpr int kIterTokens = kTile * kTilesPerIter;
// In LDS a token record takes 9 chunks of 16 bytes (144 bytes): its 8 value
// chunks, then the 16 bytes that end with its scale (record bytes 116..131),
// so the scale sits at byte 140 of the padded record.
constexpr int kChunksPerRecord = 9;
constexpr int kLdsRecord = 16 * kChunksPerRecord;
constexpr int kDmaBytes = 64 * 16;                        // one 64-lane 16-byte load
constexpr int kSlotBytes = kIterTokens * kLdsRecord;      // one iteration (9216 bytes)
constexpr int kGatherLoads = kSlotBytes / kDmaBytes;      // loads per gather (9)
constexpr int kMaxPages = kIterTokens;                    // page ids per iteration (1-token pages)

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// Cache policy of the K gather: non-temporal (the NT bit of gfx950's load
// cache-policy field).  Every K record is read once per launch, so marking its
// lines as streaming keeps them from displacing what is reused from L2 (block
// table, q, weights).  Measured on the decode workload (interleaved with the
// default policy in one process): 10.56 -> 9.80 us mean per launch; the same
// on a pool whose pages are contiguous (10.42 -> 9.84 us), which also shows
// the page scatter itself costs nothing measurable.  The per-row ring kernel
// gains more (8-token pages: 149 -> 135 us), but the shared-ring kernel at
// 128 heads loses 2-3% with it (MTP 314 -> 322 us, long context 113 -> 116 us)
// and keeps the default policy.
constexpr int kStreamK = 2;

// A lane's 32 bytes of one 128-byte q row or K record as an MFMA operand:
// the 16 bytes at p and the 16 at p + 64 (p = row + 16*kq).  The matrix
// core's K order only has to agree between q and K; this one reads each row
// as two 64-byte halves (the four lanes of a row read one contiguous half per
// load) and keeps K's LDS reads at the same bank spread.
__device__ __forceinline__ v8i load_q32(const uint8_t* p) {
  const u32x4 a = *reinterpret_cast<const u32x4*>(p);
  const u32x4 b = *reinterpret_cast<const u32x4*>(p + 64);
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
// identically, so every K index meets its partner exactly once.  Both slices
// are converted at their use: the empty asm keeps the compiler from hoisting
// the converted tiles out of the head and token loops, which would take more
// registers than q and K occupy in e4m3 (this path serves short rows only, so
// the repeated conversions cost little).
__device__ __forceinline__ v4f mfma_exact(v8i a, v8i b) {
  v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    int lo = a[2 * c], hi = a[2 * c + 1];
    int blo = b[2 * c], bhi = b[2 * c + 1];
    asm volatile("" : "+v"(lo), "+v"(hi), "+v"(blo), "+v"(bhi));
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(fp8x8_to_f16(lo, hi), fp8x8_to_f16(blo, bhi),
                                                 acc, 0, 0, 0);
  }
  return acc;
}

// Rows that see fewer tokens than this are scored on the exact-sum path.  The
// fp8 matrix core sums each run of 8 consecutive products after aligning them
// to the largest, keeping about 14 bits below it; on a row of a few tokens
// whose head-weighted sum cancels, that rounding can reach a few 1e-4 of the
// row's largest score, while rows of 32 tokens or more stay near 4e-5.
constexpr int kExactRows = 128;

// Number of 64-token iterations of a context (clamped to the grid's bound).
__device__ __forceinline__ int n_iters(int ctx, int max_tokens) {
  const int c = min(max(ctx, 0), max_tokens);
  return (c + kIterTokens - 1) / kIterTokens;
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ uint32_t ceil_div(uint32_t a, uint32_t b) { return (a + b - 1u) / b; }

// One wave's share of the work: iterations [it0, it0 + n_it) of request b
// (all wave-uniform).  A run never crosses into another request, so the wave
// loads its q rows once.
struct Run {
  int b, ctx, ctx_eff, it0, n_it;
};

// What a wave needs first: the context lengths, the batch and the grid's
// token bound.  The kernels take them as their leading scalar arguments, which
// the dispatch preloads into SGPRs (the build asks for up to 16 dwords), so
// the context-length loads issue without waiting for the argument block.
struct CtxArgs {
  const int32_t* ctx;
  int32_t batch;
  int32_t max_tokens;
};

// Iterations of request c0 + lane (0 past the batch), and its context length.
__device__ __forceinline__ int lane_iters(const CtxArgs& a, int c0, int lane, int& ctx) {
  const int b = c0 + lane;
  ctx = b < a.batch ? max(a.ctx[b], 0) : 0;
  return n_iters(ctx, a.max_tokens);
}

// Runs needed when no run is longer than P iterations: sum over the batch of
// ceil(n_b / P).
__device__ uint64_t runs_for(const CtxArgs& a, int lane, uint32_t n_first, uint32_t P) {
  uint64_t runs = wave_sum(ceil_div(n_first, P));
  for (int c0 = 64; c0 < a.batch; c0 += 64) {
    int ctx;
    runs += wave_sum(ceil_div((uint32_t)lane_iters(a, c0, lane, ctx), P));
  }
  return runs;
}

// The work split.  Every request b is cut into ceil(n_b / P) runs of nearly
// equal length (n_b iterations), with P the smallest length for which all the
// runs fit in the n_slices units the grid provides (one run per request
// always fits: the host makes n_slices >= batch).  Unit u takes the u-th run
// in request order; units past the last run have nothing to do.  Each wave
// computes the split itself from the context lengths, so the host never reads
// them.
__device__ bool find_run(const CtxArgs& a, const LogitsParams& p, int unit, int lane, Run& run) {
  int ctx0;
  const uint32_t n0 = (uint32_t)lane_iters(a, 0, lane, ctx0);
  uint64_t total = wave_sum(n0);
  uint32_t nmax = wave_max(n0);
  for (int c0 = 64; c0 < a.batch; c0 += 64) {
    int ctx;
    const uint32_t n = (uint32_t)lane_iters(a, c0, lane, ctx);
    total += wave_sum(n);
    nmax = max(nmax, wave_max(n));
  }
  if (total == 0) return false;
  const uint32_t slices = (uint32_t)p.n_slices;
  uint32_t P = (uint32_t)((total + slices - 1) / slices);
  if (runs_for(a, lane, n0, P) > slices) {
    // runs_for(lo) > slices >= runs_for(hi): bisect for the smallest fit
    uint32_t lo = P, hi = nmax;
    while (hi - lo > 1u) {
      const uint32_t mid = lo + (hi - lo) / 2u;
      if (runs_for(a, lane, n0, mid) <= slices) hi = mid;
      else lo = mid;
    }
    P = hi;
  }
  // locate unit: the request whose runs cover it
  uint32_t before = 0;
  for (int c0 = 0; c0 < a.batch; c0 += 64) {
    int ctx = ctx0;
    const uint32_t n = c0 == 0 ? n0 : (uint32_t)lane_iters(a, c0, lane, ctx);
    const uint32_t c = ceil_div(n, P);
    uint32_t chunk_runs;
    const uint32_t incl = wave_prefix(c, lane, chunk_runs);
    if (before + chunk_runs > (uint32_t)unit) {
      const uint64_t past = __ballot(before + incl > (uint32_t)unit);
      const int f = uniform(__builtin_ctzll(past));
      const uint32_t c_f = lane_of(c, f), n_f = lane_of(n, f);
      const uint32_t i = (uint32_t)unit - (before + lane_of(incl, f) - c_f);
      run.b = c0 + f;
      run.ctx = (int)lane_of((uint32_t)ctx, f);
      run.ctx_eff = min(run.ctx, a.max_tokens);
      run.it0 = (int)((uint64_t)n_f * i / c_f);
      run.n_it = (int)((uint64_t)n_f * (i + 1u) / c_f) - run.it0;
      return true;
    }
    before += chunk_runs;
  }
  return false;
}

template <int H, int JW>
struct QRegs {
  v8i qa[JW][H / 16];
  v4f wv[JW][H / 16];
};

// Load the q rows and weights of request b.  The caller ends the loads with
// an explicit full wait the compiler knows about, so no later code needs a
// compiler-inserted one (which, with LDS-bound loads in flight, would be a
// full drain inside the pipeline).
template <int H, int JW>
__device__ __forceinline__ void load_q(const LogitsParams& p, int b, int j0, int m, int kq,
                                       QRegs<H, JW>& qr) {
  constexpr int HT = H / 16;
#pragma unroll
  for (int jj = 0; jj < JW; ++jj) {
    const int j = min(j0 + jj, p.next_n - 1);  // rows past next_n are never stored
    const int64_t row = (int64_t)b * p.next_n + j;
    const uint8_t* qrow = p.q + row * (int64_t)(H * kHeadDim);
    const float* wrow = p.w + row * H;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      qr.qa[jj][ht] = load_q32(qrow + (ht * 16 + m) * kHeadDim + kq * 16);
      qr.wv[jj][ht] = *reinterpret_cast<const v4f*>(wrow + ht * 16 + kq * 4);
    }
  }
}

// q rows of request b loaded as whole lines: load i of a row moves its bytes
// [1024 i, 1024 i + 1024) (heads 8i .. 8i+7), lane l taking the 16 bytes at
// 16 l, so that every load reads 8 full 128-byte lines (load_q's operand-
// shaped loads read 16 half lines each, and the memory pipeline counts
// lines); assemble_q then builds the operands with cross-lane reads.  The
// weights are loaded as load_q does.
template <int H, int JW>
struct QLines {
  u32x4 v[JW][H / 8];
};

template <int H, int JW>
__device__ __forceinline__ void load_q_lines(const LogitsParams& p, int b, int lane, int kq,
                                             QLines<H, JW>& ql, QRegs<H, JW>& qr) {
#pragma unroll
  for (int jj = 0; jj < JW; ++jj) {
    const int j = min(jj, p.next_n - 1);  // rows past next_n are never stored
    const int64_t row = (int64_t)b * p.next_n + j;
    const u32x4* src = reinterpret_cast<const u32x4*>(p.q + row * (int64_t)(H * kHeadDim)) + lane;
    const float* wrow = p.w + row * H;
#pragma unroll
    for (int i = 0; i < H / 8; ++i) ql.v[jj][i] = src[64 * i];
#pragma unroll
    for (int ht = 0; ht < H / 16; ++ht)
      qr.wv[jj][ht] = *reinterpret_cast<const v4f*>(wrow + ht * 16 + kq * 4);
  }
}

// The MFMA operands from whole-line q loads by cross-lane reads, for a wave
// whose gather is still in flight (the slot is busy): lane (m, kq) of head
// tile ht needs bytes [16kq, 16kq+16) and [64+16kq, 64+16kq+16) of head
// 16 ht + m, which load 2 ht + m/8 holds in lanes 8 (m%8) + kq and
// 8 (m%8) + kq + 4.  A cross-lane read takes one register of every source
// lane, so each dword is read from both loads of the tile and the lane keeps
// the one of its head.  Only the q loads are waited for (the compiler counts
// the gather's loads issued after them), so this overlaps the gather.
template <int H, int JW>
__device__ __forceinline__ void assemble_q_xlane(const QLines<H, JW>& ql, int lane,
                                                 QRegs<H, JW>& qr) {
  const int m = lane & 15, kq = lane >> 4;
  const int a0 = (8 * (m & 7) + kq) * 4;  // byte index of the source lane
  const int a1 = a0 + 16;
  const bool low = m < 8;
#pragma unroll
  for (int jj = 0; jj < JW; ++jj) {
#pragma unroll
    for (int ht = 0; ht < H / 16; ++ht) {
      const u32x4 A = ql.v[jj][2 * ht], B = ql.v[jj][2 * ht + 1];
      u32x4 x0, y0, x1, y1;
      // Inline assembly with its own LDS-counter wait on purpose: the compiler
      // drains every in-flight LDS-bound load before any LDS instruction it
      // emits (it cannot tell that a cross-lane read touches no LDS memory),
      // which would wait for the gather
      asm volatile(
          "ds_bpermute_b32 %0, %16, %18\n\t"
          "ds_bpermute_b32 %1, %16, %19\n\t"
          "ds_bpermute_b32 %2, %16, %20\n\t"
          "ds_bpermute_b32 %3, %16, %21\n\t"
          "ds_bpermute_b32 %4, %16, %22\n\t"
          "ds_bpermute_b32 %5, %16, %23\n\t"
          "ds_bpermute_b32 %6, %16, %24\n\t"
          "ds_bpermute_b32 %7, %16, %25\n\t"
          "ds_bpermute_b32 %8, %17, %18\n\t"
          "ds_bpermute_b32 %9, %17, %19\n\t"
          "ds_bpermute_b32 %10, %17, %20\n\t"
          "ds_bpermute_b32 %11, %17, %21\n\t"
          "ds_bpermute_b32 %12, %17, %22\n\t"
          "ds_bpermute_b32 %13, %17, %23\n\t"
          "ds_bpermute_b32 %14, %17, %24\n\t"
          "ds_bpermute_b32 %15, %17, %25\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(x0[0]), "=&v"(x0[1]), "=&v"(x0[2]), "=&v"(x0[3]), "=&v"(y0[0]), "=&v"(y0[1]),
            "=&v"(y0[2]), "=&v"(y0[3]), "=&v"(x1[0]), "=&v"(x1[1]), "=&v"(x1[2]), "=&v"(x1[3]),
            "=&v"(y1[0]), "=&v"(y1[1]), "=&v"(y1[2]), "=&v"(y1[3])
          : "v"(a0), "v"(a1), "v"(A[0]), "v"(A[1]), "v"(A[2]), "v"(A[3]), "v"(B[0]), "v"(B[1]),
            "v"(B[2]), "v"(B[3]));
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        qr.qa[jj][ht][c] = (int)(low ? x0[c] : y0[c]);
        qr.qa[jj][ht][4 + c] = (int)(low ? x1[c] : y1[c]);
      }
    }
  }
}

// The MFMA operands from whole-line q loads, through the wave's K slot once
// the iteration's K operands have been read from it: the lines are written as
// padded rows (head h of row jj at (jj*H + h) * 144 bytes; the flat geometry
// holds at most 64 heads x rows, 9216 bytes), and lane (m, kq) of head tile
// ht reads bytes [16kq, 16kq+16) and [64+16kq, 64+16kq+16) of head 16 ht + m
// back, the 16 lanes of one kq on distinct banks as for the K operands.
template <int H, int JW>
__device__ __forceinline__ void assemble_q(const QLines<H, JW>& ql, int lane, uint8_t* slot,
                                           QRegs<H, JW>& qr) {
  static_assert(H * JW * kLdsRecord <= kSlotBytes, "q rows must fit the K slot");
  const int m = lane & 15, kq = lane >> 4;
#pragma unroll
  for (int jj = 0; jj < JW; ++jj) {
#pragma unroll
    for (int i = 0; i < H / 8; ++i) {
      const int h = 8 * i + (lane >> 3);
      *reinterpret_cast<u32x4*>(slot + (jj * H + h) * kLdsRecord + 16 * (lane & 7)) = ql.v[jj][i];
    }
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the rows are written
#pragma unroll
  for (int jj = 0; jj < JW; ++jj) {
#pragma unroll
    for (int ht = 0; ht < H / 16; ++ht) {
      const uint8_t* r = slot + (jj * H + 16 * ht + m) * kLdsRecord + 16 * kq;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(r);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(r + 64);
      qr.qa[jj][ht][0] = lo[0]; qr.qa[jj][ht][1] = lo[1];
      qr.qa[jj][ht][2] = lo[2]; qr.qa[jj][ht][3] = lo[3];
      qr.qa[jj][ht][4] = hi[0]; qr.qa[jj][ht][5] = hi[1];
      qr.qa[jj][ht][6] = hi[2]; qr.qa[jj][ht][7] = hi[3];
    }
  }
}

// Page ids of an iteration, gathered into LDS by one 4-byte-per-lane load:
// lane i moves the low 32 bits of the iteration's i-th page id (at most 64
// pages per iteration, with 1-token pages).  Only ids inside the context are
// read.
__device__ __forceinline__ void issue_ids(const LogitsParams& p, const Run& c, int it, int lane,
                                          uint32_t* ids_slot) {
  const int t0 = it * kIterTokens;
  const int lp = p.log2_page;
  const int p_first = t0 >> lp;
  const int n_pg = ((min(t0 + kIterTokens, c.ctx_eff) - 1) >> lp) - p_first + 1;
  const uint32_t* row =
      reinterpret_cast<const uint32_t*>(p.tables + (int64_t)c.b * p.table_stride + p_first);
  if (lane < n_pg) __builtin_amdgcn_global_load_lds(row + 2 * lane, LDS_PTR(ids_slot), 4, 0, 0);
}

// Page ids of a gather's 16-byte chunks, read from the iteration's LDS id
// slot.  Load i of the gather fills LDS chunks 64*i .. 64*i+63 of the slot
// (lane l: chunk 64*i + l), and chunk q belongs to record q / 9 of the
// iteration.  An iteration starts at a multiple of 64 tokens and pages hold
// 1..256 tokens (powers of two), so record x lies in page (x >> log2_page) of
// the iteration.  Only the low 32 bits of an id are staged: a pool that fits
// in device memory holds fewer than 2^32 pages even of one token (the byte
// offset id * page_bytes is still formed in 64 bits).  Inline assembly with its own LDS wait on purpose: the compiler
// cannot tell which in-flight LDS-bound loads a plain LDS read could alias and
// would drain every one of them first, while the ring's ordering already
// proves these ids have landed.
struct ChunkPages {
  uint32_t id[kGatherLoads];
};

__device__ __forceinline__ ChunkPages read_pages(const uint32_t* ids_slot, int lp,
                                                 const uint32_t (&rec)[kGatherLoads]) {
  static_assert(kGatherLoads == 9, "one ds_read_b32 per gather load below");
  const uint32_t a = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const uint32_t*)ids_slot);
  uint32_t g[kGatherLoads];
#pragma unroll
  for (int i = 0; i < kGatherLoads; ++i) g[i] = a + 4u * (rec[i] >> lp);
  ChunkPages r;
  asm volatile(
      "ds_read_b32 %0, %9\n\t"
      "ds_read_b32 %1, %10\n\t"
      "ds_read_b32 %2, %11\n\t"
      "ds_read_b32 %3, %12\n\t"
      "ds_read_b32 %4, %13\n\t"
      "ds_read_b32 %5, %14\n\t"
      "ds_read_b32 %6, %15\n\t"
      "ds_read_b32 %7, %16\n\t"
      "ds_read_b32 %8, %17\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r.id[0]), "=&v"(r.id[1]), "=&v"(r.id[2]), "=&v"(r.id[3]), "=&v"(r.id[4]),
        "=&v"(r.id[5]), "=&v"(r.id[6]), "=&v"(r.id[7]), "=&v"(r.id[8])
      : "v"(g[0]), "v"(g[1]), "v"(g[2]), "v"(g[3]), "v"(g[4]), "v"(g[5]), "v"(g[6]), "v"(g[7]),
        "v"(g[8])
      : "memory");
  return r;
}

// Byte offset, inside the iteration's run of 64 records, of the chunk lane
// `lane` moves in load i: chunk q = 64*i + lane is chunk q % 9 of record q / 9
// (value chunks at 16*c, the scale chunk at 116).  Depends only on the lane.
struct ChunkOffsets {
  uint32_t off[kGatherLoads];  // byte offset of the chunk in the iteration's records
};

// Preshuffled pages (kLayoutPreshuffled) instead hold an iteration as one
// contiguous image of 64 * 132 = 8448 bytes (64 tokens = 4 tiles of 16, each
// tile's values then its scales), so load i of lane l takes image bytes
// [1024 i + 16 l, +16); the last load's lanes past the image's 256-byte tail
// re-read that tail (inside the page) and land in unused slot bytes.
constexpr int kPreImageBytes = kIterTokens * kRecordBytes;  // 8448
constexpr int kPreTileBytes = kTile * kRecordBytes;         // 2112

__device__ __forceinline__ ChunkOffsets chunk_offsets(int lane, bool pre = false) {
  ChunkOffsets r;
  if (pre) {
#pragma unroll
    for (int i = 0; i < kGatherLoads; ++i) {
      const int b = kDmaBytes * i + 16 * lane;
      r.off[i] = (uint32_t)(b < kPreImageBytes ? b : (kGatherLoads - 1) * kDmaBytes + 16 * (lane & 15));
    }
    return r;
  }
#pragma unroll
  for (int i = 0; i < kGatherLoads; ++i) {
    const int q = 64 * i + lane;
    const int x = q / kChunksPerRecord;
    const int c = q - x * kChunksPerRecord;
    r.off[i] = (uint32_t)(x * kRecordBytes + (c < 8 ? 16 * c : kRecordBytes - 16));
  }
  return r;
}

// Issue the gather of one iteration into an LDS slot: its 64 token records,
// each as 9 chunks of 16 bytes (8 of values, then the 16 bytes ending with the
// scale), 9 loads of 16 bytes per lane in all.  A load moves the chunks of
// about 7 consecutive records, so it reads consecutive cache lines, and the
// scales come with their records instead of in a separate pass.  Every chunk
// lies inside its own record.  Exactly kGatherLoads vector memory instructions
// are issued on every call.
//  * Pages of 64 tokens or more: the iteration lies in one page, whose base is
//    wave-uniform; each load adds the lane's fixed chunk offset.  Records past
//    the context are read from the same page (it is a whole page of the pool)
//    and never used; a placeholder gather (`limit` 0, only keeping the
//    instruction count fixed) reads the pool's first 64 records.
//  * Smaller pages: each chunk takes its record's page id; chunks of records
//    at or past `limit` fetch a chunk of the pool's first record instead (one
//    cache line, inside any pool that holds a record) and never use their
//    page id.
template <int LAYOUT, int CPOL>
__device__ __forceinline__ void issue_gather(const LogitsParams& p, int it, int limit,
                                             const uint32_t* ids_slot, int lane,
                                             const ChunkOffsets& co, uint8_t* slot) {
  const int t0 = it * kIterTokens;
  const int in_page_mask = p.page_size - 1;
  if (p.log2_page >= 6) {
    const uint32_t a =
        (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const uint32_t*)ids_slot);
    uint32_t id;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(id) : "v"(a) : "memory");
    id = (uint32_t)uniform((int)id);
    const int64_t base =
        t0 < limit ? (int64_t)id * p.page_bytes + (int32_t)((t0 & in_page_mask) * kRecordBytes) : 0;
    const uint8_t* src = p.kv + base;
#pragma unroll
    for (int i = 0; i < kGatherLoads; ++i)
      __builtin_amdgcn_global_load_lds(src + co.off[i], LDS_PTR(slot + i * kDmaBytes), 16, 0, CPOL);
    return;
  }
  // Pages here hold at most 32 tokens and the iteration starts at a multiple
  // of 64, so record x of the iteration is token (x & (page_size-1)) of page
  // (x >> log2_page); the chunk's record, its place in the record and its
  // page are all derived here from one division of the chunk index (an opaque
  // copy of the lane keeps them out of the page-sized path's registers), and
  // its address is one 32x32+64-bit multiply-add
  int l = lane;
  asm volatile("" : "+v"(l));
  uint32_t rec[kGatherLoads], in_page[kGatherLoads];
  bool in_image[kGatherLoads];  // the chunk belongs to the iteration's bytes
  if constexpr (LAYOUT == kLayoutPreshuffled) {
    // preshuffled pages of 8, 16 or 32 tokens: the image is the iteration's
    // 64 / page_size pages back to back, each page_size * 132 bytes, i.e.
    // 33 * page_size / 4 chunks of 16 bytes; chunk c lies in page
    // j = c / that (a multiply by the host's ceil(2^20 / chunks per page),
    // exact for every c below 576) at byte 16 (c - j * that) of the page.
    // rec holds the page's first token (j << log2_page), as read_pages and the
    // context check below expect; chunks past the image read the pool's
    // first chunks and land in unused slot bytes.
    const uint32_t cpp = (33u * (uint32_t)p.page_size) >> 2;
#pragma unroll
    for (int i = 0; i < kGatherLoads; ++i) {
      const uint32_t c = 64u * i + (uint32_t)l;
      const uint32_t j = (c * p.pre_magic) >> 20;
      in_image[i] = c < (uint32_t)(kPreImageBytes / 16);
      rec[i] = in_image[i] ? j << p.log2_page : 0u;
      in_page[i] = (c - j * cpp) * 16u;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kGatherLoads; ++i) {
      const int q = 64 * i + l;
      const int x = q / kChunksPerRecord;
      const int c = q - x * kChunksPerRecord;
      rec[i] = (uint32_t)x;
      in_page[i] = (uint32_t)((x & in_page_mask) * kRecordBytes + (c < 8 ? 16 * c : kRecordBytes - 16));
      in_image[i] = true;
    }
  }
  const ChunkPages pg = read_pages(ids_slot, p.log2_page, rec);
  const uint32_t pb = (uint32_t)p.page_bytes;  // <= 32 records
#pragma unroll
  for (int i = 0; i < kGatherLoads; ++i) {
    const int64_t off = in_image[i] && t0 + (int)rec[i] < limit
                            ? (int64_t)((uint64_t)pg.id[i] * pb + in_page[i])
                            : (int64_t)(16 * (lane & 7));
    __builtin_amdgcn_global_load_lds(p.kv + off, LDS_PTR(slot + i * kDmaBytes), 16, 0, CPOL);
  }
}

// The gather of one iteration that lies in one page (pages of 64 tokens or
// more), from that page's id: the same loads as issue_gather's page-sized
// path.
template <int CPOL>
__device__ __forceinline__ void gather_page(const LogitsParams& p, int it, int64_t id, int lane,
                                            const ChunkOffsets& co, uint8_t* slot) {
  const int t0 = it * kIterTokens;
  const uint8_t* src =
      p.kv + id * p.page_bytes + (int32_t)((t0 & (p.page_size - 1)) * kRecordBytes);
#pragma unroll
  for (int i = 0; i < kGatherLoads; ++i)
    __builtin_amdgcn_global_load_lds(src + co.off[i], LDS_PTR(slot + i * kDmaBytes), 16, 0, CPOL);
}

// The page id of an iteration that lies in one page, by a scalar load (the
// request and iteration are wave-uniform): it is tracked by the scalar memory
// counter, so vector loads issued after it are not waited for when it is.
__device__ __forceinline__ int64_t page_id(const LogitsParams& p, const Run& c) {
  const int64_t idx =
      (int64_t)uniform(c.b) * p.table_stride + ((uniform(c.it0) * kIterTokens) >> p.log2_page);
  const __attribute__((address_space(4))) int64_t* t =
      (const __attribute__((address_space(4))) int64_t*)p.tables;
  return t[idx];
}

// Wait until at most n vector memory instructions are outstanding (n one of
// the values the ring produces, a multiple of kGatherLoads below 4 of them;
// anything smaller waits for all).
__device__ __forceinline__ void wait_vm(int n) {
  if (n >= 3 * kGatherLoads) asm volatile("s_waitcnt vmcnt(27)" ::: "memory");
  else if (n >= 2 * kGatherLoads) asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
  else if (n >= kGatherLoads) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Reduce-scatter of four per-tile partial sums over the four 16-lane rows of
// the wave: lane l of row r returns the sum, over the rows, of tile r's value
// at lanes l % 16 + 16 * r' (r' = 0..3), added as (rows 0 + 2) + (rows 1 + 3).
// The half swap pairs tiles 0/2 and 1/3 (lanes 0-31 keep the first tile's
// pair sums, lanes 32-63 the second's); the row swap then pairs the two.
// Three swaps and three adds for the four tiles.
__device__ __forceinline__ float reduce_tiles(float p0, float p1, float p2, float p3) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p2), false,
                                                  false);
  const float s02 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(p1), __float_as_uint(p3), false,
                                                  false);
  const float s13 = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(s02), __float_as_uint(s13), false,
                                                  false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// max(x, 0) on the bit pattern: positive floats are positive as int32, and
// negative ones, -0 and -inf are negative, so the integer max gives x or +0
// for every non-NaN x (a NaN with the sign bit clear passes through, as the
// definition's max(0, NaN) does).  One v_max_i32: the float max of a matrix-core
// result costs two, since the compiler first canonicalizes an operand it
// cannot prove canonical (v_max_f32 x, x).
__device__ __forceinline__ float relu_bits(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// max(y, 0) that passes NaN through, whatever its sign bit: a NaN scale makes
// the token's score NaN, as max with NaN propagation gives (the reading adopted
// for a NaN scale), where the hardware max would return 0.  -0 stays -0, which
// compares equal to 0.
__device__ __forceinline__ float relu_nan(float y) { return y < 0.f ? 0.f : y; }

// Score one iteration (64 tokens x the wave's rows) from its slot operands and
// store it.  FACTORED: every scale of the iteration is >= 0, so
// relu(s * x) = s * relu(x) and the scale multiplies the head-weighted sum once
// per token instead of once per head (2 VALU operations per MFMA output
// instead of 3); otherwise the literal form runs (relu of scale * dot per head,
// a NaN scale giving a NaN score).
template <int H, int JW, bool EXACT, bool FACTORED>
__device__ __forceinline__ void score_iteration(const LogitsParams& p, const Run& c, int it, int j0,
                                                int lane, const QRegs<H, JW>& qr,
                                                const v8i (&kb)[kTilesPerIter],
                                                const float (&sc)[kTilesPerIter]) {
  constexpr int HT = H / 16;
  const int kq = lane >> 4;
  const int t0 = it * kIterTokens;
  static_assert(kTilesPerIter == 4, "reduce_tiles takes four tiles");
  float part[JW][kTilesPerIter];
#pragma unroll
  for (int tile = 0; tile < kTilesPerIter; ++tile) {
    const float s = sc[tile];
#pragma unroll
    for (int jj = 0; jj < JW; ++jj) {
      v4f acc[HT];
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        if constexpr (EXACT) acc[ht] = mfma_exact(qr.qa[jj][ht], kb[tile]);
        else acc[ht] = mfma_fp8(qr.qa[jj][ht], kb[tile]);
      }
      float sum = 0.f;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (FACTORED)
            sum = __builtin_fmaf(qr.wv[jj][ht][i], relu_bits(acc[ht][i]), sum);
          else
            sum = __builtin_fmaf(qr.wv[jj][ht][i], relu_nan(acc[ht][i] * s), sum);
        }
      }
      part[jj][tile] = sum;
    }
  }
  if constexpr (FACTORED && !EXACT) {
    // Each matrix product is read by 8 vector instructions (4 relu, 4 fma).
    // Left to itself the scheduler reuses one result register set, so each
    // product's reads wait out its latency (an 11-cycle nop per product) and
    // the wave's matrix and vector work alternate.  This order keeps two
    // products in flight across the iteration's tiles: product g + 2 issues
    // before the reads of product g, which then find it done (measured,
    // interleaved on one box: MTP 307 -> 293 us, long context 113 -> 110 us;
    // per tile instead of per iteration 300 and 111 us; a third product in
    // flight no better).
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // 2 matrix products
#pragma unroll
    for (int g = 0; g < kTilesPerIter * HT * JW - 2; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);  // 8 vector instructions
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // the next product
    }
    __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
  }
  // this lane's row kq ends with tile kq's tokens: its scale multiplies the
  // head-weighted sum in the factored form
  // (the scales pass through an empty asm statement as plain values: a
  // select among elements of sc would become an indexed load, which puts the
  // operands in scratch memory)
  float s0 = sc[0], s1 = sc[1], s2 = sc[2], s3 = sc[3];
  asm volatile("" : "+v"(s0), "+v"(s1), "+v"(s2), "+v"(s3));
  float s_own = s0;
  s_own = kq == 1 ? s1 : s_own;
  s_own = kq == 2 ? s2 : s_own;
  s_own = kq == 3 ? s3 : s_own;
  float keep[JW];
#pragma unroll
  for (int jj = 0; jj < JW; ++jj) {
    keep[jj] = reduce_tiles(part[jj][0], part[jj][1], part[jj][2], part[jj][3]);
    if constexpr (FACTORED) keep[jj] *= s_own;
  }
  const float neg_inf = -__builtin_inff();
  const int t = t0 + lane;
#pragma unroll
  for (int jj = 0; jj < JW; ++jj) {
    const int j = j0 + jj;
    if (j >= p.next_n) break;
    const int vis = min(max(c.ctx - p.next_n + j + 1, 0), c.ctx_eff);
    float* orow = p.out + ((int64_t)c.b * p.next_n + j) * p.out_stride;
    if (t < vis)
      orow[t] = keep[jj];
    else if (t < c.ctx_eff)
      orow[t] = neg_inf;
  }
}

// The iteration's operands from its LDS slot (record x at x * 144, scale at
// byte 140 of it): per tile, this lane's 32-byte B operand (token m of the
// tile, value bytes 16*kq .. 16*kq+15 and 64+16*kq .. 64+16*kq+15, the order
// load_q32 gives q) and that token's scale.  The 144-byte
// stride keeps the 16 lanes of one kq on distinct banks.  Inline assembly with
// its own LDS wait on purpose: the compiler cannot tell which in-flight
// LDS-bound loads a plain LDS read could alias and would drain every one of
// them first (the whole ring), while the explicit vector-memory wait before
// this read already proves this slot has landed.
struct SlotOperands {
  v8i kb[kTilesPerIter];
  float sc[kTilesPerIter];
};

__device__ __forceinline__ SlotOperands read_slot(const uint8_t* slot, int lane) {
  static_assert(kTilesPerIter == 4 && kTile * kLdsRecord == 2304,
                "offsets below assume 4 tiles of 16 padded records");
  const int m = lane & 15, kq = lane >> 4;
  const uint32_t base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const uint8_t*)slot);
  // tile t's addresses are tile 0's plus t * 2304
  const uint32_t av = base + (uint32_t)(m * kLdsRecord + 16 * kq);
  const uint32_t as = base + (uint32_t)(m * kLdsRecord + kLdsRecord - 4);
  u32x4 lo0, hi0, lo1, hi1, lo2, hi2, lo3, hi3;
  SlotOperands r;
  asm volatile(
      "ds_read_b128 %0, %12\n\t"
      "ds_read_b128 %1, %12 offset:64\n\t"
      "ds_read_b128 %2, %12 offset:2304\n\t"
      "ds_read_b128 %3, %12 offset:2368\n\t"
      "ds_read_b128 %4, %12 offset:4608\n\t"
      "ds_read_b128 %5, %12 offset:4672\n\t"
      "ds_read_b128 %6, %12 offset:6912\n\t"
      "ds_read_b128 %7, %12 offset:6976\n\t"
      "ds_read_b32 %8, %13\n\t"
      "ds_read_b32 %9, %13 offset:2304\n\t"
      "ds_read_b32 %10, %13 offset:4608\n\t"
      "ds_read_b32 %11, %13 offset:6912\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(lo0), "=&v"(hi0), "=&v"(lo1), "=&v"(hi1), "=&v"(lo2), "=&v"(hi2), "=&v"(lo3),
        "=&v"(hi3), "=&v"(r.sc[0]), "=&v"(r.sc[1]), "=&v"(r.sc[2]), "=&v"(r.sc[3])
      : "v"(av), "v"(as)
      : "memory");
  const u32x4 lo[kTilesPerIter] = {lo0, lo1, lo2, lo3};
  const u32x4 hi[kTilesPerIter] = {hi0, hi1, hi2, hi3};
#pragma unroll
  for (int tile = 0; tile < kTilesPerIter; ++tile) {
    r.kb[tile][0] = lo[tile][0]; r.kb[tile][1] = lo[tile][1];
    r.kb[tile][2] = lo[tile][2]; r.kb[tile][3] = lo[tile][3];
    r.kb[tile][4] = hi[tile][0]; r.kb[tile][5] = hi[tile][1];
    r.kb[tile][6] = hi[tile][2]; r.kb[tile][7] = hi[tile][3];
  }
  return r;
}

// The iteration's operands from a slot holding a preshuffled image (64
// tokens as 4 tiles of 2112 bytes: pages of 16 tokens or more hold whole
// tiles; an 8-token page is half a tile, the tile's two pages 1056 bytes
// apart).  Lane (m, kq)'s operand is the tile's group (0, kq) and (1, kq)
// piece of token m: for whole tiles at 16 * lane and 1024 + 16 * lane (the 64
// lanes read 1 KiB contiguously, no bank conflict), its scale at
// 2048 + 4 * m; for 8-token pages the same with 8-token groups.  Inline
// assembly with its own LDS wait, as read_slot.
__device__ __forceinline__ SlotOperands read_slot_pre(const uint8_t* slot, int lane, int page_size) {
  static_assert(kPreTileBytes == 2112, "offsets below assume 2112-byte tiles");
  const int m = lane & 15, kq = lane >> 4;
  const uint32_t base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const uint8_t*)slot);
  uint32_t av, as, half;
  if (page_size >= kTile) {
    av = base + 16u * (uint32_t)lane;
    half = 1024u;
    as = base + 2048u + 4u * (uint32_t)m;
  } else {  // 8-token pages
    const uint32_t pg = (uint32_t)(m >> 3) * 1056u;
    av = base + pg + 128u * (uint32_t)kq + 16u * (uint32_t)(m & 7);
    half = 512u;
    as = base + pg + 1024u + 4u * (uint32_t)(m & 7);
  }
  const uint32_t ah = av + half;
  u32x4 lo0, hi0, lo1, hi1, lo2, hi2, lo3, hi3;
  SlotOperands r;
  asm volatile(
      "ds_read_b128 %0, %12\n\t"
      "ds_read_b128 %1, %13\n\t"
      "ds_read_b128 %2, %12 offset:2112\n\t"
      "ds_read_b128 %3, %13 offset:2112\n\t"
      "ds_read_b128 %4, %12 offset:4224\n\t"
      "ds_read_b128 %5, %13 offset:4224\n\t"
      "ds_read_b128 %6, %12 offset:6336\n\t"
      "ds_read_b128 %7, %13 offset:6336\n\t"
      "ds_read_b32 %8, %14\n\t"
      "ds_read_b32 %9, %14 offset:2112\n\t"
      "ds_read_b32 %10, %14 offset:4224\n\t"
      "ds_read_b32 %11, %14 offset:6336\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(lo0), "=&v"(hi0), "=&v"(lo1), "=&v"(hi1), "=&v"(lo2), "=&v"(hi2), "=&v"(lo3),
        "=&v"(hi3), "=&v"(r.sc[0]), "=&v"(r.sc[1]), "=&v"(r.sc[2]), "=&v"(r.sc[3])
      : "v"(av), "v"(ah), "v"(as)
      : "memory");
  const u32x4 lo[kTilesPerIter] = {lo0, lo1, lo2, lo3};
  const u32x4 hi[kTilesPerIter] = {hi0, hi1, hi2, hi3};
#pragma unroll
  for (int tile = 0; tile < kTilesPerIter; ++tile) {
    r.kb[tile][0] = lo[tile][0]; r.kb[tile][1] = lo[tile][1];
    r.kb[tile][2] = lo[tile][2]; r.kb[tile][3] = lo[tile][3];
    r.kb[tile][4] = hi[tile][0]; r.kb[tile][5] = hi[tile][1];
    r.kb[tile][6] = hi[tile][2]; r.kb[tile][7] = hi[tile][3];
  }
  return r;
}

// The iteration's operands from its slot, in the pool's layout.
template <int LAYOUT>
__device__ __forceinline__ SlotOperands read_slot_any(const LogitsParams& p, const uint8_t* slot,
                                                      int lane) {
  if constexpr (LAYOUT == kLayoutPreshuffled) return read_slot_pre(slot, lane, p.page_size);
  else return read_slot(slot, lane);
}

// Score one iteration from its operands, already read from the slot.
// WHOLE_SKIP: an iteration wholly inside the context skips clearing the
// scales of tokens past it, 12 vector instructions of ~330 (interleaved on
// the 128-head kernels: MTP 317.4 -> 308.4 us, long context 118.7 -> 114.0
// us); the single-wave kernel keeps the unconditional form (its gather and
// q loads are ordered by explicit waits, and the branch reshaped its code:
// 10.3 -> 14.6 us on decode).
template <int H, int JW, bool WHOLE_SKIP = true>
__device__ __forceinline__ void score_ops(const LogitsParams& p, const Run& c, int it, int j0,
                                          int lane, const QRegs<H, JW>& qr, SlotOperands op) {
  // the wave's first row sees the fewest tokens
  const int min_vis = min(max(c.ctx - p.next_n + j0 + 1, 0), c.ctx);
  const int t0 = it * kIterTokens + (lane & 15);
  // tokens past the context (only in a run's last iteration): scale 0, never
  // stored
  if (!WHOLE_SKIP || it * kIterTokens + kIterTokens > c.ctx_eff) {
#pragma unroll
    for (int tile = 0; tile < kTilesPerIter; ++tile)
      op.sc[tile] = t0 + tile * kTile < c.ctx_eff ? op.sc[tile] : 0.f;
  }
  bool bad = false;
#pragma unroll
  for (int tile = 0; tile < kTilesPerIter; ++tile)
    bad |= !(op.sc[tile] >= 0.f);  // NaN takes the literal form, which passes it on
  const bool factored = __ballot(bad) == 0;
  if (min_vis < kExactRows) {
    if (factored) score_iteration<H, JW, true, true>(p, c, it, j0, lane, qr, op.kb, op.sc);
    else score_iteration<H, JW, true, false>(p, c, it, j0, lane, qr, op.kb, op.sc);
  } else {
    if (factored) score_iteration<H, JW, false, true>(p, c, it, j0, lane, qr, op.kb, op.sc);
    else score_iteration<H, JW, false, false>(p, c, it, j0, lane, qr, op.kb, op.sc);
  }
}

template <int H, int JW, int LAYOUT, bool WHOLE_SKIP = true>
__device__ __forceinline__ void score(const LogitsParams& p, const Run& c, int it, int j0, int lane,
                                      const QRegs<H, JW>& qr, const uint8_t* slot) {
  score_ops<H, JW, WHOLE_SKIP>(p, c, it, j0, lane, qr, read_slot_any<LAYOUT>(p, slot, lane));
}

// H heads; JW next_n rows per wave; WAVES waves per workgroup (one workgroup
// per CU); RING iterations in flight per wave.
//
// Pipeline of one wave over its run of n iterations (refill(j) = page ids of
// iteration j+2R, then the gather of iteration j+R; R = RING):
//   prologue: ids of iterations 0..R-1 and the q rows (waited for), then
//             refill(-R) .. refill(-1) -- always R gathers, placeholders past
//             the run, so that the count of gathers in flight is fixed (one
//             slot: the q rows are loaded after the gather instead)
//   loop k:   wait for gather k; score k from its slot; refill(k)
// The ids refill(k) uses (those of iteration k+R) were issued by
// refill(k-R) before the gather of k, so "gather k has landed" (the vector
// memory counter drains in order) also proves they have landed.  Ids of
// iteration j live in id slot j % 2R, values in ring slot j % R.
template <int H, int JW, int WAVES, int RING, int LAYOUT>
__global__ __launch_bounds__(64 * WAVES) void logits_kernel(const int32_t* __restrict__ ctx_lens,
                                                            int32_t batch, int32_t max_tokens,
                                                            LogitsParams p) {
  const CtxArgs ca{ctx_lens, batch, max_tokens};
  __shared__ __attribute__((aligned(16))) uint8_t ring[WAVES][RING][kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint32_t ids[WAVES][2 * RING][kMaxPages];
  const int lane = threadIdx.x & 63;
  const int m = lane & 15;   // token within a tile (B column / A row)
  const int kq = lane >> 4;  // 32-byte quarter of the head dimension
  const int wl = uniform(threadIdx.x >> 6);
  const uint32_t nwg = gridDim.x;  // a multiple of 8
  const uint32_t wg = (blockIdx.x & 7u) * (nwg >> 3) + (blockIdx.x >> 3);
  // units are dealt wave-major over the workgroups, so that when fewer units
  // than waves have work every CU still gets its share.  When the row groups
  // of a unit fit a workgroup evenly, they take consecutive waves of one
  // workgroup: they gather the same pages, which that CU's L1 may then serve
  // once for all of them.
  const uint32_t rg = (uint32_t)p.n_rgroups;
  const uint32_t wave = (uint32_t)WAVES % rg == 0u
                            ? ((uint32_t)wl / rg) * (nwg * rg) + wg * rg + (uint32_t)wl % rg
                            : (uint32_t)wl * nwg + wg;
  const int unit = (int)(wave / (uint32_t)p.n_rgroups);
  const int j0 = (int)(wave % (uint32_t)p.n_rgroups) * JW;

  uint8_t* my_ring = &ring[wl][0][0];
  uint32_t* my_ids = &ids[wl][0][0];
  // while the context lengths are read: pull a small block table into the L2
  // of every XCD (each XCD has its own L2, and any wave may need any request's
  // page ids; workgroups are dealt round-robin over the XCDs, so blockIdx >> 3
  // numbers this XCD's workgroups) and q into L2 once (its first use waits
  // behind a gather anyway).  One 4-byte load per 128-byte line, into this
  // wave's idle ring slot: the gathers that fill the slot later are issued
  // after them, and vector memory loads complete in order.
  {
    const int64_t tline = ((int64_t)(blockIdx.x >> 3) * WAVES + wl) * 64 + lane;
    if (tline < p.warm_table_lines)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(p.tables) + tline * 128,
                                       LDS_PTR(my_ring), 4, 0, 0);
    const int64_t qline = ((int64_t)blockIdx.x * WAVES + wl) * 64 + lane;
    if (qline < p.warm_q_lines)
      __builtin_amdgcn_global_load_lds(p.q + qline * 128, LDS_PTR(my_ring + 256), 4, 0, 0);
  }
  Run run;
  if (wave >= (uint32_t)p.n_slices * (uint32_t)p.n_rgroups || !find_run(ca, p, unit, lane, run)) {
    __builtin_amdgcn_s_waitcnt(0);  // the warm-up loads write this workgroup's LDS: land them first
    return;
  }
  const int n_it = run.n_it;
  // the gather's per-lane chunk offsets: kept in registers when the wave has
  // registers to spare (4 waves per CU, or 128 q rows at two waves per SIMD),
  // recomputed at each gather otherwise (an opaque copy of the lane index keeps
  // the compiler from hoisting them)
  constexpr bool pre = LAYOUT == kLayoutPreshuffled;
  const ChunkOffsets co_kept = chunk_offsets(lane, pre);
  auto offsets = [&]() -> ChunkOffsets {
    if constexpr (WAVES <= 4 || (WAVES == 8 && H * JW == 128)) {
      return co_kept;
    } else {
      int l = lane;
      asm volatile("" : "+v"(l));
      return chunk_offsets(l, pre);
    }
  };

  // prologue
#pragma unroll
  for (int s = 0; s < RING; ++s)
    if (s < n_it) issue_ids(p, run, run.it0 + s, lane, my_ids + s * kMaxPages);
  QRegs<H, JW> qr;
  if constexpr (RING > 1) load_q<H, JW>(p, run.b, j0, m, kq, qr);
  __builtin_amdgcn_s_waitcnt(0);  // ids of the first R iterations (and q)
  int n_ids = min(n_it, RING);  // iterations whose ids were issued
#pragma unroll
  for (int s = 0; s < RING; ++s) {
    if (n_ids < n_it) {
      issue_ids(p, run, run.it0 + n_ids, lane, my_ids + (n_ids % (2 * RING)) * kMaxPages);
      ++n_ids;
    }
    issue_gather<LAYOUT, kStreamK>(p, run.it0 + s, s < n_it ? run.ctx_eff : 0, my_ids + s * kMaxPages, lane,
                 offsets(), my_ring + s * kSlotBytes);
  }
  // with one slot, the first score waits for every load anyway: q behind the
  // first gather keeps its latency off the path to the K stream
  if constexpr (RING == 1) load_q<H, JW>(p, run.b, j0, m, kq, qr);
  const int n_span = max(n_it, RING);
  for (int k0 = 0; k0 < n_it; k0 += RING) {
#pragma unroll
    for (int s = 0; s < RING; ++s) {
      const int k = k0 + s;
      if (k >= n_it) break;
      // the gathers issued after this one's (kGatherLoads instructions each;
      // page-id loads and stores issued in between only add to the count):
      // once at most that many are outstanding, iteration k's data has landed
      wait_vm(kGatherLoads * min(RING - 1, n_span - 1 - k));
      score<H, JW, LAYOUT>(p, run, run.it0 + k, j0, lane, qr, my_ring + s * kSlotBytes);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // slot reads done before refill
      if (k + RING < n_it) {
        // refill(k): ids of iteration k + 2R, then the gather of k + R
        if (n_ids < n_it) {
          issue_ids(p, run, run.it0 + n_ids, lane, my_ids + (n_ids % (2 * RING)) * kMaxPages);
          ++n_ids;
        }
        issue_gather<LAYOUT, kStreamK>(p, run.it0 + k + RING, run.ctx_eff,
                     my_ids + ((k + RING) % (2 * RING)) * kMaxPages, lane, offsets(),
                     my_ring + s * kSlotBytes);
      }
    }
  }
}

// One unit per workgroup, its next_n rows one per wave (G waves), sharing one
// ring of RING K slots: every page is gathered once for all rows.  Wave w
// issues the page ids and the gather of the iterations k with k % G == w; a
// workgroup barrier per iteration publishes slot k (its owner waited for it
// first) and frees slot k - 1 (every wave read it before the barrier) for the
// gather of k + RING - 1.  Page ids of iteration k + L are issued just before
// the gather of k, so the owner's wait for gather k proves them landed before
// their own gather is issued (L >= RING - 1).  Every wave of a workgroup runs
// the same run, hence the same number of barriers.
template <int H, int G, int RING, int LAYOUT>
__global__ __launch_bounds__(64 * G) __attribute__((amdgpu_waves_per_eu(2, 2)))
void logits_shared_kernel(const int32_t* __restrict__ ctx_lens, int32_t batch, int32_t max_tokens,
                          LogitsParams p) {
  constexpr int L = ((RING - 1 + G - 1) / G) * G;
  constexpr int NS = L / G + 1;
  static_assert(RING % G == 0 && L >= RING - 1, "shared ring layout");
  const CtxArgs ca{ctx_lens, batch, max_tokens};
  __shared__ __attribute__((aligned(16))) uint8_t ring[RING][kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint32_t ids[G][NS][kMaxPages];
  const int lane = threadIdx.x & 63;
  const int m = lane & 15;
  const int kq = lane >> 4;
  const int wl = uniform(threadIdx.x >> 6);
  const uint32_t nwg = gridDim.x;  // a multiple of 8
  const int unit = (int)((blockIdx.x & 7u) * (nwg >> 3) + (blockIdx.x >> 3));
  uint32_t* my_ids = &ids[wl][0][0];
  auto id_slot = [&](int k) { return my_ids + ((k / G) % NS) * kMaxPages; };
  {
    const int64_t tline = ((int64_t)(blockIdx.x >> 3) * G + wl) * 64 + lane;
    if (tline < p.warm_table_lines)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(p.tables) + tline * 128,
                                       LDS_PTR(my_ids), 4, 0, 0);
    const int64_t qline = ((int64_t)blockIdx.x * G + wl) * 64 + lane;
    if (qline < p.warm_q_lines)
      __builtin_amdgcn_global_load_lds(p.q + qline * 128, LDS_PTR(my_ids), 4, 0, 0);
  }
  Run run;
  if (unit >= p.n_slices || !find_run(ca, p, unit, lane, run)) {
    __builtin_amdgcn_s_waitcnt(0);
    return;
  }
  const int n_it = run.n_it;
  const ChunkOffsets co = chunk_offsets(lane, LAYOUT == kLayoutPreshuffled);
  for (int k = wl; k < L; k += G)
    if (k < n_it) issue_ids(p, run, run.it0 + k, lane, id_slot(k));
  QRegs<H, 1> qr;
  load_q<H, 1>(p, run.b, wl, m, kq, qr);
  __builtin_amdgcn_s_waitcnt(0);
  for (int k = wl; k < RING - 1; k += G) {
    if (k >= n_it) break;
    if (k + L < n_it) issue_ids(p, run, run.it0 + k + L, lane, id_slot(k + L));
    issue_gather<LAYOUT, 0>(p, run.it0 + k, run.ctx_eff, id_slot(k), lane, co, &ring[k % RING][0]);
  }
  for (int k = 0; k < n_it; ++k) {
    if (k % G == wl) {
      // own gathers issued after k's: k + G, k + 2G, ... up to k + RING - 2
      const int last = min(k + RING - 2, n_it - 1);
      wait_vm(kGatherLoads * (last > k ? (last - k) / G : 0));
    }
    __builtin_amdgcn_s_barrier();
    const int nx = k + RING - 1;
    if (nx < n_it && nx % G == wl) {
      if (nx + L < n_it) issue_ids(p, run, run.it0 + nx + L, lane, id_slot(nx + L));
      issue_gather<LAYOUT, 0>(p, run.it0 + nx, run.ctx_eff, id_slot(nx), lane, co, &ring[nx % RING][0]);
    }
    score<H, 1, LAYOUT>(p, run, run.it0 + k, wl, lane, qr, &ring[k % RING][0]);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
}

// Flat geometry for small units (all next_n rows of a request within 64 q
// rows): a work item is one 64-token iteration of one request, and every wave
// is a workgroup of its own.  The grid is at most one residency of the chip
// (16 such waves per CU), so no wave is dispatched behind the K stream, where
// its first loads would queue behind the whole gather traffic.  Workgroup g
// runs on XCD g % 8 (the dispatcher deals workgroups round-robin over the
// XCDs); XCD x takes a contiguous eighth of the request-ordered item list, and
// its waves take contiguous, nearly equal shares of that, the longer shares
// going to the waves dispatched first.  Consecutive items of a wave are then
// mostly consecutive iterations of one request, whose q rows stay in
// registers, and consecutive waves on an XCD read the same q rows and table
// lines from that XCD's L2.  One K slot per wave, refilled once its item is
// scored.  Pages of 64 tokens or more hold a whole item: its page id comes by
// a scalar load and q is requested before the gather; smaller pages stage the
// item's page ids in LDS, and the next item's ids travel with the current
// gather.  The
// host takes this geometry only when the possible iterations are at most two
// residencies, so a share holds one or two items.
// A one-iteration run: iteration it0 of request b (context ctx).  Built in one
// place from plain values, so that no field is stored on one path and not on
// another (such stores through a merged pointer keep the struct in scratch
// memory).
__device__ __forceinline__ Run item_run(const CtxArgs& a, int b, int ctx, int it0) {
  Run r;
  r.b = b;
  r.ctx = ctx;
  r.ctx_eff = min(ctx, a.max_tokens);
  r.it0 = it0;
  r.n_it = 1;
  return r;
}

// Item e of the request-ordered list (e < the list's length).
__device__ __forceinline__ Run locate_item(const CtxArgs& a, uint32_t e, int lane,
                                           uint32_t n0, int ctx0, uint32_t incl0,
                                           uint32_t chunk0) {
  uint32_t before = 0, n = n0, incl = incl0, chunk = chunk0;
  int ctx = ctx0;
  int b = 0, bctx = 0, it0 = 0;
  for (int c0 = 0; c0 < a.batch;) {
    if (before + chunk > e) {
      const uint64_t past = __ballot(before + incl > e);
      const int f = uniform(__builtin_ctzll(past));
      b = c0 + f;
      bctx = (int)lane_of((uint32_t)ctx, f);
      it0 = (int)(e - (before + lane_of(incl, f) - lane_of(n, f)));
      break;
    }
    before += chunk;
    c0 += 64;
    if (c0 >= a.batch) break;  // not reached: e lies inside the list
    n = (uint32_t)lane_iters(a, c0, lane, ctx);
    incl = wave_prefix(n, lane, chunk);
  }
  return item_run(a, b, bctx, it0);
}

// The item after `cur` (item e of the list): its next iteration, or the first
// of a later request.
__device__ __forceinline__ Run next_item(const CtxArgs& a, const Run& cur, uint32_t e,
                                         int lane, uint32_t n0, int ctx0, uint32_t incl0,
                                         uint32_t chunk0) {
  int b = cur.b, ctx = cur.ctx, it0 = cur.it0 + 1;
  if (it0 >= n_iters(cur.ctx, a.max_tokens)) {
    const Run r = locate_item(a, e, lane, n0, ctx0, incl0, chunk0);
    b = r.b;
    ctx = r.ctx;
    it0 = r.it0;
  }
  return item_run(a, b, ctx, it0);
}

template <int H, int JW, int LAYOUT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(4, 8)))
void logits_flat_kernel(const int32_t* __restrict__ ctx_lens, int32_t batch, int32_t max_tokens,
                        const int64_t* __restrict__ tables, int32_t warm_lines,
                        const uint8_t* __restrict__ q, int32_t q_lines, LogitsParams p) {
  const CtxArgs ca{ctx_lens, batch, max_tokens};
  __shared__ __attribute__((aligned(16))) uint8_t slot[kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint32_t ids[2][kMaxPages];
  const int lane = threadIdx.x;
  const int m = lane & 15;
  const int kq = lane >> 4;
  const uint32_t xcd = blockIdx.x & 7u;
  const uint32_t k = blockIdx.x >> 3;
  const uint32_t kx = gridDim.x >> 3;  // waves per XCD
  // the context lengths of the first 64 requests are requested first, by one
  // 4-byte LDS-bound load into the idle page-id slots (lanes past the batch
  // reread the last one); then a small block table is pulled into this XCD's
  // L2, and so is the eighth of a small q that this XCD's share of the
  // request-ordered items mostly needs (one 4-byte load per 128-byte line,
  // into the idle K slot; the gather that fills the slot later lands after
  // them), so that the page-id and q loads that follow the item search hit L2.
  // The warm-up is exactly two loads (lanes without a line reread the first
  // one), so vmcnt(2) proves the context lengths have landed without waiting
  // for it: the counter drains in order, while a wait the compiler derived
  // for a register load would also drain the warm-up.
  __builtin_amdgcn_global_load_lds(ctx_lens + min(lane, batch - 1), LDS_PTR(&ids[1][0]), 4, 0, 0);
  asm volatile("" ::: "memory");  // the context-length load goes first
  {
    const int64_t line = (int64_t)k * 64 + lane;
    const int64_t tl = line < warm_lines ? line : 0;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(tables) + tl * 128,
                                     LDS_PTR(slot), 4, 0, 0);
    const int32_t q8 = (q_lines + 7) >> 3;
    const int64_t ql = (int64_t)xcd * q8 + line;
    const int64_t qq = line < q8 && ql < q_lines ? ql : 0;
    __builtin_amdgcn_global_load_lds(q + qq * 128, LDS_PTR(slot + 256), 4, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0x0f70 | 2);  // vmcnt(2): the context lengths have landed
  int craw;
  {
    // inline assembly with its own LDS wait, like the ring reads: a plain LDS
    // read would make the compiler drain the warm-up loads first
    const uint32_t ca_lds =
        (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const uint32_t*)&ids[1][0]) +
        4u * (uint32_t)lane;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(craw) : "v"(ca_lds) : "memory");
  }
  // iterations of every request
  const int ctx0 = lane < batch ? max(craw, 0) : 0;
  const uint32_t n0 = (uint32_t)n_iters(ctx0, max_tokens);
  uint32_t chunk0;
  const uint32_t incl0 = wave_prefix(n0, lane, chunk0);
  uint32_t total = chunk0;
  for (int c0 = 64; c0 < ca.batch; c0 += 64) {
    int ctx;
    total += wave_sum((uint32_t)lane_iters(ca, c0, lane, ctx));
  }
  // this wave's share: items [e, e + cnt) of the list
  const uint32_t per = (total + 7u) >> 3;
  const uint32_t lo = min(xcd * per, total);
  const uint32_t nx = min(lo + per, total) - lo;
  const uint32_t a = nx / kx, r = nx % kx;
  const uint32_t cnt = a + (k < r ? 1u : 0u);
  if (cnt == 0) {
    __builtin_amdgcn_s_waitcnt(0);  // the warm-up loads write this workgroup's LDS
    return;
  }
  uint32_t e = lo + k * a + min(k, r);

  // at most two items: the grid covers at least half of the possible ones
  Run cur = locate_item(ca, e, lane, n0, ctx0, incl0, chunk0), nxt = cur;
  QRegs<H, JW> qr;
  QLines<H, JW> ql;
  if (p.log2_page >= 6) {
    // one page per item: q is requested as whole lines, then the page id by a
    // scalar load, ahead of this wave's gather (and of most waves'); q is
    // shaped into operands while the gather is in flight
    // (q first: waiting for a scalar load waits for all of them, and q's
    // addresses come from scalar loads of the arguments)
    load_q_lines<H, JW>(p, cur.b, lane, kq, ql, qr);
    asm volatile("" ::: "memory");  // every q load is issued before the gather
    const int64_t id0 = page_id(p, cur);
    gather_page<kStreamK>(p, cur.it0, id0, lane, chunk_offsets(lane, LAYOUT == kLayoutPreshuffled), slot);
    // the q loads have landed once at most the gather's loads are left (the
    // vector memory counter drains in order); the compiler would drain the
    // gather too
    __builtin_amdgcn_s_waitcnt(0x0f70 | kGatherLoads);  // vmcnt(kGatherLoads)
    assemble_q_xlane<H, JW>(ql, lane, qr);
    int64_t id1 = 0;
    if (cnt > 1) {
      nxt = next_item(ca, cur, e + 1, lane, n0, ctx0, incl0, chunk0);
      id1 = page_id(p, nxt);
    }
    __builtin_amdgcn_s_waitcnt(0);  // the gather
    score<H, JW, LAYOUT, false>(p, cur, cur.it0, 0, lane, qr, slot);
    if (cnt == 1) return;
    // the slot reads are done (read_slot waits for them): refill it.  The next
    // item's fields and the lane pass through empty asm so that its addresses
    // are formed here, not early and spilled: a spill reload between the
    // gather's loads would wait for every load issued before it.
    int l2 = lane;
    nxt.it0 = uniform(nxt.it0);
    nxt.b = uniform(nxt.b);
    asm volatile("" : "+v"(l2), "+s"(nxt.it0), "+s"(nxt.b));
    gather_page<kStreamK>(p, nxt.it0, id1, l2, chunk_offsets(l2, LAYOUT == kLayoutPreshuffled), slot);
    // a second item's q (few waves have one) takes the operand-shaped loads,
    // which need no registers beside the operands
    if (nxt.b != cur.b) load_q<H, JW>(p, nxt.b, 0, m, kq, qr);
    __builtin_amdgcn_s_waitcnt(0);
    score<H, JW, LAYOUT, false>(p, nxt, nxt.it0, 0, lane, qr, slot);
    return;
  }
  // smaller pages: the item's page ids are staged in LDS, one per lane
  issue_ids(p, cur, cur.it0, lane, ids[0]);
  __builtin_amdgcn_s_waitcnt(0);  // page ids in LDS
  issue_gather<LAYOUT, kStreamK>(p, cur.it0, cur.ctx_eff, ids[0], lane, chunk_offsets(lane, LAYOUT == kLayoutPreshuffled), slot);
  if (cnt > 1) {
    nxt = next_item(ca, cur, e + 1, lane, n0, ctx0, incl0, chunk0);
    issue_ids(p, nxt, nxt.it0, lane, ids[1]);
  }
  load_q_lines<H, JW>(p, cur.b, lane, kq, ql, qr);
  __builtin_amdgcn_s_waitcnt(0);  // the gather, q and the next item's ids
  {
    const SlotOperands op = read_slot_any<LAYOUT>(p, slot, lane);
    assemble_q<H, JW>(ql, lane, slot, qr);
    score_ops<H, JW, false>(p, cur, cur.it0, 0, lane, qr, op);
  }
  if (cnt == 1) return;
  int l2 = lane;
  nxt.it0 = uniform(nxt.it0);
  nxt.ctx_eff = uniform(nxt.ctx_eff);
  nxt.b = uniform(nxt.b);
  asm volatile("" : "+v"(l2), "+s"(nxt.it0), "+s"(nxt.ctx_eff), "+s"(nxt.b));
  issue_gather<LAYOUT, kStreamK>(p, nxt.it0, nxt.ctx_eff, ids[1], l2, chunk_offsets(l2, LAYOUT == kLayoutPreshuffled), slot);
  if (nxt.b != cur.b) load_q<H, JW>(p, nxt.b, 0, m, kq, qr);
  __builtin_amdgcn_s_waitcnt(0);
  score<H, JW, LAYOUT, false>(p, nxt, nxt.it0, 0, lane, qr, slot);
}

// Launch geometry per instantiation.  Wave units of at most 64 q rows (and at
// most 3 next_n rows, whose partial sums also take registers) run 9 waves per
// workgroup (2-3 per SIMD, so that one wave's matrix work overlaps another's
// memory stalls) with one iteration in flight each: measured on the decode
// shape, a second slot per wave made waves stall on issuing its gather behind
// the saturated memory pipeline before scoring the first, which cost more than
// the prefetch gained.  Units of 128 q rows fit two waves per SIMD (8 per
// workgroup, 2 iterations in flight each): a second wave per SIMD is what
// keeps the matrix core busy (measured faster than 2 rows per wave at 1 wave
// per SIMD, despite gathering each page once per row group; measured before
// the epilogue's schedule kept two products in flight, when a wave's own
// matrix and vector instructions barely overlapped).  Units of 192 rows
// also run two waves per SIMD: they then fill the 256 registers a wave gets
// there (a few values spill, outside the scoring loop) and were measured about
// 9% faster than one wave per SIMD with 4 iterations in flight.  Larger units
// need the registers of a whole SIMD and run 4 waves with 4 iterations in
// flight.
template <int H, int JW>
struct Geometry {
  static constexpr bool kSmall = H * JW <= 64 && JW <= 3;
  static constexpr bool kMid = H * JW == 128 || H * JW == 192;
  static constexpr int kWaves = kSmall ? 9 : (kMid ? 8 : 4);
  static constexpr int kRingDepth = kSmall ? 1 : (kMid ? 2 : 4);
};

template <int H, int JW, int LAYOUT>
hipError_t launch_one(const LogitsParams& p, const LaunchTiming& tm, hipStream_t stream) {
  if constexpr (H * JW <= 64) {
    if (p.flat_items > 0) {
      // at most one residency: 16 single-wave workgroups per CU, 32 CUs per XCD
      const int64_t per_xcd = (p.flat_items + 7) / 8;
      const uint32_t n_wg = 8u * (uint32_t)(per_xcd < 16 * 32 ? per_xcd : 16 * 32);
      auto kern = logits_flat_kernel<H, JW, LAYOUT>;
      const int32_t warm = (int32_t)p.warm_table_lines;  // at most 8192 (a 1 MiB table)
      const int32_t warm_q = (int32_t)p.warm_q_lines;    // at most 32768 (a 4 MiB q)
      if (tm.start || tm.stop)
        hipExtLaunchKernelGGL(kern, dim3(n_wg), dim3(64), 0, stream, tm.start, tm.stop, 0, p.ctx,
                              p.batch, p.max_tokens, p.tables, warm, p.q, warm_q, p);
      else
        hipLaunchKernelGGL(kern, dim3(n_wg), dim3(64), 0, stream, p.ctx, p.batch, p.max_tokens,
                           p.tables, warm, p.q, warm_q, p);
      return hipGetLastError();
    }
  }
  if constexpr (H == 128 && JW == 1) {
    const int ring = shared_ring_depth(H, JW, p.n_rgroups);
    if (ring > 0) {
      // one unit per workgroup of n_rgroups waves
      const uint32_t n_wg = ((uint32_t)p.n_slices + 7u) & ~7u;
      auto kern = ring == 8 ? logits_shared_kernel<128, 4, 8, LAYOUT> : logits_shared_kernel<128, 2, 4, LAYOUT>;
      const dim3 block(64 * p.n_rgroups);
      if (tm.start || tm.stop)
        hipExtLaunchKernelGGL(kern, dim3(n_wg), block, 0, stream, tm.start, tm.stop, 0, p.ctx,
                              p.batch, p.max_tokens, p);
      else
        hipLaunchKernelGGL(kern, dim3(n_wg), block, 0, stream, p.ctx, p.batch, p.max_tokens, p);
      return hipGetLastError();
    }
  }
  using G = Geometry<H, JW>;
  uint32_t n_wg = ((uint32_t)p.n_slices * (uint32_t)p.n_rgroups + G::kWaves - 1) / G::kWaves;
  n_wg = (n_wg + 7u) & ~7u;
  auto kern = logits_kernel<H, JW, G::kWaves, G::kRingDepth, LAYOUT>;
  if (tm.start || tm.stop)
    hipExtLaunchKernelGGL(kern, dim3(n_wg), dim3(64 * G::kWaves), 0, stream, tm.start, tm.stop, 0,
                          p.ctx, p.batch, p.max_tokens, p);
  else
    hipLaunchKernelGGL(kern, dim3(n_wg), dim3(64 * G::kWaves), 0, stream, p.ctx, p.batch,
                       p.max_tokens, p);
  return hipGetLastError();
}

// Rows per wave: at most kMaxRows(H) (the shapes logits_shape picks).
template <int H>
constexpr int kMaxRows = H >= 128 ? 1 : (H >= 64 ? 3 : 4);

template <int H, int LAYOUT>
hipError_t launch_rows(const LogitsParams& p, int jw, const LaunchTiming& tm,
                       hipStream_t stream) {
  switch (jw) {
    case 1: return launch_one<H, 1, LAYOUT>(p, tm, stream);
    case 2: if constexpr (kMaxRows<H> >= 2) return launch_one<H, 2, LAYOUT>(p, tm, stream); break;
    case 3: if constexpr (kMaxRows<H> >= 3) return launch_one<H, 3, LAYOUT>(p, tm, stream); break;
    case 4: if constexpr (kMaxRows<H> >= 4) return launch_one<H, 4, LAYOUT>(p, tm, stream); break;
  }
  return hipErrorInvalidValue;
}

// The pool's layout is a template parameter of every kernel, so each layout
// is compiled on its own (the record layout's kernels keep their registers).
template <int H>
hipError_t launch_heads(const LogitsParams& p, int jw, const LaunchTiming& tm,
                        hipStream_t stream) {
  return p.kv_layout == kLayoutPreshuffled ? launch_rows<H, kLayoutPreshuffled>(p, jw, tm, stream)
                                           : launch_rows<H, kLayoutRecords>(p, jw, tm, stream);
}

template <int H>
int ring_depth(int jw) {
  return jw <= 1 ? Geometry<H, 1>::kRingDepth
                 : jw == 2 ? Geometry<H, 2>::kRingDepth
                           : jw == 3 ? Geometry<H, 3>::kRingDepth : Geometry<H, 4>::kRingDepth;
}

template <int H>
int waves_per_cu(int jw) {
  return jw <= 1 ? Geometry<H, 1>::kWaves
                 : jw == 2 ? Geometry<H, 2>::kWaves
                           : jw == 3 ? Geometry<H, 3>::kWaves : Geometry<H, 4>::kWaves;
}

}  // namespace

LogitsShape logits_shape(int heads, int next_n) {
  LogitsShape sh;
  // rows per wave: measured per head count (at most 192 q rows of A operands)
  const int cap = heads >= 128 ? kMaxRows<128> : (heads >= 64 ? kMaxRows<64> : kMaxRows<32>);
  sh.rows_per_wave = next_n < cap ? next_n : cap;
  sh.iter_tokens = kIterTokens;
  // one workgroup per CU (its K ring fills most of the CU's LDS)
  int per_cu = 4;
  switch (heads) {
    case 16: per_cu = waves_per_cu<16>(sh.rows_per_wave); break;
    case 32: per_cu = waves_per_cu<32>(sh.rows_per_wave); break;
    case 64: per_cu = waves_per_cu<64>(sh.rows_per_wave); break;
    case 128: per_cu = waves_per_cu<128>(sh.rows_per_wave); break;
  }
  sh.target_waves = 256 * per_cu;
  // flat geometry: every row of a request in one wave of at most 64 q rows, and
  // at most two residencies of 16 single-wave workgroups per CU
  sh.flat_max_items = heads * next_n <= 64 && sh.rows_per_wave == next_n ? 2 * 16 * 256 : 0;
  return sh;
}

void persistent_geometry(int heads, int rows_per_wave, int* waves, int* ring) {
  switch (heads) {
    case 16: *waves = waves_per_cu<16>(rows_per_wave); *ring = ring_depth<16>(rows_per_wave); break;
    case 32: *waves = waves_per_cu<32>(rows_per_wave); *ring = ring_depth<32>(rows_per_wave); break;
    case 64: *waves = waves_per_cu<64>(rows_per_wave); *ring = ring_depth<64>(rows_per_wave); break;
    default: *waves = waves_per_cu<128>(rows_per_wave); *ring = ring_depth<128>(rows_per_wave); break;
  }
}

hipError_t launch_logits(const LogitsParams& p, const LogitsShape& sh, int heads,
                         const LaunchTiming& tm, hipStream_t stream) {
  switch (heads) {
    case 16: return launch_heads<16>(p, sh.rows_per_wave, tm, stream);
    case 32: return launch_heads<32>(p, sh.rows_per_wave, tm, stream);
    case 64: return launch_heads<64>(p, sh.rows_per_wave, tm, stream);
    case 128: return launch_heads<128>(p, sh.rows_per_wave, tm, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pmqa
