// Per-row top-k of the logits rows for gfx950 (MI355X).
//
// The selection that follows the logits (top_k_per_row_decode in aiter PR
// #4244, first paragraph): for each row r, the indices of the k largest scores
// among its visible tokens [0, visible(r)), -1 in the slots left over.
//
// Work split.  A row of up to 16384 scores is selected by one 1024-thread
// workgroup (when the row stride allows no longer rows).  Otherwise a row is
// cut into nseg nearly equal segments of at most 8192 scores while the grid's
// second dimension (which the caller's workspace and the merge's 16384
// candidates bound) allows, else of at most 16384, each selected by its own
// workgroup into k candidates (score, index) in the workspace; a second
// launch then selects the row's top k among its nseg * k candidates.  This is
// exact: every key of the row's top k is in its segment's top k under the
// same order (score descending, index ascending), and for any one score a
// segment lists its keys in index order, so taking equal candidates in list
// order still takes the lowest indices.  Only the visible scores
// [0, visible) are read.  Each launch has two kernels that differ only in
// their register layouts (two workgroups per CU, or 16 floats a thread at
// one per CU); the host picks them from the grid (launch_topk).
//
// A list held in registers (up to 16384 scores, 16 a thread) is first tried
// on the floats themselves (select_held): value buckets between its smallest
// and largest score, the threshold bucket (split again into value buckets,
// up to three passes in all, while it holds too many scores: heavy-tailed
// rows crowd the lowest buckets), then every score above it staged in LDS at
// its slot and the threshold bucket's few scores ranked directly.  One CU
// issues every instruction of a row, so this path keeps a fixed, small
// number of instructions per score and pass (no per-score branches or
// ballots).  Lists it cannot resolve that way (a non-finite score, all
// scores equal, a threshold bucket still crowded after three passes), longer
// rows, and in the two-per-CU split grid lists of more than 8192 scores
// (whose floats and buckets would exceed its register budget) take the
// radix passes below.
//
// One workgroup's exact select on order-preserving 32-bit keys keeps every
// step off long LDS round-trip chains, which dominate at these sizes:
//  * the keys are loaded once into registers (up to 16 a thread); longer
//    segments (a workspace too small to split the row further) stream
//    through registers chunk by chunk in every pass, the next chunk's loads
//    in flight while the current one is processed;
//  * on keys held in registers whose scores are all finite, the first pass
//    buckets by value, linearly between the smallest and largest score
//    (monotone, so still exact): on bell-shaped scores the bucket holding the
//    k-th key keeps a few dozen keys, where a radix digit (mostly sign and
//    exponent bits) keeps hundreds.  Streamed keys keep radix digits: there
//    one CU handles up to 128K keys per pass and the bucket's arithmetic costs
//    more than the pass it saves;
//  * radix passes take 11-bit digits (2048 bins) of the keys in the threshold
//    bin, starting below the bits every key shares, so scores in one binade
//    still spread over the bins instead of piling onto one LDS address;
//  * the passes stop as soon as the threshold bin is taken whole, or holds at
//    most 128 keys (256 when streamed, where a pass costs a full read): those
//    are then gathered in order and ranked against each other, each candidate
//    compared as one 64-bit value (key above inverted position) by 8 lanes (4
//    when streamed), so all 16 waves rank;
//  * each pass has two barriers: after the histogram, and after the per-wave
//    bin totals; sums, prefix sums and min/max inside a wave use DPP row
//    operations and lane reads, not LDS shuffles;
//  * the final pass writes at ordered positions (wave-major, then key order),
//    so the output is deterministic and, among keys equal to the threshold,
//    the first ones in order (the lowest indices) are taken.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "pmqa_internal.h"
#include "wave_ops.h"

namespace pmqa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;  // two bins per thread
constexpr int kSmallKeys = 8;           // keys per thread for rows up to 8192
constexpr int kLargeKeys = 16;          // keys per thread (or per chunk) beyond
constexpr int kCandCap = 256;           // threshold bins this small are ranked directly
constexpr int kCandCapHeld = 128;       // the same, for rows held in registers
constexpr int kHeldPasses = 3;          // value-bucket passes over scores held as floats
// Third word of a raw buffer resource on gfx9-family chips (gfx950): 32-bit
// elements, bounds checked against the record count in bytes.
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u << 1) == 0u) u = 0u;  // -0 and +0 are the same score
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lane_rank(uint64_t mask) {
  // number of set bits of mask below this lane
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// v, opaque to the compiler: comparisons against it are computed where they
// are used instead of 64-bit lane masks being kept in scalar registers across
// a whole pass (which spills them).
__device__ __forceinline__ int fresh(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ uint32_t high_mask(int low_bits) {
  return low_bits >= 32 ? 0u : (~0u << low_bits);
}

struct TopkShared {
  // double-buffered histogram; bins kBins + lane take the keys of positions
  // past the row (rows held as floats), one bin per lane so that their adds
  // do not serialize on one address; never read
  uint32_t hist[2][kBins + 64];
  uint32_t part[kWaves];         // per-wave bin totals / row max
  uint32_t part2[kWaves];        // row min
  uint32_t flags[kWaves];        // per-wave: a non-finite score
  uint32_t col_a[2][kWaves];     // per-wave counts of the final pass, by chunk parity
  uint32_t col_e[2][kWaves];
  alignas(16) uint32_t cand_key[kCandCap];  // keys of the threshold bin, in row order
  alignas(16) int32_t cand_idx[kCandCap];
  // the selection of a row held as floats, in output order; slots kTopkMaxK
  // + lane take the stores of keys that are not selected
  int32_t stage_idx[kTopkMaxK + 64];
  float stage_val[kTopkMaxK + 64];
};

// Keys of one chunk: thread (wave w, lane l) holds key j of the chunk at
// position chunk_base + w*64*KPT + j*64 + l (coalesced per j, wave-major
// order).  With IDX the chunk also carries each key's index in the row (the
// merge selects among candidates that came from anywhere in the row);
// otherwise a key's index is its position.
template <int KPT, bool IDX = false>
struct Chunk {
  uint32_t key[KPT];
  int32_t idx[IDX ? KPT : 1];
  int valid;  // keys j < valid are inside the row

  // The chunk at position c0 of a row of n keys (c0 < n), this thread's keys
  // at c0 + tb + 64 j.  Buffer loads with the chunk's size as their bound:
  // positions past the row read 0 (never used) with no per-key address
  // arithmetic, the 64 j offsets being immediate.
  __device__ __forceinline__ void load(const float* __restrict__ row, int n, int64_t c0, int tb) {
    const __amdgpu_buffer_rsrc_t rs = chunk_rsrc(row + c0, n - c0);
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      key[j] = order_key(__uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, 4 * (tb + 64 * j), 0, 0)));
    set_valid(n, c0 + tb);
  }

  __device__ __forceinline__ void load_idx(const int32_t* __restrict__ ids, int n, int64_t c0,
                                           int tb) {
    static_assert(IDX, "a chunk without indices");
    const __amdgpu_buffer_rsrc_t rs = chunk_rsrc(ids + c0, n - c0);
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      idx[j] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, 4 * (tb + 64 * j), 0, 0);
  }

  // a raw buffer over the chunk's keys (at most kThreads * KPT of them)
  __device__ __forceinline__ static __amdgpu_buffer_rsrc_t chunk_rsrc(const void* p, int64_t left) {
    const int64_t cnt = left < (int64_t)kThreads * KPT ? left : (int64_t)kThreads * KPT;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)(4 * cnt),
                                             kBufferFlags);
  }

  __device__ __forceinline__ void set_valid(int n, int64_t base) {
    // key j is inside the row exactly when j < valid
    const int64_t left = (int64_t)n - base;
    valid = left <= 0 ? 0 : (int)min<int64_t>((left + 63) / 64, KPT);
  }

  // the index of key j, at position pos
  __device__ __forceinline__ int32_t index(int j, int64_t pos) const {
    if constexpr (IDX) return idx[j];
    else return (int32_t)pos;
  }
};

// The float a key encodes (inverse of order_key; -0 comes back as +0).
__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Where a selected key goes: slot in [0, k) of `idx` receives its index in
// the row (a segment starts at position `base` of the row) and, when `val` is
// set, slot of `val` its score (-0 comes back as +0, the same key): a
// segment's top k as candidates of the row's merge.  One type for both uses,
// so that each key layout is compiled once per kernel.
struct SelectOut {
  int32_t* idx;
  float* val;
  int32_t base;
  __device__ __forceinline__ void put(uint32_t slot, int32_t i, uint32_t key) const {
    idx[slot] = base + i;
    if (val) val[slot] = key_value(key);
  }
  __device__ __forceinline__ void put_value(uint32_t slot, int32_t i, float v) const {
    idx[slot] = base + i;
    if (val) val[slot] = v;
  }
};

// A first pass over buckets linear in the score, for rows whose scores are all
// finite: bucket(x) = min(floor((x - lo) * scale), 2047) with lo the row's
// smallest score and scale = 2048 / (largest - smallest).  Every step is a
// monotone non-decreasing function of x (rounding included), so a key in a
// higher bucket is never smaller than one in a lower bucket, and the top k is
// still selected exactly.  Scores spread like the decode logits put a handful
// of keys in the threshold bucket, where the common-prefix radix digit (mostly
// sign and exponent bits) leaves hundreds for a second pass.
struct Buckets {
  bool on = false;
  float lo = 0.f, scale = 0.f;

  __device__ __forceinline__ void setup(uint32_t kmin, uint32_t kmax) {
    const uint32_t kNegInf = 0x007FFFFFu, kPosInf = 0xFF800000u;  // keys of -inf, +inf
    if (!(kmin > kNegInf && kmax < kPosInf && kmin < kmax)) return;
    const float l = key_value(kmin), h = key_value(kmax);
    const float span = h - l;
    const float s = (float)kBins / span;
    if (!(span > 0.f && span <= 3.0e38f && s > 0.f && s <= 3.0e38f)) return;
    on = true;
    lo = l;
    scale = s;
  }

  __device__ __forceinline__ uint32_t of(uint32_t key) const {
    const float x = key_value(key);
    return (uint32_t)__builtin_fminf((x - lo) * scale, (float)(kBins - 1));
  }

  // The bucket of a float as fma(x, scale, -lo * scale), another monotone
  // non-decreasing function of x (fma rounds once), clamped to [0, kBins - 1]
  // by one median (x near lo may come out below 0 by the rounding of
  // -lo * scale).  Rows held as floats bucket every key with this one function.
  __device__ __forceinline__ uint32_t of_value(float x, float off) const {
    return (uint32_t)(int)__builtin_amdgcn_fmed3f(__builtin_fmaf(x, scale, off), 0.f,
                                                  (float)(kBins - 1));
  }
};

// Ranks the nc keys gathered from the threshold bin (sh.cand_key, in row
// order, with their indices in sh.cand_idx) and writes the first `remaining`
// of them at slots first_eq + rank: larger keys first, equal keys in row
// order (their gather order).  A candidate compares as one 64-bit value, its
// key above its inverted position, so that one unsigned comparison orders
// both; the slots from nc to the cap hold key 0, whose values stay below every
// gathered key's (their positions come later).  T consecutive lanes share a
// candidate, each comparing it with kCap / T slots, and add their counts, so
// every wave of the workgroup takes part.
template <int kCap, class Out>
__device__ __forceinline__ void rank_bin_keys(TopkShared& sh, int nc, int remaining,
                                              uint32_t first_eq, const Out& out) {
  constexpr int T = kThreads / kCap;
  constexpr int kPer = kCap / T;
  static_assert(kCap * T == kThreads && kPer % 4 == 0 && (T & (T - 1)) == 0, "rank layout");
  const int tid = threadIdx.x;
  for (int i = nc + tid; i < kCap; i += kThreads) sh.cand_key[i] = 0u;
  __syncthreads();
  const int t = tid / T, part = tid % T;
  const uint64_t mine = ((uint64_t)sh.cand_key[t] << 32) | (uint32_t)~(uint32_t)t;
  uint32_t rank = 0;
#pragma unroll
  for (int u = 0; u < kPer; u += 4) {
    const int i = part * kPer + u;
    const uint4 o = reinterpret_cast<const uint4*>(sh.cand_key)[i >> 2];
    rank += ((((uint64_t)o.x << 32) | (uint32_t)~(uint32_t)i) > mine) ? 1u : 0u;
    rank += ((((uint64_t)o.y << 32) | (uint32_t)~(uint32_t)(i + 1)) > mine) ? 1u : 0u;
    rank += ((((uint64_t)o.z << 32) | (uint32_t)~(uint32_t)(i + 2)) > mine) ? 1u : 0u;
    rank += ((((uint64_t)o.w << 32) | (uint32_t)~(uint32_t)(i + 3)) > mine) ? 1u : 0u;
  }
#pragma unroll
  for (int d = 1; d < T; d <<= 1) rank += (uint32_t)__shfl_xor((int)rank, d);
  if (part == 0 && t < nc && rank < (uint32_t)remaining)
    out.put(first_eq + rank, sh.cand_idx[t], sh.cand_key[t]);
}

// Scores held in registers as floats: thread t holds the KPT consecutive
// scores at positions t*KPT .. t*KPT + KPT - 1 of the row, segment or
// candidate list (with IDX, also each score's index in the row), so that a
// thread-major order of the held scores is their order in the list.  A thread
// whose scores all lie inside the list loads them as 16-byte vectors; the one
// thread that straddles its end loads single scores, those past the end
// reading 0 through the buffer bound (never used).
template <int KPT, bool IDX>
struct Held {
  static_assert(KPT % 4 == 0, "16-byte loads");
  float x[KPT];
  int32_t idx[IDX ? KPT : 1];

  __device__ __forceinline__ static void load_words(const void* p, int n, int tb,
                                                    uint32_t (&w)[KPT]) {
    const __amdgpu_buffer_rsrc_t rs = Chunk<KPT, IDX>::chunk_rsrc(p, n);
    if (tb + KPT <= n) {
#pragma unroll
      for (int q = 0; q < KPT / 4; ++q) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, 4 * (tb + 4 * q), 0, 0);
        w[4 * q] = v[0];
        w[4 * q + 1] = v[1];
        w[4 * q + 2] = v[2];
        w[4 * q + 3] = v[3];
      }
    } else {
#pragma unroll
      for (int j = 0; j < KPT; ++j) w[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * (tb + j), 0, 0);
    }
  }

  __device__ __forceinline__ void load(const float* __restrict__ p, int n, int tb) {
    uint32_t w[KPT];
    load_words(p, n, tb, w);
#pragma unroll
    for (int j = 0; j < KPT; ++j) x[j] = __uint_as_float(w[j]);
  }

  __device__ __forceinline__ void load_idx(const int32_t* __restrict__ ids, int n, int tb) {
    static_assert(IDX, "scores without indices");
    uint32_t w[KPT];
    load_words(ids, n, tb, w);
#pragma unroll
    for (int j = 0; j < KPT; ++j) idx[j] = (int32_t)w[j];
  }

  __device__ __forceinline__ int32_t index(int j, int tb) const {
    if constexpr (IDX) return idx[j];
    else return tb + j;
  }
};

// The top k of n > k scores held as floats, by value buckets: buckets between
// the smallest and largest score (Buckets), the threshold bucket found from
// the histogram and, while it holds more than 128 scores that are not all
// taken, its value range cut into buckets again (at most kHeldPasses passes;
// each cut is monotone in the score too), then every score above it placed
// and the threshold bucket's scores ranked against each other.  Every phase
// is a fixed number of instructions per held score, with no per-score
// branches or ballots (the costs that dominated: one CU issues the whole
// row's instructions):
//  * positions past the list get a negative bucket, which the histogram
//    counts in an extra bin per lane and every comparison (signed) puts below
//    all buckets;
//  * each thread counts its scores above and in the threshold bucket, one
//    packed prefix sum over the wave and one over the waves give each score's
//    slot, and the selection is staged in LDS, then stored in order with
//    coalesced stores;
//  * the threshold bucket's scores (at most 128) are ranked one per lane, each
//    compared as one 64-bit value (key above inverted index), so equal scores
//    take the lowest indices, and stored at their slots while the other
//    waves copy the staged scores above the bucket.
// Returns false, having written nothing, when the row needs radix passes: a
// non-finite score, all scores equal, or more than 128 scores in a threshold
// bucket it cannot take whole after the last pass (or whose range is too
// narrow to cut).  The output is deterministic.
template <int KPT, bool IDX, bool VALS>
__device__ __forceinline__ bool select_held(int n, int k, const SelectOut& out, TopkShared& sh,
                                            const Held<KPT, IDX>& hd) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int tb = tid * KPT;                      // position of the thread's first score
  const bool full = (wave + 1) * 64 * KPT <= n;  // every position of the wave is inside

  // ---- the largest and smallest score (a non-finite one shows in the sum) ----
  float mx = -__builtin_inff(), mn = __builtin_inff(), sum = 0.f;
  auto extremes = [&](auto all) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (decltype(all)::value || tb + j < n) {
        mx = __builtin_fmaxf(mx, hd.x[j]);
        mn = __builtin_fminf(mn, hd.x[j]);
        sum += hd.x[j];
      }
    }
  };
  if (full) extremes(std::true_type{});
  else extremes(std::false_type{});
  const uint32_t wmax = wave_max(order_key(mx));
  const uint32_t wmin = wave_min(order_key(mn));
  const bool wbad = __ballot(!__builtin_isfinite(sum)) != 0;
  if (lane == 0) {
    sh.part[wave] = wmax;
    sh.part2[wave] = wmin;
    sh.flags[wave] = wbad ? 1u : 0u;
  }
  reinterpret_cast<uint2*>(sh.hist[0])[tid] = uint2{0u, 0u};
  __syncthreads();
  const uint32_t kmax = lane_of(row_max(sh.part[lane & 15]), 0);
  const uint32_t kmin = lane_of(row_min(sh.part2[lane & 15]), 0);
  const bool bad = __ballot(lane < 16 && sh.flags[lane] != 0u) != 0;
  Buckets bk;
  if (!bad) bk.setup(kmin, kmax);
  if (!bk.on) {
    __syncthreads();  // the radix passes reuse what was read above
    return false;
  }

  // ---- buckets, refined until the bucket of the k-th score is small ----
  // kb[j]: the score's bucket among the current candidates (pass 0: every
  // score), kAbove / kBelow once an earlier pass put it above / below them
  // (positions past the list start below); signed comparisons order all three
  constexpr uint32_t kAbove = 0x7FFFFFFFu, kBelow = ~0u;
  float lo = bk.lo, scale = bk.scale;
  float off = -lo * scale;
  uint32_t kb[KPT];
  auto bucket_all = [&](auto all) {
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      kb[j] = decltype(all)::value || tb + j < n ? bk.of_value(hd.x[j], off) : kBelow;
  };
  if (full) bucket_all(std::true_type{});
  else bucket_all(std::false_type{});
  const uint32_t spare = (uint32_t)(kBins + lane);
  uint32_t above = 0;              // scores above the candidates, from earlier passes
  uint32_t need = (uint32_t)k;     // rank of the k-th score among the candidates
  uint32_t bs, first_eq, cnt, remaining;
  for (int pass = 0;; ++pass) {
    uint32_t* h = sh.hist[pass & 1];
#pragma unroll
    for (int j = 0; j < KPT; ++j) atomicAdd(&h[min(kb[j], spare)], 1u);
    __syncthreads();
    // the other buffer, for a next pass (its last reads, two passes back,
    // are behind the barrier above)
    reinterpret_cast<uint2*>(sh.hist[(pass & 1) ^ 1])[tid] = uint2{0u, 0u};

    // ---- the bucket holding the need-th candidate ----
    const uint2 mine = reinterpret_cast<const uint2*>(h)[tid];  // buckets 2*tid, 2*tid+1
    const uint32_t wtot = wave_sum(mine.x + mine.y);
    if (lane == 0) sh.part[wave] = wtot;
    __syncthreads();
    const uint32_t pv = sh.part[lane & 15];
    const uint32_t pw = row_prefix(pv);
    const uint32_t t16 = lane_of(pw, 15);
    const uint32_t above_w = t16 - pw;  // candidates in higher wave spans
    const uint64_t fw = __ballot(lane < 16 && above_w < need && above_w + pv >= need);
    const int ws = min((int)__builtin_ctzll(fw), kWaves - 1);
    const uint32_t base_above = lane_of(above_w, ws);
    const uint2 hb = reinterpret_cast<const uint2*>(h)[ws * 64 + lane];
    const uint32_t s2 = hb.x + hb.y;
    uint32_t t_w;
    const uint32_t ps = wave_prefix(s2, lane, t_w);
    const uint32_t above_l = base_above + (t_w - ps);
    const uint64_t fl = __ballot(above_l < need && above_l + s2 >= need);
    const int ls = min((int)__builtin_ctzll(fl), 63);
    const uint32_t a = lane_of(above_l, ls);
    const uint32_t h0 = lane_of(hb.x, ls), h1 = lane_of(hb.y, ls);
    const uint32_t bin_hi = 2u * (uint32_t)(ws * 64 + ls) + 1u;
    uint32_t fe;
    if (a + h1 >= need) {
      bs = bin_hi; fe = a; cnt = h1;
    } else {
      bs = bin_hi - 1u; fe = a + h1; cnt = h0;
    }
    remaining = need - fe;  // taken from the threshold bucket
    first_eq = above + fe;
    if (cnt == remaining || cnt <= (uint32_t)kCandCapHeld) break;
    // too many candidates share the bucket: the next pass splits that
    // bucket's value range into kBins buckets (again monotone in the score,
    // the clamp included, so still exact), the other scores settled
    const float lo2 = lo + (float)bs / scale;
    const float scale2 = scale * (float)kBins;
    if (pass + 1 == kHeldPasses || !(scale2 <= 3.0e38f)) {
      __syncthreads();  // the radix passes reuse what was read above
      return false;
    }
    const float off2 = -lo2 * scale2;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const uint32_t sub = (uint32_t)(int)__builtin_amdgcn_fmed3f(
          __builtin_fmaf(hd.x[j], scale2, off2), 0.f, (float)(kBins - 1));
      kb[j] = kb[j] == bs ? sub : ((int)kb[j] > (int)bs ? kAbove : kBelow);
    }
    above = first_eq;
    need = remaining;
    lo = lo2;
    scale = scale2;
  }
  const bool whole = cnt == remaining;

  // ---- each score's slot: above the bucket [0, first_eq), in it after ----
  uint32_t ca = 0, ce = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    ca += (int)kb[j] > (int)bs ? 1u : 0u;
    ce += kb[j] == bs ? 1u : 0u;
  }
  const uint32_t pk = ca | (ce << 16);  // both counts stay below 2^16
  uint32_t wpk;
  const uint32_t incl = wave_prefix(pk, lane, wpk);
  if (lane == 0) sh.col_a[0][wave] = wpk;
  const uint32_t nc4 = (cnt + 3u) & ~3u;
  if (!whole && (uint32_t)tid >= cnt && (uint32_t)tid < nc4) {
    sh.cand_key[tid] = 0u;  // below every candidate's key
    sh.cand_idx[tid] = 0;
  }
  __syncthreads();
  const uint32_t wincl = lane_of(row_prefix(sh.col_a[0][lane & 15]), wave);
  const uint32_t pos = (wincl - wpk) + (incl - pk);
  uint32_t pa = pos & 0xFFFFu, pe = pos >> 16;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const bool up = (int)kb[j] > (int)bs;
    const int32_t ix = hd.index(j, tb);
    const uint32_t slot = up ? pa : (uint32_t)(kTopkMaxK + lane);
    sh.stage_idx[slot] = ix;
    if constexpr (VALS) sh.stage_val[slot] = hd.x[j];
    pa += up ? 1u : 0u;
    if (kb[j] == bs) {
      if (whole) {
        sh.stage_idx[first_eq + pe] = ix;
        if constexpr (VALS) sh.stage_val[first_eq + pe] = hd.x[j];
      } else {
        sh.cand_key[pe] = order_key(hd.x[j]);
        sh.cand_idx[pe] = ix;
      }
      ++pe;
    }
  }
  __syncthreads();

  // ---- rank the threshold bucket's scores (score desc, index asc) ----
  if (!whole && (uint32_t)tid < cnt) {
    const uint64_t me = ((uint64_t)sh.cand_key[tid] << 32) | (uint32_t)~(uint32_t)sh.cand_idx[tid];
    uint32_t rank = 0;
    for (uint32_t i = 0; i < nc4; i += 4) {
      const uint4 kk = reinterpret_cast<const uint4*>(sh.cand_key)[i >> 2];
      const uint4 ii = reinterpret_cast<const uint4*>(sh.cand_idx)[i >> 2];
      rank += ((((uint64_t)kk.x << 32) | (uint32_t)~ii.x) > me) ? 1u : 0u;
      rank += ((((uint64_t)kk.y << 32) | (uint32_t)~ii.y) > me) ? 1u : 0u;
      rank += ((((uint64_t)kk.z << 32) | (uint32_t)~ii.z) > me) ? 1u : 0u;
      rank += ((((uint64_t)kk.w << 32) | (uint32_t)~ii.w) > me) ? 1u : 0u;
    }
    // straight to its output slot: no barrier between the ranking and the
    // copy below, which the other waves start at once (decode top-k 5.29 ->
    // 5.09 us, interleaved)
    if (rank < remaining)
      out.put_value(first_eq + rank, sh.cand_idx[tid], VALS ? key_value(sh.cand_key[tid]) : 0.f);
  }

  // ---- the staged selection: the scores above the threshold bucket, or all
  // k when that bucket was taken whole (complete since the barrier above) ----
  const uint32_t staged = whole ? (uint32_t)k : first_eq;
  for (uint32_t i = tid; i < staged; i += kThreads)
    out.put_value(i, sh.stage_idx[i], VALS ? sh.stage_val[i] : 0.f);
  return true;
}

// Selects the row's top k; `ch` holds the row's first chunk (already loaded).
//
// Keys are narrowed in passes until the bin holding the k-th largest key is
// resolved.  On a row held in registers the first pass may bucket by value
// (Buckets); every later pass takes the next radix digit of the keys that lie
// in the threshold bucket and match the prefix fixed so far.  A key is then
// above the threshold when its bucket is higher, or its bucket is the
// threshold bucket and its fixed bits are higher; it is in the threshold bin
// when both are equal.
template <int KPT, bool STREAM, bool IDX, class Out>
__device__ __forceinline__ void select_row(const float* __restrict__ row, int n, int k,
                                           const Out& out, TopkShared& sh,
                                           Chunk<KPT, IDX>& ch) {
  static_assert(!(STREAM && IDX), "streamed keys carry no indices");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  constexpr int kChunk = kThreads * KPT;
  const int n_chunks = STREAM ? (n + kChunk - 1) / kChunk : 1;
  const int thread_base = wave * 64 * KPT + lane;

  // Runs body(chunk, c) over the row's chunks in order; `ch` holds chunk 0 on
  // entry.  A streamed row alternates two register chunks so that the next
  // chunk's loads are in flight while the current one is processed (a row of
  // 128K keys is 8 chunks per pass, each load a full memory latency).
  Chunk<KPT, IDX> nx;
  auto for_chunks = [&](auto&& body) {
    if constexpr (!STREAM) {
      body(ch, 0);
    } else {
      for (int c = 0; c < n_chunks; c += 2) {
        if (c + 1 < n_chunks) nx.load(row, n, (int64_t)(c + 1) * kChunk, thread_base);
        body(ch, c);
        if (c + 2 < n_chunks) ch.load(row, n, (int64_t)(c + 2) * kChunk, thread_base);
        if (c + 1 < n_chunks) body(nx, c + 1);
      }
    }
  };
  // a streamed row's later passes start again from chunk 0
  auto rewind = [&]() {
    if constexpr (STREAM) ch.load(row, n, 0, thread_base);
  };

  // ---- the row's largest and smallest key ----
  uint32_t kmax = 0u, kmin = ~0u;
  for_chunks([&](const Chunk<KPT, IDX>& cc, int) {
    const int vld = fresh(cc.valid);
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (j < vld) {
        kmax = max(kmax, cc.key[j]);
        kmin = min(kmin, cc.key[j]);
      }
    }
  });
  kmax = wave_max(kmax);
  kmin = wave_min(kmin);
  if (lane == 0) {
    sh.part[wave] = kmax;
    sh.part2[wave] = kmin;
  }
  reinterpret_cast<uint2*>(sh.hist[0])[tid] = uint2{0u, 0u};
  __syncthreads();
  kmax = lane_of(row_max(sh.part[lane & 15]), 0);
  kmin = lane_of(row_min(sh.part2[lane & 15]), 0);

  // bits every key shares are fixed from the start
  int bits_left = kmax == kmin ? 0 : 32 - __builtin_clz(kmax ^ kmin);
  uint32_t mask = high_mask(bits_left);
  uint32_t prefix = kmax & mask;
  const uint32_t mask0 = mask;
  int remaining = k;  // rank of the k-th key among the keys in the threshold bin
  bool whole_bin = false;
  int buf = 0;

  // value buckets of the held keys (all 0 when the row takes radix passes only)
  Buckets bk;
  if (!STREAM) bk.setup(kmin, kmax);
  uint32_t kb[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) kb[j] = bk.on ? bk.of(ch.key[j]) : 0u;
  uint32_t bstar = 0u;  // the threshold bucket
  bool bucket_pass = bk.on;

  // ---- passes ----
  while (bits_left > 0) {
    const int width = min(kDigitBits, bits_left);
    const int shift = bits_left - width;
    const uint32_t dmask = (1u << width) - 1u;
    uint32_t* h = sh.hist[buf];
    rewind();
    for_chunks([&](const Chunk<KPT, IDX>& cc, int) {
      const int vld = fresh(cc.valid);
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const uint32_t key = cc.key[j];
        if (bucket_pass) {
          if (j < vld) atomicAdd(&h[kb[j]], 1u);
        } else if (j < vld && kb[j] == bstar && (key & mask) == prefix) {
          atomicAdd(&h[(key >> shift) & dmask], 1u);
        }
      }
    });
    __syncthreads();
    // the other buffer was last read before this barrier: clear it for the
    // next pass
    reinterpret_cast<uint2*>(sh.hist[buf ^ 1])[tid] = uint2{0u, 0u};
    const uint2 mine = reinterpret_cast<const uint2*>(h)[tid];  // bins 2*tid, 2*tid+1
    const uint32_t wtot = wave_sum(mine.x + mine.y);
    if (lane == 0) sh.part[wave] = wtot;
    __syncthreads();

    // every wave finds the wave span, then the bin, holding the k-th key
    const uint32_t pv = sh.part[lane & 15];
    const uint32_t pw = row_prefix(pv);  // every row holds waves 0..15
    const uint32_t t16 = lane_of(pw, 15);
    const uint32_t above_w = t16 - pw;  // keys in higher wave spans
    const uint64_t fw = __ballot(lane < 16 && above_w < (uint32_t)remaining &&
                                 above_w + pv >= (uint32_t)remaining);
    const int ws = min((int)__builtin_ctzll(fw), kWaves - 1);
    const uint32_t base_above = lane_of(above_w, ws);

    const uint2 hb = reinterpret_cast<const uint2*>(h)[ws * 64 + lane];
    const uint32_t s = hb.x + hb.y;
    uint32_t t_w;
    const uint32_t ps = wave_prefix(s, lane, t_w);
    const uint32_t above_l = base_above + (t_w - ps);
    const uint64_t fl = __ballot(above_l < (uint32_t)remaining &&
                                 above_l + s >= (uint32_t)remaining);
    const int ls = min((int)__builtin_ctzll(fl), 63);
    const uint32_t a = lane_of(above_l, ls);
    const uint32_t h0 = lane_of(hb.x, ls), h1 = lane_of(hb.y, ls);
    const uint32_t bin_hi = 2u * (uint32_t)(ws * 64 + ls) + 1u;
    uint32_t digit, above, cnt;
    if (a + h1 >= (uint32_t)remaining) {
      digit = bin_hi; above = a; cnt = h1;
    } else {
      digit = bin_hi - 1u; above = a + h1; cnt = h0;
    }
    remaining -= (int)above;
    if (bucket_pass) {
      bstar = digit;
      bucket_pass = false;
    } else {
      prefix |= digit << shift;
      mask |= dmask << shift;
      bits_left = shift;
    }
    buf ^= 1;
    if (cnt == (uint32_t)remaining) {
      whole_bin = true;  // every key of this bin is in the top k
      break;
    }
    // a bin this small is ranked directly instead of refined by another
    // pass: ranking costs O(cnt^2) LDS reads, so rows held in registers (a
    // pass costs ~1 us of barriers and LDS round trips) take it only for
    // small bins, rows that stream from memory (a pass re-reads the row) for
    // larger ones
    if (bits_left > 0 && cnt <= (uint32_t)(STREAM ? kCandCap : kCandCapHeld)) break;
  }
  // the threshold bin is ranked directly unless it is taken whole or every
  // bit is fixed (its keys are then equal: row order decides)
  const bool rank_bin = !whole_bin && bits_left > 0;

  // ---- write the selection ----
  // keys above the threshold fill slots [0, k - remaining).  Keys in the
  // threshold bin take slots k - remaining + rank while rank < remaining:
  // rank in row order when the bin is taken whole or its keys are equal;
  // otherwise the bin's keys are first gathered (in row order) and each one's
  // rank among them computed below.  When the value buckets resolved the
  // threshold (no radix digit fixed after them) every key shares the fixed
  // bits, so a key's bucket alone classifies it.
  const uint32_t first_eq = (uint32_t)(k - remaining);
  const bool by_bucket = bk.on && mask == mask0;
  uint32_t run_a = 0, run_e = 0;
  auto write_pass = [&](auto fast) {
    // class of key j: above the threshold bin, or in it
    auto above = [&](const Chunk<KPT, IDX>& cc, int j, uint32_t bs, uint32_t m, uint32_t pf) {
      if constexpr (decltype(fast)::value) return kb[j] > bs;
      else return kb[j] > bs || (kb[j] == bs && (cc.key[j] & m) > pf);
    };
    auto inbin = [&](const Chunk<KPT, IDX>& cc, int j, uint32_t bs, uint32_t m, uint32_t pf) {
      if constexpr (decltype(fast)::value) return kb[j] == bs;
      else return kb[j] == bs && (cc.key[j] & m) == pf;
    };
    rewind();
    for_chunks([&](const Chunk<KPT, IDX>& cc, int c) {
      uint32_t ca = 0, ce = 0;
      const int vld = fresh(cc.valid);
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const bool ok = j < vld;
        ca += (uint32_t)__popcll(__ballot(ok && above(cc, j, bstar, mask, prefix)));
        ce += (uint32_t)__popcll(__ballot(ok && inbin(cc, j, bstar, mask, prefix)));
      }
      if (lane == 0) {
        sh.col_a[c & 1][wave] = ca;
        sh.col_e[c & 1][wave] = ce;
      }
      __syncthreads();
      const uint32_t pa = row_prefix(sh.col_a[c & 1][lane & 15]);
      const uint32_t pe = row_prefix(sh.col_e[c & 1][lane & 15]);
      const uint32_t ta = lane_of(pa, 15), te = lane_of(pe, 15);
      uint32_t off_a = run_a + lane_of(pa, wave) - ca;  // exclusive over waves
      uint32_t off_e = run_e + lane_of(pe, wave) - ce;
      const int64_t base = (int64_t)c * kChunk + thread_base;
      // the threshold passes through an empty asm statement, so that the
      // classes below are computed again instead of the first loop's 2 * KPT
      // ballots being kept live across the barrier
      uint32_t bs = bstar, m = mask, pf = prefix;
      asm volatile("" : "+v"(bs), "+v"(m), "+v"(pf));
      const int vld2 = fresh(cc.valid);
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const bool ok = j < vld2;
        const bool fa = ok && above(cc, j, bs, m, pf);
        const bool fe = ok && inbin(cc, j, bs, m, pf);
        const uint64_t ma = __ballot(fa);
        const uint64_t me = __ballot(fe);
        const int32_t idx = cc.index(j, base + 64 * j);
        if (fa) out.put(off_a + (uint32_t)lane_rank(ma), idx, cc.key[j]);
        if (fe) {
          const uint32_t rank = off_e + (uint32_t)lane_rank(me);
          if (rank_bin) {
            sh.cand_key[rank] = cc.key[j];
            sh.cand_idx[rank] = idx;
          } else if (rank < (uint32_t)remaining) {
            out.put(first_eq + rank, idx, cc.key[j]);
          }
        }
        off_a += (uint32_t)__popcll(ma);
        off_e += (uint32_t)__popcll(me);
      }
      run_a += ta;
      run_e += te;
    });
  };
  if (by_bucket) write_pass(std::true_type{});
  else write_pass(std::false_type{});
  if (!rank_bin) return;
  rank_bin_keys<STREAM ? kCandCap : kCandCapHeld>(sh, (int)run_e, remaining, first_eq, out);
}

// The top-k's parameters inside a kernel, built from its scalar arguments.
struct TopkArgs {
  const float* logits;
  int64_t row_stride;
  const int32_t* ctx;
  int32_t next_n;
  int32_t k;
  int32_t* out_idx;
  float* cand_val;   // workspace: [rows, seg_grid, k] candidate scores
  int32_t* cand_idx;  // workspace: [rows, seg_grid, k] candidate indices
  int32_t seg_grid;   // segments per row in the stage-1 grid (1: no split)
};

// Visible scores of row r (a row never reads past its stride).
__device__ __forceinline__ int row_len(const int32_t* __restrict__ ctx_lens, int r, int next_n,
                                       int64_t row_stride) {
  const int b = r / next_n;
  const int j = r - b * next_n;
  const int ctx = max(ctx_lens[b], 0);
  const int n = min(max(ctx - next_n + j + 1, 0), ctx);
  return (int64_t)n > row_stride ? (int)row_stride : n;
}

// Selects n > k scores held in registers (with IDX, candidates with their
// row indices at `ids`): value-bucket passes when they resolve the row, else the
// radix passes over the same scores as keys.  VALS: `out` takes the selected
// scores too (a segment's candidates), else only their indices.
template <int KPT, bool IDX, bool VALS>
__device__ __forceinline__ void held_or_radix(const float* __restrict__ vals,
                                              const int32_t* __restrict__ ids, int n, int k,
                                              const SelectOut& out, TopkShared& sh) {
  {
    Held<KPT, IDX> hd;
    hd.load(vals, n, (int)threadIdx.x * KPT);
    if constexpr (IDX) hd.load_idx(ids, n, (int)threadIdx.x * KPT);
    if (select_held<KPT, IDX, VALS>(n, k, out, sh, hd)) return;
  }
  // the radix passes take the scores again, in their own layout (a rare path:
  // a non-finite score, all scores equal, or many scores in one bucket)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tb = wave * 64 * KPT + lane;
  Chunk<KPT, IDX> ch;
  ch.load(vals, n, 0, tb);
  if constexpr (IDX) ch.load_idx(ids, n, 0, tb);
  select_row<KPT, false>(vals, n, k, out, sh, ch);
}

// Selects n keys at `row` (positions 0..n-1) into `out`, with the register
// layout their count calls for.  Without STREAM the caller guarantees n <=
// kTopkSegmentKeys (the keys fit the registers).  Without WIDE_HELD, lists of
// more than 8192 keys skip the value-bucket select on floats (its 16 floats and
// 16 buckets a thread would take the register budget of two workgroups per
// CU, which the split grid needs) and take the radix passes on keys.
template <bool STREAM, bool WIDE_HELD = true, bool VALS = false>
__device__ __forceinline__ void select_keys(const float* __restrict__ row, int n, int k,
                                            const SelectOut& out, TopkShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (n <= kThreads * kSmallKeys) {
    held_or_radix<kSmallKeys, false, VALS>(row, nullptr, n, k, out, sh);
  } else if (WIDE_HELD && (!STREAM || n <= kThreads * kLargeKeys)) {
    held_or_radix<kLargeKeys, false, VALS>(row, nullptr, n, k, out, sh);
  } else if (!STREAM || n <= kThreads * kLargeKeys) {
    Chunk<kLargeKeys> ch;
    ch.load(row, n, 0, wave * 64 * kLargeKeys + lane);
    select_row<kLargeKeys, false>(row, n, k, out, sh, ch);
  } else {
    Chunk<kLargeKeys> ch;
    ch.load(row, n, 0, wave * 64 * kLargeKeys + lane);
    select_row<kLargeKeys, true>(row, n, k, out, sh, ch);
  }
}

// Stage 1.  Workgroup (r, s) selects segment s of row r: the whole row when
// it has one segment (the result goes straight to out_idx), otherwise k
// candidates of the segment into the workspace.  Segments hold at most
// kTopkSegmentKeys keys, except that STREAM (a grid of one segment per row,
// the workspace too small to split anything, on rows the stride allows to be
// longer) selects any row whole, streaming it through the registers.  With
// more than one segment per row, a row that would need more segments than
// the grid has is left to the merge launch, which selects it whole, so the
// stage keeps only the register-resident layouts.  SPLIT: the grid may split
// rows (its segments stage their candidates' scores); otherwise every row
// is one segment and only indices are staged.  WIDE (split grids): segments
// of more than 8192 scores also take the value-bucket select on floats.
template <bool STREAM, bool SPLIT, bool WIDE = false>
__device__ __forceinline__ void stage1(const TopkArgs& a, TopkShared& sh) {
  const int r = blockIdx.x;
  const int s = blockIdx.y;
  const int n = row_len(a.ctx, r, a.next_n, a.row_stride);
  const int k = a.k;
  int32_t* out = a.out_idx + (int64_t)r * k;
  if (n <= k) {
    if (s == 0)
      for (int i = threadIdx.x; i < k; i += kThreads) out[i] = i < n ? i : -1;
    return;
  }
  const int grid = a.seg_grid;  // the launch grid's second dimension
  const int nseg = topk_row_segments(n, grid);
  if (nseg == 0) return;  // selected whole by the merge launch
  if (s >= nseg) return;
  // a row of one segment selects straight into out_idx; otherwise nearly
  // equal segments (each holds more than k scores) select k candidates each
  // into the workspace
  const int64_t s0 = (int64_t)n * s / nseg, s1 = (int64_t)n * (s + 1) / nseg;
  const int64_t slot = ((int64_t)r * grid + s) * k;
  const float* seg = a.logits + (int64_t)r * a.row_stride + s0;
  if constexpr (SPLIT) {
    // one instantiation for both cases (its register budget is that of two
    // workgroups per CU): a row of one segment stages values it never stores
    const SelectOut so = nseg == 1 ? SelectOut{out, nullptr, 0}
                                   : SelectOut{a.cand_idx + slot, a.cand_val + slot, (int32_t)s0};
    select_keys<false, WIDE, true>(seg, (int)(s1 - s0), k, so, sh);
  } else {
    select_keys<STREAM, true, false>(seg, n, k, SelectOut{out, nullptr, 0}, sh);
  }
}

// Stage 1 for grids of one segment per row.  Every parameter is a scalar
// argument; the dispatch preloads the first 14 dwords into SGPRs (all the
// user SGPRs left beside the argument pointer; the build asks for up to 16),
// i.e. everything but the candidate indices, which only the last step of a
// split row writes.  So no wave waits for a scalar load of its argument
// block, or of the grid size, before its first load.  Rows here are never
// split, so no candidate values are staged.
template <bool STREAM>
__global__ __launch_bounds__(kThreads) void topk_kernel(
    const float* __restrict__ logits, int64_t row_stride, const int32_t* __restrict__ ctx,
    int32_t next_n, int32_t k, int32_t seg_grid, int32_t* __restrict__ out_idx,
    float* __restrict__ cand_val, int32_t* __restrict__ cand_idx) {
  __shared__ TopkShared sh;
  stage1<STREAM, false>(TopkArgs{logits, row_stride, ctx, next_n, k, out_idx, cand_val, cand_idx,
                                 seg_grid},
                        sh);
}

// Stage 1 for grids that split rows: many workgroups, so two should share a
// CU.  The register-resident select needs 52 VGPRs (eight waves per SIMD fit)
// but about 93 SGPRs, and on gfx950 a second 1024-thread workgroup then does
// not fit a CU (measured: one workgroup per CU at 93-97 SGPRs, two at 80 and
// below), so the compiler is held to 80 SGPRs (it moves the rest to VGPR
// lanes).  Measured on the MTP, small-pages and long-context workloads: 15%
// less time than one workgroup per CU.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_num_sgpr(80)))
void topk_split_kernel(const float* __restrict__ logits, int64_t row_stride,
                       const int32_t* __restrict__ ctx, int32_t next_n, int32_t k,
                       int32_t seg_grid, int32_t* __restrict__ out_idx,
                       float* __restrict__ cand_val, int32_t* __restrict__ cand_idx) {
  __shared__ TopkShared sh;
  stage1<false, true>(TopkArgs{logits, row_stride, ctx, next_n, k, out_idx, cand_val, cand_idx,
                               seg_grid},
                      sh);
}

// Stage 1 for split grids whose segments may hold more than 8192 scores
// (rows longer than 8192 times the grid's segments): such segments take the
// value-bucket select on 16 floats a thread, which leaves room for one
// workgroup per CU, instead of the radix passes (measured on 65K-131K-score
// rows in 8 segments: a segment's workgroup took 11-25 us in the radix
// passes).
__global__ __launch_bounds__(kThreads) void topk_split_wide_kernel(
    const float* __restrict__ logits, int64_t row_stride, const int32_t* __restrict__ ctx,
    int32_t next_n, int32_t k, int32_t seg_grid, int32_t* __restrict__ out_idx,
    float* __restrict__ cand_val, int32_t* __restrict__ cand_idx) {
  __shared__ TopkShared sh;
  stage1<false, true, true>(TopkArgs{logits, row_stride, ctx, next_n, k, out_idx, cand_val,
                                     cand_idx, seg_grid},
                            sh);
}

// Stage 2 (launched when the grid has more than one segment per row).
// Workgroup r selects the top k of row r among its segments' nseg * k
// candidates (at most kTopkMergeKeys: the host caps the segments), held in
// registers with their indices; or, for a row longer than the grid's
// segments can hold, the whole row, streamed.  Rows of one segment or none
// were finished in stage 1.  SMALL (seg_grid * k <= 8192, so every row has
// at most 8192 candidates): only the 8-a-thread layouts are compiled, a row
// left whole streamed 8 keys a thread at a time, so that the registers leave
// room for two workgroups per CU.
template <bool SMALL>
__device__ __forceinline__ void merge_row(const TopkArgs& a, TopkShared& sh) {
  const int r = blockIdx.x;
  const int n = row_len(a.ctx, r, a.next_n, a.row_stride);
  const int k = a.k;
  if (n <= k) return;
  const int nseg = topk_row_segments(n, a.seg_grid);
  const SelectOut out{a.out_idx + (int64_t)r * k, nullptr, 0};
  if (nseg == 0) {
    const float* row = a.logits + (int64_t)r * a.row_stride;
    if constexpr (SMALL) {
      // streamed 8 keys a thread at a time (the registers of this kernel)
      const int tb = (int)(threadIdx.x >> 6) * 64 * kSmallKeys + (int)(threadIdx.x & 63);
      Chunk<kSmallKeys> ch;
      ch.load(row, n, 0, tb);
      select_row<kSmallKeys, true>(row, n, k, out, sh, ch);
    } else {
      select_keys<true>(row, n, k, out, sh);
    }
    return;
  }
  if (nseg < 2) return;
  const int m = nseg * k;
  const int64_t slot = (int64_t)r * a.seg_grid * k;
  const float* cv = a.cand_val + slot;
  const int32_t* ci = a.cand_idx + slot;
  if (m <= kThreads * kSmallKeys) {
    held_or_radix<kSmallKeys, true, false>(cv, ci, m, k, out, sh);
  } else if constexpr (!SMALL) {
    held_or_radix<kLargeKeys, true, false>(cv, ci, m, k, out, sh);
  }
}

__global__ __launch_bounds__(kThreads) void topk_merge_kernel(
    const float* __restrict__ logits, int64_t row_stride, const int32_t* __restrict__ ctx,
    int32_t next_n, int32_t k, int32_t seg_grid, int32_t* __restrict__ out_idx,
    float* __restrict__ cand_val, int32_t* __restrict__ cand_idx) {
  __shared__ TopkShared sh;
  merge_row<false>(TopkArgs{logits, row_stride, ctx, next_n, k, out_idx, cand_val, cand_idx,
                            seg_grid},
                   sh);
}

// The merge of grids whose rows have at most 8192 candidates each, held to
// 80 SGPRs as the split stage is, so that two workgroups share a CU.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_num_sgpr(80), amdgpu_waves_per_eu(8)))
void topk_merge_small_kernel(const float* __restrict__ logits, int64_t row_stride,
                             const int32_t* __restrict__ ctx, int32_t next_n, int32_t k,
                             int32_t seg_grid, int32_t* __restrict__ out_idx,
                             float* __restrict__ cand_val, int32_t* __restrict__ cand_idx) {
  __shared__ TopkShared sh;
  merge_row<true>(TopkArgs{logits, row_stride, ctx, next_n, k, out_idx, cand_val, cand_idx,
                           seg_grid},
                  sh);
}

}  // namespace

static_assert(kTopkSegmentKeys == kThreads * kLargeKeys, "a segment is held in registers");
static_assert(kTopkMergeKeys == kThreads * kLargeKeys, "the merge is held in registers");

// Scratch of the allocation-free top-k: the candidates of split rows, in a
// fixed device array (one copy per GPU, held until the process ends), for
// callers that cannot allocate.  Calls on one GPU share it; nothing in it has
// to start at zero (a call writes every candidate it reads).
static __device__ __align__(256) uint8_t scratch[kTopkScratchBytes];

hipError_t topk_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    // the array's name is a host-side stand-in: its device address (this
    // device's copy) comes from the runtime, once per device
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_topk(const TopkParams& p, const LaunchTiming& tm, hipStream_t stream) {
  const uint32_t rows = (uint32_t)p.batch * (uint32_t)p.next_n;
  const dim3 grid(rows, (uint32_t)p.seg_grid);
  const bool merge = p.seg_grid > 1;
  // with one segment per row, rows longer than the registers hold are
  // streamed by stage 1 itself (when the stride allows such rows); with more,
  // the merge launch takes them
  const int64_t longest = p.row_stride < INT32_MAX ? p.row_stride : INT32_MAX;
  const bool stream_keys = !merge && longest > kTopkSegmentKeys;
  // Which split-stage kernel (both select any segment exactly): segments of
  // more than 8192 scores come from rows longer than 8192 per segment of the
  // grid.  A grid narrower than the merge allows was bounded by the caller's
  // workspace, sized for the caller's longest row, so its segments are
  // expected to hold at most 8192 scores (the two-per-CU kernel); a grid at
  // the merge's limit on rows whose stride allows longer segments takes the
  // kernel that holds 16 floats a thread.
  const int64_t merge_cap = kTopkMergeKeys / p.k;
  const bool wide = merge && p.seg_grid >= merge_cap &&
                    (longest + kTopkSplitKeys - 1) / kTopkSplitKeys > p.seg_grid;
  // a merge of at most 8192 candidates a row fits two workgroups per CU
  const bool small_merge = (int64_t)p.seg_grid * p.k <= kThreads * kSmallKeys;
  auto kern = merge ? (wide ? topk_split_wide_kernel : topk_split_kernel)
                    : (stream_keys ? topk_kernel<true> : topk_kernel<false>);
  auto merge_kern = small_merge ? topk_merge_small_kernel : topk_merge_kernel;
  if (tm.start || tm.stop)
    hipExtLaunchKernelGGL(kern, grid, dim3(kThreads), 0, stream, tm.start,
                          merge ? nullptr : tm.stop, 0, p.logits, p.row_stride, p.ctx, p.next_n,
                          p.k, p.seg_grid, p.out_idx, p.cand_val, p.cand_idx);
  else
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, stream, p.logits, p.row_stride, p.ctx,
                       p.next_n, p.k, p.seg_grid, p.out_idx, p.cand_val, p.cand_idx);
  if (merge) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (tm.start || tm.stop)
      hipExtLaunchKernelGGL(merge_kern, dim3(rows), dim3(kThreads), 0, stream, nullptr,
                            tm.stop, 0, p.logits, p.row_stride, p.ctx, p.next_n, p.k, p.seg_grid,
                            p.out_idx, p.cand_val, p.cand_idx);
    else
      hipLaunchKernelGGL(merge_kern, dim3(rows), dim3(kThreads), 0, stream, p.logits,
                         p.row_stride, p.ctx, p.next_n, p.k, p.seg_grid, p.out_idx, p.cand_val,
                         p.cand_idx);
  }
  return hipGetLastError();
}

}  // namespace pmqa
