"""K-cache producer (oracle; test infrastructure only).

What it computes: the records that the paged K cache holds, written from new
K rows.  For every token i with a cache slot s_i (the flat row of the page
pool, page * page_size + offset in page):

* ``amax = max_d |k_i[d]|`` and ``scale_i = amax / 448`` in float32 (1 when
  that quotient is 0), the per-token quantisation the workloads use for K;
* ``code_i[d] = e4m3fn(clamp(k_i[d] / scale_i, -448, 448))`` with the quotient
  rounded to float32 and the e4m3fn value chosen by round-to-nearest, ties to
  the even code;
* the record at byte ``s_i * (head_dim + 4)`` of the pool: the head_dim codes,
  then scale_i as a little-endian float32 (the record layout the paged cache
  uses: the last 4 bytes of each token row hold its fp32 scale, aiter PR #4244
  reproducer).  Slots are Python ints, so offsets past 2^31 bytes are exact
  (ATOM PR #2533: the cache writers compute slots in int64).  Slots outside
  ``[0, num_slots)`` are skipped (padding tokens carry -1).

Readings: the pages name the producer only through its slots (ATOM PR #2533);
the quantisation recipe (per-token fp32 scale = amax/448, e4m3fn codes) is that
of the workloads' K.  The division is the plain reading of "quantised with
scale": code = e4m3fn(k / scale), taken in float32 (the precision of the k rows
and of the scale), after which the choice of code is exact.

Independent of the HIP path: its own encoder (nearest value over the decoded
code table), its own bf16 widening and its own record addressing.
"""
import numpy as np

from .fp8 import E4M3FN_TABLE
from .layout import preshuffled_offsets

E4M3FN_MAX = 448.0
_POS_VALUES = E4M3FN_TABLE[:0x7F]  # codes 0x00..0x7E: every finite value >= 0, increasing


def e4m3fn_encode(y) -> np.ndarray:
    """Round finite values inside [-448, 448] to e4m3fn codes (uint8).

    Round to nearest, ties to the code whose mantissa is even (the code's last
    bit), following the format's definition: the candidates are the two finite
    magnitudes that bracket |y|; the sign bit is copied from y, so -0 and
    negative values that round to zero give 0x80.
    """
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)) or np.any(np.abs(y) > E4M3FN_MAX):
        raise ValueError("e4m3fn_encode takes finite values inside +-448")
    mag = np.abs(y)
    # index of the largest code whose value is <= mag
    lo = np.searchsorted(_POS_VALUES, mag, side="right") - 1
    hi = np.minimum(lo + 1, len(_POS_VALUES) - 1)
    d_lo = mag - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - mag
    pick_hi = (hi != lo) & ((d_hi < d_lo) | ((d_hi == d_lo) & (lo % 2 == 1)))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(y), code | np.uint8(0x80), code).astype(np.uint8)


def bf16_to_float32(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32: the bf16 bits are the high half."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def quantize_tokens(k) -> tuple:
    """Per-token quantisation of float32 rows [n, D] -> (codes uint8 [n, D], scales float32 [n])."""
    k = np.asarray(k, dtype=np.float32)
    n, d = k.shape
    codes = np.zeros((n, d), dtype=np.uint8)
    scales = np.zeros(n, dtype=np.float32)
    for i in range(n):
        amax = np.float32(np.max(np.abs(k[i]))) if d else np.float32(0.0)
        scale = np.float32(amax / np.float32(E4M3FN_MAX))  # float32 quotient
        if scale == np.float32(0.0):
            scale = np.float32(1.0)
        y = (k[i] / scale).astype(np.float32)  # float32 quotients
        y = np.clip(y, np.float32(-E4M3FN_MAX), np.float32(E4M3FN_MAX))
        codes[i] = e4m3fn_encode(y)
        scales[i] = scale
    return codes, scales


def record_offset(slot: int, head_dim: int) -> int:
    """Byte offset of cache row `slot` (Python int arithmetic: never wraps)."""
    return int(slot) * (int(head_dim) + 4)


def write_k_cache(pool: np.ndarray, k, slot_mapping, head_dim: int, layout: str = "records",
                  page_size: int = 0) -> np.ndarray:
    """Write the records of rows k [n, head_dim] (float32) at their slots into the
    uint8 pool (in place; returns it).  The pool holds num_slots = len(pool) //
    (head_dim + 4) rows; slots outside [0, num_slots) are skipped.  With
    layout="preshuffled" (and the pool's page_size) each token's codes and
    scale go to the byte offsets ``oracle.layout`` defines instead."""
    k = np.asarray(k, dtype=np.float32)
    codes, scales = quantize_tokens(k)
    rec = head_dim + 4
    num_slots = len(pool) // rec
    for i, s in enumerate(np.asarray(slot_mapping, dtype=np.int64).tolist()):
        if s < 0 or s >= num_slots:
            continue
        sb = np.frombuffer(np.asarray([scales[i]], dtype="<f4").tobytes(), dtype=np.uint8)
        if layout == "preshuffled":
            voff, soff = preshuffled_offsets([s], page_size, head_dim)
            pool[voff[0]] = codes[i]
            pool[int(soff[0]):int(soff[0]) + 4] = sb
            continue
        off = record_offset(s, head_dim)
        pool[off:off + head_dim] = codes[i]
        pool[off + head_dim:off + rec] = sb
    return pool
