"""Literal fp64 CPU computation of paged MQA logits and the per-row top-k.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain numpy; one request
at a time; no tiling, fusion or reordering beyond the definition.

Inputs are the raw arrays the path consumes (uint8 codes, fp32 weights, int32
context lengths, int64 block tables, a flat uint8 K cache).  The K cache is read
as per-token records ``[D e4m3fn codes][fp32 scale, little endian]``: the pages
describe the cache as ``[num_blocks, block_size, 1, D+4]`` fp8 bytes whose last
4 bytes per token the kernel views as one fp32 scale (aiter PR #4244,
reproducer input construction).  Token ``s`` of page ``p`` therefore starts at
byte ``(p*page_size + s)*(D+4)``; this is the reading adopted (a per-page
"all values, then all scales" split, which the gfx1250 loader's load order in
aiter PR #6626 section 1 could suggest, is not).
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

from .fp8 import e4m3fn_to_float64
from .layout import preshuffled_offsets

NEG_INF_BITS = 0xFF800000


def visible_len(ctx: int, next_n: int, j: int) -> int:
    """Tokens visible to MTP position ``j`` of a request with ``ctx`` tokens.

    Reading adopted for the causal mask: the ``next_n`` query rows of a request
    are the last ``next_n`` positions of its context, so position ``j`` sees
    tokens ``t <= ctx - next_n + j``.  Clamped to ``[0, ctx]``, so a request
    with an empty context (aiter PR #6626, "Accuracy", tests one under MTP with
    three positions) gives its rows no visible token.  For next_n = 1 every row
    sees its whole context.
    """
    v = int(ctx) - int(next_n) + int(j) + 1
    return max(0, min(v, int(ctx)))


def gather_request(kv_cache: np.ndarray, table_row: np.ndarray, ctx: int,
                   page_size: int, head_dim: int, layout: str = "records"):
    """Collect the ``ctx`` tokens of one request through its block table.

    Returns (K float64 [ctx, D], scale float64 [ctx]).  Only the first
    ``ceil(ctx/page_size)`` table entries are read; page ids are int64 and the
    byte address ``(id*page_size + slot)*(D+4)`` is formed in 64-bit integers,
    as the int64-id fix requires (ATOM PR #2533 "Address Triton decode KV rows
    with int64 ids": an int32 id times the row size wraps at 2^31).  With
    ``layout="preshuffled"`` the same cache rows are read at the byte offsets
    ``oracle.layout`` defines.
    """
    ctx = int(ctx)
    rec = head_dim + 4
    if ctx <= 0:
        return np.zeros((0, head_dim)), np.zeros(0)
    n_pages = (ctx + page_size - 1) // page_size
    pages = np.asarray(table_row[:n_pages], dtype=np.int64)
    t = np.arange(ctx, dtype=np.int64)
    rec_index = pages[t // page_size] * np.int64(page_size) + (t % page_size)
    if layout == "preshuffled":
        flat = kv_cache.reshape(-1)
        voff, soff = preshuffled_offsets(rec_index, page_size, head_dim)
        codes = flat[voff]  # [ctx, D] uint8
        sb = flat[soff[:, None] + np.arange(4, dtype=np.int64)[None, :]]  # [ctx, 4]
        k = e4m3fn_to_float64(codes)
        scale = np.ascontiguousarray(sb).view("<f4").reshape(ctx).astype(np.float64)
        return k, scale
    if layout != "records":
        raise ValueError(f"unknown layout {layout}")
    records = kv_cache.reshape(-1, rec)[rec_index]  # [ctx, D+4] uint8
    k = e4m3fn_to_float64(records[:, :head_dim])
    scale = np.ascontiguousarray(records[:, head_dim:]).view("<f4").reshape(ctx).astype(np.float64)
    return k, scale


def request_logits(q_req: np.ndarray, w_req: np.ndarray, k: np.ndarray,
                   scale: np.ndarray, next_n: int) -> List[np.ndarray]:
    """Scores of one request's ``next_n`` rows over their visible tokens.

    ``logit[j, t] = sum_h w[j, h] * max(0, scale_t * sum_d q[j, h, d] * k[t, d])``
    in fp64.  The dot of two e4m3fn vectors of length <= 128 is exact in fp64
    (every product is a multiple of 2^-18 below 2^18 in magnitude), so the
    matmul's summation order cannot change it.
    """
    ctx = k.shape[0]
    q = e4m3fn_to_float64(q_req)  # [next_n, H, D]
    w = np.asarray(w_req, dtype=np.float64)  # [next_n, H]
    out = []
    for j in range(next_n):
        vis = visible_len(ctx, next_n, j)
        dots = q[j] @ k[:vis].T  # [H, vis]
        act = np.maximum(scale[None, :vis] * dots, 0.0)
        out.append(w[j] @ act)  # [vis]
    return out


def _row_base(row: int, out_row_stride: int) -> int:
    """Element offset of an output row: 64-bit (Python int) row * stride.

    aiter PR #4244, "Fix": the row must be folded into the base address in
    64-bit; a 32-bit byte offset ``row*stride*4`` drops every store at or past
    2^31 bytes.
    """
    return int(row) * int(out_row_stride)


def _store(out: np.ndarray, row: int, out_row_stride: int, col0: int,
           values: np.ndarray) -> None:
    """Write ``values`` at columns ``[col0, col0+len)`` of output row ``row``."""
    if len(values) == 0:
        return
    base = _row_base(row, out_row_stride) + int(col0)
    out[base : base + len(values)] = values


def paged_mqa_logits(q, kv_cache, weights, context_lens, block_tables,
                     page_size: int, next_n: int, out: Optional[np.ndarray] = None,
                     out_row_stride: Optional[int] = None,
                     requests: Optional[Sequence[int]] = None,
                     layout: str = "records") -> List[Optional[np.ndarray]]:
    """Oracle for the whole logits step.

    Returns a list with one fp64 array per output row ``r = b*next_n + j``
    (its visible scores), or None for rows of requests not in ``requests``.
    If ``out`` (a flat float32 buffer) is given, row ``r`` is written the way the
    op writes it: float32 scores on ``[0, visible)``, -inf on
    ``[visible, ctx)``, and no write at ``t >= ctx`` (the reproducer in aiter
    PR #4244 compares only the first ``context_len`` columns; reading adopted:
    nothing past the context is written).  ``layout`` names the byte layout of
    ``kv_cache``: "records" (per-token records) or "preshuffled" (``oracle.layout``).
    """
    B = int(np.asarray(context_lens).shape[0])
    q = np.asarray(q)
    H, D = q.shape[1], q.shape[2]
    rows: List[Optional[np.ndarray]] = [None] * (B * next_n)
    reqs = range(B) if requests is None else requests
    for b in reqs:
        ctx = int(context_lens[b])
        k, scale = gather_request(kv_cache, block_tables[b], ctx, page_size, D, layout)
        r0 = b * next_n
        res = request_logits(q[r0 : r0 + next_n], weights[r0 : r0 + next_n], k, scale, next_n)
        for j in range(next_n):
            rows[r0 + j] = res[j]
            if out is not None:
                vis = len(res[j])
                _store(out, r0 + j, out_row_stride, 0, res[j].astype(np.float32))
                _store(out, r0 + j, out_row_stride, vis,
                       np.full(ctx - vis, -np.inf, dtype=np.float32))
    return rows


def topk_per_row(row_values: Sequence[np.ndarray], k: int) -> np.ndarray:
    """Top-k token indices per row (the follow-on ``top_k_per_row_decode``).

    Each entry of ``row_values`` holds one row's candidate scores (its visible
    tokens only).  Order: score descending, then index ascending (reading
    adopted for ties; the pages do not state one).  The first ``min(k, n)``
    indices are returned, the rest of the k slots are -1.
    """
    out = np.full((len(row_values), k), -1, dtype=np.int32)
    for r, v in enumerate(row_values):
        if v is None:
            continue
        v = np.asarray(v, dtype=np.float64)
        n = len(v)
        order = np.lexsort((np.arange(n), -v))
        m = min(k, n)
        out[r, :m] = order[:m]
    return out
