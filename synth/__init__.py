"""Seeded synthetic inputs for the FP8 paged MQA logits + per-row top-k path.

This module only *produces bytes*: fp8 query codes, a paged fp8 K cache with one
fp32 scale per token, weights, context lengths and int64 block tables.  It holds
none of the scoring arithmetic (no dot products, no relu, no masking, no top-k),
so the CPU oracle and the HIP path can both be fed from it without sharing any
of the method's code.

Layout produced (the reading of the pages' tensor shapes, aiter PR #4244
"fix silent tail-row drop in deepgemm_fp8_paged_mqa_logits at large output
stride", the standalone reproducer's input construction):

* ``q``            uint8 ``[B*next_n, H, D]``  e4m3fn codes, row ``r = b*next_n + j``
* ``kv_cache``     uint8 flat ``[num_pages * page_size * (D+4)]``; token ``s`` of
                   page ``p`` is the record at byte ``(p*page_size + s)*(D+4)``:
                   D e4m3fn codes, then the token's fp32 scale (little endian)
* ``weights``      float32 ``[B*next_n, H]``
* ``context_lens`` int32 ``[B]``
* ``block_tables`` int64 ``[B, W]``; entries past ``ceil(ctx/page_size)`` point at
                   a poison page (NaN codes, NaN scale) that must never be used.

Quantisation of K (generator only): per token ``scale = amax/448`` (1 when the
token is all zero), codes = round-to-nearest-even e4m3fn of ``x/scale`` after
clamping to +-448 (torch's CPU cast is the rounding routine).  Both sides read
the stored bytes, so this rounding never enters a parity comparison.

Draw order from ``numpy.random.default_rng(seed)`` (PCG64): context lengths,
page permutation, q, then K request by request (for the log-normal workload
the per-token factors of a request are drawn before its normals), then weights.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch

E4M3_MAX = 448.0
POISON_CODE = 0x7F  # e4m3fn NaN
POISON_SCALE_BITS = 0x7FC00000  # fp32 quiet NaN


@dataclasses.dataclass
class Workload:
    """One synthetic batch of the path's inputs (all host numpy arrays)."""

    name: str
    batch: int
    next_n: int
    heads: int
    head_dim: int
    page_size: int
    num_pages: int
    context_lens: np.ndarray  # int32 [B]
    block_tables: np.ndarray  # int64 [B, W]
    kv_cache: np.ndarray  # uint8 flat
    q: np.ndarray  # uint8 [B*next_n, H, D]
    weights: np.ndarray  # float32 [B*next_n, H]
    topk: int
    out_row_stride: int  # fp32 elements between output rows
    poison_page: int
    extra_tables: dict = dataclasses.field(default_factory=dict)

    @property
    def rows(self) -> int:
        return self.batch * self.next_n

    @property
    def record_bytes(self) -> int:
        return self.head_dim + 4

    def visible_lens(self) -> np.ndarray:
        """Per-row count of scored tokens (host helper for sizing/metrics only).

        Uses the MTP convention adopted for the causal mask: the next_n query
        positions are the last next_n positions of the context.
        """
        ctx = self.context_lens.astype(np.int64)
        out = np.empty(self.rows, dtype=np.int64)
        for j in range(self.next_n):
            out[j :: self.next_n] = np.clip(ctx - self.next_n + j + 1, 0, ctx)
        return out

    def scored_tokens(self) -> int:
        return int(self.visible_lens().sum())

    def kv_tokens(self) -> int:
        return int(self.context_lens.astype(np.int64).sum())


def quantize_e4m3fn(x: np.ndarray) -> np.ndarray:
    """RNE cast of float32 values (already inside +-448) to e4m3fn codes."""
    x = np.clip(np.asarray(x, dtype=np.float32), -E4M3_MAX, E4M3_MAX)
    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def quantize_tokens(x: np.ndarray):
    """Per-token (row) quantisation: returns (codes uint8 [n, D], scales f32 [n])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=1) if x.shape[0] else np.zeros(0, np.float32)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    scale[scale == 0] = np.float32(1.0)
    codes = quantize_e4m3fn(x / scale[:, None])
    return codes, scale


def _poison_pool(num_pages: int, page_size: int, head_dim: int) -> np.ndarray:
    rec = head_dim + 4
    pool = np.full(num_pages * page_size * rec, POISON_CODE, dtype=np.uint8)
    recs = pool.reshape(num_pages * page_size, rec)
    recs[:, head_dim:] = np.frombuffer(
        np.uint32(POISON_SCALE_BITS).astype("<u4").tobytes(), dtype=np.uint8
    )
    return pool


def build_workload(
    name: str,
    *,
    batch: int,
    next_n: int,
    heads: int,
    head_dim: int,
    page_size: int,
    context_lens: Optional[Sequence[int]] = None,
    ctx_range: Optional[tuple] = None,
    table: str = "permuted",  # "identity" | "permuted"
    pool_pages: Optional[int] = None,
    table_width: Optional[int] = None,
    weights_dist: str = "normal",  # "uniform" U(0,1) | "normal" N(0,1)/sqrt(H)
    lognormal_scales: bool = False,
    topk: int = 2048,
    out_row_stride: Optional[int] = None,
    seed: int = 0,
    ctx_fixups: Optional[dict] = None,
    zero_every: int = 0,
    padded_width: Optional[int] = None,
    neg_scale_blocks: float = 0.0,
    nan_scale_tokens: int = 0,
) -> Workload:
    """Build one workload; see the module docstring for layout and draw order.

    ``neg_scale_blocks`` (a fraction) and ``nan_scale_tokens`` (a count per
    request) perturb the stored scales after every other draw, so the rest of
    the workload is unchanged: each 64-token block of a request is picked with
    that probability, and inside a picked block every token's scale is negated
    with probability 1/2 (blocks of mixed signs next to blocks of scales >= 0);
    then that many distinct tokens per request get a NaN scale.  The codes are
    untouched."""
    rng = np.random.default_rng(seed)
    D, H, ps, B = head_dim, heads, page_size, batch
    rec = D + 4

    # 1. context lengths
    if context_lens is not None:
        ctx = np.asarray(context_lens, dtype=np.int64)
        assert ctx.shape == (B,)
    else:
        lo, hi = ctx_range
        ctx = rng.integers(lo, hi + 1, size=B, dtype=np.int64)
    if zero_every:
        ctx[::zero_every] = 0
    if ctx_fixups:
        for i, v in ctx_fixups.items():
            ctx[i] = v
    npages_req = (ctx + ps - 1) // ps
    W = int(table_width) if table_width is not None else max(1, int(npages_req.max()))
    assert W >= int(npages_req.max())
    n_used = int(npages_req.sum())

    # 2. page assignment
    tables = np.empty((B, W), dtype=np.int64)
    if table == "identity":
        num_pages = B * W + 1 if pool_pages is None else pool_pages
        assert num_pages >= B * W + 1
        poison = B * W
        for b in range(B):
            tables[b] = np.arange(b * W, (b + 1) * W, dtype=np.int64)
            tables[b, npages_req[b]:] = poison
    else:
        num_pages = pool_pages if pool_pages is not None else n_used + 1
        assert num_pages >= n_used + 1, "pool too small"
        perm = rng.permutation(num_pages).astype(np.int64)
        poison = int(perm[n_used])
        tables[:] = poison
        pos = 0
        for b in range(B):
            n = int(npages_req[b])
            tables[b, :n] = perm[pos : pos + n]
            pos += n

    # 3. q
    q_f = rng.standard_normal((B * next_n, H, D), dtype=np.float32)
    q = quantize_e4m3fn(q_f).reshape(B * next_n, H, D)

    # 4. K, request by request, scattered into the pool through the table
    pool = _poison_pool(num_pages, ps, D)
    recs = pool.reshape(num_pages * ps, rec)
    for b in range(B):
        n = int(ctx[b])
        if n == 0:
            continue
        if lognormal_scales:
            f = np.exp(rng.standard_normal(n)).astype(np.float32)
        x = rng.standard_normal((n, D), dtype=np.float32)
        if lognormal_scales:
            x *= f[:, None]
        codes, scales = quantize_tokens(x)
        t = np.arange(n, dtype=np.int64)
        rows = tables[b, t // ps] * ps + (t % ps)
        recs[rows, :D] = codes
        recs[rows, D:] = scales.astype("<f4").view(np.uint8).reshape(n, 4)

    # 5. weights
    if weights_dist == "uniform":
        w = rng.random((B * next_n, H), dtype=np.float32)
    else:
        w = (rng.standard_normal((B * next_n, H), dtype=np.float32) / np.float32(math.sqrt(H))).astype(np.float32)

    # 6. optional scale perturbations (sign flips, NaN), after every other draw
    if neg_scale_blocks > 0.0 or nan_scale_tokens > 0:
        for b in range(B):
            n = int(ctx[b])
            if n == 0:
                continue
            t = np.arange(n, dtype=np.int64)
            rows = tables[b, t // ps] * ps + (t % ps)
            sc = recs[rows, D:].copy().view("<f4").reshape(n)
            if neg_scale_blocks > 0.0:
                picked = rng.random((n + 63) // 64) < neg_scale_blocks
                flip = picked[t // 64] & (rng.random(n) < 0.5)
                sc = np.where(flip, -sc, sc).astype(np.float32)
            if nan_scale_tokens > 0:
                sc[rng.choice(n, min(n, nan_scale_tokens), replace=False)] = np.float32(np.nan)
            recs[rows, D:] = sc.astype("<f4").view(np.uint8).reshape(n, 4)

    wl = Workload(
        name=name,
        batch=B,
        next_n=next_n,
        heads=H,
        head_dim=D,
        page_size=ps,
        num_pages=num_pages,
        context_lens=ctx.astype(np.int32),
        block_tables=tables,
        kv_cache=pool,
        q=q,
        weights=w,
        topk=topk,
        out_row_stride=int(out_row_stride) if out_row_stride is not None else max(1, int(ctx.max()) if B else 1),
        poison_page=poison,
    )
    if padded_width is not None:
        assert padded_width >= W
        padded = np.full((B, padded_width), poison, dtype=np.int64)
        padded[:, :W] = tables
        wl.extra_tables["padded"] = padded
    return wl


# The five workloads of the path, by number.  Sizes and distributions follow the
# configurations the measurements are quoted on; where a recipe leaves a detail
# open the choice is fixed here once (pool sizes, weights for 3-5, seeds).
CONFIG_NAMES = {
    1: "tiny_decode",
    2: "decode_b64",
    3: "mtp_wide_output",
    4: "small_pages",
    5: "long_context",
}


def make_config(cfg: int, seed: int = 0, table: str = "permuted") -> Workload:
    """Workload `cfg` (1-5).  `table` = "identity" lays each request's pages out
    contiguously in the same pool (workloads 2-5; the first is identity
    already), for comparing a scattered page stream with a contiguous one."""
    assert table in ("permuted", "identity")
    if cfg == 1:
        # B=2, next_n=1, H=64, D=128, 64-token pages, ctx [1000, 1024], identity table
        return build_workload(
            "tiny_decode", batch=2, next_n=1, heads=64, head_dim=128, page_size=64,
            context_lens=[1000, 1024], table="identity", weights_dist="uniform",
            topk=256, out_row_stride=1024, seed=seed,
        )
    if cfg == 2:
        # B=64 decode, ctx U[1,8192], permuted table over a 10,000-page pool
        return build_workload(
            "decode_b64", batch=64, next_n=1, heads=64, head_dim=128, page_size=64,
            ctx_range=(1, 8192), table=table, pool_pages=10_000, table_width=128,
            topk=2048, out_row_stride=8192, seed=seed,
        )
    if cfg == 3:
        # B=256, next_n=4 (1024 rows), H=128, 256-token pages, out [1024, 1<<20]
        return build_workload(
            "mtp_wide_output", batch=256, next_n=4, heads=128, head_dim=128, page_size=256,
            ctx_range=(2, 32768), table=table, pool_pages=40_960, table_width=128,
            topk=2048, out_row_stride=1 << 20, seed=seed,
        )
    if cfg == 4:
        # B=128, next_n=3, 8-token pages, ctx U[0,65536] with zeros and edge lengths,
        # a 2^21-page pool so that used pages sit past 2^31 bytes
        return build_workload(
            "small_pages", batch=128, next_n=3, heads=64, head_dim=128, page_size=8,
            ctx_range=(0, 65536), table=table, pool_pages=1 << 21, table_width=8192,
            zero_every=16, ctx_fixups={1: 1, 2: 7, 3: 8, 4: 9, 5: 65536},
            topk=2048, out_row_stride=65536, seed=seed, padded_width=16384,
        )
    if cfg == 5:
        # B=32, next_n=2, H=128, ctx U[65536,131072], log-normal per-token scales
        return build_workload(
            "long_context", batch=32, next_n=2, heads=128, head_dim=128, page_size=64,
            ctx_range=(65536, 131072), table=table, pool_pages=1 << 17, table_width=2048,
            lognormal_scales=True, topk=2048, out_row_stride=131072, seed=seed,
        )
    raise ValueError(f"unknown config {cfg}")


def preshuffle_pool(pool: np.ndarray, page_size: int, head_dim: int = 128) -> np.ndarray:
    """The same pool in the preshuffled page layout (a byte permutation of each
    page): tiles of R = min(page_size, 16) tokens; a tile holds, for each of the
    8 16-byte pieces of a 128-byte row (piece g = bytes [16g, 16g+16)), that
    piece of its R tokens in token order, then the R fp32 scales."""
    assert head_dim == 128
    P = int(page_size)
    R = min(P, 16)
    rec = head_dim + 4
    x = np.asarray(pool, dtype=np.uint8).reshape(-1, P // R, R, rec)
    vals = x[..., :head_dim].reshape(x.shape[0], P // R, R, 8, 16).transpose(0, 1, 3, 2, 4)
    scl = x[..., head_dim:]
    tiles = np.concatenate([vals.reshape(x.shape[0], P // R, 8 * R * 16),
                            scl.reshape(x.shape[0], P // R, R * 4)], axis=2)
    return np.ascontiguousarray(tiles).reshape(-1)


def make_logit_rows(rows: int, width: int, lens: Sequence[int], seed: int = 0,
                    ties: int = 0) -> np.ndarray:
    """Synthetic fp32 score rows for exercising a per-row top-k on its own.

    Row r holds N(0,1) values on [0, lens[r]); the rest is -inf (never a
    candidate).  With ``ties > 0`` every value is snapped to a grid of ``ties``
    levels so that many exact ties sit at any k-th boundary.
    """
    rng = np.random.default_rng(seed)
    out = np.full((rows, width), -np.inf, dtype=np.float32)
    for r in range(rows):
        n = int(lens[r])
        v = rng.standard_normal(n).astype(np.float32)
        if ties:
            v = (np.round(v * ties) / ties).astype(np.float32)
        out[r, :n] = v
    return out
