"""Invariants and properties of the CPU oracle (CPU only).

Each is exact (bit-identical) in the oracle:
* identity vs randomly permuted block table holding the same logical K;
* compact vs wide output row stride, and one shot vs the batch split in halves
  (the reproducer in aiter PR #4244 compares exactly these);
* power-of-two scaling of every token scale or every weight scales the scores;
* MTP prefix: row j equals a next_n=1 run over the visible prefix;
* masking: -inf bits exactly on [visible, ctx), untouched at t >= ctx and for
  empty contexts;
* row coverage of a [1024, 1<<20] fp32 output, with a negative control that
  plants a 32-bit byte-offset store in the oracle and must reproduce the first
  untouched rows the page prints (512 at 1<<20 columns, 895 at 600000);
* int64 page ids: a page whose byte offset passes 2^31 is read correctly, with
  a negative control that plants an int32 id * record-size product in the
  oracle's gather and must reproduce the wrap boundary ATOM PR #2533 prints
  (row 3,728,270 of 576-byte records, block 233,016 of 16) and this path's own
  (page 2,033,602 of 8-token pages).
"""
import math

import numpy as np
import pytest

import oracle
import oracle.paged_mqa as opm
import synth
from tests.handcase import load_golden

SENTINEL = np.float32(12345.0)


def small(seed=0, **kw):
    args = dict(batch=5, next_n=2, heads=16, head_dim=32, page_size=4, ctx_range=(0, 37),
                table="permuted", topk=8, seed=seed)
    args.update(kw)
    return synth.build_workload("small", **args)


def run(wl, tables=None, stride=None, requests=None, scale_w=1.0):
    stride = stride or wl.out_row_stride
    out = np.full(wl.rows * stride, SENTINEL, dtype=np.float32)
    rows = oracle.paged_mqa_logits(wl.q, wl.kv_cache, wl.weights * np.float32(scale_w),
                                   wl.context_lens, wl.block_tables if tables is None else tables,
                                   wl.page_size, wl.next_n, out=out, out_row_stride=stride,
                                   requests=requests)
    return rows, out.reshape(wl.rows, stride)


@pytest.mark.parametrize("ps", [1, 2, 8])
def test_identity_vs_permuted_table(ps):
    """Same logical K, pages placed by a random permutation or in order."""
    b = small(seed=11, page_size=ps, ctx_range=(1, 40), table="permuted", pool_pages=400)
    W = b.block_tables.shape[1]
    npg = (b.context_lens.astype(np.int64) + ps - 1) // ps
    rec = b.head_dim + 4
    ident_pool = np.zeros((b.batch * W + 1) * ps * rec, dtype=np.uint8)
    ident_tab = np.full((b.batch, W), b.batch * W, dtype=np.int64)
    src = b.kv_cache.reshape(-1, ps * rec)
    dst = ident_pool.reshape(-1, ps * rec)
    for r in range(b.batch):
        for i in range(int(npg[r])):
            dst[r * W + i] = src[b.block_tables[r, i]]
            ident_tab[r, i] = r * W + i
    assert not np.array_equal(ident_tab, b.block_tables)
    rows_p, _ = run(b)
    rows_i = oracle.paged_mqa_logits(b.q, ident_pool, b.weights, b.context_lens, ident_tab,
                                     ps, b.next_n)
    for x, y in zip(rows_p, rows_i):
        assert np.array_equal(x, y)
    assert sum(len(x) for x in rows_p) > 0


@pytest.mark.parametrize("ps", [2, 8, 64])
def test_token_level_table_reads_the_same_rows(ps):
    """The pool read through its page table, and read through a token-level
    table (page_size 1: entry t is the pool row page * ps + t % ps), give the
    same scores: the paging changes addresses only."""
    b = small(seed=12, page_size=ps, ctx_range=(1, 150), table="permuted")
    ctx = b.context_lens.astype(np.int64)
    tok = np.full((b.batch, int(ctx.max())), b.poison_page * ps, dtype=np.int64)
    for r in range(b.batch):
        t = np.arange(ctx[r])
        tok[r, : ctx[r]] = b.block_tables[r, t // ps] * ps + t % ps
    rows_p, _ = run(b)
    rows_t = oracle.paged_mqa_logits(b.q, b.kv_cache, b.weights, b.context_lens, tok, 1, b.next_n)
    for x, y in zip(rows_p, rows_t):
        assert np.array_equal(x, y)
    # a wrong in-page offset (t // ps in place of t % ps) reads other rows
    bad = tok.copy()
    for r in range(b.batch):
        t = np.arange(ctx[r])
        bad[r, : ctx[r]] = b.block_tables[r, t // ps] * ps + (t // ps) % ps
    rows_b = oracle.paged_mqa_logits(b.q, b.kv_cache, b.weights, b.context_lens, bad, 1, b.next_n)
    assert any(not np.array_equal(x, y) for x, y in zip(rows_p, rows_b))


def test_compact_vs_wide_stride_and_batch_split():
    wl = small(seed=2, batch=8, ctx_range=(1, 50))
    compact = int(wl.context_lens.max())
    r1, o1 = run(wl, stride=compact)
    r2, o2 = run(wl, stride=1000)
    for r in range(wl.rows):
        ctx = int(wl.context_lens[r // wl.next_n])
        assert np.array_equal(o1[r, :ctx], o2[r, :ctx])
        assert np.all(o2[r, ctx:] == SENTINEL)
    # batch split: halves, each with its own slice of every input
    h = wl.batch // 2
    parts = []
    for lo, hi in [(0, h), (h, wl.batch)]:
        rows = oracle.paged_mqa_logits(
            wl.q[lo * wl.next_n: hi * wl.next_n], wl.kv_cache,
            wl.weights[lo * wl.next_n: hi * wl.next_n], wl.context_lens[lo:hi],
            wl.block_tables[lo:hi], wl.page_size, wl.next_n)
        parts.extend(rows)
    for x, y in zip(parts, r1):
        assert np.array_equal(x, y)


def test_power_of_two_scaling():
    wl = small(seed=5)
    r1, _ = run(wl)
    r2, _ = run(wl, scale_w=0.25)
    for x, y in zip(r1, r2):
        assert np.array_equal(x * 0.25, y)
    # scale every token's fp32 scale by 8: edit the stored scale bytes
    pool = wl.kv_cache.copy()
    recs = pool.reshape(-1, wl.head_dim + 4)
    sc = recs[:, wl.head_dim:].copy().view("<f4")
    finite = np.isfinite(sc)
    sc[finite] *= np.float32(8.0)
    recs[:, wl.head_dim:] = sc.view(np.uint8)
    r3 = oracle.paged_mqa_logits(wl.q, pool, wl.weights, wl.context_lens, wl.block_tables,
                                 wl.page_size, wl.next_n)
    for x, y in zip(r1, r3):
        assert np.array_equal(x * 8.0, y)


def test_mtp_prefix_property():
    wl = small(seed=9, next_n=3, ctx_range=(0, 30))
    rows, _ = run(wl)
    for b in range(wl.batch):
        ctx = int(wl.context_lens[b])
        for j in range(wl.next_n):
            vis = oracle.visible_len(ctx, wl.next_n, j)
            r = b * wl.next_n + j
            single = oracle.paged_mqa_logits(
                wl.q[r:r + 1], wl.kv_cache, wl.weights[r:r + 1],
                np.array([vis], np.int32), wl.block_tables[b:b + 1], wl.page_size, 1)
            assert np.array_equal(single[0], rows[r])


def test_visible_len_cases():
    assert [oracle.visible_len(3, 2, j) for j in range(2)] == [2, 3]
    assert [oracle.visible_len(1, 3, j) for j in range(3)] == [0, 0, 1]
    assert [oracle.visible_len(0, 3, j) for j in range(3)] == [0, 0, 0]
    assert oracle.visible_len(100, 1, 0) == 100


def test_masking_bits_and_untouched_tail():
    wl = small(seed=4, next_n=3, ctx_range=(0, 20), zero_every=2)
    stride = 32
    rows, out = run(wl, stride=stride)
    bits = out.view(np.uint32)
    for r in range(wl.rows):
        b, j = divmod(r, wl.next_n)
        ctx = int(wl.context_lens[b])
        vis = oracle.visible_len(ctx, wl.next_n, j)
        assert np.all(np.isfinite(out[r, :vis]))
        assert np.all(bits[r, vis:ctx] == oracle.NEG_INF_BITS)
        assert np.all(out[r, ctx:] == SENTINEL)
        if ctx == 0:
            assert np.all(out[r] == SENTINEL)
    assert (wl.context_lens == 0).any()


def test_poison_never_reaches_output():
    # the poison page holds NaN codes and NaN scales; any read of a table entry
    # past ceil(ctx/page_size), or of a page tail past ctx, would show as NaN
    wl = small(seed=12, page_size=8, ctx_range=(1, 60))
    rows, out = run(wl)
    for r in range(wl.rows):
        ctx = int(wl.context_lens[r // wl.next_n])
        assert not np.isnan(out[r, :ctx]).any()


def _coverage_case(stride):
    """B=256, next_n=4 (1024 rows), tiny heads: coverage is about addressing."""
    return synth.build_workload("coverage", batch=256, next_n=4, heads=1, head_dim=4,
                                page_size=2, ctx_range=(1, 4), table="identity", topk=4,
                                out_row_stride=stride, seed=1)


def _first_untouched(out2):
    touched = (out2 != SENTINEL).any(axis=1)
    bad = np.nonzero(~touched)[0]
    return (int(bad[0]) if len(bad) else None), touched


@pytest.mark.slow
def test_full_row_coverage_wide_output_and_negative_control(monkeypatch):
    fixtures = load_golden("row_coverage.json")["cases"]
    stride = fixtures[0]["row_stride"]
    assert stride == 1 << 20
    wl = _coverage_case(stride)
    _, out = run(wl)  # [1024, 1<<20] fp32 = 4 GiB on the host
    first, touched = _first_untouched(out)
    assert first is None and touched.all()
    del out

    # negative control: an emulated 32-bit byte-offset store drops every write
    # whose byte offset row*stride*4 + col*4 reaches 2^31
    def store32(out, row, out_row_stride, col0, values):
        for c, v in enumerate(values):
            off = (row * out_row_stride + col0 + c) * 4
            if off >= 2 ** 31:
                continue  # dropped, like an out-of-range buffer store
            out[off // 4] = v

    monkeypatch.setattr(opm, "_store", store32)
    for case in fixtures:
        wl = _coverage_case(case["row_stride"])
        _, out = run(wl)
        first, _ = _first_untouched(out)
        assert first == case["first_untouched_row"]
        assert first == math.ceil(2 ** 31 / (4 * case["row_stride"]))
        del out


def test_int64_page_ids_past_2gib():
    """A page whose byte offset passes 2^31 (and 2^32) is read at the right place."""
    D, ps = 4, 2
    rec = D + 4
    page_bytes = ps * rec
    hi_page = (2 ** 32) // page_bytes + 5  # byte offset past 2^32
    num_pages = hi_page + 1
    pool = np.zeros(num_pages * page_bytes, dtype=np.uint8)  # lazily backed
    from tests.handcase import codes_of
    kv = codes_of([1.0, 2.0, 3.0, 4.0])
    off = hi_page * page_bytes
    pool[off:off + D] = kv
    pool[off + D:off + rec] = np.frombuffer(np.float32(0.5).tobytes(), np.uint8)
    q = codes_of([1.0, 1.0, 1.0, 1.0]).reshape(1, 1, D)
    rows = oracle.paged_mqa_logits(q, pool, np.ones((1, 1), np.float32),
                                   np.array([1], np.int32), np.array([[hi_page]], np.int64), ps, 1)
    assert rows[0].tolist() == [5.0]  # (1+2+3+4) * 0.5


def _offset_int32(row_id, row_bytes):
    """The byte offset row_id * row_bytes as a product in int32 arithmetic
    (two's complement wrap), the failure ATOM PR #2533 describes."""
    v = (int(row_id) * int(row_bytes)) & 0xFFFFFFFF
    return v - (1 << 32) if v >= 1 << 31 else v


def _gather_int32(kv_cache, table_row, ctx, page_size, head_dim, layout="records"):
    """The oracle's gather with the planted mistake: each record's byte offset is
    the int32 product of its cache row id and the record size.  A wrapped
    (negative) offset lands outside the pool: its values read back as NaN."""
    rec = head_dim + 4
    flat = kv_cache.reshape(-1)
    k = np.full((ctx, head_dim), np.nan)
    scale = np.full(ctx, np.nan)
    for t in range(ctx):
        row = int(table_row[t // page_size]) * page_size + t % page_size
        off = _offset_int32(row, rec)
        if 0 <= off and off + rec <= flat.size:
            k[t] = oracle.e4m3fn_to_float64(flat[off:off + head_dim])
            scale[t] = float(np.frombuffer(flat[off + head_dim:off + rec].tobytes(), "<f4")[0])
    return k, scale


def test_int32_row_ids_wrap_where_the_page_says(monkeypatch):
    """Negative control for int64 ids.  ATOM PR #2533 (description) reports that a
    token-level table of int32 ids multiplied by the 576-byte MLA row stride
    wraps for rows past 2**31 / 576 = 3,728,270, i.e. from block 233,016 of 16
    tokens.  Planting that int32 product in the oracle's gather reproduces the
    boundary exactly: the last row below it is read correctly, the first row
    past it is not, while the real (int64) oracle reads both.  The same planted
    gather on this path's own records (132 bytes, 8-token pages) goes wrong
    from page ceil(2^31 / 1056) = 2,033,602, the boundary the small-pages
    workload's pool is sized to cross."""
    assert 2 ** 31 // 576 == 3_728_270
    first_bad = next(r for r in range(3_728_260, 3_728_280) if _offset_int32(r, 576) < 0)
    assert first_bad == 3_728_270 + 1 and first_bad // 16 == 233_016
    assert _offset_int32(3_728_270, 576) == 3_728_270 * 576

    # MLA-sized records (572 codes + the fp32 scale = 576 bytes), token-level
    # table, a pool past the boundary (lazily backed zeros)
    from tests.handcase import codes_of
    D, rows_in_pool = 572, first_bad + 2
    pool = np.zeros(rows_in_pool * (D + 4), dtype=np.uint8)
    ids = [first_bad - 1, first_bad]
    for i, r in enumerate(ids):
        off = r * (D + 4)
        pool[off:off + D] = codes_of([float(i + 1)] * D)
        pool[off + D:off + D + 4] = np.frombuffer(np.float32(1.0).tobytes(), np.uint8)
    q = codes_of([1.0] * D).reshape(1, 1, D)
    args = (q, pool, np.ones((1, 1), np.float32), np.array([2], np.int32),
            np.array([ids], np.int64), 1, 1)
    good = oracle.paged_mqa_logits(*args)[0]
    assert good.tolist() == [572.0, 1144.0]
    monkeypatch.setattr(opm, "gather_request", _gather_int32)
    bad = oracle.paged_mqa_logits(*args)[0]
    assert bad[0] == 572.0 and np.isnan(bad[1])
    monkeypatch.undo()

    # this path's records: 8-token pages of 132-byte records
    ps, D = 8, 128
    page_bytes = ps * (D + 4)
    boundary = -(-(2 ** 31) // page_bytes)
    assert boundary == 2_033_602
    assert _offset_int32(boundary * ps, D + 4) < 0 <= _offset_int32(boundary * ps - 1, D + 4)
    pool = np.zeros((boundary + 1) * page_bytes, dtype=np.uint8)
    for i, pg in enumerate((boundary - 1, boundary)):
        off = pg * page_bytes
        pool[off:off + D] = codes_of([float(i + 1)] * D)
        pool[off + D:off + D + 4] = np.frombuffer(np.float32(0.5).tobytes(), np.uint8)
    q = codes_of([1.0] * D).reshape(1, 1, D)
    args = (q, pool, np.ones((1, 1), np.float32), np.array([9], np.int32),
            np.array([[boundary - 1, boundary]], np.int64), ps, 1)
    good = oracle.paged_mqa_logits(*args)[0]
    assert good[0] == 64.0 and good[8] == 128.0
    monkeypatch.setattr(opm, "gather_request", _gather_int32)
    bad = oracle.paged_mqa_logits(*args)[0]
    assert bad[0] == 64.0 and np.isnan(bad[8])
