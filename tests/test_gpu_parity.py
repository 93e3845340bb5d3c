"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small cases are compared element by element on every row (several 16-token
tiles, 64-token iterations and 256-token wave units, with ragged tails, every
page size, head count and next_n class, zero contexts, scales of both signs
and NaN scales).  The five workloads run at full size in the launch
configuration the benchmark times, every row compared with the oracle, plus
properties that hold at any size: full-row coverage of the [1024, 1<<20]
output, no write past a context, bit-identical results across compact and
padded tables, output strides, batch splits, table permutations and repeat
runs.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import (SENTINEL_BITS, check_rows, check_topk, check_untouched_rows,
                          new_out, oracle_rows, run_logits, say, upload)

pytestmark = pytest.mark.gpu


def topk_gpu(pm, wl, out, k=None, ctx=None):
    k = k or wl.topk
    idx = torch.full((wl.rows, k), -7, dtype=torch.int32, device="cuda")
    say(f"[gpu] topk_per_row {wl.name} rows={wl.rows} k={k} stride={out.shape[1]}")
    pm.topk_per_row(out, ctx, k, idx, next_n=wl.next_n)
    torch.cuda.synchronize()
    return idx


SMALL = [
    dict(batch=3, next_n=1, heads=64, page_size=64, ctx_range=(1, 700)),
    dict(batch=4, next_n=2, heads=128, page_size=256, ctx_range=(2, 1500)),
    dict(batch=6, next_n=3, heads=64, page_size=8, ctx_range=(0, 900), zero_every=3),
    dict(batch=5, next_n=4, heads=32, page_size=16, ctx_range=(0, 600)),
    dict(batch=5, next_n=1, heads=16, page_size=32, ctx_range=(1, 520)),
    dict(batch=4, next_n=2, heads=64, page_size=128, ctx_range=(100, 1100)),
    dict(batch=3, next_n=5, heads=64, page_size=64, ctx_range=(0, 400)),
    dict(batch=3, next_n=3, heads=128, page_size=8, ctx_range=(1, 300)),
    # 128 heads with 4 rows per request: one shared K ring per request, runs
    # shorter and longer than its 8 slots, small pages and empty contexts
    dict(batch=6, next_n=4, heads=128, page_size=8, ctx_range=(0, 700), zero_every=3),
    dict(batch=4, next_n=4, heads=128, page_size=64, context_lens=[1, 64, 450, 1100]),
    dict(batch=4, next_n=4, heads=16, page_size=256, ctx_range=(0, 800)),
    dict(batch=2, next_n=1, heads=64, page_size=16,
         context_lens=[1, 15]),
    dict(batch=7, next_n=2, heads=32, page_size=8,
         context_lens=[0, 1, 2, 16, 17, 255, 257]),
    # token-level tables (1-token pages) and the other pages below 8 tokens
    dict(batch=4, next_n=2, heads=64, page_size=1, ctx_range=(1, 400)),
    dict(batch=5, next_n=1, heads=128, page_size=1, context_lens=[0, 1, 63, 64, 65]),
    dict(batch=3, next_n=3, heads=32, page_size=2, ctx_range=(0, 300)),
    dict(batch=4, next_n=1, heads=16, page_size=4, ctx_range=(1, 500)),
]


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_small_cases_every_row(gpu_lib, case):
    kw = dict(SMALL[case])
    for seed in (0, 1):
        wl = synth.build_workload(f"small{case}", head_dim=128, table="permuted", topk=64,
                                  seed=seed, **kw)
        wl.out_row_stride = int(max(1, wl.context_lens.max())) + 37
        d = upload(wl)
        out = run_logits(gpu_lib, wl, d, label=f"seed={seed}")
        ref = oracle_rows(wl)
        check_rows(wl, out, ref)
        for k in (1, 16, 64):
            idx = topk_gpu(gpu_lib, wl, out, k=k, ctx=d["ctx"])
            check_topk(idx, ref, k)


def test_config1_tiny_decode(gpu_lib):
    wl = synth.make_config(1)
    d = upload(wl)
    out = run_logits(gpu_lib, wl, d)
    ref = oracle_rows(wl)
    worst = check_rows(wl, out, ref)
    say(f"config1 worst rel err {worst:.3e}")
    idx = topk_gpu(gpu_lib, wl, out, ctx=d["ctx"])
    check_topk(idx, ref, wl.topk)


@pytest.fixture(scope="module")
def cfg2():
    return synth.make_config(2)


def test_config2_decode_all_rows(gpu_lib, cfg2):
    wl = cfg2
    d = upload(wl)
    out = run_logits(gpu_lib, wl, d)
    ref = oracle_rows(wl)
    worst = check_rows(wl, out, ref)
    say(f"config2 worst rel err {worst:.3e}")
    idx = topk_gpu(gpu_lib, wl, out, ctx=d["ctx"])
    check_topk(idx, ref, wl.topk)


def test_invariants_bit_identical(gpu_lib, cfg2):
    """Strides, batch split, table permutation and repeat runs change nothing."""
    wl = cfg2
    d = upload(wl)
    a = run_logits(gpu_lib, wl, d, label="ref")
    b = run_logits(gpu_lib, wl, d, label="repeat")
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    wide = run_logits(gpu_lib, wl, d, stride=wl.out_row_stride + 4099, label="wide")
    assert torch.equal(a.view(torch.int32), wide[:, : wl.out_row_stride].view(torch.int32))
    assert bool((wide[:, wl.out_row_stride:].view(torch.int32) == SENTINEL_BITS).all())
    # batch split: two launches over the halves
    h = wl.batch // 2
    for lo, hi in ((0, h), (h, wl.batch)):
        part = new_out((hi - lo) * wl.next_n, wl.out_row_stride)
        say(f"[gpu] paged_mqa_logits batch split [{lo},{hi})")
        nn = wl.next_n
        gpu_lib.paged_mqa_logits(d["q"][lo * nn:hi * nn], d["kv"], d["w"][lo * nn:hi * nn],
                                 d["ctx"][lo:hi].contiguous(), d["tab"][lo:hi].contiguous(),
                                 wl.page_size, nn, part)
        torch.cuda.synchronize()
        assert torch.equal(part.view(torch.int32), a[lo * nn:hi * nn].view(torch.int32))
    # identity table over a re-laid pool holding the same pages
    ps, W = wl.page_size, wl.block_tables.shape[1]
    npg = (wl.context_lens.astype(np.int64) + ps - 1) // ps
    rec = ps * (wl.head_dim + 4)
    src = wl.kv_cache.reshape(-1, rec)
    pool = np.zeros(((wl.batch * W) + 1, rec), dtype=np.uint8)
    tab = np.full((wl.batch, W), wl.batch * W, dtype=np.int64)
    for r in range(wl.batch):
        for i in range(int(npg[r])):
            pool[r * W + i] = src[wl.block_tables[r, i]]
            tab[r, i] = r * W + i
    d2 = dict(d)
    d2["kv"] = torch.from_numpy(pool.reshape(-1)).cuda()
    d2["tab"] = torch.from_numpy(tab).cuda()
    c = run_logits(gpu_lib, wl, d2, label="identity-table")
    assert torch.equal(a.view(torch.int32), c.view(torch.int32))


@pytest.fixture(scope="module")
def cfg3():
    return synth.make_config(3)


def test_config3_wide_output_rows_past_2gib(gpu_lib, cfg3):
    wl = cfg3
    d = upload(wl)
    out = run_logits(gpu_lib, wl, d)  # [1024, 1<<20] fp32: rows >= 512 start past 2^31 bytes
    # every row is touched, nothing is written past a context (checked on the GPU)
    bits = out.view(torch.int32)
    ctx_rows = d["ctx"].repeat_interleave(wl.next_n)
    cols = torch.arange(out.shape[1], device="cuda")
    for r0 in range(0, wl.rows, 64):
        blk = bits[r0 : r0 + 64]
        untouched = (blk == SENTINEL_BITS)
        assert bool((~untouched).any(dim=1).all()), f"untouched row in [{r0}, {r0 + 64})"
        past = cols[None, :] >= ctx_rows[r0 : r0 + 64, None]
        assert not bool((past & ~untouched).any()), f"write past a context in [{r0}, {r0 + 64})"
    # every request vs the oracle (rows on both sides of the 2^31-byte boundary)
    ref = oracle_rows(wl)
    worst = check_rows(wl, out, ref)
    say(f"config3 worst rel err {worst:.3e} over all {wl.rows} rows")
    idx = topk_gpu(gpu_lib, wl, out, ctx=d["ctx"])
    check_topk(idx, ref, wl.topk)


@pytest.fixture(scope="module")
def cfg4():
    return synth.make_config(4)


def test_config4_small_pages_compact_and_padded(gpu_lib, cfg4):
    wl = cfg4
    d = upload(wl)
    out = run_logits(gpu_lib, wl, d, label="compact")
    dp = dict(d)
    dp["tab"] = torch.from_numpy(wl.extra_tables["padded"]).cuda()
    outp = run_logits(gpu_lib, wl, dp, label="padded")
    assert torch.equal(out.view(torch.int32), outp.view(torch.int32))
    boundary = -(-(2 ** 31) // (wl.page_size * (wl.head_dim + 4)))
    npg = (wl.context_lens.astype(np.int64) + 7) // 8
    high = [b for b in range(wl.batch) if (wl.block_tables[b, : npg[b]] >= boundary).any()]
    assert high
    zero = [b for b in range(wl.batch) if wl.context_lens[b] == 0]
    # every request vs the oracle, including those reading pages past 2^31 bytes
    ref = oracle_rows(wl)
    worst = check_rows(wl, out, ref)
    check_untouched_rows(wl, out, zero)
    say(f"config4 worst rel err {worst:.3e} over all {wl.rows} rows ({len(high)} requests "
        f"read pages past 2^31 bytes)")
    idx = topk_gpu(gpu_lib, wl, out, ctx=d["ctx"])
    check_topk(idx, ref, wl.topk)
    zrows = [r for b in zero for r in range(b * wl.next_n, (b + 1) * wl.next_n)]
    assert bool((idx[zrows] == -1).all())


def token_level_table(wl, table=None):
    """The same cache rows addressed one token per page: entry t of request b is
    the pool row of its token t (page * page_size + t % page_size); entries past
    the context point at the poison page's first row."""
    tab = wl.block_tables if table is None else table
    ctx = wl.context_lens.astype(np.int64)
    out = np.full((wl.batch, max(1, int(ctx.max()))), wl.poison_page * wl.page_size, dtype=np.int64)
    for b in range(wl.batch):
        t = np.arange(ctx[b])
        out[b, : ctx[b]] = tab[b, t // wl.page_size] * wl.page_size + t % wl.page_size
    return out


def test_token_level_table_matches_paged(gpu_lib, cfg4):
    """Reading the 8-token-page workload's pool through a token-level table
    (page_size 1) gives bit-identical logits: per-token arithmetic does not
    depend on how the rows are paged.  The pool holds 16.7M rows, so token ids
    pass 2^31 / 132 and their byte offsets pass 2^31."""
    wl = cfg4
    d = upload(wl)
    out8 = run_logits(gpu_lib, wl, d, label="8-token pages")
    tok = token_level_table(wl)
    assert tok.max() >= 2 ** 31 // (wl.head_dim + 4)
    out1 = new_out(wl.rows, wl.out_row_stride)
    say(f"[gpu] paged_mqa_logits token-level table {tok.shape}")
    gpu_lib.paged_mqa_logits(d["q"], d["kv"], d["w"], d["ctx"], torch.from_numpy(tok).cuda(), 1,
                             wl.next_n, out1)
    torch.cuda.synchronize()
    assert torch.equal(out8.view(torch.int32), out1.view(torch.int32))


def test_config5_long_context(gpu_lib):
    wl = synth.make_config(5)
    d = upload(wl)
    out = run_logits(gpu_lib, wl, d)
    ref = oracle_rows(wl)
    worst = check_rows(wl, out, ref)
    say(f"config5 worst rel err {worst:.3e} over all {wl.rows} rows")
    idx = topk_gpu(gpu_lib, wl, out, ctx=d["ctx"])
    check_topk(idx, ref, wl.topk)


@pytest.mark.parametrize("ties", [0, 3])
def test_topk_synthetic_rows(gpu_lib, ties):
    """The top-k alone on seeded score rows: exact sets (same fp32 inputs on both
    sides), lowest indices among equal scores, every row length class."""
    lens = [0, 1, 100, 2047, 2048, 2049, 4000, 8192, 8193, 16384, 16385, 32768, 32769,
            40000, 131072]
    width = max(lens)
    dense = synth.make_logit_rows(len(lens), width, lens, seed=5, ties=ties)
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    logits = torch.from_numpy(dense).cuda()
    for k in (1, 7, 2048):
        idx = torch.full((len(lens), k), -7, dtype=torch.int32, device="cuda")
        say(f"[gpu] topk_per_row synthetic ties={ties} k={k}")
        gpu_lib.topk_per_row(logits, ctx, k, idx, next_n=1)
        torch.cuda.synchronize()
        want = oracle.topk_per_row([dense[r, :n] for r, n in enumerate(lens)], k)
        got = idx.cpu().numpy()
        for r, n in enumerate(lens):
            m = min(k, n)
            assert sorted(got[r, :m].tolist()) == sorted(want[r, :m].tolist()), f"row {r} n={n} k={k}"
            assert np.all(got[r, m:] == -1)


@pytest.mark.parametrize("split", [True, False])
def test_topk_special_rows(gpu_lib, split):
    """Rows the score distribution never produces but the op accepts: one value
    repeated (every key ties), both zeros (equal scores), infinities, subnormals
    and both signs, extremes whose difference overflows, a heavy tail, values a
    few ulps apart, at lengths on each side of the register-resident limits.
    With a full workspace the 40000- and 100000-score rows are split (and the
    shorter rows go through the split grid: at k = 2048 the grid that holds
    16 floats a thread, whose 100000-score rows have segments of 12500; at
    smaller k the two-per-CU grid and merge); with none, every row is one
    workgroup's, the shorter rows through the one-pass select on floats and
    its fallbacks."""
    rng = np.random.default_rng(11)
    rows = []
    for n in (3000, 9000, 40000, 100000):
        rows.append(np.full(n, 1.5, dtype=np.float32))
        z = np.where(rng.random(n) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
        z[rng.choice(n, 50, replace=False)] = 1.0
        rows.append(z)
        mix = rng.standard_normal(n).astype(np.float32) * np.float32(1e30)
        pick = rng.choice(n, 40, replace=False)
        mix[pick[:10]] = np.inf
        mix[pick[10:20]] = -np.inf
        mix[pick[20:30]] = np.float32(1e-45)
        mix[pick[30:40]] = np.float32(-1e-45)
        rows.append(mix)
        two = np.where(rng.random(n) < 0.7, np.float32(-2.0), np.float32(3.0)).astype(np.float32)
        rows.append(two)
        # finite, but the span between the extremes overflows float32
        rows.append(np.clip(rng.standard_normal(n) * 2e38, -3.4e38, 3.4e38).astype(np.float32))
        # a heavy tail: most scores share the lowest value bucket
        rows.append(np.exp(rng.standard_normal(n) * 6.0).astype(np.float32))
        # eight distinct values one ulp apart
        rows.append((np.float32(1.0) + rng.integers(0, 8, n).astype(np.float32)
                     * np.float32(2.0 ** -23)).astype(np.float32))
        # subnormals only (the bucket scale would overflow)
        rows.append((rng.integers(-20, 21, n).astype(np.float32) * np.float32(1e-45)).astype(np.float32))
    lens = [len(r) for r in rows]
    width = max(lens)
    dense = np.full((len(rows), width), -np.inf, dtype=np.float32)
    for i, r in enumerate(rows):
        dense[i, : len(r)] = r
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    logits = torch.from_numpy(dense).cuda()
    for k in (1, 100, 2048):
        idx = torch.full((len(rows), k), -7, dtype=torch.int32, device="cuda")
        say(f"[gpu] topk_per_row special rows k={k} split={split}")
        ws = None if split else torch.empty(0, dtype=torch.uint8, device="cuda")
        gpu_lib.topk_per_row(logits, ctx, k, idx, next_n=1, workspace=ws)
        torch.cuda.synchronize()
        want = oracle.topk_per_row(rows, k)
        got = idx.cpu().numpy()
        for r, n in enumerate(lens):
            m = min(k, n)
            assert sorted(got[r, :m].tolist()) == sorted(want[r, :m].tolist()), f"row {r} n={n} k={k}"
            assert np.all(got[r, m:] == -1)


@pytest.mark.parametrize("shape", [
    dict(batch=5, next_n=1, heads=64, page_size=64),   # single-wave geometry, page-sized items
    dict(batch=64, next_n=2, heads=32, page_size=8),   # single-wave geometry, small pages
    dict(batch=5, next_n=3, heads=64, page_size=8),    # persistent geometry, 192-row units
    dict(batch=3, next_n=1, heads=128, page_size=256),  # persistent geometry, 128-row units
    dict(batch=3, next_n=4, heads=128, page_size=64),  # shared-ring geometry
])
def test_all_contexts_empty(gpu_lib, shape):
    """A batch whose every context is empty: nothing is scored, every output
    row keeps its sentinel, and the top-k rows are all -1."""
    wl = synth.build_workload("empty", head_dim=128, table="permuted", topk=16, seed=5,
                              context_lens=[0] * shape["batch"], **shape)
    wl.out_row_stride = 512
    d = upload(wl)
    out = run_logits(gpu_lib, wl, d, label="all empty")
    check_untouched_rows(wl, out, range(wl.batch))
    idx = topk_gpu(gpu_lib, wl, out, ctx=d["ctx"])
    assert np.all(idx.cpu().numpy() == -1)


@pytest.mark.parametrize("heads", [16, 32, 64, 128])
def test_short_rows_meet_row_tolerance(gpu_lib, heads):
    """Rows that see only a few tokens, with sign-cancelling weights: the row's
    largest score can be small next to its terms, which is where an inexact sum
    of products would show."""
    lens = [1, 2, 3, 4, 5, 8, 16, 127, 128, 129, 130, 131] * 40
    wl = synth.build_workload("short", batch=len(lens), next_n=2, heads=heads, head_dim=128,
                              page_size=16, context_lens=lens, table="permuted", topk=4,
                              seed=heads)
    d = upload(wl)
    out = run_logits(gpu_lib, wl, d)
    worst = check_rows(wl, out, oracle_rows(wl))
    say(f"short rows H={heads}: worst rel err {worst:.3e}")


def test_graph_replay_matches_eager(gpu_lib, cfg2):
    """The step captured as a HIP graph (as the benchmark replays it) gives the
    eager results on every replay, with eager work and syncs in between."""
    wl = cfg2
    d = upload(wl)
    out_e = run_logits(gpu_lib, wl, d, label="eager")
    idx_e = topk_gpu(gpu_lib, wl, out_e, ctx=d["ctx"])
    out = new_out(wl.rows, wl.out_row_stride)
    idx = torch.full((wl.rows, wl.topk), -7, dtype=torch.int32, device="cuda")
    g = torch.cuda.CUDAGraph()
    say("[gpu] capture logits + topk graph")
    with torch.cuda.graph(g):
        gpu_lib.paged_mqa_logits(d["q"], d["kv"], d["w"], d["ctx"], d["tab"], wl.page_size,
                                 wl.next_n, out)
        gpu_lib.topk_per_row(out, d["ctx"], wl.topk, idx, next_n=wl.next_n)
    want = np.sort(idx_e.cpu().numpy(), axis=1)
    for rep in range(4):
        out.view(torch.int32).fill_(SENTINEL_BITS)
        idx.fill_(-7)
        torch.cuda.synchronize()
        say(f"[gpu] graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), out_e.view(torch.int32)), f"replay {rep}"
        assert np.array_equal(np.sort(idx.cpu().numpy(), axis=1), want), f"replay {rep}"
        run_logits(gpu_lib, wl, d, label="eager between replays")


def test_check_inputs_flags_device_preconditions(gpu_lib):
    """The debug check of device-resident preconditions: clean inputs pass;
    an out-of-pool id, a negative id and contexts longer than the output row
    or the table row are reported (lowest request first); entries past a
    context are never looked at."""
    wl = synth.make_config(2)
    tab = wl.block_tables.copy()
    ctx = wl.context_lens.copy()
    num_pages = wl.kv_cache.shape[0] if wl.kv_cache.ndim > 1 else wl.kv_cache.size // (wl.page_size * 132)
    npg = (ctx.astype(np.int64) + wl.page_size - 1) // wl.page_size
    for b in range(wl.batch):
        tab[b, npg[b]:] = -5  # unused entries: anything goes
    d_ctx = torch.from_numpy(ctx).cuda()
    say("[gpu] pmqa_check_inputs clean")
    assert gpu_lib.check_inputs(d_ctx, torch.from_numpy(tab).cuda(), wl.page_size,
                                wl.out_row_stride, num_pages) == (0, wl.batch)
    bad = tab.copy()
    bad[7, 0] = num_pages             # past the pool
    bad[3, npg[3] - 1] = -1           # negative id, last used entry
    bad_ctx = ctx.copy()
    bad_ctx[20] = wl.out_row_stride + 1               # longer than the output row
    bad_ctx[40] = bad.shape[1] * wl.page_size + 64    # longer than the table row
    say("[gpu] pmqa_check_inputs planted")
    got = gpu_lib.check_inputs(torch.from_numpy(bad_ctx).cuda(), torch.from_numpy(bad).cuda(),
                               wl.page_size, wl.out_row_stride, num_pages)
    assert got == (4, 3), got
    # the same pool through token-level tables (page_size 1): ids are pool rows
    tok = token_level_table(wl)
    rows = num_pages * wl.page_size
    say("[gpu] pmqa_check_inputs token-level clean")
    assert gpu_lib.check_inputs(d_ctx, torch.from_numpy(tok).cuda(), 1, wl.out_row_stride,
                                rows) == (0, wl.batch)
    tok_bad = tok.copy()
    tok_bad[11, int(ctx[11]) - 1] = rows  # the last used entry past the pool
    say("[gpu] pmqa_check_inputs token-level planted")
    assert gpu_lib.check_inputs(d_ctx, torch.from_numpy(tok_bad).cuda(), 1, wl.out_row_stride,
                                rows) == (1, 11)


FLAT = [
    # batch > 64 (the item search walks several 64-request chunks) and more
    # 64-token iterations than one residency of single-wave workgroups (4096),
    # so shares of two items occur, some crossing into the next request
    dict(batch=200, next_n=1, heads=64, page_size=64, ctx_range=(1280, 2560), stride=2560),
    dict(batch=160, next_n=2, heads=32, page_size=16, ctx_range=(1200, 3200), stride=3200),
    dict(batch=130, next_n=4, heads=16, page_size=128, ctx_range=(2000, 4032), stride=4032,
         zero_every=10),
]


@pytest.mark.parametrize("case", range(len(FLAT)))
def test_flat_geometry_two_item_shares(gpu_lib, case):
    """Decode shapes launched on the flat geometry (every row of a request in
    one wave, at most 8192 possible iterations), every row against the oracle."""
    kw = dict(FLAT[case])
    stride = kw.pop("stride")
    ps = kw["page_size"]
    wl = synth.build_workload(f"flat{case}", head_dim=128, table="permuted", topk=512,
                              seed=11 + case, table_width=-(-stride // ps), **kw)
    wl.out_row_stride = stride
    max_iters = wl.batch * (-(-min(wl.block_tables.shape[1] * ps, stride) // 64))
    items = int(sum(-(-int(c) // 64) for c in wl.context_lens))
    assert wl.heads * wl.next_n <= 64 and max_iters <= 8192 and items > 4096
    d = upload(wl)
    out = run_logits(gpu_lib, wl, d, label=f"items={items}")
    ref = oracle_rows(wl)
    worst = check_rows(wl, out, ref)
    say(f"flat case {case}: {items} items, worst rel err {worst:.3e}")
    idx = topk_gpu(gpu_lib, wl, out, ctx=d["ctx"])
    check_topk(idx, ref, wl.topk)


def test_randomized_small_workloads(gpu_lib):
    """Seeded random shapes across every axis the kernels dispatch on (heads,
    next_n, page size, batch, context mix incl. zeros, output stride, table
    width), every row against the oracle, logits and top-k."""
    rng = np.random.default_rng(2024)
    for trial in range(12):
        heads = int(rng.choice([16, 32, 64, 128]))
        next_n = int(rng.integers(1, 6))
        ps = int(rng.choice([8, 16, 32, 64, 128, 256]))
        batch = int(rng.integers(1, 9))
        ctx = rng.integers(0, 1300, size=batch)
        ctx[rng.random(batch) < 0.2] = 0
        wl = synth.build_workload(f"rand{trial}", batch=batch, next_n=next_n, heads=heads,
                                  head_dim=128, page_size=ps, context_lens=ctx.tolist(),
                                  table="permuted", topk=int(rng.choice([1, 32, 100])),
                                  seed=int(rng.integers(1 << 30)),
                                  table_width=int(-(-max(1, ctx.max()) // ps)) + int(rng.integers(0, 3)))
        wl.out_row_stride = int(max(1, ctx.max())) + int(rng.integers(0, 50))
        say(f"[gpu] random trial {trial}: H={heads} next_n={next_n} ps={ps} B={batch} "
            f"ctx={ctx.tolist()} stride={wl.out_row_stride} k={wl.topk}")
        d = upload(wl)
        out = run_logits(gpu_lib, wl, d, label=f"trial={trial}")
        ref = oracle_rows(wl)
        check_rows(wl, out, ref)
        idx = topk_gpu(gpu_lib, wl, out, ctx=d["ctx"])
        check_topk(idx, ref, wl.topk)


# One shape per logits kernel family (the flat single-wave grid, the persistent
# grid at 64 and 128 heads, the shared K ring at 128 heads with 2 or 4 rows).
FAMILIES = [
    dict(heads=64, next_n=1, family="logits_flat_kernel"),
    dict(heads=64, next_n=3, family="logits_kernel"),
    dict(heads=128, next_n=1, family="logits_kernel"),
    dict(heads=128, next_n=2, family="logits_shared_kernel"),
    dict(heads=128, next_n=4, family="logits_shared_kernel"),
]


@pytest.mark.parametrize("page_size", [8, 64])
@pytest.mark.parametrize("case", range(len(FAMILIES)))
def test_signed_and_nan_scales(gpu_lib, case, page_size):
    """Scales of both signs: 64-token blocks whose scales are all >= 0 sit next
    to blocks with negated scales, so iterations take both the factored form
    (s * relu(dot)) and the literal one (relu(s * dot)); rows shorter than 128
    visible tokens (the exact-sum path) and longer ones.  Then NaN scales: the
    rows that see such a token score NaN exactly there, as the oracle does."""
    c = FAMILIES[case]
    lens = [1, 5, 40, 127, 128, 131, 200, 700, 1500, 2100]
    for nan_tokens in (0, 2):
        wl = synth.build_workload(f"signed{case}", batch=len(lens), next_n=c["next_n"],
                                  heads=c["heads"], head_dim=128, page_size=page_size,
                                  context_lens=lens, table="permuted", topk=100,
                                  seed=31 + case, neg_scale_blocks=0.4,
                                  nan_scale_tokens=nan_tokens)
        wl.out_row_stride = 2112
        name = gpu_lib.logits_kernel(wl.batch, wl.next_n, page_size, wl.out_row_stride, wl.heads,
                                     wl.block_tables.shape[1])
        assert name.startswith(c["family"] + "<"), name
        npg = (wl.context_lens.astype(np.int64) + page_size - 1) // page_size
        scales = np.concatenate([oracle.gather_request(wl.kv_cache, wl.block_tables[b],
                                                       int(wl.context_lens[b]), page_size, 128)[1]
                                 for b in range(wl.batch)])
        assert (scales < 0).any() and (scales > 0).any() and npg.sum() > 0
        d = upload(wl)
        out = run_logits(gpu_lib, wl, d, label=f"{name} nan_tokens={nan_tokens}")
        ref = oracle_rows(wl)
        worst = check_rows(wl, out, ref)
        say(f"{name} ps={page_size} nan_tokens={nan_tokens}: worst rel err {worst:.3e}")
        if nan_tokens == 0:
            idx = topk_gpu(gpu_lib, wl, out, ctx=d["ctx"])
            check_topk(idx, ref, wl.topk)
        else:
            assert any(np.isnan(r).any() for r in ref if r is not None)


@pytest.mark.parametrize("case", [0, 1, 3])
def test_negative_context_lens_count_as_zero(gpu_lib, case):
    """Negative context lengths count as 0 (as the oracle's visible length does):
    those requests' rows stay untouched and their top-k rows are all -1; the
    other requests are unaffected."""
    c = FAMILIES[case]
    lens = [0, 300, 0, 0, 77, 1000]
    neg = np.array([-5, 300, -1, -(2 ** 31), 77, 1000], dtype=np.int32)
    wl = synth.build_workload("negctx", batch=len(lens), next_n=c["next_n"], heads=c["heads"],
                              head_dim=128, page_size=64, context_lens=lens, table="permuted",
                              topk=32, seed=77)
    wl.out_row_stride = 1024
    wl.context_lens = neg
    d = upload(wl)
    out = run_logits(gpu_lib, wl, d, label="negative context lengths")
    ref = oracle_rows(wl)
    check_rows(wl, out, ref)
    check_untouched_rows(wl, out, [0, 2, 3])
    idx = topk_gpu(gpu_lib, wl, out, ctx=d["ctx"])
    check_topk(idx, ref, wl.topk)
    rows = [r for b in (0, 2, 3) for r in range(b * wl.next_n, (b + 1) * wl.next_n)]
    assert bool((idx[rows] == -1).all())


@pytest.mark.parametrize("case", [0, 1, 3])
def test_contexts_past_the_table_row_and_output_row(gpu_lib, case):
    """Contexts longer than the output row and than the table row (a broken
    precondition) are contained: a row is scored on [0, min(visible, ctx_eff)),
    ctx_eff = min(ctx, table width * page_size, row stride), -inf up to ctx_eff,
    and nothing is written past its row (the columns past ctx_eff and a guard
    row after the output keep their sentinel).  The scores are those of the
    same tokens under a context the table covers."""
    c = FAMILIES[case]
    ps, stride = 64, 1024
    covered = [100, 900, 1280, 1280, 1280]        # what the 20-page table rows hold
    true_ctx = [100, 900, 1300, 2000, 1 << 20]     # what the caller claims
    wl = synth.build_workload("pastrow", batch=len(covered), next_n=c["next_n"],
                              heads=c["heads"], head_dim=128, page_size=ps,
                              context_lens=covered, table="permuted", topk=16, seed=5)
    assert wl.block_tables.shape[1] * ps == 1280
    ref = oracle_rows(wl)  # per-token scores over the covered tokens
    d = upload(wl)
    d["ctx"] = torch.tensor(true_ctx, dtype=torch.int32, device="cuda")
    big = new_out(wl.rows + 1, stride)
    out = big[: wl.rows]
    say(f"[gpu] paged_mqa_logits past-row contexts {true_ctx} stride={stride} ({c['family']})")
    gpu_lib.paged_mqa_logits(d["q"], d["kv"], d["w"], d["ctx"], d["tab"], ps, wl.next_n, out)
    torch.cuda.synchronize()
    bits = big.view(torch.int32).cpu().numpy()
    vals = big.cpu().numpy()
    assert np.all(bits[wl.rows] == SENTINEL_BITS), "guard row written"
    nn = wl.next_n
    for b in range(wl.batch):
        ctx_eff = min(true_ctx[b], 1280, stride)
        for j in range(nn):
            r = b * nn + j
            vis = min(max(true_ctx[b] - nn + j + 1, 0), ctx_eff)
            want = ref[r][:vis]
            assert len(ref[r]) >= vis
            got = vals[r, :vis].astype(np.float64)
            tol = 2e-4 * float(np.max(np.abs(want))) if vis else 0.0
            assert np.all(np.abs(got - want) <= tol), f"row {r}"
            assert np.all(bits[r, vis:ctx_eff] == np.int32(-8388608)), f"row {r}: mask"
            assert np.all(bits[r, ctx_eff:] == SENTINEL_BITS), f"row {r}: write past ctx_eff"


def test_binding_rejects_an_empty_table_row(gpu_lib):
    """A [B, 0] block table holds no page: the binding refuses it (B > 0) before
    anything is enqueued, and accepts it for an empty batch."""
    wl = synth.build_workload("w0", batch=2, next_n=1, heads=64, head_dim=128, page_size=64,
                              context_lens=[10, 20], table="permuted", topk=4, seed=1)
    d = upload(wl)
    out = new_out(2, 64)
    with pytest.raises(ValueError):
        gpu_lib.paged_mqa_logits(d["q"], d["kv"], d["w"], d["ctx"],
                                 torch.empty((2, 0), dtype=torch.int64, device="cuda"), 64, 1, out)
    assert bool((out.view(torch.int32) == SENTINEL_BITS).all())
    e = torch.empty((0, 0), dtype=torch.int64, device="cuda")
    gpu_lib.paged_mqa_logits(d["q"][:0], d["kv"], d["w"][:0], d["ctx"][:0], e, 64, 1,
                             new_out(0, 64))


def _topk_exact(gpu_lib, dense, lens, k, workspace, label):
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    logits = torch.from_numpy(dense).cuda()
    idx = torch.full((len(lens), k), -7, dtype=torch.int32, device="cuda")
    say(f"[gpu] topk_per_row {label} k={k} workspace={workspace.numel()} B")
    gpu_lib.topk_per_row(logits, ctx, k, idx, next_n=1, workspace=workspace)
    torch.cuda.synchronize()
    want = oracle.topk_per_row([dense[r, :n] for r, n in enumerate(lens)], k)
    got = idx.cpu().numpy()
    for r, n in enumerate(lens):
        m = min(k, n)
        assert sorted(got[r, :m].tolist()) == sorted(want[r, :m].tolist()), f"row {r} n={n} k={k}"
        assert np.all(got[r, m:] == -1)
    return got


@pytest.mark.parametrize("ties", [0, 3])
def test_topk_segments_and_workspace_sizes(gpu_lib, ties):
    """Rows longer than one segment are split over workgroups into candidates
    in the workspace (segments of at most 8192 scores while the grid has
    room, else of at most 16384), then merged: exact sets for every
    workspace size (none: one workgroup per row, streamed; room for a few
    segments; the full split), with many equal scores at the k-th boundary
    spread over segments (lowest indices win), at lengths on both sides of
    the segment multiples and of the switch to longer segments."""
    lens = [16383, 16384, 16385, 20000, 32768, 32769, 50000, 65536, 98304, 131072, 200000, 5,
            8193, 24577, 65537]
    width = max(lens)
    dense = synth.make_logit_rows(len(lens), width, lens, seed=9, ties=ties)
    rows = len(lens)
    for k in (1, 7, 100, 2048):
        # none; room for 4 segments of 8192 (at k = 2048 the merge of at most
        # 8192 candidates, which streams rows longer than 4 * 16384 itself);
        # room for 5; the full split
        sizes = [0, gpu_lib.topk_workspace_size(rows, k, 32768),
                 gpu_lib.topk_workspace_size(rows, k, 40000),
                 gpu_lib.topk_workspace_size(rows, k, width)]
        assert 0 < sizes[1] < sizes[2] < sizes[3]
        for nbytes in sizes:
            ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
            _topk_exact(gpu_lib, dense, lens, k, ws, f"segments ties={ties}")


def test_topk_merge_graph_replay(gpu_lib):
    """The two top-k launches (segments, then the merge) captured in a graph
    give the eager indices on every replay, with eager work in between."""
    lens = [70000, 131072, 1000, 40000]
    dense = synth.make_logit_rows(len(lens), max(lens), lens, seed=4, ties=0)
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    logits = torch.from_numpy(dense).cuda()
    k = 2048
    ws = torch.empty(gpu_lib.topk_workspace_size(len(lens), k, max(lens)), dtype=torch.uint8,
                     device="cuda")
    eager = _topk_exact(gpu_lib, dense, lens, k, ws, "eager before capture")
    idx = torch.full((len(lens), k), -7, dtype=torch.int32, device="cuda")
    g = torch.cuda.CUDAGraph()
    say("[gpu] capture the two top-k launches")
    with torch.cuda.graph(g):
        gpu_lib.topk_per_row(logits, ctx, k, idx, next_n=1, workspace=ws)
    for rep in range(3):
        idx.fill_(-7)
        torch.cuda.synchronize()
        say(f"[gpu] top-k graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(np.sort(idx.cpu().numpy(), axis=1), np.sort(eager, axis=1))
        _topk_exact(gpu_lib, dense, lens, k, ws, "eager between replays")


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_topk_random_shapes(gpu_lib, seed):
    """Random batches of rows (lengths from 0 to past the split thresholds,
    a few with many ties; bell-shaped, one-sided or two-sided heavy-tailed
    scores, the tails crowding a few value buckets so that the select cuts
    them again or falls back), random k, stride and workspace size (none, part
    of a full split, a full split): exact sets against the oracle every
    time."""
    rng = np.random.default_rng(1000 + seed)
    for trial in range(4):
        rows = int(rng.integers(1, 40))
        k = int(rng.choice([1, 3, 64, 100, 500, 1024, 2047, 2048]))
        cls = rng.integers(0, 4, rows)
        lens = np.where(cls == 0, rng.integers(0, 3000, rows),
                        np.where(cls == 1, rng.integers(3000, 16385, rows),
                                 np.where(cls == 2, rng.integers(16385, 70000, rows),
                                          rng.integers(0, 2 * k + 2, rows)))).astype(np.int64)
        stride = int(max(1, lens.max()) + rng.integers(0, 300))
        dense = synth.make_logit_rows(rows, stride, lens.tolist(), seed=int(rng.integers(1 << 30)),
                                      ties=int(rng.choice([0, 0, 4])))
        tail = int(rng.integers(0, 3))
        if tail == 1:    # one-sided heavy tail (positions past a row are never read)
            dense = np.exp(dense.astype(np.float64) * 4.0).astype(np.float32)
        elif tail == 2:  # heavy tails on both sides
            dense = np.sinh(dense.astype(np.float64) * 4.0).astype(np.float32)
        full = gpu_lib.topk_workspace_size(rows, k, stride)
        nbytes = int(rng.choice([0, full // 3, full])) if full else 0
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        say(f"[gpu] top-k random shapes seed={seed} trial={trial} rows={rows} k={k} "
            f"stride={stride} workspace={nbytes}/{full} tail={tail}")
        _topk_exact(gpu_lib, dense, lens.tolist(), k, ws, f"random seed={seed} trial={trial}")
