"""Checks of the seeded input generator (CPU only): layout, determinism, the
structure each workload asks for (table kinds, zero contexts, pages past 2^31
bytes), and that poison fills every record no request owns."""
import numpy as np
import pytest

import synth


def test_deterministic_and_seeded():
    a = synth.make_config(1)
    b = synth.make_config(1)
    c = synth.make_config(1, seed=1)
    assert np.array_equal(a.kv_cache, b.kv_cache) and np.array_equal(a.q, b.q)
    assert not np.array_equal(a.q, c.q)


def test_config1_shape_and_identity_table():
    wl = synth.make_config(1)
    assert (wl.batch, wl.next_n, wl.heads, wl.head_dim, wl.page_size) == (2, 1, 64, 128, 64)
    assert wl.context_lens.tolist() == [1000, 1024]
    assert wl.block_tables[0, :16].tolist() == list(range(16))
    assert wl.block_tables[1, :16].tolist() == list(range(16, 32))
    assert wl.q.shape == (2, 64, 128) and wl.weights.shape == (2, 64)
    assert (wl.weights >= 0).all() and (wl.weights < 1).all()
    assert wl.topk == 256


def test_config2_permuted_pool():
    wl = synth.make_config(2)
    ctx = wl.context_lens
    assert ctx.min() >= 1 and ctx.max() <= 8192 and wl.num_pages == 10_000
    used = np.concatenate([wl.block_tables[b, : (int(c) + 63) // 64] for b, c in enumerate(ctx)])
    assert len(np.unique(used)) == len(used)  # no page shared
    assert wl.poison_page not in set(used.tolist())
    assert not np.array_equal(np.sort(used), used)  # permuted


def test_quantisation_scale_and_range():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 128)).astype(np.float32)
    x[3] = 0
    codes, scale = synth.quantize_tokens(x)
    assert scale[3] == 1.0
    import torch
    deq = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert np.isfinite(deq).all() and np.abs(deq).max() <= 448
    # the largest element of each nonzero token maps to +-448
    nz = np.arange(50) != 3
    assert np.all(np.abs(deq[nz]).max(axis=1) == 448)


def test_poison_fills_unowned_records():
    wl = synth.build_workload("t", batch=3, next_n=1, heads=16, head_dim=32, page_size=8,
                              context_lens=[5, 0, 17], table="permuted", pool_pages=12, seed=0)
    rec = 36
    recs = wl.kv_cache.reshape(-1, rec)
    owned = set()
    for b, c in enumerate(wl.context_lens):
        for t in range(int(c)):
            owned.add(int(wl.block_tables[b, t // 8]) * 8 + t % 8)
    for i in range(recs.shape[0]):
        if i not in owned:
            assert np.all(recs[i, :32] == 0x7F)
            assert np.isnan(recs[i, 32:].view("<f4")[0])
    # unused table entries point at the poison page
    assert wl.block_tables[1, 0] == wl.poison_page
    assert wl.block_tables[0, 1] == wl.poison_page


@pytest.mark.slow
def test_config4_small_pages_structure():
    wl = synth.make_config(4)
    ctx = wl.context_lens
    assert wl.page_size == 8 and wl.next_n == 3 and wl.num_pages == 1 << 21
    assert (ctx[::16] == 0).all() and ctx[1:6].tolist() == [1, 7, 8, 9, 65536]
    assert wl.block_tables.shape == (128, 8192)
    assert wl.extra_tables["padded"].shape == (128, 16384)
    boundary = -(-(2 ** 31) // (8 * 132))  # first page whose byte offset passes 2^31
    used = np.concatenate([wl.block_tables[b, : (int(c) + 7) // 8] for b, c in enumerate(ctx)])
    assert (used >= boundary).any()
