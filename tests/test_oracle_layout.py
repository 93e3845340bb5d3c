"""Pins of the oracle's preshuffled page layout (CPU only).

* hand-derived byte positions (tests/golden/preshuffled_layout.json), with a
  planted mistake (the (half, quarter) groups taken in the other order) that
  must fail them;
* for every page size the layout is a permutation of the page's bytes (each
  byte of a page is the home of exactly one code or scale byte);
* the same K rows written by the oracle's K-cache writer in both layouts give
  the same codes and scales back and bit-identical logits.
"""
import numpy as np
import pytest

import oracle
import oracle.layout as olay
from tests.handcase import load_golden


@pytest.mark.parametrize("case", load_golden("preshuffled_layout.json")["cases"],
                         ids=lambda c: f"ps{c['page_size']}-slot{c['slot']}")
def test_golden_positions(case):
    v, s = oracle.preshuffled_offsets([case["slot"]], case["page_size"])
    assert int(v[0, case["d"]]) == case["value_byte"]
    assert int(s[0]) == case["scale_byte"]


def test_planted_group_order_fails_the_golden(monkeypatch):
    def swapped(slots, page_size, head_dim=128):
        s = np.asarray(slots, dtype=np.int64).reshape(-1)
        P, R, rec = np.int64(page_size), np.int64(olay.tile_rows(page_size)), np.int64(head_dim + 4)
        page, u = s // P, s % P
        ts = page * P * rec + (u // R) * R * rec
        m = u % R
        d = np.arange(head_dim, dtype=np.int64)
        h, q, b = d // 64, (d % 64) // 16, d % 16
        vals = ts[:, None] + ((q * 2 + h)[None, :] * R + m[:, None]) * 16 + b[None, :]  # wrong order
        return vals, ts + 128 * R + 4 * m
    cases = load_golden("preshuffled_layout.json")["cases"]
    bad = sum(int(swapped([c["slot"]], c["page_size"])[0][0, c["d"]]) != c["value_byte"] for c in cases)
    assert bad >= 2  # d = 101 in two of the cases; the other two coincide under the swap


@pytest.mark.parametrize("page_size", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_layout_is_a_permutation_of_each_page(page_size):
    rec = 132
    slots = np.arange(2 * page_size)  # two pages
    v, s = oracle.preshuffled_offsets(slots, page_size)
    home = np.concatenate([v.reshape(-1), (s[:, None] + np.arange(4)[None, :]).reshape(-1)])
    assert np.array_equal(np.sort(home), np.arange(2 * page_size * rec))


@pytest.mark.parametrize("page_size", [8, 16, 64, 256])
def test_both_layouts_hold_the_same_tokens(page_size):
    rng = np.random.default_rng(page_size)
    n_pages, D = 4, 128
    n = n_pages * page_size
    k = (rng.standard_normal((n, D)) * np.exp(rng.standard_normal((n, 1)))).astype(np.float32)
    slots = rng.permutation(n)
    rec_pool = np.zeros(n * 132, np.uint8)
    pre_pool = np.zeros(n * 132, np.uint8)
    oracle.write_k_cache(rec_pool, k, slots, D)
    oracle.write_k_cache(pre_pool, k, slots, D, layout="preshuffled", page_size=page_size)
    assert not np.array_equal(rec_pool, pre_pool)
    table = np.arange(n_pages, dtype=np.int64)[rng.permutation(n_pages)]
    ctx = n - 3
    k_r, s_r = oracle.gather_request(rec_pool, table, ctx, page_size, D)
    k_p, s_p = oracle.gather_request(pre_pool, table, ctx, page_size, D, layout="preshuffled")
    assert np.array_equal(k_r, k_p) and np.array_equal(s_r, s_p)
    H, nn = 4, 2
    q = rng.integers(0, 256, size=(nn, H, D), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x3C
    w = rng.standard_normal((nn, H)).astype(np.float32)
    ctxs = np.array([ctx], np.int32)
    a = oracle.paged_mqa_logits(q, rec_pool, w, ctxs, table[None, :], page_size, nn)
    b = oracle.paged_mqa_logits(q, pre_pool, w, ctxs, table[None, :], page_size, nn,
                                layout="preshuffled")
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
