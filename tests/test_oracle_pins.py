"""Pins of the CPU oracle against things other than itself (CPU only).

* e4m3fn decoding: every code against torch's float8_e4m3fn cast (a library
  routine) and against the format's published spot values;
* exactness: the oracle's fp64 dots against exact rational brute force
  (fractions.Fraction) on random tiny inputs, including subnormal and max codes;
* worked examples derived by hand (tests/golden/worked_examples.json);
* the textbook reduction: with one head, unit weight and unit scale, and
  non-negative operands, the score is the plain product Q.K^T, checked by an
  integer double loop over the logical tokens.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle.fp8 import E4M3FN_TABLE
from tests.handcase import assemble, expected_value, load_golden


# ---------------------------------------------------------------- fp8 decoding

def test_e4m3fn_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = E4M3FN_TABLE
    nan_ref = np.isnan(ref)
    assert np.array_equal(nan_ref, np.isnan(ours))
    assert np.array_equal(ref[~nan_ref], ours[~nan_ref])
    # exactly two NaN codes, no infinities
    assert nan_ref.sum() == 2 and nan_ref[0x7F] and nan_ref[0xFF]
    assert not np.isinf(ours).any()


@pytest.mark.parametrize("code,value", [
    (0x38, 1.0), (0x40, 2.0), (0x44, 3.0), (0x48, 4.0), (0x30, 0.5), (0x28, 0.25),
    (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x7E, 448.0),
    (0xB8, -1.0), (0xC0, -2.0), (0xC4, -3.0), (0xFE, -448.0), (0x00, 0.0),
])
def test_e4m3fn_spot_values(code, value):
    assert oracle.e4m3fn_to_float64(np.uint8(code)) == value


def test_e4m3fn_negative_zero_and_nan():
    assert math.copysign(1.0, float(E4M3FN_TABLE[0x80])) == -1.0
    assert np.isnan(E4M3FN_TABLE[0x7F]) and np.isnan(E4M3FN_TABLE[0xFF])


# ---------------------------------------------------------------- exactness

def _frac_of_code(c):
    v = float(E4M3FN_TABLE[c])
    return Fraction(v)


def _frac_logit(qc, kc, s, w):
    """Exact rational score for one token: sum_h w_h * relu(s * (q_h . k))."""
    total = Fraction(0)
    for h in range(qc.shape[0]):
        dot = sum((_frac_of_code(a) * _frac_of_code(b) for a, b in zip(qc[h], kc)), Fraction(0))
        y = Fraction(float(s)) * dot
        total += Fraction(float(w[h])) * max(y, Fraction(0))
    return total


def _finite_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E  # keep finite
    return c


@pytest.mark.parametrize("seed", range(6))
def test_dot_exact_against_fractions(seed):
    rng = np.random.default_rng(seed)
    D = [8, 32, 128][seed % 3]
    n = 5
    qc = _finite_codes(rng, (1, 1, D))
    kc = _finite_codes(rng, (n, D))
    k = oracle.e4m3fn_to_float64(kc)
    # unit scale, unit weight, one head: the score is relu(dot), so exactness of
    # the dot shows bit-for-bit
    rows = oracle.request_logits(qc, np.ones((1, 1), np.float32), k, np.ones(n), 1)
    for t in range(n):
        exact = _frac_logit(qc[0], kc[t], 1.0, [1.0])
        assert Fraction(float(rows[0][t])) == exact


def test_dot_exact_cancellation():
    # q = [448, 448, 2^-9 x126], k = [448, -448, 2^-9 x126]: 448^2 cancels and
    # the 126 subnormal products survive exactly: 126 * 2^-18.
    D = 128
    qv = np.array([448.0, 448.0] + [2.0 ** -9] * 126)
    kv = np.array([448.0, -448.0] + [2.0 ** -9] * 126)
    from tests.handcase import codes_of
    qc = codes_of(qv).reshape(1, 1, D)
    kc = codes_of(kv).reshape(1, D)
    rows = oracle.request_logits(qc, np.ones((1, 1), np.float32),
                                 oracle.e4m3fn_to_float64(kc), np.ones(1), 1)
    assert rows[0][0] == 126 * 2.0 ** -18


@pytest.mark.parametrize("seed", range(4))
def test_full_score_close_to_fractions(seed):
    """Several heads, random scales and weights: the only roundings left are the
    fp64 product with the scale and the weighted sum, so the oracle is within a
    few ulps of the exact rational value."""
    rng = np.random.default_rng(100 + seed)
    H, D, n = 4, 16, 6
    qc = _finite_codes(rng, (1, H, D))
    kc = _finite_codes(rng, (n, D))
    # scales of both signs: relu acts on scale * dot, so a negative scale
    # selects the heads whose dot is negative
    s = ((rng.random(n) - 0.5) * 6).astype(np.float32)
    w = rng.standard_normal((1, H)).astype(np.float32)
    rows = oracle.request_logits(qc, w, oracle.e4m3fn_to_float64(kc), s.astype(np.float64), 1)
    for t in range(n):
        exact = _frac_logit(qc[0], kc[t], s[t], w[0])
        mag = sum(abs(Fraction(float(w[0, h]))) for h in range(H)) * 448 * 448 * D * abs(Fraction(float(s[t])))
        assert abs(Fraction(float(rows[0][t])) - exact) <= mag * Fraction(1, 2 ** 50)


def test_negative_scale_golden_rejects_a_factored_relu(monkeypatch):
    """Plant s * relu(dot) (right only for s >= 0) in the oracle: the hand-derived
    negative-scale example must then fail, so the golden pins the order of scale
    and relu."""
    import oracle.paged_mqa as opm

    ex = [e for e in load_golden("worked_examples.json")["examples"]
          if e["name"].startswith("E5_")][0]
    a = assemble(ex)

    def factored(q_req, w_req, k, scale, next_n):
        q = oracle.e4m3fn_to_float64(q_req)
        w = np.asarray(w_req, dtype=np.float64)
        out = []
        for j in range(next_n):
            vis = oracle.visible_len(k.shape[0], next_n, j)
            act = np.maximum(q[j] @ k[:vis].T, 0.0) * scale[None, :vis]
            out.append(w[j] @ act)
        return out

    want = [expected_value(v) for v in ex["expected_rows"][0]]
    rows = oracle.paged_mqa_logits(a["q"], a["kv_cache"], a["weights"], a["context_lens"],
                                   a["block_tables"], a["page_size"], 1)
    assert rows[0].tolist() == want
    monkeypatch.setattr(opm, "request_logits", factored)
    planted = oracle.paged_mqa_logits(a["q"], a["kv_cache"], a["weights"], a["context_lens"],
                                      a["block_tables"], a["page_size"], 1)
    assert planted[0].tolist() != want
    assert planted[0].tolist() == [-0.25, 0.5, 0.0]


# ---------------------------------------------------------------- worked examples

@pytest.mark.parametrize("ex", load_golden("worked_examples.json")["examples"],
                         ids=lambda e: e["name"])
def test_worked_examples(ex):
    a = assemble(ex)
    B = len(ex["requests"])
    nn = a["next_n"]
    stride = max(4, max(r["ctx"] for r in ex["requests"]) + 2)
    sentinel = np.float32(12345.0)
    out = np.full(B * nn * stride, sentinel, dtype=np.float32)
    rows = oracle.paged_mqa_logits(a["q"], a["kv_cache"], a["weights"], a["context_lens"],
                                   a["block_tables"], a["page_size"], nn, out=out,
                                   out_row_stride=stride)
    out2 = out.reshape(B * nn, stride)
    for r, exp in enumerate(ex["expected_rows"]):
        exp = [expected_value(v) for v in exp]
        ctx = ex["requests"][r // nn]["ctx"]
        assert len(exp) == ctx
        got = out2[r, :ctx].astype(np.float64)
        assert np.array_equal(got, np.asarray(exp), equal_nan=True), (r, got, exp)
        assert np.all(out2[r, ctx:] == sentinel)
        if "expected_visible" in ex:
            assert len(rows[r]) == ex["expected_visible"][r]
    for k, exp_sets in ex.get("topk", {}).items():
        idx = oracle.topk_per_row(rows, int(k))
        for r, e in enumerate(exp_sets):
            assert sorted(idx[r].tolist()) == sorted(e)


def test_worked_example_e1_order():
    ex = load_golden("worked_examples.json")["examples"][0]
    a = assemble(ex)
    rows = oracle.paged_mqa_logits(a["q"], a["kv_cache"], a["weights"], a["context_lens"],
                                   a["block_tables"], a["page_size"], 1)
    assert oracle.topk_per_row(rows, 4)[0].tolist() == [2, 0, 1, -1]


# ---------------------------------------------------------------- textbook reduction

@pytest.mark.parametrize("page_size", [1, 2, 4])
def test_single_head_is_plain_product(page_size):
    """H=1, w=1, s=1, non-negative codes: score == sum_d q_d k_td (integer loop)."""
    rng = np.random.default_rng(7)
    D, ctx = 8, 11
    q_int = rng.integers(0, 8, size=D)
    k_int = rng.integers(0, 8, size=(ctx, D))
    from tests.handcase import codes_of
    n_pages = (ctx + page_size - 1) // page_size
    perm = rng.permutation(n_pages + 1)
    ex = {
        "heads": 1, "head_dim": D, "page_size": page_size, "next_n": 1,
        "q": [[q_int.astype(float).tolist()]], "weights": [[1.0]],
        "requests": [{"ctx": ctx, "tokens": k_int.astype(float).tolist(),
                      "scales": [1.0] * ctx, "table": perm[:n_pages].tolist()}],
        "num_pages": n_pages + 1,
    }
    a = assemble(ex)
    rows = oracle.paged_mqa_logits(a["q"], a["kv_cache"], a["weights"], a["context_lens"],
                                   a["block_tables"], page_size, 1)
    expect = [sum(int(q_int[d]) * int(k_int[t, d]) for d in range(D)) for t in range(ctx)]
    assert rows[0].tolist() == [float(e) for e in expect]


def test_one_hot_weight_picks_one_head():
    rng = np.random.default_rng(3)
    H, D, ctx, ps = 4, 16, 9, 4
    qc = _finite_codes(rng, (1, H, D))
    kc = _finite_codes(rng, (ctx, D))
    s = (rng.random(ctx) + 0.5).astype(np.float32)
    k = oracle.e4m3fn_to_float64(kc)
    for h in range(H):
        w = np.zeros((1, H), np.float32)
        w[0, h] = 1.0
        rows = oracle.request_logits(qc, w, k, s.astype(np.float64), 1)
        for t in range(ctx):
            dot = sum(_frac_of_code(a) * _frac_of_code(b) for a, b in zip(qc[0, h], kc[t]))
            want = max(Fraction(float(s[t])) * dot, Fraction(0))
            # one rounding (scale * dot) in fp64
            assert rows[0][t] == float(want)
