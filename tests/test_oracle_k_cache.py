"""Pins of the oracle's K-cache producer against things other than itself (CPU only).

* a hand-derived worked example (tests/golden/k_cache_example.json): plain
  values, a zero token, an exact power-of-two scale, ties between codes in the
  normal and subnormal ranges, a negative value that rounds to zero, a skipped
  padding slot and a slot past the pool;
* the encoder against torch's float8_e4m3fn cast (a library routine) on every
  midpoint between adjacent codes, its neighbours one float32 ulp away, and
  random values over the whole range;
* the encoder's round trip on every finite code, and its tie rule on values
  chosen by hand;
* the per-token quantisation against the input generator's own (which
  quantises with torch's cast), and against properties any correct quantiser
  has: the largest element maps to +-448, and the dequantised value is within
  half a code step of the input;
* bf16 widening against torch's bfloat16 -> float32 conversion;
* record offsets in exact integer arithmetic past 2^31 bytes.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.fp8 import E4M3FN_TABLE

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "k_cache_example.json")


def _torch_cast(y):
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(y, dtype=np.float32)))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_worked_example_records():
    g = json.load(open(GOLDEN))
    d = g["head_dim"]
    pool = np.full(g["num_slots"] * (d + 4), g["sentinel"], dtype=np.uint8)
    k = np.array([t["k"] for t in g["tokens"]], dtype=np.float32)
    slots = [t["slot"] for t in g["tokens"]]
    oracle.write_k_cache(pool, k, slots, d)
    rows = [pool[i * (d + 4):(i + 1) * (d + 4)].tobytes().hex() for i in range(g["num_slots"])]
    assert rows == g["expected_rows_hex"]


def test_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = E4M3FN_TABLE[codes]
    assert np.array_equal(oracle.e4m3fn_encode(vals), codes)


@pytest.mark.parametrize("value,code", [
    (1.0625, 0x38),    # halfway 1.0 (0x38) / 1.125 (0x39): even code 0x38
    (1.1875, 0x3A),    # halfway 1.125 / 1.25: even code 0x3A
    (400.0, 0x7C),     # halfway 384 (0x7C) / 416 (0x7D)
    (432.0, 0x7E),     # halfway 416 (0x7D) / 448 (0x7E)
    (2.0 ** -10, 0x00),  # halfway 0 / 2^-9 (smallest subnormal)
    (3 * 2.0 ** -10, 0x02),  # halfway 2^-9 (0x01) / 2^-8 (0x02)
    (-3 * 2.0 ** -10, 0x82),
    (-1e-30, 0x80),    # rounds to zero, keeps the sign
    (1.06, 0x38), (1.07, 0x39), (447.0, 0x7E), (-448.0, 0xFE),
])
def test_encode_hand_values(value, code):
    assert int(oracle.e4m3fn_encode(np.float32(value))) == code


def test_encode_matches_torch_cast():
    vals = E4M3FN_TABLE[:0x7F]  # finite magnitudes, increasing
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)  # exact in float32
    assert np.array_equal(mids.astype(np.float64), (vals[:-1] + vals[1:]) / 2)
    up = np.nextafter(mids, np.float32(np.inf))
    down = np.nextafter(mids, np.float32(0))
    rng = np.random.default_rng(3)
    rand = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 5000),  # subnormal range
        np.exp(rng.uniform(-30, 6, 5000)) * rng.choice([-1, 1], 5000),
    ]).astype(np.float32)
    rand = np.clip(rand, -448, 448)
    y = np.concatenate([mids, up, down, -mids, -up, -down, rand, [0.0, -0.0]]).astype(np.float32)
    y = np.clip(y, np.float32(-448), np.float32(448))
    assert np.array_equal(oracle.e4m3fn_encode(y), _torch_cast(y))


def test_encode_rejects_out_of_range():
    for bad in (np.float32(449.0), np.float32(np.nan), np.float32(np.inf)):
        with pytest.raises(ValueError):
            oracle.e4m3fn_encode(bad)


def test_quantize_matches_generator():
    rng = np.random.default_rng(4)
    k = rng.standard_normal((300, 128)).astype(np.float32)
    k *= np.exp(rng.standard_normal((300, 1)) * 2).astype(np.float32)
    k[5] = 0.0
    k[6] = np.float32(1e-44)  # amax/448 underflows to 0: scale 1
    k[7] = np.float32(1e-42)  # amax/448 is a subnormal scale
    codes, scales = oracle.quantize_tokens(k)
    g_codes, g_scales = synth.quantize_tokens(k)
    assert np.array_equal(codes, g_codes)
    assert np.array_equal(scales.view(np.uint32), g_scales.view(np.uint32))
    assert scales[5] == 1.0 and scales[6] == 1.0
    assert 0.0 < scales[7] < np.finfo(np.float32).tiny


def test_quantize_properties():
    rng = np.random.default_rng(5)
    k = (rng.standard_normal((200, 128)) * np.exp(rng.uniform(-20, 20, (200, 1)))).astype(np.float32)
    codes, scales = oracle.quantize_tokens(k)
    amax_at = np.argmax(np.abs(k), axis=1)
    top = codes[np.arange(200), amax_at]
    assert np.all((top & 0x7F) == 0x7E)  # the largest element is +-448
    dq = E4M3FN_TABLE[codes] * scales[:, None].astype(np.float64)
    x = k.astype(np.float64)
    # half a code step: 2^-4 relative in the normal range, 2^-10 * scale below
    bound = (np.abs(x) * 2.0 ** -4 + 2.0 ** -10 * scales[:, None]) * (1 + 1e-6)
    assert np.all(np.abs(dq - x) <= bound)


def test_bf16_widening_matches_torch():
    rng = np.random.default_rng(6)
    bits = rng.integers(0, 1 << 16, 50000, dtype=np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]  # finite patterns
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(oracle.bf16_to_float32(bits).view(np.uint32), ref.view(np.uint32))


def test_record_offsets_past_2_31():
    assert oracle.record_offset(2 ** 31, 128) == 2 ** 31 * 132
    assert oracle.record_offset(16_268_816, 128) == 16_268_816 * 132 > 2 ** 31
    assert oracle.record_offset(0, 128) == 0


def test_slots_outside_the_pool_are_skipped():
    pool = np.full(3 * 132, 0x55, dtype=np.uint8)
    k = np.ones((3, 128), dtype=np.float32)
    oracle.write_k_cache(pool, k, [-1, 3, 1 << 40], 128)
    assert np.all(pool == 0x55)
    oracle.write_k_cache(pool, k, [-1, 1, 7], 128)
    assert np.all(pool[:132] == 0x55) and np.all(pool[264:] == 0x55)
    assert np.all(pool[132:260] == 0x7E)  # 1 / (1/448) = 448
