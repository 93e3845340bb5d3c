"""OCP FP8 E4M3FN decoding to fp64 (oracle; test infrastructure only).

Reading adopted: the pages call the query/K element type ``dtypes.fp8``
without naming the encoding (aiter PR #4244, reproducer input construction).
On gfx950 (the CDNA target named in aiter PR #6626, section 1 "gfx950 already
supports 8-token pages") that type is OCP E4M3FN: sign bit, 4 exponent bits
with bias 7, 3 mantissa bits, no infinities, NaN = S.1111.111, largest
finite value 448.  The per-token quantisation scale amax/448 fits that range.

Decoding is exact: every code maps to a dyadic rational that fp64 holds.
"""
import numpy as np


def _decode_one(code: int) -> float:
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        # subnormal: 0.mmm * 2^(1-7)
        return sign * (man / 8.0) * 2.0 ** (-6)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


E4M3FN_TABLE = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)
E4M3FN_TABLE.setflags(write=False)


def e4m3fn_to_float64(codes) -> np.ndarray:
    """Decode uint8 e4m3fn codes (any shape) to float64."""
    return E4M3FN_TABLE[np.asarray(codes, dtype=np.uint8)]
