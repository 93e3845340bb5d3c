"""Assemble hand-written cases (golden worked examples) into the path's raw arrays.

Test helper: builds the byte-level inputs exactly as a caller would lay them
out, from logical token values, scales and a block table chosen by the test.
"""
import json
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def codes_of(values):
    """e4m3fn codes of values that are exactly representable (checked)."""
    v = np.asarray(values, dtype=np.float32)
    c = torch.from_numpy(np.ascontiguousarray(v)).to(torch.float8_e4m3fn)
    back = c.to(torch.float32).numpy()
    assert np.array_equal(back, v), "hand value not representable in e4m3fn"
    return c.view(torch.uint8).numpy().copy()


def assemble(ex):
    """Return dict(q, kv_cache, weights, context_lens, block_tables, page_size, next_n, H, D)."""
    H, D, ps, nn = ex["heads"], ex["head_dim"], ex["page_size"], ex["next_n"]
    reqs = ex["requests"]
    B = len(reqs)
    rec = D + 4
    num_pages = ex["num_pages"]
    pool = np.full(num_pages * ps * rec, 0x7F, dtype=np.uint8)
    recs = pool.reshape(num_pages * ps, rec)
    recs[:, D:] = np.frombuffer(np.uint32(0x7FC00000).astype("<u4").tobytes(), dtype=np.uint8)
    W = max(len(r["table"]) for r in reqs)
    tables = np.zeros((B, W), dtype=np.int64)
    ctx = np.zeros(B, dtype=np.int32)
    for b, r in enumerate(reqs):
        tables[b, : len(r["table"])] = r["table"]
        ctx[b] = r["ctx"]
        for t in range(r["ctx"]):
            if "tokens" in r:
                kc = codes_of(r["tokens"][t])
            else:
                kc = np.full(D, ex["k_code_fill"], dtype=np.uint8)
            row = r["table"][t // ps] * ps + t % ps
            recs[row, :D] = kc
            recs[row, D:] = np.frombuffer(np.float32(r["scales"][t]).astype("<f4").tobytes(), dtype=np.uint8)
    if "q" in ex:
        q = codes_of(np.asarray(ex["q"], dtype=np.float32)).reshape(B * nn, H, D)
    else:
        q = np.full((B * nn, H, D), ex["q_code_fill"], dtype=np.uint8)
    w = np.asarray(ex["weights"], dtype=np.float32).reshape(B * nn, H)
    return dict(q=q, kv_cache=pool, weights=w, context_lens=ctx, block_tables=tables,
                page_size=ps, next_n=nn, H=H, D=D)


def expected_value(v):
    """A golden value: a number, or the strings "-inf" / "nan"."""
    return float(v)
