"""GPU parity of the K-cache producer (quantize_k_cache) against the oracle.

The records are bytes decided by floating point (a scale and e4m3fn codes), so
the comparison is bit-exact over the whole pool: written records, and every
byte the call must leave alone (the slots of skipped tokens, untouched rows).
Rows mix bell-shaped values over many magnitudes with hand-built cases: a zero
row, rows whose scale underflows or is subnormal, rows whose quotients sit
exactly halfway between two codes (scale 1 via an element of 448) or one
float32 ulp either side, negative values that round to zero.  A second test
writes rows past 2^31 bytes of the pool; a third feeds the produced cache to
paged_mqa_logits; a fourth replays the producer from a captured HIP graph.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.fp8 import E4M3FN_TABLE
from tests.parity import check_rows, oracle_rows, run_logits, say, upload

pytestmark = pytest.mark.gpu

D = 128
REC = D + 4
POOL_FILL = 0xA5


def _special_rows():
    mags = E4M3FN_TABLE[:0x7F]
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    vals = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)),
                           np.nextafter(mids, np.float32(0)), np.float32([-1e-30, -0.0, 1e-30])])
    vals = np.concatenate([vals, -vals]).astype(np.float32)
    rows = []
    for i in range(0, len(vals), D - 1):
        r = np.zeros(D, dtype=np.float32)
        chunk = vals[i:i + D - 1]
        r[:len(chunk)] = chunk
        r[D - 1] = 448.0  # amax 448: scale exactly 1, quotients exact
        rows.append(r)
    rows.append(np.zeros(D, dtype=np.float32))            # amax 0: scale 1
    rows.append(np.full(D, 1e-44, dtype=np.float32))       # scale underflows to 0: 1
    rows.append(np.full(D, -1e-42, dtype=np.float32))      # subnormal scale
    rows.append(np.linspace(-3e38, 3e38, D).astype(np.float32))  # near the float32 limit
    return np.stack(rows)


def _rows(seed, n):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((n, D)) * np.exp(rng.normal(0.0, 3.0, (n, 1)))
    return np.concatenate([_special_rows(), k.astype(np.float32)])


def _bf16_bits(k32):
    # round-to-nearest-even float32 -> bfloat16 on the host (torch CPU cast)
    return torch.from_numpy(k32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_k_cache_matches_oracle(gpu_lib, dtype):
    for seed in (0, 1):
        k32 = _rows(seed, 700)
        n = k32.shape[0]
        num_slots = n + 300
        rng = np.random.default_rng(100 + seed)
        slots = rng.permutation(num_slots)[:n].astype(np.int64)
        slots[rng.choice(n, 25, replace=False)] = -1           # padding tokens
        slots[rng.choice(n, 10, replace=False)] = num_slots + 7  # past the pool
        if dtype == "bf16":
            bits = _bf16_bits(k32)
            k_host = oracle.bf16_to_float32(bits)
            k_dev = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        else:
            k_host = k32
            k_dev = torch.from_numpy(k32).cuda()
        want = np.full(num_slots * REC, POOL_FILL, dtype=np.uint8)
        oracle.write_k_cache(want, k_host, slots, D)
        pool = torch.full((num_slots * REC,), POOL_FILL, dtype=torch.uint8, device="cuda")
        say(f"[gpu] quantize_k_cache {dtype} seed={seed} tokens={n} slots={num_slots}")
        gpu_lib.quantize_k_cache(k_dev.view(n, D), torch.from_numpy(slots).cuda(), pool)
        torch.cuda.synchronize()
        got = pool.cpu().numpy()
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (
            f"{bad.size} bytes differ; first at slot {bad[0] // REC} byte {bad[0] % REC}: "
            f"gpu {got[bad[0]]:#04x} oracle {want[bad[0]]:#04x}")


def test_k_cache_rows_past_2_31_bytes(gpu_lib):
    # a pool of 17M rows (2.24 GB): rows >= 2^31 / 132 = 16,268,815.5 start past 2^31 bytes
    num_slots = 17_000_000
    slots = np.array([16_268_815, 16_268_816, 16_999_999, 5, 12_345_678], dtype=np.int64)
    k32 = _rows(7, len(slots))[-len(slots):]
    pool = torch.full((num_slots * REC,), POOL_FILL, dtype=torch.uint8, device="cuda")
    say(f"[gpu] quantize_k_cache large pool slots={slots.tolist()}")
    gpu_lib.quantize_k_cache(torch.from_numpy(k32).cuda(), torch.from_numpy(slots).cuda(), pool)
    torch.cuda.synchronize()
    want = np.full(len(slots) * REC, POOL_FILL, dtype=np.uint8)
    oracle.write_k_cache(want, k32, np.arange(len(slots)), D)
    for i, s in enumerate(slots.tolist()):
        got = pool[s * REC:(s + 1) * REC].cpu().numpy()
        assert np.array_equal(got, want[i * REC:(i + 1) * REC]), f"slot {s}"
        # the neighbouring rows stay untouched
        for nb in (s - 1, s + 1):
            if 0 <= nb < num_slots and nb not in slots:
                assert np.all(pool[nb * REC:(nb + 1) * REC].cpu().numpy() == POOL_FILL)
    del pool
    torch.cuda.empty_cache()


def test_k_cache_feeds_logits(gpu_lib):
    """The produced cache read back by paged_mqa_logits: every record of each
    request's context is written by the producer through the request's block
    table, then the logits are compared with the oracle's on the oracle's pool
    (which the first test shows to be byte-identical)."""
    wl = synth.build_workload("kcache_e2e", batch=4, next_n=2, heads=64, head_dim=D,
                              page_size=16, ctx_range=(1, 600), table="permuted", topk=64, seed=3)
    ctx = wl.context_lens.astype(np.int64)
    slots = np.concatenate([
        wl.block_tables[b, np.arange(ctx[b]) // wl.page_size] * wl.page_size
        + np.arange(ctx[b]) % wl.page_size for b in range(wl.batch)]).astype(np.int64)
    rng = np.random.default_rng(9)
    k32 = (rng.standard_normal((len(slots), D)) * np.exp(rng.normal(0, 1, (len(slots), 1)))).astype(np.float32)
    pool_dev = torch.from_numpy(wl.kv_cache.copy()).cuda()
    gpu_lib.quantize_k_cache(torch.from_numpy(k32).cuda(), torch.from_numpy(slots).cuda(), pool_dev)
    torch.cuda.synchronize()
    oracle.write_k_cache(wl.kv_cache, k32, slots, D)
    assert np.array_equal(pool_dev.cpu().numpy(), wl.kv_cache)
    d = upload(wl)
    d["kv"] = pool_dev
    out = run_logits(gpu_lib, wl, d, label="produced cache")
    check_rows(wl, out, oracle_rows(wl))


def test_k_cache_graph_replay(gpu_lib):
    """The producer captured in a HIP graph and replayed with new rows copied into
    the captured input between replays (the way a serving loop drives it): every
    replay writes what the oracle writes for the rows of that replay."""
    n, num_slots = 300, 400
    rng = np.random.default_rng(21)
    slots = torch.from_numpy(rng.permutation(num_slots)[:n].astype(np.int64)).cuda()
    k_in = torch.zeros((n, D), dtype=torch.float32, device="cuda")
    pool = torch.full((num_slots * REC,), POOL_FILL, dtype=torch.uint8, device="cuda")
    gpu_lib.quantize_k_cache(k_in, slots, pool)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("[gpu] capture quantize_k_cache graph")
    with torch.cuda.graph(g):
        gpu_lib.quantize_k_cache(k_in, slots, pool)
    for rep in range(3):
        k32 = _rows(30 + rep, n)[-n:]
        k_in.copy_(torch.from_numpy(k32))
        pool.fill_(POOL_FILL)
        torch.cuda.synchronize()
        say(f"[gpu] producer graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        want = np.full(num_slots * REC, POOL_FILL, dtype=np.uint8)
        oracle.write_k_cache(want, k32, slots.cpu().numpy(), D)
        assert np.array_equal(pool.cpu().numpy(), want), f"replay {rep}"
