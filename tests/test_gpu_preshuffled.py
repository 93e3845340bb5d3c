"""GPU parity of the preshuffled page layout (paged_mqa_logits_preshuffled and
quantize_k_cache_preshuffled).

The same tokens in either layout must give bit-identical logits (the per-token
arithmetic is the same; only where the bytes come from differs), on every
kernel family and on page sizes 8 to 256; the logits also meet the oracle,
which reads the preshuffled pool through its own definition of the layout.
The producer's preshuffled pool is compared byte for byte with the oracle's
writer.  The MTP and long-context workloads run at full size in both layouts.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import check_rows, check_topk, new_out, say, upload
from tests.test_gpu_k_cache import POOL_FILL, REC, D, _bf16_bits, _rows

pytestmark = pytest.mark.gpu

FAMILIES = [
    dict(heads=64, next_n=1, family="logits_flat_kernel"),
    dict(heads=64, next_n=3, family="logits_kernel"),
    dict(heads=128, next_n=1, family="logits_kernel"),
    dict(heads=128, next_n=4, family="logits_shared_kernel"),
]


def _run(gpu_lib, wl, d, layout, label):
    out = new_out(wl.rows, wl.out_row_stride)
    say(f"[gpu] paged_mqa_logits {layout} {label} B={wl.batch} next_n={wl.next_n} H={wl.heads} "
        f"ps={wl.page_size} stride={wl.out_row_stride}")
    gpu_lib.paged_mqa_logits(d["q"], d["kv"], d["w"], d["ctx"], d["tab"], wl.page_size, wl.next_n,
                             out, layout=layout)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("page_size", [8, 16, 32, 64, 256])
@pytest.mark.parametrize("case", range(len(FAMILIES)))
def test_preshuffled_matches_records_and_oracle(gpu_lib, case, page_size):
    c = FAMILIES[case]
    lens = [1, 5, 64, 127, 200, 700, 1500, 2100]
    wl = synth.build_workload(f"pre{case}", batch=len(lens), next_n=c["next_n"], heads=c["heads"],
                              head_dim=128, page_size=page_size, context_lens=lens,
                              table="permuted", topk=100, seed=50 + case)
    wl.out_row_stride = 2112
    name = gpu_lib.logits_kernel(wl.batch, wl.next_n, page_size, wl.out_row_stride, wl.heads,
                                 wl.block_tables.shape[1])
    assert name.startswith(c["family"] + "<"), name
    d = upload(wl)
    rec = _run(gpu_lib, wl, d, "records", name)
    pre_pool = synth.preshuffle_pool(wl.kv_cache, page_size)
    dp = dict(d)
    dp["kv"] = torch.from_numpy(pre_pool).cuda()
    pre = _run(gpu_lib, wl, dp, "preshuffled", name)
    assert torch.equal(rec.view(torch.int32), pre.view(torch.int32))
    ref = oracle.paged_mqa_logits(wl.q, pre_pool, wl.weights, wl.context_lens, wl.block_tables,
                                  page_size, wl.next_n, layout="preshuffled")
    worst = check_rows(wl, pre, ref)
    idx = torch.full((wl.rows, wl.topk), -7, dtype=torch.int32, device="cuda")
    gpu_lib.topk_per_row(pre, d["ctx"], wl.topk, idx, next_n=wl.next_n)
    torch.cuda.synchronize()
    check_topk(idx, ref, wl.topk)
    say(f"{name} ps={page_size}: bit-identical to records, worst rel err {worst:.3e}")


@pytest.mark.parametrize("page_size", [8, 64, 256])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_preshuffled_producer_matches_oracle(gpu_lib, dtype, page_size):
    k32 = _rows(3, 500)
    n = k32.shape[0]
    num_pages = -(-(n + 300) // page_size)
    num_slots = num_pages * page_size
    rng = np.random.default_rng(7)
    slots = rng.permutation(num_slots)[:n].astype(np.int64)
    slots[rng.choice(n, 20, replace=False)] = -1
    slots[rng.choice(n, 8, replace=False)] = num_slots + 3
    if dtype == "bf16":
        bits = _bf16_bits(k32)
        k_host = oracle.bf16_to_float32(bits)
        k_dev = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        k_host = k32
        k_dev = torch.from_numpy(k32).cuda()
    want = np.full(num_slots * REC, POOL_FILL, dtype=np.uint8)
    oracle.write_k_cache(want, k_host, slots, D, layout="preshuffled", page_size=page_size)
    pool = torch.full((num_slots * REC,), POOL_FILL, dtype=torch.uint8, device="cuda")
    say(f"[gpu] quantize_k_cache_preshuffled {dtype} ps={page_size} tokens={n} slots={num_slots}")
    gpu_lib.quantize_k_cache(k_dev.view(n, D), torch.from_numpy(slots).cuda(), pool,
                             page_size=page_size)
    torch.cuda.synchronize()
    got = pool.cpu().numpy()
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} bytes differ, first at byte {bad[0]}"


def test_preshuffled_producer_feeds_logits(gpu_lib):
    """Both producers write the same tokens through the same table; the two
    pools then give bit-identical logits."""
    wl = synth.build_workload("pre_e2e", batch=5, next_n=2, heads=64, head_dim=D, page_size=32,
                              ctx_range=(1, 900), table="permuted", topk=64, seed=8)
    ctx = wl.context_lens.astype(np.int64)
    slots = np.concatenate([
        wl.block_tables[b, np.arange(ctx[b]) // wl.page_size] * wl.page_size
        + np.arange(ctx[b]) % wl.page_size for b in range(wl.batch)]).astype(np.int64)
    rng = np.random.default_rng(10)
    k = torch.from_numpy((rng.standard_normal((len(slots), D))).astype(np.float32)).cuda()
    s = torch.from_numpy(slots).cuda()
    rec_pool = torch.from_numpy(wl.kv_cache.copy()).cuda()
    pre_pool = torch.from_numpy(synth.preshuffle_pool(wl.kv_cache, wl.page_size)).cuda()
    gpu_lib.quantize_k_cache(k, s, rec_pool)
    gpu_lib.quantize_k_cache(k, s, pre_pool, page_size=wl.page_size)
    torch.cuda.synchronize()
    d = upload(wl)
    d["kv"] = rec_pool
    a = _run(gpu_lib, wl, d, "records", "produced")
    d["kv"] = pre_pool
    b = _run(gpu_lib, wl, d, "preshuffled", "produced")
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("cfg", [3, 5])
def test_full_workloads_in_both_layouts(gpu_lib, cfg):
    wl = synth.make_config(cfg)
    d = upload(wl)
    rec = _run(gpu_lib, wl, d, "records", f"config {cfg}")
    dp = dict(d)
    dp["kv"] = torch.from_numpy(synth.preshuffle_pool(wl.kv_cache, wl.page_size)).cuda()
    del d["kv"]
    pre = _run(gpu_lib, wl, dp, "preshuffled", f"config {cfg}")
    assert torch.equal(rec.view(torch.int32), pre.view(torch.int32))
