"""GPU parity of the fused step, paged_mqa_logits_topk: the logits launch folds
each row's extremes into statistics at the start of the workspace and the
top-k launch sets its buckets from them.

Every case compares the logits and the top-k with the oracle (tests/parity.py
tolerances), and checks that the call leaves the statistics zero.  With a
zeroed workspace the results are also identical to the two separate calls
(the statistics are then exactly the extremes the top-k would find itself):
array for array when rows are not split, row sets otherwise.  A workspace of
random bytes, calls in a row on one workspace, rows long enough to be split
and merged, and signed scales must all still give the oracle's sets.
"""
import numpy as np
import pytest
import torch

import synth
from tests.parity import check_rows, check_topk, new_out, oracle_rows, run_logits, say, upload

pytestmark = pytest.mark.gpu


def _stats_bytes(rows):
    return (rows * 8 + 255) // 256 * 256


def _workspace(gpu_lib, wl, fill=None, seed=0):
    n = gpu_lib.logits_topk_workspace_size(wl.rows, wl.topk, wl.out_row_stride)
    if fill is None:
        return torch.zeros(n, dtype=torch.uint8, device="cuda")
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g).cuda()


def _fused(gpu_lib, wl, d, ws, label=""):
    out = new_out(wl.rows, wl.out_row_stride)
    idx = torch.full((wl.rows, wl.topk), -7, dtype=torch.int32, device="cuda")
    say(f"[gpu] paged_mqa_logits_topk {label} {wl.name} B={wl.batch} next_n={wl.next_n} "
        f"H={wl.heads} ps={wl.page_size} k={wl.topk} workspace={ws.numel()} B")
    gpu_lib.paged_mqa_logits_topk(d["q"], d["kv"], d["w"], d["ctx"], d["tab"], wl.page_size,
                                  wl.next_n, out, wl.topk, idx, workspace=ws)
    torch.cuda.synchronize()
    return out, idx


def _check(wl, out, idx, ws, ref=None):
    ref = oracle_rows(wl) if ref is None else ref
    check_rows(wl, out, ref)
    check_topk(idx, ref, wl.topk)
    # two words a row; the padding up to _stats_bytes is never touched
    assert bool((ws[:8 * wl.rows] == 0).all()), "row statistics not cleared"
    return ref


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_fused_matches_oracle_and_the_two_calls(gpu_lib, cfg):
    wl = synth.make_config(cfg)
    d = upload(wl)
    ws = _workspace(gpu_lib, wl)
    out, idx = _fused(gpu_lib, wl, d, ws, "zeroed workspace")
    ref = _check(wl, out, idx, ws)
    out2 = run_logits(gpu_lib, wl, d, label="two calls")
    idx2 = torch.full_like(idx, -7)
    gpu_lib.topk_per_row(out2, d["ctx"], wl.topk, idx2, next_n=wl.next_n)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), out2.view(torch.int32))
    if wl.out_row_stride <= 16384:
        assert torch.equal(idx, idx2)
    else:
        # split rows: a segment's buckets span the row's range instead of its
        # own, which can reorder its candidates, never change the set
        assert torch.equal(torch.sort(idx, dim=1).values, torch.sort(idx2, dim=1).values)
    # the statistics a first call leaves make a second call identical again
    out3, idx3 = _fused(gpu_lib, wl, d, ws, "reused workspace")
    assert torch.equal(idx3, idx) and torch.equal(out3.view(torch.int32), out.view(torch.int32))
    del ref


def test_fused_random_workspace_then_smaller_call(gpu_lib):
    """Garbage statistics only widen the bucket range: exact sets, and the
    call clears them; then a smaller call on the same workspace."""
    wl = synth.make_config(2)
    d = upload(wl)
    ws = _workspace(gpu_lib, wl, fill="random", seed=5)
    out, idx = _fused(gpu_lib, wl, d, ws, "random workspace")
    _check(wl, out, idx, ws)
    small = synth.build_workload("fused_small", batch=5, next_n=2, heads=64, head_dim=128,
                                 page_size=64, ctx_range=(1, 5000), topk=512, seed=11)
    ds = upload(small)
    out_s, idx_s = _fused(gpu_lib, small, ds, ws, "smaller call, same workspace")
    _check(small, out_s, idx_s, ws)


@pytest.mark.parametrize("fill", [None, "random"])
def test_fused_split_rows(gpu_lib, fill):
    """Rows of 20K-70K scores are cut into segments (their workgroups read the
    statistics) and merged (the merge clears them)."""
    wl = synth.build_workload("fused_long", batch=3, next_n=2, heads=64, head_dim=128,
                              page_size=64, context_lens=[70000, 20000, 45000], topk=2048,
                              seed=4)
    d = upload(wl)
    assert gpu_lib.logits_topk_workspace_size(wl.rows, wl.topk, wl.out_row_stride) > \
        _stats_bytes(wl.rows), "rows this long are split"
    ws = _workspace(gpu_lib, wl, fill=fill, seed=9)
    out, idx = _fused(gpu_lib, wl, d, ws, f"split rows, {fill or 'zeroed'} workspace")
    _check(wl, out, idx, ws)


def test_fused_signed_scales(gpu_lib):
    """Negative scores and blocks of negative scales: the statistics' keys
    order negative scores correctly."""
    wl = synth.build_workload("fused_signed", batch=6, next_n=2, heads=64, head_dim=128,
                              page_size=16, ctx_range=(100, 9000), topk=700, seed=3,
                              neg_scale_blocks=0.5)
    d = upload(wl)
    ws = _workspace(gpu_lib, wl)
    out, idx = _fused(gpu_lib, wl, d, ws, "signed scales")
    _check(wl, out, idx, ws)


def test_fused_statistics_only_minimum_workspace(gpu_lib):
    """A workspace of just the statistics: long rows are selected unsplit
    (streamed), still exact."""
    wl = synth.build_workload("fused_nosplit", batch=2, next_n=1, heads=64, head_dim=128,
                              page_size=64, context_lens=[40000, 3000], topk=1000, seed=8)
    d = upload(wl)
    ws = torch.full((_stats_bytes(wl.rows),), 0xFF, dtype=torch.uint8, device="cuda")
    out, idx = _fused(gpu_lib, wl, d, ws, "statistics-only workspace")
    _check(wl, out, idx, ws)
    assert np.isfinite(out.cpu().numpy()[0, :40000]).all()
