"""The allocation-free top-k (topk_per_row_noalloc, through the C ABI) against
the workspace entry point topk_per_row.

Both split rows the same way (the no-alloc call as topk_per_row does with a
workspace of topk_per_row_workspace_size(rows, k, row stride) bytes), so their
outputs must be identical arrays; the index sets are also checked against the
oracle.  Two calls in a row, the second on a smaller input, since every call on
a GPU shares the library's one scratch array; then a size whose split needs
more than the scratch holds is refused before anything is enqueued.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import say

pytestmark = pytest.mark.gpu

ERR_WORKSPACE = 4


def _noalloc(lib, logits, ctx, k, idx, next_n=1):
    rows = logits.shape[0]
    return lib.topk_per_row_noalloc(logits.data_ptr(), ctx.data_ptr(), k, idx.data_ptr(),
                                    rows // next_n, next_n, logits.shape[1],
                                    torch.cuda.current_stream().cuda_stream)


def test_noalloc_matches_topk_per_row_twice(gpu_lib):
    lib = gpu_lib.load_library()
    cases = [  # the second call is smaller (fewer rows, shorter stride)
        dict(lens=[70000, 131072, 1000, 16385, 98304, 0, 40000, 131072] * 8, k=2048, ties=0, seed=3),
        dict(lens=[30000, 5, 16384, 32769, 2049], k=100, ties=3, seed=4),
    ]
    for c in cases:
        lens, k = c["lens"], c["k"]
        width = max(lens)
        dense = synth.make_logit_rows(len(lens), width, lens, seed=c["seed"], ties=c["ties"])
        logits = torch.from_numpy(dense).cuda()
        ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
        need = gpu_lib.topk_workspace_size(len(lens), k, width)
        assert 0 < need <= 64 << 20
        ref = torch.full((len(lens), k), -7, dtype=torch.int32, device="cuda")
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        say(f"[gpu] topk_per_row rows={len(lens)} width={width} k={k} workspace={need}")
        gpu_lib.topk_per_row(logits, ctx, k, ref, next_n=1, workspace=ws)
        got = torch.full((len(lens), k), -9, dtype=torch.int32, device="cuda")
        say(f"[gpu] topk_per_row_noalloc rows={len(lens)} width={width} k={k}")
        assert _noalloc(lib, logits, ctx, k, got) == 0
        torch.cuda.synchronize()
        g, r = got.cpu().numpy(), ref.cpu().numpy()
        assert np.array_equal(g, r)
        want = oracle.topk_per_row([dense[i, :n] for i, n in enumerate(lens)], k)
        for i, n in enumerate(lens):
            m = min(k, n)
            assert sorted(g[i, :m].tolist()) == sorted(want[i, :m].tolist()), f"row {i} n={n}"
            assert np.all(g[i, m:] == -1)


def test_noalloc_refuses_a_split_beyond_the_scratch(gpu_lib):
    lib = gpu_lib.load_library()
    rows, k, stride = 1024, 2048, 1 << 20
    assert gpu_lib.topk_workspace_size(rows, k, stride) > 64 << 20
    # a buffer of the stride claimed (nothing may be read from it, but a launch
    # would still stay inside it)
    logits = torch.empty((rows, stride), dtype=torch.float32, device="cuda")
    ctx = torch.full((rows,), 16, dtype=torch.int32, device="cuda")
    idx = torch.full((rows, k), -9, dtype=torch.int32, device="cuda")
    st = lib.topk_per_row_noalloc(logits.data_ptr(), ctx.data_ptr(), k, idx.data_ptr(), rows, 1,
                                  stride, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == ERR_WORKSPACE
    assert bool((idx == -9).all())
