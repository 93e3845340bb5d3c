"""Shared helpers of the GPU parity tests: upload a workload, run the HIP path
through the C ABI, and compare with the CPU oracle at the stated tolerance.

Tolerance (logits): per row, max_t |gpu - oracle| <= 2e-4 * max_t |oracle| over
the visible tokens (NaN exactly where the oracle is NaN, the tolerance taken
over the rest); -inf bits exact on [visible, ctx); the sentinel exact past
the context.  Top-k: index sets equal, except that indices in the symmetric
difference must score within that same tolerance of the oracle's k-th value.
"""
import sys

import numpy as np
import torch

import oracle

REL_TOL = 2e-4
SENTINEL_BITS = 0x7FA5A5A5  # a NaN payload no computed score can take
NEG_INF_BITS = 0xFF800000


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def upload(wl, table=None):
    dev = torch.device("cuda", 0)
    t = wl.block_tables if table is None else table
    return dict(
        q=torch.from_numpy(wl.q).to(dev).view(torch.float8_e4m3fn),
        kv=torch.from_numpy(wl.kv_cache).to(dev),
        w=torch.from_numpy(wl.weights).to(dev),
        ctx=torch.from_numpy(wl.context_lens).to(dev),
        tab=torch.from_numpy(np.ascontiguousarray(t)).to(dev),
    )


def new_out(rows, stride):
    out = torch.empty((rows, stride), dtype=torch.int32, device="cuda")
    out.fill_(SENTINEL_BITS - (1 << 32) if SENTINEL_BITS >= 1 << 31 else SENTINEL_BITS)
    return out.view(torch.float32)


def run_logits(pm, wl, d, stride=None, label=""):
    stride = stride or wl.out_row_stride
    out = new_out(wl.rows, stride)
    say(f"[gpu] paged_mqa_logits {label} {wl.name} B={wl.batch} next_n={wl.next_n} H={wl.heads} "
        f"ps={wl.page_size} stride={stride} table={tuple(d['tab'].shape)}")
    pm.paged_mqa_logits(d["q"], d["kv"], d["w"], d["ctx"], d["tab"], wl.page_size, wl.next_n, out)
    torch.cuda.synchronize()
    return out


def oracle_rows(wl, requests=None, table=None):
    return oracle.paged_mqa_logits(wl.q, wl.kv_cache, wl.weights, wl.context_lens,
                                   wl.block_tables if table is None else table, wl.page_size,
                                   wl.next_n, requests=requests)


def check_rows(wl, out_gpu, rows_oracle, requests=None, stride=None):
    """Compare the listed requests' rows (all if None); returns the worst ratio."""
    stride = stride or wl.out_row_stride
    reqs = range(wl.batch) if requests is None else requests
    worst = 0.0
    for b in reqs:
        ctx = max(int(wl.context_lens[b]), 0)  # negative lengths count as 0
        ctx_eff = min(ctx, stride)
        r0 = b * wl.next_n
        g = out_gpu[r0 : r0 + wl.next_n].cpu().numpy()
        bits = g.view(np.uint32)
        for j in range(wl.next_n):
            r = r0 + j
            ref = rows_oracle[r]
            vis = len(ref)
            assert vis == oracle.visible_len(ctx, wl.next_n, j)
            got = g[j, :vis].astype(np.float64)
            if vis:
                # a NaN scale makes its token's score NaN (the oracle's relu
                # passes NaN on): NaN exactly where the oracle has it
                nan_ref = np.isnan(ref)
                assert np.array_equal(np.isnan(got), nan_ref), f"row {r}: NaN positions differ"
                got, ref_f = got[~nan_ref], ref[~nan_ref]
                assert np.all(np.isfinite(got)), f"row {r}: non-finite score"
                scale = float(np.max(np.abs(ref_f))) if ref_f.size else 0.0
                err = float(np.max(np.abs(got - ref_f))) if ref_f.size else 0.0
                if scale == 0.0:
                    assert err == 0.0, f"row {r}: all-zero row, err {err}"
                else:
                    ratio = err / scale
                    worst = max(worst, ratio)
                    assert ratio <= REL_TOL, f"row {r} (b={b}, j={j}): max err {err} vs row max {scale}"
            assert np.all(bits[j, vis:ctx_eff] == NEG_INF_BITS), f"row {r}: mask not -inf"
            assert np.all(bits[j, ctx_eff:] == SENTINEL_BITS), f"row {r}: write past the context"
    return worst


def check_untouched_rows(wl, out_gpu, requests):
    for b in requests:
        r0 = b * wl.next_n
        bits = out_gpu[r0 : r0 + wl.next_n].cpu().numpy().view(np.uint32)
        assert np.all(bits == SENTINEL_BITS)


def check_topk(idx_gpu, rows_oracle, k, rows=None):
    """Set comparison with the tie window at the k-th boundary."""
    idx = idx_gpu.cpu().numpy()
    ref_idx = oracle.topk_per_row(rows_oracle, k)
    sel = range(len(rows_oracle)) if rows is None else rows
    for r in sel:
        ref_vals = rows_oracle[r]
        if ref_vals is None:
            continue
        n = len(ref_vals)
        m = min(k, n)
        g = idx[r]
        assert np.all(g[m:] == -1), f"row {r}: padding"
        gs = g[:m]
        assert len(np.unique(gs)) == m, f"row {r}: duplicate indices"
        assert np.all((gs >= 0) & (gs < n)), f"row {r}: index out of range"
        diff = set(gs.tolist()) ^ set(ref_idx[r, :m].tolist())
        if diff:
            vk = float(ref_vals[ref_idx[r, m - 1]])
            tol = REL_TOL * float(np.max(np.abs(ref_vals)))
            for i in diff:
                assert abs(float(ref_vals[i]) - vk) <= tol, (
                    f"row {r}: index {i} (score {ref_vals[i]}) differs beyond the tie window "
                    f"around the k-th score {vk}")
