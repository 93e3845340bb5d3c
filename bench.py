#!/usr/bin/env python3
"""Benchmark of the FP8 paged MQA logits + per-row top-k step on one MI355X.

One step = paged_mqa_logits then topk_per_row over one batch of the decode
workload (B=64 requests, next_n=1, H=64, D=128, 64-token pages, context
lengths U[1,8192], a randomly permuted 10,000-page pool, top-k 2048).  Inputs
are synthetic and seeded, resident in HBM before timing starts.  Sixteen
copies of the inputs and outputs are rotated so that consecutive steps never
find their K pages in the 256 MB last-level cache.

Prints one JSON line.  `value` is context tokens scored per second over the
whole step, timed over replays of one HIP graph holding one step per rotated
input set (the kernels back to back, as in a serving forward pass that
captures every layer's indexer step in one graph); `roofline` describes
the logits kernel (HBM-bound at this shape), its duration the mean of the
events its dispatches record at kernel start and end over the same number of
eager steps.  Every timed region follows `settle_s` seconds of untimed steps
(the GPU's clocks take tens of milliseconds of load to reach their sustained
level), then the W warm-up steps.  `cpu_baseline` is the CPU oracle (numpy
fp64) on a bounded sample; `device_copy` is a plain 512 MiB device copy (1 GiB
moved; context for the HBM roofline); `per_config` times the other four workloads (logits
and top-k launch durations from dispatch-recorded events over rotated input
sets, their throughput and roofline fractions); `token_level_tables` times the
logits on the same pools read through token-level tables (page_size 1);
`preshuffled_layout` (also in each per_config entry) times the logits on the
same pools rewritten in the preshuffled page layout; `k_cache_producer` times
the K-cache producer (quantize_k_cache) that writes new K rows into the cache,
at a decode step's rows and at prefill-sized chunks.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "context tokens scored/s (TFLOP/s fp8) + % MFMA/HBM roofline, 1×MI355X"
HBM_PEAK_GBPS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
N_SETS = 16
KERNEL_SOURCES = ["fp8_paged_mqa_block_amd/csrc/logits_gfx950.hip",
                  "fp8_paged_mqa_block_amd/csrc/pmqa_host.hip"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_b64_traffic.md")


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch has loaded (ctypes)."""

    def __init__(self):
        import ctypes

        self.ct = ctypes
        self.rt = ctypes.CDLL("libamdhip64.so.7")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        h = self.ct.c_void_p()
        assert self.rt.hipEventCreate(self.ct.byref(h)) == 0
        return h.value

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        assert self.rt.hipEventElapsedTime(self.ct.byref(ms), a, b) == 0
        return float(ms.value)

    def destroy(self, h):
        self.rt.hipEventDestroy(h)


def kernel_digest():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(wl):
    """Bytes the logits step must move: every K record of every context token,
    one table entry per page, the fp32 outputs on [0, ctx) of every row, and
    each row's q and weights."""
    ctx = wl.context_lens.astype(int)
    pages = sum((c + wl.page_size - 1) // wl.page_size for c in ctx)
    k_bytes = int(ctx.sum()) * (wl.head_dim + 4)
    out_bytes = int(ctx.sum()) * 4 * wl.next_n
    table_bytes = pages * 8
    row_bytes = wl.rows * (wl.heads * wl.head_dim + 4 * wl.heads) + 4 * wl.batch
    return k_bytes + out_bytes + table_bytes + row_bytes


def topk_bytes(wl):
    vis = wl.visible_lens()
    return int(vis.sum()) * 4 + wl.rows * wl.topk * 4 + 4 * wl.batch


def read_traffic(digest):
    """HBM bytes per logits launch from the committed rocprofv3 counter runs,
    or None when the kernel sources changed since they were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m = re.search(r"kernel_digest:\s*([0-9a-f]+)", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != digest:
        return None
    return float(t.group(1))


def pm_rows_per_wave(wl):
    cap = 1 if wl.heads >= 128 else (3 if wl.heads >= 64 else 4)
    return min(wl.next_n, cap)


def logits_kernel_name(wl):
    """The logits kernel the library launches for this workload (asked of the
    library itself, which takes the launch geometry from the same sizes)."""
    import fp8_paged_mqa_block_amd as pm

    return pm.logits_kernel(wl.batch, wl.next_n, wl.page_size, wl.out_row_stride, wl.heads,
                            wl.block_tables.shape[1], head_dim=wl.head_dim)


def measure_copy(dev, mib=512, reps=20):
    """Context for the roofline: a plain device-to-device copy of `mib` MiB
    (torch's copy kernel), bytes read + written per second, mean over reps."""
    import torch

    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    for _ in range(3):
        dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    sec = a.elapsed_time(b) * 1e-3 / reps
    del src, dst
    gbps = 2 * n / sec / 1e9
    return {"bytes": 2 * n, "GBps": gbps, "frac_of_peak": gbps / HBM_PEAK_GBPS}


def measure_token_level(lib, wl, sets, hip, sh, reps=100):
    """The logits launch on the same rotated pools read through token-level
    tables (page_size 1: entry t is the pool row of token t), as a dense table
    of cache row ids addresses them.  Algorithmic bytes as for the paged call,
    with one 8-byte table entry per token."""
    import copy

    import numpy as np
    import torch

    ctx = wl.context_lens.astype(np.int64)
    tok = np.full((wl.batch, max(1, int(ctx.max()))), wl.poison_page * wl.page_size, dtype=np.int64)
    for b in range(wl.batch):
        t = np.arange(ctx[b])
        tok[b, : ctx[b]] = wl.block_tables[b, t // wl.page_size] * wl.page_size + t % wl.page_size
    tabs = [torch.from_numpy(tok).to(d["kv"].device) for d in sets]
    largs = [(d["q"].data_ptr(), d["kv"].data_ptr(), d["w"].data_ptr(), d["ctx"].data_ptr(),
              t.data_ptr(), 1, wl.next_n, d["out"].data_ptr(), wl.out_row_stride, wl.batch,
              wl.heads, wl.head_dim, tok.shape[1], sh) for d, t in zip(sets, tabs)]
    settle(lib, largs, None)
    ev = [(hip.create(), hip.create()) for _ in range(reps)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(ev):
        assert lib.paged_mqa_logits_timed(*largs[i % len(largs)], a, b) == 0
    torch.cuda.synchronize()
    us = np.array([hip.elapsed_ms(a, b) for a, b in ev]) * 1e3
    for a, b in ev:
        hip.destroy(a)
        hip.destroy(b)
    w1 = copy.copy(wl)
    w1.page_size = 1
    nbytes = algorithmic_bytes(w1)
    gbps = nbytes / (us.mean() * 1e-6) / 1e9
    return {"workload": f"{wl.name} through token-level tables (page_size 1)",
            "logits_us_mean": float(us.mean()), "logits_us_median": float(np.median(us)),
            "algorithmic_bytes": nbytes, "GBps": gbps, "hbm_frac": gbps / HBM_PEAK_GBPS}


def measure_k_cache(lib, wl, hip, dev, sh, sizes=(16384, 131072), reps=50):
    """The K-cache producer on new bf16 K rows written at permuted slots of a
    pool the size of the workload's: one decode step's rows (batch*next_n), a
    prefill chunk of 16384 batched tokens, and 131072 tokens (where the kernel
    leaves its latency floor for the bandwidth regime).  Algorithmic bytes per
    token: 2*D read + 8 of slot + D+4 written."""
    import numpy as np
    import torch

    rng = np.random.default_rng(11)
    num_slots = wl.num_pages * wl.page_size
    pool = torch.zeros(num_slots * (wl.head_dim + 4), dtype=torch.uint8, device=dev)
    gen = torch.Generator().manual_seed(11)
    out = {}
    for n in (wl.rows,) + tuple(sizes):
        k = torch.randn((n, wl.head_dim), generator=gen).to(torch.bfloat16).to(dev)
        slots = torch.from_numpy(rng.choice(num_slots, n, replace=False).astype(np.int64)).to(dev)
        args = (k.data_ptr(), 1, slots.data_ptr(), n, wl.head_dim, pool.data_ptr(), num_slots, sh)
        for _ in range(5):
            assert lib.quantize_k_cache(*args) == 0
        ev = [(hip.create(), hip.create()) for _ in range(reps)]
        torch.cuda.synchronize()
        for a, b in ev:
            assert lib.quantize_k_cache_timed(*args, a, b) == 0
        torch.cuda.synchronize()
        us = np.array([hip.elapsed_ms(a, b) for a, b in ev]) * 1e3
        for a, b in ev:
            hip.destroy(a)
            hip.destroy(b)
        nbytes = n * (2 * wl.head_dim + 8 + wl.head_dim + 4)
        gbps = nbytes / (us.mean() * 1e-6) / 1e9
        out[f"tokens_{n}"] = {"us_mean": float(us.mean()), "us_median": float(np.median(us)),
                              "algorithmic_bytes": nbytes, "GBps": gbps,
                              "hbm_frac": gbps / HBM_PEAK_GBPS}
    del pool
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def make_sets(wl, n_sets, dev):
    """n_sets device copies of the workload's inputs and outputs (rotated so
    that consecutive steps never find their pages in the last-level cache),
    and one top-k workspace sized for the workload's longest visible row
    (shared: the steps run in order on one stream)."""
    import torch

    import fp8_paged_mqa_block_amd as pm

    sets = []
    q = torch.from_numpy(wl.q).to(dev)
    w = torch.from_numpy(wl.weights).to(dev)
    ctx = torch.from_numpy(wl.context_lens).to(dev)
    tab = torch.from_numpy(wl.block_tables).to(dev)
    kv0 = torch.from_numpy(wl.kv_cache).to(dev)
    for s in range(n_sets):
        kv = kv0 if s == 0 else kv0.clone()
        out = torch.empty((wl.rows, wl.out_row_stride), dtype=torch.float32, device=dev)
        idx = torch.empty((wl.rows, wl.topk), dtype=torch.int32, device=dev)
        sets.append(dict(q=q.clone(), w=w.clone(), ctx=ctx.clone(), tab=tab.clone(), kv=kv,
                         out=out, idx=idx))
    del kv0
    ws_bytes = pm.topk_workspace_size(wl.rows, wl.topk, int(wl.visible_lens().max(initial=0)))
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    return sets, ws, ws_bytes


def launch_args(wl, sets, ws, ws_bytes, sh):
    """Raw C-ABI argument tuples of the logits and top-k calls, per set."""
    W = wl.block_tables.shape[1]
    largs = [(d["q"].data_ptr(), d["kv"].data_ptr(), d["w"].data_ptr(), d["ctx"].data_ptr(),
              d["tab"].data_ptr(), wl.page_size, wl.next_n, d["out"].data_ptr(),
              wl.out_row_stride, wl.batch, wl.heads, wl.head_dim, W, sh) for d in sets]
    targs = [(d["out"].data_ptr(), d["ctx"].data_ptr(), wl.topk, d["idx"].data_ptr(), wl.batch,
              wl.next_n, wl.out_row_stride, ws.data_ptr() if ws_bytes else None, ws_bytes, sh)
             for d in sets]
    return largs, targs


def warm_set(i, warmup, n_sets):
    """Set of warm-up step i: the warm-up ends on the last set, so the timed
    rotation (which starts at set 0) first reaches the sets touched longest ago."""
    return (i - warmup) % n_sets


# Untimed load before any timed region, in seconds of wall time.  The GPU's
# clocks reach their sustained level only after tens of milliseconds of
# load: interleaved rounds of 25 launches measured the MTP workload's logits
# at 365, 365, 336, 320, 312, 312 us and the long-context workload's at 137,
# 127, 122, 119, 116, 116 us, so a short timed region right after setup
# would time the ramp, not the steady state a serving loop runs in.
SETTLE_S = 0.1


def settle(lib, largs, targs, seconds=SETTLE_S, logits_fn=None):
    """Untimed steps (logits then top-k over the rotated sets; no top-k when
    targs is None) until `seconds` of wall time have passed; returns the
    number of steps run.  `logits_fn` replaces paged_mqa_logits."""
    import torch

    lfn = logits_fn or lib.paged_mqa_logits
    n = len(largs)
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            assert lfn(*largs[i % n]) == 0
            if targs is not None:
                assert lib.topk_per_row(*targs[i % n]) == 0
            i += 1
        torch.cuda.synchronize()
    return i


def time_steps(lib, largs, targs, hip, steps, warmup, logits_fn=None):
    """Eager steps (logits then top-k per rotated set): warm-up, then `steps`
    steps whose kernels record dispatch events.  Returns per-launch ms lists.
    `logits_fn` replaces paged_mqa_logits_timed (the preshuffled layout's)."""
    import torch

    lfn = logits_fn or lib.paged_mqa_logits_timed
    n = len(largs)
    spare = [hip.create() for _ in range(4)]
    for i in range(warmup):
        s = warm_set(i, warmup, n)
        assert lfn(*largs[s], spare[0], spare[1]) == 0
        assert lib.topk_per_row_timed(*targs[s], spare[2], spare[3]) == 0
    events = [[hip.create() for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        e = events[i]
        assert lfn(*largs[i % n], e[0], e[1]) == 0
        assert lib.topk_per_row_timed(*targs[i % n], e[2], e[3]) == 0
    torch.cuda.synchronize()
    time_steps.wall_s = time.perf_counter() - t0
    logits_ms = [hip.elapsed_ms(e[0], e[1]) for e in events]
    topk_ms = [hip.elapsed_ms(e[2], e[3]) for e in events]
    for e in events + [spare]:
        for h in e:
            hip.destroy(h)
    return logits_ms, topk_ms


def roof_of(wl, logits_s):
    """Binding roof of the logits launch: HBM or fp8 MFMA, by arithmetic intensity."""
    flops = 2.0 * wl.heads * wl.head_dim * wl.scored_tokens()
    abytes = algorithmic_bytes(wl)
    gbps = abytes / logits_s / 1e9
    tflops = flops / logits_s / 1e12
    mfma_bound = flops / abytes > FP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    return dict(bound="mfma" if mfma_bound else "hbm", algorithmic_bytes=abytes,
                algorithmic_flops=flops, hbm_GBps=gbps, hbm_frac=gbps / HBM_PEAK_GBPS,
                tflops=tflops, mfma_frac=tflops / FP8_PEAK_TFLOPS,
                frac=(tflops / FP8_PEAK_TFLOPS) if mfma_bound else (gbps / HBM_PEAK_GBPS))


def measure_config(lib, cfg, hip, dev, sh, steps=20, warmup=5, rounds=3):
    """One workload's logits and top-k launches, timed eagerly over rotated sets
    (16 for the small decode shape, 3 for the large ones, whose single step
    already exceeds the last-level cache), after the settle phase, over
    `rounds` rounds of `steps` launches each."""
    import numpy as np
    import torch

    import synth

    t0 = time.perf_counter()
    wl = synth.make_config(cfg)
    gen_s = time.perf_counter() - t0
    n_sets = 16 if cfg == 1 else 3
    sets, ws, ws_bytes = make_sets(wl, n_sets, dev)
    largs, targs = launch_args(wl, sets, ws, ws_bytes, sh)
    torch.cuda.synchronize()
    settle(lib, largs, targs)
    logits_ms, topk_ms = [], []
    for _ in range(rounds):
        lg, tk = time_steps(lib, largs, targs, hip, steps, warmup)
        logits_ms += lg
        topk_ms += tk
    lg_s = float(np.mean(logits_ms)) * 1e-3
    tk_s = float(np.mean(topk_ms)) * 1e-3
    roof = roof_of(wl, lg_s)
    tbytes = topk_bytes(wl)
    scored = wl.scored_tokens()
    res = {
        "workload": wl.name, "batch": wl.batch, "next_n": wl.next_n, "heads": wl.heads,
        "page_size": wl.page_size, "topk": wl.topk, "scored_tokens": scored,
        "kernel": logits_kernel_name(wl),
        "logits_us": {"mean": lg_s * 1e6, "median": float(np.median(logits_ms)) * 1e3},
        "topk_us": {"mean": tk_s * 1e6, "median": float(np.median(topk_ms)) * 1e3},
        "step_us": (lg_s + tk_s) * 1e6,
        "tokens_per_s": scored / (lg_s + tk_s),
        "logits_tokens_per_s": scored / lg_s,
        "tflops": roof["tflops"],
        "logits_roofline": roof,
        "topk_GBps": tbytes / tk_s / 1e9,
        "topk_hbm_frac": tbytes / tk_s / 1e9 / HBM_PEAK_GBPS,
        "topk_algorithmic_bytes": tbytes,
        "topk_workspace_bytes": ws_bytes,
        "rotated_sets": n_sets, "launches": steps * rounds, "settle_s": SETTLE_S,
        "generate_s": gen_s,
    }
    res["preshuffled_layout"] = measure_preshuffled(lib, wl, sets, targs, hip, sh, steps * rounds,
                                                    warmup)
    del sets, ws, largs, targs
    torch.cuda.empty_cache()
    return res


def measure_preshuffled(lib, wl, sets, targs, hip, sh, steps=20, warmup=5):
    """The logits launch on the same pools rewritten in the preshuffled page
    layout (paged_mqa_logits_preshuffled; bit-identical results), timed as the
    record layout's."""
    import numpy as np
    import torch

    import synth

    pre = torch.from_numpy(synth.preshuffle_pool(wl.kv_cache, wl.page_size)).to(sets[0]["kv"].device)
    for d in sets:
        d["kv"].copy_(pre)
    del pre
    W = wl.block_tables.shape[1]
    largs = [(d["q"].data_ptr(), d["kv"].data_ptr(), d["w"].data_ptr(), d["ctx"].data_ptr(),
              d["tab"].data_ptr(), wl.page_size, wl.next_n, d["out"].data_ptr(),
              wl.out_row_stride, wl.batch, wl.heads, wl.head_dim, W, sh) for d in sets]
    torch.cuda.synchronize()
    settle(lib, largs, targs, logits_fn=lib.paged_mqa_logits_preshuffled)
    lg, _ = time_steps(lib, largs, targs, hip, steps, warmup, lib.paged_mqa_logits_preshuffled_timed)
    m = float(np.mean(lg)) * 1e-3
    return {"logits_us": {"mean": m * 1e6, "median": float(np.median(lg)) * 1e3},
            "logits_roofline": roof_of(wl, m)}


def cpu_baseline(wl, min_seconds=10.0, max_reps=400):
    import oracle
    from threadpoolctl import threadpool_info

    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    reps = 0
    t0 = time.perf_counter()
    while True:
        rows = oracle.paged_mqa_logits(wl.q, wl.kv_cache, wl.weights, wl.context_lens,
                                       wl.block_tables, wl.page_size, wl.next_n)
        oracle.topk_per_row(rows, wl.topk)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or reps >= max_reps:
            break
    return {
        "value": wl.scored_tokens() * reps / el,
        "unit": "tokens/s",
        "cores": int(threads),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"the whole {wl.name} workload (logits + top-k, {wl.scored_tokens()} scored tokens) "
                  f"run {reps}x in {el:.1f} s, numpy fp64 on {threads} BLAS threads",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, help="workload number (2 = decode B=64)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sets", type=int, default=N_SETS)
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the step (no copy, token-level or producer measurements): "
                         "for profiler runs whose per-kernel figures must cover the step alone")
    ap.add_argument("--table", choices=("permuted", "identity"), default="permuted",
                    help="page order of the workload's pool (identity: each request's pages "
                         "contiguous, for comparison with the permuted pool)")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip timing the other workloads")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this path runs on a single MI355X; --gpus {args.gpus} "
              "is not supported (requests shard by request across GPUs with no exchange, "
              "so N GPUs run N independent copies of this step)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fp8_paged_mqa_block_amd as pm
    import synth

    lib = pm.load_library()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    wl = synth.make_config(args.config, table=args.table)
    rows, stride, k = wl.rows, wl.out_row_stride, wl.topk
    print(f"[bench] workload {wl.name}: B={wl.batch} next_n={wl.next_n} H={wl.heads} "
          f"ps={wl.page_size} scored={wl.scored_tokens()} sets={args.sets}", file=sys.stderr,
          flush=True)

    sets, ws, ws_bytes = make_sets(wl, args.sets, dev)
    # check once through the binding, then launch through the raw C ABI in the loop
    pm.paged_mqa_logits(sets[0]["q"].view(torch.float8_e4m3fn), sets[0]["kv"], sets[0]["w"],
                        sets[0]["ctx"], sets[0]["tab"], wl.page_size, wl.next_n, sets[0]["out"])
    pm.topk_per_row(sets[0]["out"], sets[0]["ctx"], k, sets[0]["idx"], next_n=wl.next_n,
                    workspace=ws[:ws_bytes])
    torch.cuda.synchronize()

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        print(f"[bench] calibration copies: 3 x {args.calibrate_copy_mib} MiB", file=sys.stderr,
              flush=True)

    stream = torch.cuda.current_stream(dev)
    sh = int(stream.cuda_stream)
    largs, targs = launch_args(wl, sets, ws, ws_bytes, sh)
    hip = HipEvents()

    # Kernel durations: dispatch-recorded start/end events of every launch over
    # `steps` eager steps (the same rotated inputs), after the settle phase.
    torch.cuda.synchronize()
    settle(lib, largs, targs)
    logits_ms, topk_ms = time_steps(lib, largs, targs, hip, args.steps, args.warmup)
    eager_elapsed = time_steps.wall_s

    # Step throughput: W warm-up steps, then exactly K timed steps, each a
    # sequence of steps over the rotated input sets (logits then top-k each)
    # captured in one HIP graph, as a serving forward pass captures its
    # layers' indexer steps in one graph; the timed region holds the kernels
    # back to back.
    cap = torch.cuda.Stream(dev)

    def capture(set_of_step, n_steps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                csh = int(torch.cuda.current_stream(dev).cuda_stream)
                for i in range(n_steps):
                    a = list(largs[set_of_step(i)]); a[-1] = csh
                    t = list(targs[set_of_step(i)]); t[-1] = csh
                    assert lib.paged_mqa_logits(*a) == 0 and lib.topk_per_row(*t) == 0
        return g

    # the warm-up ends on the last set, so the timed steps (sets 0, 1, ...)
    # start on the sets touched longest ago
    nw = max(args.warmup, 1)
    warm_graph = capture(lambda i: warm_set(i, nw, len(sets)), nw)
    timed_graph = capture(lambda i: i % len(sets), args.steps)
    torch.cuda.synchronize()
    settle(lib, largs, targs)  # the captures left the GPU idle
    warm_graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    timed_graph.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    graph_steps = args.steps
    step_ms = elapsed * 1e3 / graph_steps

    scored = wl.scored_tokens()
    flops = 2.0 * wl.heads * wl.head_dim * scored
    value = scored * graph_steps / elapsed
    lg_avg_s = float(np.mean(logits_ms)) * 1e-3
    abytes = algorithmic_bytes(wl)
    achieved = abytes / lg_avg_s / 1e9
    digest = kernel_digest()
    traffic = read_traffic(digest)

    ai = flops / abytes
    if ai > FP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9):
        roof = {"bound": "mfma", "achieved": flops / lg_avg_s / 1e12, "peak": FP8_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof.update({
        "traffic": traffic,
        "kernel": logits_kernel_name(wl),
        "algorithmic_bytes_per_launch": abytes,
        "algorithmic_flops_per_launch": flops,
        "hbm_GBps": achieved,
        "hbm_frac": achieved / HBM_PEAK_GBPS,
        "mfma_frac": flops / lg_avg_s / 1e12 / FP8_PEAK_TFLOPS,
        "kernel_digest": digest,
    })
    res = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": SETTLE_S,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": wl.name, "page_order": args.table, "batch": wl.batch, "next_n": wl.next_n,
                   "heads": wl.heads, "head_dim": wl.head_dim, "page_size": wl.page_size,
                   "context_lens": "U[1,8192]" if args.config == 2 else "see workload",
                   "topk": k, "scored_tokens_per_step": scored, "rotated_input_sets": args.sets,
                   "topk_workspace_bytes": ws_bytes},
        "tflops": flops * graph_steps / elapsed / 1e12,
        "eager_ms_per_step": eager_elapsed * 1e3 / args.steps,
        "logits_us": {"mean": lg_avg_s * 1e6, "median": float(np.median(logits_ms)) * 1e3},
        "topk_us": {"mean": float(np.mean(topk_ms)) * 1e3, "median": float(np.median(topk_ms)) * 1e3},
        "logits_tflops": flops / lg_avg_s / 1e12,
        "topk_GBps": topk_bytes(wl) / (float(np.mean(topk_ms)) * 1e-3) / 1e9,
        "topk_hbm_frac": topk_bytes(wl) / (float(np.mean(topk_ms)) * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "roofline": roof,
    }
    if not args.no_extras:
        res["device_copy"] = measure_copy(dev)
        res["token_level_tables"] = measure_token_level(lib, wl, sets, hip, sh)
        res["k_cache_producer"] = measure_k_cache(lib, wl, hip, dev, sh)
        res["preshuffled_layout"] = measure_preshuffled(lib, wl, sets, targs, hip, sh, 100, 10)
    if not args.no_per_config:
        del sets, ws, largs, targs
        torch.cuda.empty_cache()
        res["per_config"] = {}
        for cfg in (1, 3, 4, 5):
            if cfg == args.config:
                continue
            print(f"[bench] per_config: workload {cfg}", file=sys.stderr, flush=True)
            res["per_config"][synth.CONFIG_NAMES[cfg]] = measure_config(lib, cfg, hip, dev, sh)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(res, default=lambda o: o.item() if hasattr(o, "item") else str(o)), flush=True)


if __name__ == "__main__":
    main()
