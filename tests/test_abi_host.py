"""The C-ABI library on the host (CPU only, no GPU needed).

Loads libpmqa.so, checks that every symbol include/pmqa.h declares is exported,
and drives the host-side argument checks: each invalid argument returns its
status code before anything is enqueued (so these calls never touch a GPU).
"""
import ctypes
import os
import re
import subprocess

import pytest

import fp8_paged_mqa_block_amd as pm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_ALIGN = range(7)


def header_symbols():
    text = open(os.path.join(ROOT, "include", "pmqa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(\w+)\s*\(", text, flags=re.M)) - {"if"})


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pm.library_path()):
        pytest.fail("libpmqa.so not built: run python -m fp8_paged_mqa_block_amd.build")
    return pm.load_library()


def test_header_declares_the_exports():
    assert header_symbols() == sorted(pm.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", pm.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for sym in header_symbols():
        assert sym in exported, sym
        assert hasattr(lib, sym)


def test_status_strings_and_version(lib):
    for s in range(7):
        assert lib.pmqa_status_string(s)
    assert lib.pmqa_status_string(99) == b"unknown status"
    assert lib.pmqa_version() >= 100


# A fake, suitably aligned "device" address: the checks below all fail before
# the library could dereference or launch anything.
P = 0x10000


def logits(lib, **kw):
    a = dict(q=P, kv=P, w=P, ctx=P, tab=P, ps=64, nn=1, out=P, ors=1024, b=2, h=64, d=128,
             ts=16, stream=None)
    a.update(kw)
    return lib.paged_mqa_logits(a["q"], a["kv"], a["w"], a["ctx"], a["tab"], a["ps"], a["nn"],
                                a["out"], a["ors"], a["b"], a["h"], a["d"], a["ts"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), ERR_NULL), (dict(kv=None), ERR_NULL), (dict(w=None), ERR_NULL),
    (dict(ctx=None), ERR_NULL), (dict(tab=None), ERR_NULL), (dict(out=None), ERR_NULL),
    (dict(nn=0), ERR_SHAPE), (dict(b=-1), ERR_SHAPE), (dict(ors=0), ERR_SHAPE),
    (dict(ts=0), ERR_SHAPE), (dict(ps=0), ERR_SHAPE), (dict(ps=3), ERR_SHAPE), (dict(ps=24), ERR_SHAPE), (dict(ps=-8), ERR_SHAPE),
    (dict(ps=512), ERR_SHAPE), (dict(d=64), ERR_UNSUPPORTED), (dict(h=48), ERR_UNSUPPORTED),
    (dict(h=256), ERR_UNSUPPORTED), (dict(q=P + 8), ERR_ALIGN), (dict(w=P + 4), ERR_ALIGN),
    (dict(kv=P + 2), ERR_ALIGN), (dict(out=P + 2), ERR_ALIGN), (dict(tab=P + 4), ERR_ALIGN),
    (dict(b=0, q=None, kv=None), OK),
])
def test_logits_host_checks(lib, kw, status):
    assert logits(lib, **kw) == status


def topk(lib, **kw):
    a = dict(lg=P, ctx=P, k=2048, out=P, b=4, nn=1, rs=8192, ws=P, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.topk_per_row(a["lg"], a["ctx"], a["k"], a["out"], a["b"], a["nn"], a["rs"],
                            a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(lg=None), ERR_NULL), (dict(ctx=None), ERR_NULL), (dict(out=None), ERR_NULL),
    (dict(k=0), ERR_SHAPE), (dict(k=2049), ERR_SHAPE), (dict(nn=0), ERR_SHAPE),
    (dict(rs=0), ERR_SHAPE), (dict(b=-3), ERR_SHAPE), (dict(lg=P + 2), ERR_ALIGN),
    (dict(out=P + 1), ERR_ALIGN), (dict(b=0, lg=None), OK),
    # a workspace is optional (0 bytes, NULL), but a size needs memory behind it
    (dict(ws=None), ERR_WORKSPACE), (dict(ws=None, b=0), ERR_WORKSPACE),
    (dict(ws=P + 8), ERR_ALIGN), (dict(ws=P + 8, wsb=0, lg=None), ERR_NULL),
    (dict(ws=P + 8, wsb=0, b=0), OK),
])
def test_topk_host_checks(lib, kw, status):
    assert topk(lib, **kw) == status


@pytest.mark.parametrize("rows,k,max_len,want", [
    (64, 2048, 8192, 0),            # rows of one segment are never split
    (64, 2048, 16384, 0),
    (64, 2048, 16385, 64 * 3 * 2048 * 8),     # longer rows: segments of <= 8192
    (64, 2048, 131072, 64 * 8 * 2048 * 8),
    (64, 2048, 1 << 20, 64 * 8 * 2048 * 8),   # the merge holds 8 segments of 2048
    (1024, 2048, 32768, 1024 * 4 * 2048 * 8),
    (5, 100, 1 << 20, 5 * 128 * 100 * 8),     # 128 segments of 8192; 12800 candidates
    (5, 1, 1 << 20, 5 * 128 * 1 * 8),
    (0, 16, 1 << 20, 0),
    (-1, 16, 100000, 0), (4, 0, 100000, 0), (4, 2049, 100000, 0), (4, 16, -1, 0),
])
def test_topk_workspace_size(lib, rows, k, max_len, want):
    assert lib.topk_per_row_workspace_size(rows, k, max_len) == want
    assert pm.topk_workspace_size(rows, k, max_len) == want if rows >= 0 else True


def test_binding_rejects_wrong_dtypes_before_the_library():
    import torch
    t = torch.zeros(4, dtype=torch.float32)
    with pytest.raises(ValueError):
        pm.paged_mqa_logits(t, t, t, t, t, 64, 1, t)


def check(lib, **kw):
    a = dict(ctx=P, tab=P, b=4, ps=64, ts=16, ors=1024, np=100, res=P, stream=None)
    a.update(kw)
    return lib.pmqa_check_inputs(a["ctx"], a["tab"], a["b"], a["ps"], a["ts"], a["ors"], a["np"],
                                 a["res"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(res=None), ERR_NULL), (dict(ctx=None), ERR_NULL), (dict(tab=None), ERR_NULL),
    (dict(b=-1), ERR_SHAPE), (dict(ps=12), ERR_SHAPE), (dict(ts=0), ERR_SHAPE),
    (dict(ors=0), ERR_SHAPE), (dict(np=0), ERR_SHAPE), (dict(res=P + 2), ERR_ALIGN),
    (dict(tab=P + 4), ERR_ALIGN),
])
def test_check_inputs_host_checks(lib, kw, status):
    assert check(lib, **kw) == status


def kcache(lib, **kw):
    a = dict(k=P, dt=0, sl=P, n=16, d=128, kv=P, ns=1000, stream=None)
    a.update(kw)
    return lib.quantize_k_cache(a["k"], a["dt"], a["sl"], a["n"], a["d"], a["kv"], a["ns"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(k=None), ERR_NULL), (dict(sl=None), ERR_NULL), (dict(kv=None), ERR_NULL),
    (dict(n=-1), ERR_SHAPE), (dict(ns=-1), ERR_SHAPE), (dict(dt=2), ERR_UNSUPPORTED),
    (dict(dt=-1), ERR_UNSUPPORTED), (dict(d=64), ERR_UNSUPPORTED), (dict(k=P + 8), ERR_ALIGN),
    (dict(sl=P + 4), ERR_ALIGN), (dict(kv=P + 2), ERR_ALIGN),
    (dict(n=0, k=None, sl=None, kv=None), OK), (dict(dt=1, n=0), OK),
])
def test_quantize_k_cache_host_checks(lib, kw, status):
    assert kcache(lib, **kw) == status


def test_quantize_k_cache_binding_rejects_wrong_dtypes():
    import torch
    k = torch.zeros(4, 128, dtype=torch.float16)
    with pytest.raises(ValueError):
        pm.quantize_k_cache(k, torch.zeros(4, dtype=torch.int64), torch.zeros(1320, dtype=torch.uint8))


@pytest.mark.parametrize("sizes, name", [
    # the five workloads' shapes: (batch, next_n, page_size, out_row_stride, heads, table width)
    ((2, 1, 64, 1024, 64, 16), "logits_flat_kernel<64,1>"),
    ((64, 1, 64, 8192, 64, 128), "logits_flat_kernel<64,1>"),
    ((256, 4, 256, 1 << 20, 128, 128), "logits_shared_kernel<128,4,8>"),
    ((128, 3, 8, 65536, 64, 8192), "logits_kernel<64,3,8,2>"),
    ((32, 2, 64, 131072, 128, 2048), "logits_shared_kernel<128,2,4>"),
    # the single-wave geometry's bound: at most 8192 possible 64-token iterations
    ((64, 1, 64, 8256, 64, 129), "logits_kernel<64,1,9,1>"),
    ((128, 1, 64, 4096, 64, 64), "logits_flat_kernel<64,1>"),
    ((16, 4, 16, 2048, 16, 128), "logits_flat_kernel<16,4>"),
    ((16, 3, 16, 2048, 32, 128), "logits_kernel<32,3,4,4>"),
    # 128 heads: next_n 3 keeps one ring per wave, 1 row per request the flat geometry
    ((8, 3, 64, 4096, 128, 64), "logits_kernel<128,1,8,2>"),
])
def test_logits_kernel_names(lib, sizes, name):
    """The launch geometry paged_mqa_logits takes for given sizes (host only)."""
    batch, next_n, ps, stride, heads, width = sizes
    assert pm.logits_kernel(batch, next_n, ps, stride, heads, width) == name


def test_logits_kernel_name_errors(lib):
    buf = ctypes.create_string_buffer(8)
    assert lib.pmqa_logits_kernel(2, 1, 64, 1024, 64, 128, 16, None, 8) == ERR_NULL
    # the name does not fit
    assert lib.pmqa_logits_kernel(2, 1, 64, 1024, 64, 128, 16, buf, len(buf)) == ERR_SHAPE
    big = ctypes.create_string_buffer(64)
    assert lib.pmqa_logits_kernel(2, 1, 64, 1024, 96, 128, 16, big, 64) == ERR_UNSUPPORTED
    assert lib.pmqa_logits_kernel(2, 1, 48, 1024, 64, 128, 16, big, 64) == ERR_SHAPE


def noalloc(lib, **kw):
    a = dict(lg=P, ctx=P, k=2048, out=P, b=64, nn=1, rs=131072, stream=None)
    a.update(kw)
    return lib.topk_per_row_noalloc(a["lg"], a["ctx"], a["k"], a["out"], a["b"], a["nn"], a["rs"],
                                    a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(lg=None), ERR_NULL), (dict(ctx=None), ERR_NULL), (dict(out=None), ERR_NULL),
    (dict(k=0), ERR_SHAPE), (dict(nn=0), ERR_SHAPE), (dict(rs=0), ERR_SHAPE), (dict(b=-1), ERR_SHAPE),
    # the split the stride calls for needs more than the library's scratch:
    # 1024 rows * 8 segments * 2048 candidates * 8 bytes = 128 MiB > 64 MiB
    (dict(b=1024, rs=1 << 20), ERR_WORKSPACE), (dict(b=1024, rs=1 << 20, lg=None), ERR_WORKSPACE),
    (dict(b=0), OK), (dict(b=0, lg=None), OK),
])
def test_topk_noalloc_host_checks(lib, kw, status):
    assert noalloc(lib, **kw) == status


def test_noalloc_scratch_size_in_header_matches_a_full_split():
    text = open(os.path.join(ROOT, "include", "pmqa.h")).read()
    m = re.search(r"#define PMQA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == 64 << 20
    # the long-context and small-pages workloads' full splits fit; the MTP workload's stride does not
    assert pm.topk_workspace_size(64, 2048, 131072) <= 64 << 20
    assert pm.topk_workspace_size(384, 2048, 65536) <= 64 << 20
    assert pm.topk_workspace_size(1024, 2048, 1 << 20) > 64 << 20


@pytest.mark.parametrize("ps,status", [(1, ERR_UNSUPPORTED), (2, ERR_UNSUPPORTED),
                                       (4, ERR_UNSUPPORTED), (12, ERR_SHAPE), (0, ERR_SHAPE)])
def test_preshuffled_page_sizes(lib, ps, status):
    assert lib.paged_mqa_logits_preshuffled(P, P, P, P, P, ps, 1, P, 1024, 2, 64, 128, 16,
                                            None) == status
    assert lib.quantize_k_cache_preshuffled(P, 0, P, 4, 128, P, 64, ps, None) == status


def test_preshuffled_producer_needs_whole_pages(lib):
    assert lib.quantize_k_cache_preshuffled(P, 0, P, 4, 128, P, 100, 64, None) == ERR_SHAPE
