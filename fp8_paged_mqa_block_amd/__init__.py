"""FP8 paged MQA logits + per-row top-k on MI355X (gfx950).

A thin ctypes binding over ``libpmqa.so`` (C ABI in ``include/pmqa.h``).  It only
checks and marshals arguments: every step of the computation runs in the
library's HIP kernels.  torch tensors provide the device memory and the
stream.  There is no fallback: when the library is missing or no GPU is
visible the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "PmqaError",
    "load_library",
    "library_path",
    "logits_kernel",
    "paged_mqa_logits",
    "topk_per_row",
    "topk_workspace_size",
    "check_inputs",
    "quantize_k_cache",
    "EXPORTS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libpmqa.so")
_lib: Optional[ctypes.CDLL] = None

# Every symbol include/pmqa.h declares.
EXPORTS = ("paged_mqa_logits", "paged_mqa_logits_timed", "paged_mqa_logits_preshuffled",
           "paged_mqa_logits_preshuffled_timed", "quantize_k_cache_preshuffled",
           "topk_per_row", "topk_per_row_timed",
           "topk_per_row_workspace_size", "topk_per_row_noalloc", "pmqa_check_inputs",
           "quantize_k_cache",
           "quantize_k_cache_timed", "pmqa_status_string", "pmqa_version", "pmqa_logits_kernel")

# pmqa_dtype codes of the K rows quantize_k_cache accepts
_K_DTYPES = {torch.float32: 0, torch.bfloat16: 1}

_STATUS = {0: "PMQA_OK", 1: "PMQA_ERR_NULL", 2: "PMQA_ERR_SHAPE", 3: "PMQA_ERR_UNSUPPORTED",
           4: "PMQA_ERR_WORKSPACE", 5: "PMQA_ERR_HIP", 6: "PMQA_ERR_ALIGNMENT"}


class PmqaError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {_STATUS.get(status, status)} ({msg})")
        self.status = status


def logits_kernel(batch: int, next_n: int, page_size: int, out_row_stride: int,
                  num_heads: int, block_table_stride: int, head_dim: int = 128) -> str:
    """Name of the logits kernel paged_mqa_logits launches for these sizes
    (host only; see pmqa_logits_kernel in include/pmqa.h)."""
    buf = ctypes.create_string_buffer(64)
    st = load_library().pmqa_logits_kernel(batch, next_n, page_size, out_row_stride, num_heads,
                                           head_dim, block_table_stride, buf, len(buf))
    _check("pmqa_logits_kernel", st)
    return buf.value.decode()


def library_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load libpmqa.so (built in-tree by fp8_paged_mqa_block_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with `python -m fp8_paged_mqa_block_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    c_i32, c_i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    lib.paged_mqa_logits.restype = ctypes.c_int
    lib.paged_mqa_logits.argtypes = [vp, vp, vp, vp, vp, c_i32, c_i32, vp, c_i64, c_i32, c_i32,
                                     c_i32, c_i64, vp]
    lib.paged_mqa_logits_timed.restype = ctypes.c_int
    lib.paged_mqa_logits_timed.argtypes = lib.paged_mqa_logits.argtypes + [vp, vp]
    lib.paged_mqa_logits_preshuffled.restype = ctypes.c_int
    lib.paged_mqa_logits_preshuffled.argtypes = lib.paged_mqa_logits.argtypes
    lib.paged_mqa_logits_preshuffled_timed.restype = ctypes.c_int
    lib.paged_mqa_logits_preshuffled_timed.argtypes = lib.paged_mqa_logits_timed.argtypes
    lib.quantize_k_cache_preshuffled.restype = ctypes.c_int
    lib.quantize_k_cache_preshuffled.argtypes = [vp, c_i32, vp, c_i32, c_i32, vp, c_i64, c_i32, vp]
    lib.topk_per_row.restype = ctypes.c_int
    lib.topk_per_row.argtypes = [vp, vp, c_i32, vp, c_i32, c_i32, c_i64, vp, ctypes.c_size_t, vp]
    lib.topk_per_row_timed.restype = ctypes.c_int
    lib.topk_per_row_timed.argtypes = lib.topk_per_row.argtypes + [vp, vp]
    lib.topk_per_row_noalloc.restype = ctypes.c_int
    lib.topk_per_row_noalloc.argtypes = [vp, vp, c_i32, vp, c_i32, c_i32, c_i64, vp]
    lib.topk_per_row_workspace_size.restype = ctypes.c_size_t
    lib.topk_per_row_workspace_size.argtypes = [c_i32, c_i32, c_i64]
    lib.pmqa_check_inputs.restype = ctypes.c_int
    lib.pmqa_check_inputs.argtypes = [vp, vp, c_i32, c_i32, c_i64, c_i64, c_i64, vp, vp]
    lib.quantize_k_cache.restype = ctypes.c_int
    lib.quantize_k_cache.argtypes = [vp, c_i32, vp, c_i32, c_i32, vp, c_i64, vp]
    lib.quantize_k_cache_timed.restype = ctypes.c_int
    lib.quantize_k_cache_timed.argtypes = lib.quantize_k_cache.argtypes + [vp, vp]
    lib.pmqa_status_string.restype = ctypes.c_char_p
    lib.pmqa_status_string.argtypes = [ctypes.c_int]
    lib.pmqa_version.restype = ctypes.c_int32
    lib.pmqa_version.argtypes = []
    lib.pmqa_logits_kernel.restype = ctypes.c_int
    lib.pmqa_logits_kernel.argtypes = [c_i32, c_i32, c_i32, c_i64, c_i32, c_i32, c_i64,
                                       ctypes.c_char_p, c_i32]
    _lib = lib
    return lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        msg = load_library().pmqa_status_string(status).decode()
        raise PmqaError(fn, status, msg)


def _stream_handle(t: torch.Tensor, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return int(stream.cuda_stream)


def _need(cond: bool, what: str) -> None:
    if not cond:
        raise ValueError(what)


def _byte_view(t: torch.Tensor, name: str) -> torch.Tensor:
    _need(t.dtype in (torch.uint8, torch.float8_e4m3fn), f"{name} must be uint8 or float8_e4m3fn, got {t.dtype}")
    return t


def paged_mqa_logits(q: torch.Tensor, kv_cache: torch.Tensor, weights: torch.Tensor,
                     context_lens: torch.Tensor, block_tables: torch.Tensor, page_size: int,
                     next_n: int, out: torch.Tensor, stream=None,
                     layout: str = "records") -> torch.Tensor:
    """Enqueue the logits step; writes ``out`` in place and returns it.

    q            [B*next_n, H, 128] or [B, next_n, H, 128], e4m3fn (or its uint8 bytes), contiguous
    kv_cache     page pool [num_pages, page_size, 132] bytes (any contiguous shape)
    weights      [B*next_n, H] float32, contiguous
    context_lens [B] int32
    block_tables [B, W] int64, contiguous (W entries per request)
    out          [B*next_n, cols] float32, contiguous (cols = the row stride)
    layout       "records" (paged_mqa_logits) or "preshuffled" (paged_mqa_logits_preshuffled)
    """
    lib = load_library()
    _byte_view(q, "q")
    _byte_view(kv_cache, "kv_cache")
    for name, t in (("q", q), ("kv_cache", kv_cache), ("weights", weights),
                    ("context_lens", context_lens), ("block_tables", block_tables), ("out", out)):
        _need(t.is_cuda, f"{name} must be a device tensor")
    _need(weights.dtype == torch.float32, "weights must be float32")
    _need(context_lens.dtype == torch.int32, "context_lens must be int32")
    _need(block_tables.dtype == torch.int64, "block_tables must be int64 (int32 ids wrap past 2^31 bytes)")
    _need(out.dtype == torch.float32, "out must be float32")
    _need(q.is_contiguous() and kv_cache.is_contiguous() and weights.is_contiguous()
          and context_lens.is_contiguous(), "q, kv_cache, weights, context_lens must be contiguous")
    B = context_lens.shape[0]
    _need(context_lens.dim() == 1, "context_lens must be 1-D")
    if q.dim() == 4:
        _need(q.shape[0] == B and q.shape[1] == next_n, "q [B, next_n, H, D] does not match")
        q = q.reshape(B * next_n, q.shape[2], q.shape[3])
    _need(q.dim() == 3 and q.shape[0] == B * next_n, "q must be [B*next_n, H, D]")
    H, D = int(q.shape[1]), int(q.shape[2])
    _need(tuple(weights.shape) == (B * next_n, H), "weights must be [B*next_n, H]")
    # the row stride doubles as the row's capacity in the C ABI, so rows must be
    # exactly as wide as their stride
    _need(block_tables.dim() == 2 and block_tables.shape[0] == B and block_tables.is_contiguous(),
          "block_tables must be a contiguous [B, W] tensor")
    _need(out.dim() == 2 and out.shape[0] == B * next_n and out.is_contiguous(),
          "out must be a contiguous [B*next_n, cols] tensor")
    ts = block_tables.shape[1]
    # a [B, 0] table cannot hold any page: the stride it would pass (1) would
    # let the kernel read an entry the tensor does not have
    _need(ts >= 1 or B == 0, "block_tables must have at least one entry per request")
    _need(layout in ("records", "preshuffled"), f"unknown layout {layout}")
    fn = lib.paged_mqa_logits if layout == "records" else lib.paged_mqa_logits_preshuffled
    st = fn(q.data_ptr(), kv_cache.data_ptr(), weights.data_ptr(),
                              context_lens.data_ptr(), block_tables.data_ptr(), int(page_size),
                              int(next_n), out.data_ptr(), int(out.shape[1]), int(B), H, D,
                              int(max(ts, 1)), _stream_handle(out, stream))
    _check("paged_mqa_logits", st)
    return out


def topk_workspace_size(rows: int, k: int, max_row_len: int) -> int:
    """Workspace bytes with which topk_per_row splits rows of up to max_row_len
    visible scores fully (host only; see topk_per_row_workspace_size in include/pmqa.h)."""
    return int(load_library().topk_per_row_workspace_size(int(rows), int(k), int(max_row_len)))


def topk_per_row(logits: torch.Tensor, context_lens: torch.Tensor, k: int, out_idx: torch.Tensor,
                 next_n: int = 1, workspace: Optional[torch.Tensor] = None,
                 max_row_len: Optional[int] = None, stream=None) -> torch.Tensor:
    """Enqueue the per-row top-k; writes ``out_idx`` [B*next_n, k] int32 in place and returns it.

    ``workspace`` is a device uint8 tensor the selection may use for the
    candidates of long rows.  When None, one is allocated (torch's caching
    allocator) of topk_workspace_size(rows, k, max_row_len), max_row_len
    defaulting to the row stride; pass an explicit tensor (any size, 0
    included) to control the memory.
    """
    lib = load_library()
    for name, t in (("logits", logits), ("context_lens", context_lens), ("out_idx", out_idx)):
        _need(t.is_cuda, f"{name} must be a device tensor")
    _need(logits.dtype == torch.float32 and logits.dim() == 2 and logits.is_contiguous(),
          "logits must be a contiguous 2-D float32 tensor")
    _need(context_lens.dtype == torch.int32 and context_lens.dim() == 1 and context_lens.is_contiguous(),
          "context_lens must be contiguous 1-D int32")
    B = context_lens.shape[0]
    _need(logits.shape[0] == B * next_n, "logits must have B*next_n rows")
    _need(out_idx.dtype == torch.int32 and out_idx.is_contiguous()
          and tuple(out_idx.shape) == (B * next_n, k), "out_idx must be contiguous int32 [B*next_n, k]")
    if workspace is None:
        size = topk_workspace_size(B * next_n, k, logits.shape[1] if max_row_len is None else max_row_len)
        workspace = torch.empty(max(size, 1), dtype=torch.uint8, device=logits.device)
    _need(workspace.is_cuda and workspace.dtype == torch.uint8 and workspace.is_contiguous(),
          "workspace must be a contiguous uint8 device tensor")
    nbytes = int(workspace.numel())
    st = lib.topk_per_row(logits.data_ptr(), context_lens.data_ptr(), int(k), out_idx.data_ptr(),
                          int(B), int(next_n), int(logits.shape[1]),
                          workspace.data_ptr() if nbytes else None, nbytes,
                          _stream_handle(out_idx, stream))
    _check("topk_per_row", st)
    return out_idx


def quantize_k_cache(k: torch.Tensor, slot_mapping: torch.Tensor, kv_cache: torch.Tensor,
                     stream=None, page_size: int = 0) -> torch.Tensor:
    """Enqueue the K-cache producer: quantise rows of k into the records of kv_cache
    at their slots (in place; returns kv_cache).

    k            [num_tokens, 128] float32 or bfloat16, contiguous
    slot_mapping [num_tokens] int64 cache rows (page * page_size + offset); rows
                 outside the pool (e.g. -1 for padding) are skipped
    kv_cache     page pool bytes (uint8 or float8_e4m3fn, any contiguous shape);
                 its byte size / 132 is the number of cache rows
    page_size    0: per-token records (quantize_k_cache); otherwise the pool's
                 page size, writing the preshuffled page layout
                 (quantize_k_cache_preshuffled)
    """
    lib = load_library()
    _byte_view(kv_cache, "kv_cache")
    for name, t in (("k", k), ("slot_mapping", slot_mapping), ("kv_cache", kv_cache)):
        _need(t.is_cuda, f"{name} must be a device tensor")
    _need(k.dtype in _K_DTYPES, f"k must be float32 or bfloat16, got {k.dtype}")
    _need(k.dim() == 2 and k.is_contiguous(), "k must be a contiguous [num_tokens, head_dim] tensor")
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.dim() == 1 and slot_mapping.is_contiguous()
          and slot_mapping.shape[0] == k.shape[0], "slot_mapping must be contiguous int64 [num_tokens]")
    _need(kv_cache.is_contiguous(), "kv_cache must be contiguous")
    num_slots = kv_cache.numel() // (int(k.shape[1]) + 4)
    if page_size:
        st = lib.quantize_k_cache_preshuffled(k.data_ptr(), _K_DTYPES[k.dtype], slot_mapping.data_ptr(),
                                              int(k.shape[0]), int(k.shape[1]), kv_cache.data_ptr(),
                                              int(num_slots), int(page_size),
                                              _stream_handle(kv_cache, stream))
    else:
        st = lib.quantize_k_cache(k.data_ptr(), _K_DTYPES[k.dtype], slot_mapping.data_ptr(),
                                  int(k.shape[0]), int(k.shape[1]), kv_cache.data_ptr(), int(num_slots),
                                  _stream_handle(kv_cache, stream))
    _check("quantize_k_cache", st)
    return kv_cache


def check_inputs(context_lens: torch.Tensor, block_tables: torch.Tensor, page_size: int,
                 out_row_stride: int, num_pages: int, stream=None):
    """Debug check of the device-resident preconditions (synchronises).

    Returns ``(violations, first)``: the number of requests whose context does
    not fit its table row or output row, or that use a page id outside
    ``[0, num_pages)``, and the lowest such request index (``B`` when none).
    """
    lib = load_library()
    _need(context_lens.is_cuda and block_tables.is_cuda, "inputs must be device tensors")
    _need(context_lens.dtype == torch.int32 and context_lens.dim() == 1 and context_lens.is_contiguous(),
          "context_lens must be contiguous 1-D int32")
    B = context_lens.shape[0]
    _need(block_tables.dtype == torch.int64 and block_tables.dim() == 2 and block_tables.shape[0] == B
          and block_tables.is_contiguous(), "block_tables must be a contiguous [B, W] int64 tensor")
    _need(block_tables.shape[1] >= 1 or B == 0, "block_tables must have at least one entry per request")
    result = torch.empty(2, dtype=torch.int32, device=context_lens.device)
    st = lib.pmqa_check_inputs(context_lens.data_ptr(), block_tables.data_ptr(), int(B), int(page_size),
                               int(max(block_tables.shape[1], 1)), int(out_row_stride), int(num_pages),
                               result.data_ptr(), _stream_handle(result, stream))
    _check("pmqa_check_inputs", st)
    r = result.cpu()
    return int(r[0]), int(r[1])

