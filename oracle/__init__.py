"""CPU oracle for the FP8 paged MQA logits + per-row top-k path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or run
anything in this package; only the tests, the smoke entry point and the CPU
baseline leg of the benchmark use it.  It shares no code with the HIP path: it
has its own fp8 decoder, its own page gather and its own address arithmetic,
all in plain numpy fp64 (Python ints for addresses).

What it computes (the plain definition, written out):

* ``logit[r, t] = sum_h w[r, h] * relu(scale_t * (q[r, h, :] . k_t))`` for the
  tokens a row may see, ``-inf`` for the masked tail of the context, and
  nothing at all past the context (those output columns are left untouched);
* the top-k token indices per row, ties broken by ascending index, padded
  with -1 when a row sees fewer than k tokens;
* the K-cache records the logits read, produced from new K rows (per-token
  scale amax/448, e4m3fn codes by round-to-nearest-even, records written at
  int64 slots): ``oracle.k_cache``;
* the preshuffled page layout (a format of this path: tiles of min(page, 16)
  tokens whose operand pieces are contiguous): ``oracle.layout``, read by the
  gather and written by the K-cache writer.

Sources: the op and its tensors are those of ``deepgemm_fp8_paged_mqa_logits``
(aiter PR #4244 "fix silent tail-row drop in deepgemm_fp8_paged_mqa_logits at
large output stride": bug description, root cause, and the reproducer's
inputs), with its output feeding ``top_k_per_row_decode`` (same page, first
paragraph).  The pages do not print the score formula; the formula above is
the DSA indexer score adopted as the reading.  See each function for the
passage it follows and the readings where the pages are silent.

Pins (what ties this oracle to something other than itself) live in
``tests/test_oracle_*.py``: every e4m3fn code against torch's float8 cast
and the format's published spot values, exact rational brute force of the
dots, hand-derived worked examples under ``tests/golden/``, the matmul
reduction, and invariants (table permutation, output stride, batch split,
power-of-two scaling, MTP prefix, row coverage with an emulated 32-bit
store as negative control).
"""
from .fp8 import e4m3fn_to_float64, E4M3FN_TABLE  # noqa: F401
from .paged_mqa import (  # noqa: F401
    visible_len,
    gather_request,
    request_logits,
    paged_mqa_logits,
    topk_per_row,
    NEG_INF_BITS,
)
from .layout import preshuffled_offsets, tile_rows  # noqa: F401,E402
from .k_cache import (  # noqa: F401,E402
    e4m3fn_encode,
    bf16_to_float32,
    quantize_tokens,
    record_offset,
    write_k_cache,
)
