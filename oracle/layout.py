"""The preshuffled page layout of the K cache (test infrastructure only).

The pages name a preshuffled K-page layout only through a library call that
reshapes each page into (min(page, 16), 16) tiles (aiter PR #6626, section 1,
the loader of 8-token pages) and never define its permutation, so this is a
format of this path's own, with the same idea: a page is cut into tiles of
R = min(page_size, 16) tokens, and inside a tile the bytes are ordered so that
a matrix-core operand of one token is a run of contiguous 16-byte pieces.

Definition (head_dim D = 128, record size D + 4 = 132 bytes per token, so a
page keeps page_size * 132 bytes and pools are sized exactly as in the record
layout).  Cache row s (page p = s // P, token u = s % P of the page):

* tile t = u // R of page p starts at byte p * P * 132 + t * R * 132;
* m = u % R is the token's place in its tile;
* value byte d of the token (code of element d) sits at
  tile_start + ((h * 4 + q) * R + m) * 16 + b with h = d // 64, q = (d % 64) // 16,
  b = d % 16: the tile holds 8 groups (h, q), each the 16-byte pieces of its R
  tokens in token order;
* the token's fp32 scale (little endian) sits at tile_start + 128 * R + 4 * m:
  the R scales follow the tile's values, in token order.

This is plain addressing written from that definition; it shares nothing with
the HIP path.
"""
import numpy as np

HEAD_DIM = 128


def tile_rows(page_size: int) -> int:
    """Tokens per tile: min(page_size, 16)."""
    return min(int(page_size), 16)


def preshuffled_offsets(slots, page_size: int, head_dim: int = HEAD_DIM):
    """Byte offsets of cache rows `slots` in a preshuffled pool: (values
    [n, head_dim] int64, scales [n] int64).  Python-int-safe: int64 throughout."""
    if head_dim != HEAD_DIM:
        raise ValueError("the preshuffled layout is defined for head_dim 128")
    s = np.asarray(slots, dtype=np.int64).reshape(-1)
    P = np.int64(page_size)
    R = np.int64(tile_rows(page_size))
    rec = np.int64(head_dim + 4)
    page, u = s // P, s % P
    tile_start = page * P * rec + (u // R) * R * rec
    m = u % R
    d = np.arange(head_dim, dtype=np.int64)
    h, q, b = d // 64, (d % 64) // 16, d % 16
    values = tile_start[:, None] + ((h * 4 + q)[None, :] * R + m[:, None]) * 16 + b[None, :]
    scales = tile_start + 128 * R + 4 * m
    return values, scales
