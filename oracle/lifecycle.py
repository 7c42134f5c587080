"""Page lifecycle operations on a paged KV pool — CPU oracle (test
infrastructure only).

What they compute:

* swap out / swap in (MoE-Infinity PR #183, "What landed", serving-lifecycle
  bullet: pages leave the GPU and come back with their INT8 scales). In the
  page layout of ``oracle.pages`` a token's scales live in the same page as
  its codes, so moving whole pages moves both. Swap-out copies pages
  ``block_ids[i]`` of the pool, in order, into a contiguous array; swap-in
  copies such an array back into (possibly other) pages. An out-of-range
  block id is skipped (that entry is neither read nor written).

* front trim that keeps sink tokens (mlxcel PR #717 and its follow-up on the
  same page: ``trim_front_keep_sink(n, keep)`` drops the n tokens that follow
  the first ``keep`` positions instead of the n oldest, so the first tokens
  (attention sinks) survive; the INT8 scales move with their tokens). For a
  sequence of length L the result holds positions ``0 .. keep-1`` unchanged
  followed by the old positions ``keep + n .. L-1``; the new length is
  ``L - n``. Readings (listed in the design doc): n is clamped to
  ``[0, max(L - keep, 0)]``; the tokens are rewritten through the
  sequence's unchanged block table; slots at or past the new length keep
  whatever they held (they are no longer part of the sequence).
"""

from __future__ import annotations

import numpy as np

from .pages import (KV_16BIT, KV_INT8_STATIC, KV_INT8_SYM, _v_index, int8_token_bytes,
                    page_bytes)


def swap_out_pages(pool: np.ndarray, block_ids) -> np.ndarray:
    """Pages ``block_ids`` of the pool, in order: [n, page_bytes] uint8.
    Entries with an out-of-range id stay zero."""
    ids = np.asarray(block_ids, dtype=np.int64)
    out = np.zeros((len(ids), pool.shape[1]), dtype=np.uint8)
    ok = (ids >= 0) & (ids < pool.shape[0])
    out[ok] = pool[ids[ok]]
    return out


def swap_in_pages(pool: np.ndarray, block_ids, pages: np.ndarray) -> None:
    """Write ``pages[i]`` into page ``block_ids[i]`` of the pool (in order;
    out-of-range ids are skipped)."""
    ids = np.asarray(block_ids, dtype=np.int64)
    for i, blk in enumerate(ids):
        if 0 <= blk < pool.shape[0]:
            pool[blk] = pages[i]


def _token_byte_index(kv_format: int, block_size: int, head_dim: int, num_kv_heads: int,
                      page_len: int, blk: np.ndarray, pos: np.ndarray, head: int) -> np.ndarray:
    """Flat pool byte indexes [n, bytes_per_token] of every byte that belongs
    to token slot ``pos`` of page ``blk`` for KV head ``head`` (K row, V
    entries, and for per-token INT8 the two scales)."""
    d = head_dim
    dd = np.arange(d)
    if kv_format == KV_INT8_SYM:
        page0 = (blk * page_len)[:, None]
        parts = [page0 + i for i in int8_token_bytes(block_size, num_kv_heads, d, head, pos)]
    elif kv_format == KV_INT8_STATIC:
        base = blk * page_len + head * 2 * block_size * d
        parts = [base[:, None] + pos[:, None] * d + dd,
                 base[:, None] + block_size * d + _v_index(pos[:, None], dd[None, :], d)]
    elif kv_format == KV_16BIT:
        base = blk * page_len + head * 4 * block_size * d
        two = np.arange(2)
        k_el = pos[:, None] * d + dd                                   # element index
        v_el = block_size * d + _v_index(pos[:, None], dd[None, :], d)
        parts = [(base[:, None, None] + 2 * k_el[:, :, None] + two).reshape(len(pos), -1),
                 (base[:, None, None] + 2 * v_el[:, :, None] + two).reshape(len(pos), -1)]
    else:
        raise ValueError("unknown format")
    return np.concatenate(parts, axis=1)


def trim_keep_sink(kv_format: int, pool: np.ndarray, block_tables, context_lens, trim_lens,
                   keep: int, block_size: int, num_kv_heads: int, head_dim: int):
    """Drop ``trim_lens[b]`` tokens after the first ``keep`` of every
    sequence b, in place. Returns the new context lengths (int32 [B])."""
    if keep < 0:
        raise ValueError("keep must be >= 0")
    if pool.shape[1] != page_bytes(kv_format, block_size, num_kv_heads, head_dim):
        raise ValueError("pool page size does not match the shape")
    flat = pool.reshape(-1)
    new_lens = np.asarray(context_lens, dtype=np.int64).copy()
    for b, L in enumerate(np.asarray(context_lens, dtype=np.int64)):
        n = int(min(max(int(trim_lens[b]), 0), max(int(L) - keep, 0)))
        new_lens[b] = L - n
        if n == 0 or keep + n >= L:  # nothing dropped, or nothing left to move
            continue
        src = np.arange(keep + n, L)            # old positions that survive after the sink
        dst = np.arange(keep, L - n)            # their new positions
        row = np.asarray(block_tables[b], dtype=np.int64)
        for h in range(num_kv_heads):
            si = _token_byte_index(kv_format, block_size, head_dim, num_kv_heads, pool.shape[1],
                                   row[src // block_size], src % block_size, h)
            di = _token_byte_index(kv_format, block_size, head_dim, num_kv_heads, pool.shape[1],
                                   row[dst // block_size], dst % block_size, h)
            flat[di] = flat[si].copy()         # read every source before any write
    return new_lens.astype(np.int32)
