"""Paged KV-pool byte layout — CPU oracle (test infrastructure only).

The pages fix only the byte totals: an INT8 page holds the INT8 payload plus
one FP16 scale per (layer, page, KV head, token), 33,280 bytes for
(block_size 16, 8 KV heads, head_dim 128) against 65,536 bytes for an FP16
page (MoE-Infinity PR #183, "Precision & memory"). Those totals require one
scale for K and a separate one for V per token and head. The byte order
inside a page is not on the pages; this module implements the layout that the
library's C header documents, written out again here from that description
(no code or constant is shared with the library):

INT8 page (``page_bytes = Hkv * (2*bs*D + 4*bs)``): the codes of every KV
head first, then the scales of every KV head:

    head h's codes at h * 2*bs*D:
        K codes   int8  [bs][D]           token-major
        V codes   int8  [bs/4][D][4]      groups of 4 tokens, dimension-major
                                          inside a group: byte (p//4)*4D + 4d + p%4
    head h's scales at Hkv * 2*bs*D + h * 4*bs, one 16-byte record per group
    of 4 tokens (g = p//4, at 16*g):
        K scales  fp16  [4]               token 4g + i at 2*i
        V scales  fp16  [4]               token 4g + i at 8 + 2*i

16-bit page (fp16 or bf16, same dtype as the model), per KV head h (head
block of ``4*bs*D`` bytes, ``page_bytes = Hkv * 4*bs*D``):

    K   [bs][D]                       token-major
    V   [bs/4][D][4]                  same token grouping as the INT8 V codes

INT8 page with static scales (one calibrated scalar for K and one for V per
layer, held by the caller; no per-token scales in the page), per KV head h
(head block of ``2*bs*D`` bytes, ``page_bytes = Hkv * 2*bs*D`` — half the
16-bit page, the one-byte-per-element saving of InfiniLM PR #553, "Benchmark
/ Performance Impact"):

    K codes   int8  [bs][D]           token-major
    V codes   int8  [bs/4][D][4]      as in the per-token INT8 page

A token at logical position t of a sequence lives in physical page
``block_table[t // bs]`` at slot ``t % bs``; a write addresses it by
``slot = page * bs + t % bs`` (paged decode, MoE-Infinity PR #183, "What
landed").
"""

from __future__ import annotations

import numpy as np

KV_INT8_SYM = 1
KV_16BIT = 2
KV_INT8_STATIC = 3


def page_bytes(kv_format: int, block_size: int, num_kv_heads: int, head_dim: int) -> int:
    """Bytes of one page (all KV heads of one layer, ``block_size`` tokens)."""
    if block_size <= 0 or block_size % 4 or num_kv_heads <= 0 or head_dim <= 0:
        raise ValueError("page_bytes: bad shape")
    if kv_format == KV_INT8_SYM:
        return num_kv_heads * (2 * block_size * head_dim + 4 * block_size)
    if kv_format == KV_16BIT:
        return num_kv_heads * 4 * block_size * head_dim
    if kv_format == KV_INT8_STATIC:
        return num_kv_heads * 2 * block_size * head_dim
    raise ValueError("page_bytes: unknown format")


def int8_layout(block_size: int, num_kv_heads: int, head_dim: int) -> dict:
    """Byte offsets of an INT8 page's regions: each KV head's code block
    (``code_bytes`` long, K codes then V codes) and scale block
    (``scale_bytes`` long) after all code blocks."""
    bs, d = block_size, head_dim
    return {"code_bytes": 2 * bs * d, "v_codes": bs * d,
            "scales": num_kv_heads * 2 * bs * d, "scale_bytes": 4 * bs}


def _int8_scale_offset(pos, is_v: int):
    """Byte offset of token ``pos``'s K (is_v=0) or V (is_v=1) scale inside
    its head's scale block: 16-byte records per group of 4 tokens."""
    return (pos // 4) * 16 + 8 * is_v + 2 * (pos % 4)


def int8_token_bytes(block_size: int, num_kv_heads: int, head_dim: int, head: int, pos):
    """Byte indexes inside an INT8 page of token slot(s) ``pos`` (array [n])
    of KV head ``head``: K codes [n, D], V codes [n, D], K scale [n, 2] and V
    scale [n, 2] (little-endian fp16)."""
    lay = int8_layout(block_size, num_kv_heads, head_dim)
    d = head_dim
    pos = np.asarray(pos, dtype=np.int64)[:, None]
    dd = np.arange(d)[None, :]
    two = np.arange(2)[None, :]
    code = head * lay["code_bytes"]
    sc = lay["scales"] + head * lay["scale_bytes"]
    return (code + pos * d + dd,
            code + lay["v_codes"] + _v_index(pos, dd, d),
            sc + _int8_scale_offset(pos, 0) + two,
            sc + _int8_scale_offset(pos, 1) + two)


def new_pool(kv_format: int, num_blocks: int, block_size: int, num_kv_heads: int,
             head_dim: int, fill: int = 0) -> np.ndarray:
    """A zero (or ``fill``) byte pool of shape [num_blocks, page_bytes]."""
    pb = page_bytes(kv_format, block_size, num_kv_heads, head_dim)
    return np.full((num_blocks, pb), fill, dtype=np.uint8)


def _v_index(pos: np.ndarray, d: np.ndarray, head_dim: int) -> np.ndarray:
    """Element index of V[pos][d] inside the grouped V sub-array."""
    return (pos // 4) * (4 * head_dim) + d * 4 + (pos % 4)


def _slot_split(slot_mapping, num_blocks, block_size):
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = slots >= 0  # negative slot: padding token, not written
    if np.any(slots[keep] >= num_blocks * block_size):
        raise ValueError("slot out of range")
    return keep, slots // block_size, slots % block_size


def write_int8_tokens(pool: np.ndarray, k_codes, k_scales, v_codes, v_scales,
                      slot_mapping, block_size: int) -> None:
    """Store codes [T,Hkv,D] and scales [T,Hkv] of K and V at their slots.

    Tokens with a negative slot are padding and are skipped. When two tokens
    name the same slot, the later one wins (plain sequential semantics).
    """
    t_n, hkv, d = k_codes.shape
    if pool.shape[1] != page_bytes(KV_INT8_SYM, block_size, hkv, d):
        raise ValueError("pool page size does not match the shape")
    keep, blk, pos = _slot_split(slot_mapping, pool.shape[0], block_size)
    flat = pool.reshape(-1)
    kc = np.ascontiguousarray(k_codes).view(np.uint8)
    vc = np.ascontiguousarray(v_codes).view(np.uint8)
    ks = np.ascontiguousarray(k_scales.astype(np.float16)).view(np.uint8).reshape(t_n, hkv, 2)
    vs = np.ascontiguousarray(v_scales.astype(np.float16)).view(np.uint8).reshape(t_n, hkv, 2)
    tt = np.nonzero(keep)[0]
    page0 = (blk[tt] * pool.shape[1])[:, None]          # [n, 1]
    for h in range(hkv):
        ki, vi, ksi, vsi = int8_token_bytes(block_size, hkv, d, h, pos[tt])
        flat[page0 + ki] = kc[tt, h]
        flat[page0 + vi] = vc[tt, h]
        flat[page0 + ksi] = ks[tt, h]
        flat[page0 + vsi] = vs[tt, h]


def write_16bit_tokens(pool: np.ndarray, k_bits, v_bits, slot_mapping,
                       block_size: int) -> None:
    """Store 16-bit K/V (uint16 bit patterns [T,Hkv,D]) at their slots."""
    t_n, hkv, d = k_bits.shape
    hb_w = 2 * block_size * d  # 16-bit words per head block
    if pool.shape[1] != hkv * 2 * hb_w:
        raise ValueError("pool page size does not match the shape")
    keep, blk, pos = _slot_split(slot_mapping, pool.shape[0], block_size)
    words = pool.view(np.uint16).reshape(-1)
    wpp = pool.shape[1] // 2
    dd = np.arange(d)
    tt = np.nonzero(keep)[0]
    p = pos[tt]
    for h in range(hkv):
        base = blk[tt] * wpp + h * hb_w
        words[base[:, None] + p[:, None] * d + dd[None, :]] = np.asarray(k_bits)[tt, h]
        words[base[:, None] + block_size * d + _v_index(p[:, None], dd[None, :], d)] = \
            np.asarray(v_bits)[tt, h]


def _seq_positions(block_table_row, context_len, block_size):
    t = np.arange(context_len)
    blk = np.asarray(block_table_row, dtype=np.int64)[t // block_size]
    return blk, t % block_size


def gather_int8_sequence(pool: np.ndarray, block_table_row, context_len: int,
                         block_size: int, num_kv_heads: int, head_dim: int,
                         heads=None):
    """Read back (k_codes, k_scales, v_codes, v_scales) of one sequence.

    Shapes: codes [L, H, D] int8, scales [L, H] float16, in logical token
    order following the block table; H = len(heads) (default: all KV heads).
    """
    d = head_dim
    heads = list(range(num_kv_heads)) if heads is None else list(heads)
    blk, pos = _seq_positions(block_table_row, context_len, block_size)
    flat = pool.reshape(-1)
    page0 = (blk * pool.shape[1])[:, None]                          # [L, 1]
    kc, vc, ks, vs = [], [], [], []
    for h in heads:
        ki, vi, ksi, vsi = int8_token_bytes(block_size, num_kv_heads, d, h, pos)
        kc.append(flat[page0 + ki])
        vc.append(flat[page0 + vi])
        ks.append(flat[page0 + ksi])
        vs.append(flat[page0 + vsi])
    kc = np.stack(kc, axis=1).view(np.int8)
    vc = np.stack(vc, axis=1).view(np.int8)
    ks = np.ascontiguousarray(np.stack(ks, axis=1)).view(np.float16)[..., 0]
    vs = np.ascontiguousarray(np.stack(vs, axis=1)).view(np.float16)[..., 0]
    return kc, ks, vc, vs


def gather_16bit_sequence(pool: np.ndarray, block_table_row, context_len: int,
                          block_size: int, num_kv_heads: int, head_dim: int,
                          heads=None):
    """Read back K and V bit patterns [L, H, D] (uint16) of one sequence."""
    d = head_dim
    hb_w = 2 * block_size * d
    heads = list(range(num_kv_heads)) if heads is None else list(heads)
    blk, pos = _seq_positions(block_table_row, context_len, block_size)
    words = pool.view(np.uint16).reshape(-1)
    wpp = pool.shape[1] // 2
    dd = np.arange(d)
    k, v = [], []
    for h in heads:
        base = blk * wpp + h * hb_w
        k.append(words[base[:, None] + pos[:, None] * d + dd])
        v.append(words[base[:, None] + block_size * d + _v_index(pos[:, None], dd[None, :], d)])
    return np.stack(k, axis=1), np.stack(v, axis=1)


def write_int8_static_tokens(pool: np.ndarray, k_codes, v_codes, slot_mapping,
                             block_size: int) -> None:
    """Store static-scale codes [T,Hkv,D] of K and V at their slots
    (negative slot: padding, skipped; a repeated slot: the later token wins)."""
    t_n, hkv, d = k_codes.shape
    hb = 2 * block_size * d
    if pool.shape[1] != hkv * hb:
        raise ValueError("pool page size does not match the shape")
    keep, blk, pos = _slot_split(slot_mapping, pool.shape[0], block_size)
    flat = pool.reshape(-1)
    kc = np.ascontiguousarray(k_codes).view(np.uint8)
    vc = np.ascontiguousarray(v_codes).view(np.uint8)
    dd = np.arange(d)
    tt = np.nonzero(keep)[0]
    p = pos[tt]
    for h in range(hkv):
        base = blk[tt] * pool.shape[1] + h * hb
        flat[base[:, None] + p[:, None] * d + dd[None, :]] = kc[tt, h]
        flat[base[:, None] + block_size * d + _v_index(p[:, None], dd[None, :], d)] = vc[tt, h]


def gather_int8_static_sequence(pool: np.ndarray, block_table_row, context_len: int,
                                block_size: int, num_kv_heads: int, head_dim: int,
                                heads=None):
    """Read back (k_codes, v_codes) [L, H, D] int8 of one sequence."""
    d = head_dim
    hb = 2 * block_size * d
    heads = list(range(num_kv_heads)) if heads is None else list(heads)
    blk, pos = _seq_positions(block_table_row, context_len, block_size)
    flat = pool.reshape(-1)
    dd = np.arange(d)
    kc, vc = [], []
    for h in heads:
        base = blk * pool.shape[1] + h * hb
        kc.append(flat[base[:, None] + pos[:, None] * d + dd])
        vc.append(flat[base[:, None] + block_size * d + _v_index(pos[:, None], dd[None, :], d)])
    return np.stack(kc, axis=1).view(np.int8), np.stack(vc, axis=1).view(np.int8)
