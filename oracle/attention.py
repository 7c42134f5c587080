"""Decode attention over a paged KV pool — CPU oracle (test infrastructure only).

What it computes (MoE-Infinity PR #183, "What landed": paged decode over INT8
payload + FP16 scales with FP32 accumulation, MHA and GQA, checked against an
FP32-dequantized scaled-dot-product-attention oracle; "Scope & fallback": MHA
and GQA validated):

for each sequence b and query head h, with G = Hq / Hkv and g = h // G,

    k_t = K codes[t, g, :] * K scale[t, g]      (binary32, exact)
    v_t = V codes[t, g, :] * V scale[t, g]      (binary32, exact)
    logit_t = sm_scale * <q[b, h, :], k_t>      for t < context_len[b]
    p = softmax(logit)                          (max-subtracted)
    out[b, h, :] = sum_t p_t v_t

All sums are taken in FP64, so the oracle's own rounding error is negligible
next to the GPU's FP32 arithmetic.

Readings (also in the design doc): query head h reads KV head h // G (contiguous
groups); sm_scale is a call parameter (the workloads use 1/sqrt(D));
context_len 0 gives a zero output row; all-zero tokens are attended like any
other token (logit 0), nothing is masked except positions >= context_len.
"""

from __future__ import annotations

import numpy as np

from .pages import gather_16bit_sequence, gather_int8_sequence, gather_int8_static_sequence
from .quant import as_f32, dequantize_rows, dequantize_static


def bits_to_f32(bits: np.ndarray, kv_dtype: str) -> np.ndarray:
    """16-bit patterns (uint16) of fp16 or bf16 values -> float32 (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    if kv_dtype == "f16":
        return bits.view(np.float16).astype(np.float32)
    if kv_dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32)
    raise ValueError(kv_dtype)


def attend_one_sequence(q, k, v, sm_scale: float) -> np.ndarray:
    """Attention of one decode query over one sequence's keys and values.

    q [Hq, D]; k, v [L, Hkv, D] (already dequantized, any float dtype);
    returns out [Hq, D] in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    hq, d = q.shape
    L, hkv = k.shape[0], k.shape[1]
    if hq % hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    group = hq // hkv
    out = np.zeros((hq, d), dtype=np.float64)
    if L == 0:
        return out
    for h in range(hq):
        g = h // group
        logits = float(sm_scale) * (k[:, g, :] @ q[h])          # [L]
        w = np.exp(logits - logits.max())
        out[h] = (w @ v[:, g, :]) / w.sum()
    return out


def decode_int8_from_pool(pool, block_tables, context_lens, q, sm_scale: float,
                          block_size: int, num_kv_heads: int, head_dim: int,
                          pairs=None) -> np.ndarray:
    """Reference output of the INT8 paged decode.

    q [B, Hq, D] (fp16/bf16/fp32 array or tensor). Returns float64
    [B, Hq, D]; when ``pairs`` (a list of (b, h)) is given, only those rows
    are computed and the others stay NaN.
    """
    qf = as_f32(q)
    B, hq, d = qf.shape
    group = hq // num_kv_heads
    out = np.full((B, hq, d), np.nan)
    want = {}
    for b, h in (pairs if pairs is not None else [(b, h) for b in range(B) for h in range(hq)]):
        want.setdefault(b, set()).add(h)
    for b, hs in want.items():
        L = int(context_lens[b])
        gs = sorted({h // group for h in hs})
        kc, ks, vc, vs = gather_int8_sequence(pool, block_tables[b], L, block_size,
                                              num_kv_heads, head_dim, heads=gs)
        k = dequantize_rows(kc, ks)
        v = dequantize_rows(vc, vs)
        for h in sorted(hs):
            j = gs.index(h // group)
            out[b, h] = attend_one_sequence(qf[b, h][None], k[:, j:j + 1], v[:, j:j + 1],
                                            sm_scale)[0]
    return out


def decode_16bit_from_pool(pool, block_tables, context_lens, q, sm_scale: float,
                           block_size: int, num_kv_heads: int, head_dim: int,
                           kv_dtype: str, pairs=None) -> np.ndarray:
    """Reference output of the 16-bit (fp16/bf16 KV) paged decode control."""
    qf = as_f32(q)
    B, hq, d = qf.shape
    group = hq // num_kv_heads
    out = np.full((B, hq, d), np.nan)
    want = {}
    for b, h in (pairs if pairs is not None else [(b, h) for b in range(B) for h in range(hq)]):
        want.setdefault(b, set()).add(h)
    for b, hs in want.items():
        L = int(context_lens[b])
        gs = sorted({h // group for h in hs})
        kb, vb = gather_16bit_sequence(pool, block_tables[b], L, block_size,
                                       num_kv_heads, head_dim, heads=gs)
        k = bits_to_f32(kb, kv_dtype)
        v = bits_to_f32(vb, kv_dtype)
        for h in sorted(hs):
            j = gs.index(h // group)
            out[b, h] = attend_one_sequence(qf[b, h][None], k[:, j:j + 1], v[:, j:j + 1],
                                            sm_scale)[0]
    return out


def decode_int8_static_from_pool(pool, block_tables, context_lens, q, sm_scale: float,
                                 k_scale, v_scale, block_size: int, num_kv_heads: int,
                                 head_dim: int, pairs=None) -> np.ndarray:
    """Reference output of the paged decode over static-scale INT8 pages:
    the same attention with k_t = cK_t * k_scale and v_t = cV_t * v_scale
    (one scalar each for the whole layer; InfiniLM PR #553, "Summary";
    TensorRT-LLM PR #18953, "Summary"). Returns float64 [B, Hq, D]; rows
    outside ``pairs`` stay NaN."""
    qf = as_f32(q)
    B, hq, d = qf.shape
    group = hq // num_kv_heads
    out = np.full((B, hq, d), np.nan)
    want = {}
    for b, h in (pairs if pairs is not None else [(b, h) for b in range(B) for h in range(hq)]):
        want.setdefault(b, set()).add(h)
    for b, hs in want.items():
        L = int(context_lens[b])
        gs = sorted({h // group for h in hs})
        kc, vc = gather_int8_static_sequence(pool, block_tables[b], L, block_size,
                                             num_kv_heads, head_dim, heads=gs)
        k = dequantize_static(kc, k_scale)
        v = dequantize_static(vc, v_scale)
        for h in sorted(hs):
            j = gs.index(h // group)
            out[b, h] = attend_one_sequence(qf[b, h][None], k[:, j:j + 1], v[:, j:j + 1],
                                            sm_scale)[0]
    return out


def _sequence_kv(kind, pool, bt_row, L, block_size, num_kv_heads, head_dim, heads,
                 kv_dtype=None, k_scale=None, v_scale=None):
    """Dequantized K, V [L, len(heads), D] of one sequence, any page format."""
    if kind == "int8":
        kc, ks, vc, vs = gather_int8_sequence(pool, bt_row, L, block_size, num_kv_heads,
                                              head_dim, heads=heads)
        return dequantize_rows(kc, ks), dequantize_rows(vc, vs)
    if kind == "static":
        kc, vc = gather_int8_static_sequence(pool, bt_row, L, block_size, num_kv_heads,
                                             head_dim, heads=heads)
        return dequantize_static(kc, k_scale), dequantize_static(vc, v_scale)
    kb, vb = gather_16bit_sequence(pool, bt_row, L, block_size, num_kv_heads, head_dim,
                                   heads=heads)
    return bits_to_f32(kb, kv_dtype), bits_to_f32(vb, kv_dtype)


def decode_multi_from_pool(kind: str, pool, block_tables, context_lens, q, sm_scale: float,
                           block_size: int, num_kv_heads: int, head_dim: int, kv_dtype=None,
                           k_scale=None, v_scale=None, triples=None) -> np.ndarray:
    """Reference output of a paged decode with T query tokens per sequence
    (speculative verification or a short chunk decoded against the cache;
    mlxcel PR #717, "Server integration": INT8 chunked prefill followed by
    decode).

    q [B, T, Hq, D]. The T new tokens are the last T positions of each
    sequence (context_lens[b] counts them): query token j sits at position
    p = context_lens[b] - T + j and attends to positions 0..p (causal among
    the new tokens); p < 0 gives a zero row. ``kind`` is "int8", "static" or
    "16bit" (with ``kv_dtype``). Returns float64 [B, T, Hq, D]; rows outside
    ``triples`` (a list of (b, j, h)) stay NaN.
    """
    qf = as_f32(q)
    B, T, hq, d = qf.shape
    group = hq // num_kv_heads
    out = np.full((B, T, hq, d), np.nan)
    want = {}
    for b, j, h in (triples if triples is not None else
                    [(b, j, h) for b in range(B) for j in range(T) for h in range(hq)]):
        want.setdefault(b, set()).add((j, h))
    for b, jh in want.items():
        L = int(context_lens[b])
        gs = sorted({h // group for _, h in jh})
        k, v = _sequence_kv(kind, pool, block_tables[b], L, block_size, num_kv_heads,
                            head_dim, gs, kv_dtype, k_scale, v_scale)
        for j, h in sorted(jh):
            n = L - T + j + 1  # positions this query token sees
            i = gs.index(h // group)
            if n <= 0:
                out[b, j, h] = 0.0
                continue
            out[b, j, h] = attend_one_sequence(qf[b, j, h][None], k[:n, i:i + 1],
                                               v[:n, i:i + 1], sm_scale)[0]
    return out
