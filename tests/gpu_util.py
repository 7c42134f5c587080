"""Helpers for the GPU parity tests: move a workload to the device, run the
library's kernels through the C ABI, and build the oracle's own pools from the
same host inputs."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle

FILL = 0x5A  # pool bytes no write should touch keep this value


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import paged_decode_attention_kv_amd as P
    flags = P.pdakv_capabilities()
    assert flags & P.CAP_GFX950, "the library targets gfx950"
    return P


def to_dev(t: torch.Tensor) -> torch.Tensor:
    """Copy a host tensor to the GPU keeping its strides (views of a fused
    buffer stay views of a device copy of that buffer)."""
    if t.is_contiguous():
        return t.to("cuda")
    base = t._base if t._base is not None else t
    assert base.is_contiguous()
    dbase = base.to("cuda")
    return torch.as_strided(dbase, t.size(), t.stride(), t.storage_offset())


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda")


def gpu_pool(P, wl, fmt, guard_pages: int = 0):
    """Allocate a pool (FILL bytes) and write every phase with the library.

    Returns (pool, full): ``pool`` is the view passed to the library; ``full``
    includes ``guard_pages`` extra pages on each side."""
    pb = P.pdakv_page_bytes(fmt, wl.block_size, wl.num_kv_heads, wl.head_dim)
    full = torch.full((wl.num_blocks + 2 * guard_pages, pb), FILL, dtype=torch.uint8,
                      device="cuda")
    pool = full[guard_pages:guard_pages + wl.num_blocks]
    write = P.kv_quant_int8_sym_write if fmt == P.KV_INT8_SYM else P.kv_write_16bit
    for ph in wl.phases:
        write(to_dev(ph.k), to_dev(ph.v), dev_i32(ph.slot_mapping), pool, wl.num_blocks)
    return pool, full


def oracle_pool(wl, fmt) -> np.ndarray:
    pool = oracle.new_pool(fmt, wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim,
                           fill=FILL)
    for ph in wl.phases:
        if fmt == oracle.KV_INT8_SYM:
            kc, ks = oracle.quantize_rows(ph.k)
            vc, vs = oracle.quantize_rows(ph.v)
            oracle.write_int8_tokens(pool, kc, ks, vc, vs, ph.slot_mapping, wl.block_size)
        else:
            oracle.write_16bit_tokens(pool, bits16(ph.k), bits16(ph.v), ph.slot_mapping,
                                      wl.block_size)
    return pool


def gpu_decode(P, wl, pool, fmt, out_dtype=torch.float32, q=None, context_lens=None,
               block_tables=None, max_context_len=None, err_flag=None, out=None):
    q = to_dev(wl.q) if q is None else q
    ctx = dev_i32(wl.context_lens if context_lens is None else context_lens)
    bt = dev_i32(wl.block_tables if block_tables is None else block_tables)
    maxl = wl.max_context_len if max_context_len is None else max_context_len
    if out is None:
        out = torch.empty((wl.num_seqs, wl.num_q_heads, wl.head_dim), dtype=out_dtype,
                          device="cuda")
    ws = P.alloc_workspace(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, maxl)
    fn = P.paged_attn_decode_int8 if fmt == P.KV_INT8_SYM else P.paged_attn_decode_fp16
    fn(out, q, pool, pool.shape[0], bt, ctx, wl.num_kv_heads, maxl, wl.sm_scale, ws,
       err_flag=err_flag)
    return out


def oracle_decode(wl, pool_host, fmt, pairs=None):
    if fmt == oracle.KV_INT8_SYM:
        return oracle.decode_int8_from_pool(pool_host, wl.block_tables, wl.context_lens, wl.q,
                                            wl.sm_scale, wl.block_size, wl.num_kv_heads,
                                            wl.head_dim, pairs=pairs)
    return oracle.decode_16bit_from_pool(pool_host, wl.block_tables, wl.context_lens, wl.q,
                                         wl.sm_scale, wl.block_size, wl.num_kv_heads,
                                         wl.head_dim, wl.kv_dtype, pairs=pairs)


def oracle_pair_from_sources(wl, b: int, h: int, fmt) -> np.ndarray:
    """Oracle output row (b, h) computed straight from the source K/V of
    sequence b (quantize -> dequantize -> attend), without any page pool."""
    g = h // (wl.num_q_heads // wl.num_kv_heads)
    k, v = wl.tokens_of_seq(b)
    k, v = k[:, g:g + 1], v[:, g:g + 1]
    if fmt == oracle.KV_INT8_SYM:
        kc, ks = oracle.quantize_rows(k)
        vc, vs = oracle.quantize_rows(v)
        kf, vf = oracle.dequantize_rows(kc, ks), oracle.dequantize_rows(vc, vs)
    else:
        kf, vf = oracle.as_f32(k), oracle.as_f32(v)
    q = oracle.as_f32(wl.q[b, h:h + 1])
    return oracle.attend_one_sequence(q, kf, vf, wl.sm_scale)[0]


MAX_ABS_TOL = 2e-3  # decode outputs vs the FP32-dequantized oracle (FP32 output)


def calibrated_scales(wl, shrink: float = 1.0):
    """Static K and V scales for a workload, the input the static-scale
    variant takes: the absolute maximum of all K (or V) values the workload
    writes, divided by 127 and by ``shrink`` (shrink > 1 makes the largest
    values saturate), as binary32. The calibration itself happens outside the
    path (the pages take calibrated scales from a checkpoint)."""
    ak = max(float(ph.k.float().abs().max()) for ph in wl.phases if ph.k.numel())
    av = max(float(ph.v.float().abs().max()) for ph in wl.phases if ph.v.numel())
    return float(np.float32(ak / 127.0 / shrink)), float(np.float32(av / 127.0 / shrink))


def oracle_static_pool(wl, k_scale: float, v_scale: float) -> np.ndarray:
    pool = oracle.new_pool(oracle.KV_INT8_STATIC, wl.num_blocks, wl.block_size,
                           wl.num_kv_heads, wl.head_dim, fill=FILL)
    for ph in wl.phases:
        oracle.write_int8_static_tokens(pool, oracle.quantize_static(ph.k, k_scale),
                                        oracle.quantize_static(ph.v, v_scale), ph.slot_mapping,
                                        wl.block_size)
    return pool
