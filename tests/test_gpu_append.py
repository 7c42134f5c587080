"""GPU parity of the fused append + decode step (the newest token of every
sequence is quantized and written inside the decode launch): the pool it
leaves is bit-identical to the oracle's after writing every phase, and the
output matches the oracle's decode over all tokens."""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import (FILL, MAX_ABS_TOL, dev_i32, oracle_decode, oracle_pair_from_sources,
                            oracle_pool, require_gpu, to_dev)
from workloads import build, make_config

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    return require_gpu()


def _say(msg):
    print(msg, flush=True)


def _fused(P, wl, fmt, out_dtype=torch.float32):
    """Write every phase but the last with the library, then run the fused
    step with the last phase (one token per sequence) as the new tokens."""
    last = wl.phases[-1]
    assert np.all(last.counts == 1)
    pb = P.pdakv_page_bytes(fmt, wl.block_size, wl.num_kv_heads, wl.head_dim)
    pool = torch.full((wl.num_blocks, pb), FILL, dtype=torch.uint8, device="cuda")
    write = P.kv_quant_int8_sym_write if fmt == P.KV_INT8_SYM else P.kv_write_16bit
    for ph in wl.phases[:-1]:
        if len(ph.slot_mapping):
            write(to_dev(ph.k), to_dev(ph.v), dev_i32(ph.slot_mapping), pool, wl.num_blocks)
    out = torch.empty((wl.num_seqs, wl.num_q_heads, wl.head_dim), dtype=out_dtype, device="cuda")
    ws = P.alloc_workspace(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                           wl.max_context_len)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    fn = (P.paged_attn_decode_int8_append if fmt == P.KV_INT8_SYM
          else P.paged_attn_decode_fp16_append)
    fn(out, to_dev(wl.q), to_dev(last.k), to_dev(last.v), pool, wl.num_blocks,
       dev_i32(wl.block_tables), dev_i32(wl.context_lens), wl.num_kv_heads, wl.max_context_len,
       wl.sm_scale, ws, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return out, pool


def _check(P, wl, fmt_name):
    fmt = P.KV_INT8_SYM if fmt_name == "int8" else P.KV_16BIT
    ofmt = oracle.KV_INT8_SYM if fmt_name == "int8" else oracle.KV_16BIT
    out, pool = _fused(P, wl, fmt)
    host = oracle_pool(wl, ofmt)
    assert np.array_equal(pool.cpu().numpy(), host), "pool after the fused step differs"
    want = oracle_decode(wl, host, ofmt)
    d = float(np.max(np.abs(out.cpu().numpy().astype(np.float64) - want)))
    _say(f"  max abs diff {d:.3e}")
    assert d <= MAX_ABS_TOL
    return out, pool


@pytest.mark.parametrize("fmt_name", ["int8", "16bit"])
@pytest.mark.parametrize("idx,scale", [(3, 0.05), (5, 0.2)])
def test_fused_append_matches_write_then_decode(P, fmt_name, idx, scale):
    """Batched step (prefill + one appended token per sequence; c5's K/V are
    strided views of a fused QKV buffer)."""
    wl = make_config(idx, scale)
    _say(f"fused append {fmt_name}: config {idx} scale {scale}")
    _check(P, wl, fmt_name)


@pytest.mark.parametrize("fmt_name", ["int8", "16bit"])
def test_fused_append_page_boundaries(P, fmt_name):
    """New tokens at positions 0, 15, 16 and inside a page, with GQA 4 and
    MHA-like shapes."""
    for hq, hkv, d, dt in ((32, 8, 128, "f16"), (14, 2, 64, "bf16")):
        wl = build("app", 41, [("prefill", [0, 15, 16, 300, 1]), ("append", [1] * 5)], hq, hkv,
                   d, dt, "outlier", shuffle=True, spare_blocks=2)
        _say(f"fused append boundaries {fmt_name}: {hq}/{hkv}/{d} {dt} lens {wl.context_lens}")
        _check(P, wl, fmt_name)


def test_fused_append_then_plain_decode_agree(P):
    """The pool the fused step leaves decodes (unfused) to the same rows."""
    wl = make_config(3, 0.05)
    out, pool = _fused(P, wl, P.KV_INT8_SYM)
    ws = P.alloc_workspace(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                           wl.max_context_len)
    again = torch.empty_like(out)
    P.paged_attn_decode_int8(again, to_dev(wl.q), pool, wl.num_blocks, dev_i32(wl.block_tables),
                             dev_i32(wl.context_lens), wl.num_kv_heads, wl.max_context_len,
                             wl.sm_scale, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, again)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_fused_append_non_finite_rows_are_flagged(P, dtype):
    """A new K or V row holding a NaN or an infinity has no valid scale: the
    fused append flags it (PDAKV_EFLAG_SCALE_RANGE) and leaves that (slot, KV
    head) as it was, exactly as the writer does with the same rows; the other
    rows are written as the oracle writes them."""
    hq, hkv, d = 8, 2, 128
    wl = build("nonfinite", 62, [("prefill", [5, 37, 16]), ("append", [1, 1, 1])], hq, hkv, d,
               dtype, "outlier", shuffle=True, spare_blocks=1)
    last = wl.phases[-1]
    last.k[0, 1, 7] = float("nan")    # sequence 0, KV head 1: NaN in K
    last.v[1, 0, 100] = float("inf")  # sequence 1, KV head 0: infinity in V
    bad = {(0, 1), (1, 0)}
    ref = None
    for route in ("writer", "fused"):
        _say(f"non-finite append {dtype}: {route}")
        pb = P.pdakv_page_bytes(P.KV_INT8_SYM, 16, hkv, d)
        pool = torch.full((wl.num_blocks, pb), FILL, dtype=torch.uint8, device="cuda")
        P.kv_quant_int8_sym_write(to_dev(wl.phases[0].k), to_dev(wl.phases[0].v),
                                  dev_i32(wl.phases[0].slot_mapping), pool, wl.num_blocks)
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        if route == "writer":
            P.kv_quant_int8_sym_write(to_dev(last.k), to_dev(last.v), dev_i32(last.slot_mapping),
                                      pool, wl.num_blocks, err_flag=err)
        else:
            out = torch.empty((wl.num_seqs, hq, d), dtype=torch.float32, device="cuda")
            ws = P.alloc_workspace(wl.num_seqs, hq, hkv, d, wl.max_context_len)
            P.paged_attn_decode_int8_append(out, to_dev(wl.q), to_dev(last.k), to_dev(last.v),
                                            pool, wl.num_blocks, dev_i32(wl.block_tables),
                                            dev_i32(wl.context_lens), hkv, wl.max_context_len,
                                            wl.sm_scale, ws, err_flag=err)
        torch.cuda.synchronize()
        assert int(err.item()) == P.EFLAG_SCALE_RANGE
        host = pool.cpu().numpy()
        for b in range(wl.num_seqs):
            L = int(wl.context_lens[b])
            kc, ks, vc, vs = oracle.gather_int8_sequence(host, wl.block_tables[b], L, 16, hkv, d)
            for g in range(hkv):
                if (b, g) in bad:
                    # untouched: the pool's fill bytes
                    assert np.all(kc[L - 1, g].view(np.uint8) == FILL)
                    assert np.all(vc[L - 1, g].view(np.uint8) == FILL)
                    assert np.all(ks[L - 1, g:g + 1].view(np.uint8) == FILL)
                    assert np.all(vs[L - 1, g:g + 1].view(np.uint8) == FILL)
                else:
                    wkc, wks = oracle.quantize_rows(last.k[b, g:g + 1])
                    wvc, wvs = oracle.quantize_rows(last.v[b, g:g + 1])
                    assert np.array_equal(kc[L - 1, g], wkc[0])
                    assert np.array_equal(vc[L - 1, g], wvc[0])
                    assert ks[L - 1, g].view(np.uint16) == wks[0].view(np.uint16)
                    assert vs[L - 1, g].view(np.uint16) == wvs[0].view(np.uint16)
        if ref is None:
            ref = host
        else:
            assert np.array_equal(host, ref)  # fused append == writer, byte for byte
