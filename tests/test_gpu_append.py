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


@pytest.mark.slow
@pytest.mark.parametrize("fmt_name", ["int8", "16bit"])
def test_full_size_fused_append_sampled(P, fmt_name):
    """The batched step at full size (64 sequences, contexts 1K-8K, shuffled
    pages) in the launch shape the bench times: the fused append + decode
    call. Sampled sequences' newest tokens are read back from the pool and
    compared with the oracle's codes and scales (INT8) or the source values
    (16-bit), and sampled output rows with the oracle's attention over each
    sequence's source K/V, newest token included."""
    fmt = P.KV_INT8_SYM if fmt_name == "int8" else P.KV_16BIT
    wl = make_config(3)
    _say(f"full-size fused append {fmt_name}: {wl.num_seqs} seqs, max ctx {wl.max_context_len}")
    out, pool = _fused(P, wl, fmt)
    out = out.cpu().numpy()
    assert not np.isnan(out).any()
    host = pool.cpu().numpy()
    last = wl.phases[-1]
    rng = np.random.default_rng(17)
    seqs = rng.choice(wl.num_seqs, 4, replace=False)
    for b in seqs:
        L = int(wl.context_lens[b])
        if fmt == P.KV_INT8_SYM:
            kc, ks, vc, vs = oracle.gather_int8_sequence(host, wl.block_tables[b], L, 16,
                                                         wl.num_kv_heads, wl.head_dim)
            wkc, wks = oracle.quantize_rows(last.k[b])
            wvc, wvs = oracle.quantize_rows(last.v[b])
            assert np.array_equal(kc[L - 1], wkc) and np.array_equal(vc[L - 1], wvc)
            assert np.array_equal(ks[L - 1].view(np.uint16), wks.view(np.uint16))
            assert np.array_equal(vs[L - 1].view(np.uint16), wvs.view(np.uint16))
        else:
            k16, v16 = oracle.gather_16bit_sequence(host, wl.block_tables[b], L, 16,
                                                    wl.num_kv_heads, wl.head_dim)
            assert np.array_equal(k16[L - 1], last.k[b].view(torch.int16).numpy().view(np.uint16))
            assert np.array_equal(v16[L - 1], last.v[b].view(torch.int16).numpy().view(np.uint16))
    worst = 0.0
    for b in seqs:
        for h in rng.choice(wl.num_q_heads, 3, replace=False):
            want = oracle_pair_from_sources(wl, int(b), int(h), oracle.KV_INT8_SYM if
                                            fmt == P.KV_INT8_SYM else oracle.KV_16BIT)
            worst = max(worst, float(np.max(np.abs(out[b, h] - want))))
    _say(f"  worst sampled max abs diff {worst:.3e}")
    assert worst <= MAX_ABS_TOL
