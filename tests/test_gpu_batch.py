"""GPU parity with more than 64 sequences per call: the context lengths are
scanned 64 per step, so batches of 150 and 300 sequences exercise the
later chunks, the hand-over of a wave's run from one chunk's sequences to the
next, and empty sequences at chunk edges; every decode entry point is
checked against the oracle."""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import (FILL, MAX_ABS_TOL, calibrated_scales, dev_i32, gpu_decode,
                            gpu_pool, oracle_decode, oracle_pool, oracle_static_pool,
                            require_gpu, to_dev)
from workloads import build, multi_query

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    return require_gpu()


def _say(msg):
    print(msg, flush=True)


def _lens(B, seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 120, B)
    for b in (0, 63, 64, 65, 127, 128, B - 1):  # empty sequences at chunk edges
        if b < B:
            lens[b] = 0
    lens[B // 2] = 900  # one long sequence in the middle chunk
    return lens


def _maxdiff(out, want):
    got = out.float().cpu().numpy().astype(np.float64)
    m = ~np.isnan(want)
    return float(np.max(np.abs(got[m] - want[m])))


@pytest.mark.parametrize("B", [150, 300])
@pytest.mark.parametrize("fmt_name", ["int8", "16bit"])
def test_many_sequences_decode(P, B, fmt_name):
    wl = build(f"batch{B}", B, [("prefill", _lens(B, B))], 16, 4, 64, "bf16", "outlier",
               shuffle=True, spare_blocks=2)
    fmt, ofmt = ((P.KV_INT8_SYM, oracle.KV_INT8_SYM) if fmt_name == "int8"
                 else (P.KV_16BIT, oracle.KV_16BIT))
    _say(f"{B} sequences, {fmt_name}")
    pool, _ = gpu_pool(P, wl, fmt)
    out = gpu_decode(P, wl, pool, fmt)
    want = oracle_decode(wl, oracle_pool(wl, ofmt), ofmt)
    assert _maxdiff(out, want) <= MAX_ABS_TOL
    for b in np.nonzero(wl.context_lens == 0)[0]:
        assert torch.all(out[b] == 0)


def test_many_sequences_fused_append(P):
    B = 200
    lens = _lens(B, 7)
    wl = build("batch-append", 8, [("prefill", np.maximum(lens - 1, 0)), ("append", [1] * B)],
               32, 8, 128, "f16", "outlier", shuffle=True, spare_blocks=2)
    pb = P.pdakv_page_bytes(P.KV_INT8_SYM, 16, 8, 128)
    pool = torch.full((wl.num_blocks, pb), FILL, dtype=torch.uint8, device="cuda")
    pre = wl.phases[0]
    if len(pre.slot_mapping):
        P.kv_quant_int8_sym_write(to_dev(pre.k), to_dev(pre.v), dev_i32(pre.slot_mapping), pool,
                                  wl.num_blocks)
    new = wl.phases[1]
    out = torch.empty((B, 32, 128), dtype=torch.float32, device="cuda")
    ws = P.alloc_workspace(B, 32, 8, 128, wl.max_context_len)
    P.paged_attn_decode_int8_append(out, to_dev(wl.q), to_dev(new.k), to_dev(new.v), pool,
                                    wl.num_blocks, dev_i32(wl.block_tables),
                                    dev_i32(wl.context_lens), 8, wl.max_context_len,
                                    wl.sm_scale, ws)
    torch.cuda.synchronize()
    host = oracle_pool(wl, oracle.KV_INT8_SYM)
    assert np.array_equal(pool.cpu().numpy(), host)
    assert _maxdiff(out, oracle_decode(wl, host, oracle.KV_INT8_SYM)) <= MAX_ABS_TOL


def test_many_sequences_static_and_multi(P):
    B = 150
    wl = build("batch-sm", 9, [("prefill", _lens(B, 9))], 16, 4, 64, "f16", "normal",
               shuffle=True, spare_blocks=2)
    ks, vs = calibrated_scales(wl)
    pb = P.pdakv_page_bytes(P.KV_INT8_STATIC, 16, 4, 64)
    spool = torch.full((wl.num_blocks, pb), FILL, dtype=torch.uint8, device="cuda")
    ph = wl.phases[0]
    P.kv_quant_int8_static_write(to_dev(ph.k), to_dev(ph.v), dev_i32(ph.slot_mapping), spool,
                                 wl.num_blocks, ks, vs)
    out = torch.empty((B, 16, 64), dtype=torch.float32, device="cuda")
    ws = P.alloc_workspace(B, 16, 4, 64, wl.max_context_len)
    P.paged_attn_decode_int8_static(out, to_dev(wl.q), spool, wl.num_blocks,
                                    dev_i32(wl.block_tables), dev_i32(wl.context_lens), 4,
                                    wl.max_context_len, wl.sm_scale, ks, vs, ws)
    torch.cuda.synchronize()
    host = oracle_static_pool(wl, ks, vs)
    assert np.array_equal(spool.cpu().numpy(), host)
    want = oracle.decode_int8_static_from_pool(host, wl.block_tables, wl.context_lens, wl.q,
                                               wl.sm_scale, ks, vs, 16, 4, 64)
    assert _maxdiff(out, want) <= MAX_ABS_TOL
    # three query tokens per sequence over the per-token INT8 pool
    pool, _ = gpu_pool(P, wl, P.KV_INT8_SYM)
    q = multi_query(wl, 3, seed=11)
    outm = torch.empty((B, 3, 16, 64), dtype=torch.float32, device="cuda")
    wsm = P.alloc_multi_workspace(B, 3, 16, 4, 64, wl.max_context_len)
    P.paged_attn_decode_int8_multi(outm, to_dev(q), pool, wl.num_blocks,
                                   dev_i32(wl.block_tables), dev_i32(wl.context_lens), 4,
                                   wl.max_context_len, wl.sm_scale, wsm)
    torch.cuda.synchronize()
    wantm = oracle.decode_multi_from_pool("int8", oracle_pool(wl, oracle.KV_INT8_SYM),
                                          wl.block_tables, wl.context_lens, q, wl.sm_scale, 16,
                                          4, 64)
    assert _maxdiff(outm, wantm) <= MAX_ABS_TOL
