"""Element-wise GPU parity at the full sizes the bench times.

The batched step (64 sequences, contexts 1K-8K + 1 appended token, shuffled
pages) and the 32K workload (8 sequences of 32,768 tokens, bf16
log-magnitude rows), in the launch configuration the bench uses:

* the whole pool the library writes equals the oracle's byte for byte (INT8
  codes and FP16 scales, static-scale codes, 16-bit values);
* every (sequence, query head) output row of the decode calls -- INT8, the
  FP16-KV control, static scales, and the fused append + decode call of the
  batched step -- is within the 2e-3 bound of the oracle's FP64 attention over
  the oracle's own pool.

The oracle results are computed once per module and shared by the tests."""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import (FILL, MAX_ABS_TOL, calibrated_scales, dev_i32, gpu_decode,
                            gpu_pool, oracle_decode, oracle_pool, oracle_static_pool,
                            require_gpu, to_dev)
from workloads import make_config

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def P():
    return require_gpu()


def _say(msg):
    print(msg, flush=True)


class _Cache:
    """Workloads and oracle results of one configuration at a time."""

    def __init__(self):
        self.idx, self.items = None, {}

    def get(self, idx, key, make):
        if idx != self.idx:
            self.idx, self.items = idx, {}
        if key not in self.items:
            self.items[key] = make()
        return self.items[key]


_C = _Cache()


def _wl(idx):
    return _C.get(idx, "wl", lambda: make_config(idx))


def _host_pool(idx, fmt):
    return _C.get(idx, ("pool", fmt), lambda: oracle_pool(_wl(idx), fmt))


def _want(idx, fmt):
    return _C.get(idx, ("out", fmt), lambda: oracle_decode(_wl(idx), _host_pool(idx, fmt), fmt))


def _scales(idx):
    return _C.get(idx, "scales", lambda: calibrated_scales(_wl(idx)))


def _host_static(idx):
    return _C.get(idx, "static", lambda: oracle_static_pool(_wl(idx), *_scales(idx)))


def _want_static(idx):
    wl = _wl(idx)
    ks, vs = _scales(idx)
    return _C.get(idx, "static_out", lambda: oracle.decode_int8_static_from_pool(
        _host_static(idx), wl.block_tables, wl.context_lens, wl.q, wl.sm_scale, ks, vs,
        wl.block_size, wl.num_kv_heads, wl.head_dim))


def _same_pool(got, want, what):
    g = got.cpu().numpy()
    assert g.shape == want.shape
    bad = np.nonzero(g != want)
    assert bad[0].size == 0, (f"{what}: {bad[0].size} bytes differ, first at page "
                              f"{bad[0][0]} byte {bad[1][0]}")


def _rows_within(out, want, what):
    g = out.float().cpu().numpy().astype(np.float64)
    assert g.shape == want.shape and not np.isnan(want).any()
    assert not np.isnan(g).any(), what
    per_row = np.abs(g - want).max(axis=-1)  # [B, Hq]
    worst = float(per_row.max())
    b, h = np.unravel_index(int(per_row.argmax()), per_row.shape)
    _say(f"  {what}: {per_row.size} rows, max abs diff {worst:.3e} (row {b}, head {h})")
    assert worst <= MAX_ABS_TOL, what


def _fmt(P, name):
    return {"int8": (P.KV_INT8_SYM, oracle.KV_INT8_SYM),
            "16bit": (P.KV_16BIT, oracle.KV_16BIT)}[name]


def _pool_and_decode(P, idx, fmt_name):
    fmt, ofmt = _fmt(P, fmt_name)
    wl = _wl(idx)
    _say(f"full size {wl.name} {fmt_name}: {wl.num_seqs} seqs, max ctx {wl.max_context_len}")
    pool, _ = gpu_pool(P, wl, fmt)
    _same_pool(pool, _host_pool(idx, ofmt), f"{fmt_name} pool")
    out = gpu_decode(P, wl, pool, fmt)
    _rows_within(out, _want(idx, ofmt), f"{fmt_name} decode")


def _static_pool_and_decode(P, idx):
    wl = _wl(idx)
    ks, vs = _scales(idx)
    _say(f"full size {wl.name} static scales {ks:.4g} / {vs:.4g}")
    pb = P.pdakv_page_bytes(P.KV_INT8_STATIC, 16, wl.num_kv_heads, wl.head_dim)
    pool = torch.full((wl.num_blocks, pb), FILL, dtype=torch.uint8, device="cuda")
    for ph in wl.phases:
        P.kv_quant_int8_static_write(to_dev(ph.k), to_dev(ph.v), dev_i32(ph.slot_mapping), pool,
                                     wl.num_blocks, ks, vs)
    _same_pool(pool, _host_static(idx), "static pool")
    out = torch.empty((wl.num_seqs, wl.num_q_heads, wl.head_dim), dtype=torch.float32,
                      device="cuda")
    ws = P.alloc_workspace(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                           wl.max_context_len)
    P.paged_attn_decode_int8_static(out, to_dev(wl.q), pool, wl.num_blocks,
                                    dev_i32(wl.block_tables), dev_i32(wl.context_lens),
                                    wl.num_kv_heads, wl.max_context_len, wl.sm_scale, ks, vs, ws)
    _rows_within(out, _want_static(idx), "static decode")


# ---- the batched step (64 sequences) --------------------------------------

@pytest.mark.parametrize("fmt_name", ["int8", "16bit"])
def test_batched_step_pool_and_decode(P, fmt_name):
    _pool_and_decode(P, 3, fmt_name)


@pytest.mark.parametrize("fmt_name", ["int8", "16bit"])
def test_batched_step_fused_append(P, fmt_name):
    """The bench's headline launch: every phase but the appended token
    written, then the fused append + decode call. The pool it leaves and
    every output row against the oracle."""
    fmt, ofmt = _fmt(P, fmt_name)
    wl = _wl(3)
    last = wl.phases[-1]
    assert np.all(last.counts == 1)
    _say(f"full size fused append {fmt_name}")
    pb = P.pdakv_page_bytes(fmt, 16, wl.num_kv_heads, wl.head_dim)
    pool = torch.full((wl.num_blocks, pb), FILL, dtype=torch.uint8, device="cuda")
    write = P.kv_quant_int8_sym_write if fmt == P.KV_INT8_SYM else P.kv_write_16bit
    for ph in wl.phases[:-1]:
        write(to_dev(ph.k), to_dev(ph.v), dev_i32(ph.slot_mapping), pool, wl.num_blocks)
    out = torch.empty((wl.num_seqs, wl.num_q_heads, wl.head_dim), dtype=torch.float32,
                      device="cuda")
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
    _same_pool(pool, _host_pool(3, ofmt), f"{fmt_name} pool after the fused step")
    _rows_within(out, _want(3, ofmt), f"{fmt_name} fused append + decode")


def test_batched_step_static(P):
    _static_pool_and_decode(P, 3)


# ---- 32K context (8 sequences) ----------------------------------------------

@pytest.mark.parametrize("fmt_name", ["int8", "16bit"])
def test_32k_pool_and_decode(P, fmt_name):
    _pool_and_decode(P, 4, fmt_name)


def test_32k_static(P):
    _static_pool_and_decode(P, 4)
