"""GPU checks of the one-token decode's split of units over waves and the
merge of their partials: repeated calls on one workspace give identical
rows, one workspace serves calls of different shapes in turn, and waves
whose share is close to the 128-page limit of a pass (several segments,
padded to whole page pairs) keep every partial. Outputs against the
oracle's decode of the same pool bytes."""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import (MAX_ABS_TOL, dev_i32, gpu_decode, gpu_pool, oracle_decode,
                            require_gpu, to_dev)
from workloads import build, make_config

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    return require_gpu()


def _say(msg):
    print(msg, flush=True)


def _decode(P, wl, pool, ws, fmt=None):
    out = torch.empty((wl.num_seqs, wl.num_q_heads, wl.head_dim), dtype=torch.float32,
                      device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    fn = P.paged_attn_decode_int8 if fmt in (None, P.KV_INT8_SYM) else P.paged_attn_decode_fp16
    fn(out, to_dev(wl.q), pool, wl.num_blocks, dev_i32(wl.block_tables),
       dev_i32(wl.context_lens), wl.num_kv_heads, wl.max_context_len, wl.sm_scale, ws,
       err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return out


def _diff(out, want):
    got = out.cpu().numpy().astype(np.float64)
    assert not np.isnan(got).any()
    return float(np.max(np.abs(got - want)))


def test_repeated_calls_on_one_workspace_are_identical(P):
    wl = make_config(3, 0.1)
    pool, _ = gpu_pool(P, wl, P.KV_INT8_SYM)
    ws = P.alloc_workspace(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                           wl.max_context_len)
    _say(f"repeated calls: {wl.num_seqs} sequences, max context {wl.max_context_len}")
    outs = [_decode(P, wl, pool, ws) for _ in range(4)]
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    want = oracle_decode(wl, pool.cpu().numpy(), oracle.KV_INT8_SYM)
    assert _diff(outs[0], want) <= MAX_ABS_TOL


def test_one_workspace_serves_calls_of_several_shapes(P):
    """Three shapes in turn on one workspace (sized for the largest), each
    call against the oracle; the partials of one shape cover the places
    where another shape's records lie."""
    shapes = [build("ws-a", 71, [("prefill", [3000, 17, 4100, 800, 2222, 64])], 32, 8, 128,
                    "f16", "outlier", shuffle=True, spare_blocks=2),
              build("ws-b", 72, [("prefill", [40000, 9000])], 16, 2, 128, "bf16", "outlier",
                    shuffle=True, spare_blocks=2),
              build("ws-c", 73, [("prefill", [700] * 40)], 32, 8, 128, "f16", "normal",
                    shuffle=True, spare_blocks=2)]
    need = max(P.pdakv_decode_workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads,
                                              w.head_dim, w.max_context_len) for w in shapes)
    ws = torch.zeros(need // 4, dtype=torch.float32, device="cuda")
    pools = [gpu_pool(P, w, P.KV_INT8_SYM)[0] for w in shapes]
    wants = [oracle_decode(w, p.cpu().numpy(), oracle.KV_INT8_SYM) for w, p in zip(shapes, pools)]
    for rnd in range(2):
        for i in (0, 1, 2, 1, 0):
            _say(f"round {rnd} shape {i}")
            assert _diff(_decode(P, shapes[i], pools[i], ws), wants[i]) <= MAX_ABS_TOL


@pytest.mark.parametrize("fmt_name", ["int8", "16bit"])
def test_wave_shares_near_the_pass_limit(P, fmt_name):
    """Eight sequences of about 64K tokens at 8 KV heads: 262,072 items over
    2,048 waves, 128 pages each; units of 4,093 to 4,096 pages start inside
    the waves' runs at odd offsets, so with page pairs a run's second segment
    does not fit the pass and starts the next one (cutting it would give
    its unit two partials in one slot)."""
    lens = [65519, 65535, 65519, 65503, 65519, 65535, 65519, 65487]
    wl = build("pass-limit", 903, [("prefill", lens)], 8, 8, 128, "f16", "outlier",
               shuffle=True, spare_blocks=3)
    fmt = P.KV_INT8_SYM if fmt_name == "int8" else P.KV_16BIT
    waves, ppw = P.pdakv_decode_plan(fmt, wl.num_seqs, wl.num_kv_heads, wl.head_dim,
                                     wl.max_context_len)
    _say(f"pass limit {fmt_name}: {waves} waves, up to {ppw} pages each")
    assert ppw == 128
    pool, _ = gpu_pool(P, wl, fmt)
    out = gpu_decode(P, wl, pool, fmt)
    want = oracle_decode(wl, pool.cpu().numpy(),
                         oracle.KV_INT8_SYM if fmt_name == "int8" else oracle.KV_16BIT)
    d = _diff(out, want)
    _say(f"  max abs diff {d:.3e}")
    assert d <= MAX_ABS_TOL
