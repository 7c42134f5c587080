"""GPU parity of the one-token INT8 decode kernels that take two pages per
softmax update (head size 128, query groups of 1 to 8 heads: the 16 matrix
columns hold the group once for each page of a pair, so a page pair shares
one softmax step) against the oracle, at shapes that run the grid kernels
(more than 64 (sequence, KV head) units): groups of 1, 2, 3, 5, 7 and 8
heads; ragged lengths with odd page counts (a pass pads each segment to
whole pairs with a page that holds no item); many segments per wave and per
pass; the fused append's new token in the first or the second page of a
pair; per-token and static scales."""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import (MAX_ABS_TOL, calibrated_scales, dev_i32, gpu_decode, gpu_pool,
                            oracle_decode, oracle_pool, oracle_static_pool, require_gpu,
                            to_dev)
from tests.test_gpu_append import _check as check_fused_int8
from tests.test_gpu_append import _fused
from tests.test_gpu_static import (_gpu_static_decode, _gpu_static_pool, _max_diff,
                                   _oracle_decode)
from workloads import build

pytestmark = pytest.mark.gpu

HKV = 8
GROUPS = [1, 2, 3, 5, 7, 8]
# 12 sequences x 8 KV heads = 96 units; page counts 0..126, many odd, so the
# waves' runs (about 4 pages each) start and end inside units at odd offsets
SHORT = [0, 1, 15, 16, 17, 31, 32, 33, 257, 700, 1029, 2001]
# 9 x 8 units, about 33,000 pages: 17 pages per wave (odd), several units per pass
LONG = [16001, 9999, 1, 17, 12345, 255, 20001, 8191, 33]
# final lengths of the fused-append cases: the new token opens a page (1, 17,
# 33, 49, 1025), fills one (16, 32, 48) or sits inside one
APPEND = [1, 16, 17, 32, 33, 48, 49, 300, 513, 1024, 1025, 2000]


@pytest.fixture(scope="module")
def P():
    return require_gpu()


def _say(msg):
    print(msg, flush=True)


def _wl(name, seed, lens, g, dt="f16", append=False):
    phases = ([("prefill", [L - 1 for L in lens]), ("append", [1] * len(lens))] if append
              else [("prefill", lens)])
    return build(name, seed, phases, g * HKV, HKV, 128, dt, "outlier", shuffle=True,
                 spare_blocks=3)


def _check_decode(P, wl, fmt_name):
    if fmt_name == "int8":
        pool, _ = gpu_pool(P, wl, P.KV_INT8_SYM)
        out = gpu_decode(P, wl, pool, P.KV_INT8_SYM)
        want = oracle_decode(wl, oracle_pool(wl, oracle.KV_INT8_SYM), oracle.KV_INT8_SYM)
        got = out.cpu().numpy().astype(np.float64)
        assert not np.isnan(got).any()
        d = float(np.max(np.abs(got - want)))
    else:
        ks, vs = calibrated_scales(wl)
        pool = _gpu_static_pool(P, wl, ks, vs)
        host = oracle_static_pool(wl, ks, vs)
        assert np.array_equal(pool.cpu().numpy(), host)
        out = _gpu_static_decode(P, wl, pool, ks, vs)
        d = _max_diff(out, _oracle_decode(wl, host, ks, vs))
    _say(f"  max abs diff {d:.3e}")
    assert d <= MAX_ABS_TOL
    for b, L in enumerate(wl.context_lens):
        if L == 0:
            assert torch.all(out[b] == 0)


@pytest.mark.parametrize("fmt_name", ["int8", "static"])
@pytest.mark.parametrize("g", GROUPS)
def test_pair_groups_ragged(P, g, fmt_name):
    wl = _wl("pair-short", 500 + g, SHORT, g)
    _say(f"pair decode {fmt_name}: group {g}, lens {SHORT}")
    _check_decode(P, wl, fmt_name)


@pytest.mark.parametrize("fmt_name", ["int8", "static"])
@pytest.mark.parametrize("g,dt", [(4, "f16"), (7, "bf16")])
def test_pair_long_odd_share(P, g, dt, fmt_name):
    wl = _wl("pair-long", 600 + g, LONG, g, dt)
    _say(f"pair decode {fmt_name}: group {g} {dt}, lens {LONG}")
    _check_decode(P, wl, fmt_name)


@pytest.mark.parametrize("g", [1, 4, 7])
def test_pair_fused_append_int8(P, g):
    """The pool the fused step leaves equals the oracle's, its output is
    within the bound, and the plain decode of that pool gives the same rows
    bit for bit."""
    wl = _wl("pair-append", 700 + g, APPEND, g, append=True)
    _say(f"pair fused append int8: group {g}, final lens {APPEND}")
    check_fused_int8(P, wl, "int8")
    out, pool = _fused(P, wl, P.KV_INT8_SYM)
    again = gpu_decode(P, wl, pool, P.KV_INT8_SYM)
    assert torch.equal(out, again)


@pytest.mark.parametrize("g", [2, 7])
def test_pair_fused_append_static(P, g):
    wl = _wl("pair-append-static", 800 + g, APPEND, g, "bf16", append=True)
    ks, vs = calibrated_scales(wl)
    last = wl.phases[-1]
    _say(f"pair fused append static: group {g}, final lens {APPEND}")
    pool = _gpu_static_pool(P, wl, ks, vs, phases=wl.phases[:-1])
    out = torch.empty((wl.num_seqs, wl.num_q_heads, wl.head_dim), dtype=torch.float32,
                      device="cuda")
    ws = P.alloc_workspace(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                           wl.max_context_len)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    P.paged_attn_decode_int8_static_append(
        out, to_dev(wl.q), to_dev(last.k), to_dev(last.v), pool, wl.num_blocks,
        dev_i32(wl.block_tables), dev_i32(wl.context_lens), wl.num_kv_heads,
        wl.max_context_len, wl.sm_scale, ks, vs, ws, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    host = oracle_static_pool(wl, ks, vs)
    assert np.array_equal(pool.cpu().numpy(), host)
    d = _max_diff(out, _oracle_decode(wl, host, ks, vs))
    _say(f"  max abs diff {d:.3e}")
    assert d <= MAX_ABS_TOL
    assert torch.equal(out, _gpu_static_decode(P, wl, pool, ks, vs))


@pytest.mark.parametrize("fmt_name", ["int8", "static"])
def test_pair_many_short_units_several_passes(P, fmt_name):
    """2,000 sequences of 0 to 40 tokens (one to three pages, most counts odd):
    a wave's run of about a dozen pages crosses many units, so a pass reaches
    its segment limit and the wave takes several passes, each segment padded
    to whole pairs."""
    rng = np.random.default_rng(901)
    lens = rng.integers(0, 41, 2000).tolist()
    wl = _wl("pair-many", 902, lens, 4)
    _say(f"pair decode {fmt_name}: 2,000 short sequences, {sum(lens)} tokens")
    _check_decode(P, wl, fmt_name)
