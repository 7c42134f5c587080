"""Pins for the oracle's multi-token decode (CPU only).

T query tokens per sequence are the sequence's last T positions; token j
attends to the positions up to its own (causal among the new tokens). Checked
against an independent pure-Python FP64 brute force (math.fsum over explicit
per-token position lists) for the three page formats, closed forms (a query
token that sees one position returns that position's value; a token before
the start of the sequence gives zeros), and the single-token decode where the
two coincide (T = 1; the last query token).
"""

import math

import numpy as np
import pytest

import oracle
from oracle import KV_16BIT, KV_INT8_STATIC, KV_INT8_SYM
from tests.test_oracle_attention import _brute_attention


def _case(rng, kind, lens, T, hq, hkv, d, bs=16):
    """Pool of the given format holding random K/V for sequences of lengths
    ``lens``; returns (pool, block_tables, q [B, T, Hq, D], k, v) with k/v the
    per-sequence dequantized values as Python lists [L][hkv][d]."""
    nblk = [max(1, math.ceil(L / bs)) for L in lens]
    total = sum(nblk) + 2
    perm = rng.permutation(total)
    bt = np.zeros((len(lens), max(nblk)), np.int32)
    off = 0
    for b, n in enumerate(nblk):
        bt[b, :n] = perm[off:off + n]
        off += n
    fmt = {"int8": KV_INT8_SYM, "static": KV_INT8_STATIC, "16bit": KV_16BIT}[kind]
    pool = oracle.new_pool(fmt, total, bs, hkv, d, fill=0x33)
    ks, vs = 0.031, 0.027
    keys, vals = [], []
    for b, L in enumerate(lens):
        xk = rng.standard_normal((L, hkv, d)).astype(np.float16).astype(np.float32)
        xv = rng.standard_normal((L, hkv, d)).astype(np.float16).astype(np.float32)
        t = np.arange(L)
        slots = bt[b, t // bs] * bs + t % bs
        if kind == "int8":
            kc, kss = oracle.quantize_rows(xk)
            vc, vss = oracle.quantize_rows(xv)
            oracle.write_int8_tokens(pool, kc, kss, vc, vss, slots, bs)
            kf = kc.astype(np.float64) * kss.astype(np.float64)[..., None]
            vf = vc.astype(np.float64) * vss.astype(np.float64)[..., None]
        elif kind == "static":
            kc, vc = oracle.quantize_static(xk, ks), oracle.quantize_static(xv, vs)
            oracle.write_int8_static_tokens(pool, kc, vc, slots, bs)
            kf = kc.astype(np.float64) * float(np.float32(ks))
            vf = vc.astype(np.float64) * float(np.float32(vs))
        else:
            oracle.write_16bit_tokens(pool, xk.astype(np.float16).view(np.uint16),
                                      xv.astype(np.float16).view(np.uint16), slots, bs)
            kf, vf = xk.astype(np.float64), xv.astype(np.float64)
        keys.append(kf.tolist())
        vals.append(vf.tolist())
    q = (rng.standard_normal((len(lens), T, hq, d)) * 2).astype(np.float16)
    return pool, bt, q, keys, vals, ks, vs


def _run(kind, pool, bt, lens, q, sm, hkv, d, ks, vs):
    return oracle.decode_multi_from_pool(kind, pool, bt, np.array(lens), q, sm, 16, hkv, d,
                                         kv_dtype="f16", k_scale=ks, v_scale=vs)


@pytest.mark.parametrize("kind", ["int8", "static", "16bit"])
@pytest.mark.parametrize("T,hq,hkv,d", [(3, 8, 2, 64), (4, 4, 4, 64), (2, 7, 1, 128)])
def test_multi_matches_pure_python_brute_force(kind, T, hq, hkv, d):
    rng = np.random.default_rng(T * 100 + hq + d)
    lens = [T + 14, 33, T]  # a query that starts mid-page, one past a page, one at position 0
    pool, bt, q, keys, vals, ks, vs = _case(rng, kind, lens, T, hq, hkv, d)
    sm = 1.0 / math.sqrt(d)
    got = _run(kind, pool, bt, lens, q, sm, hkv, d, ks, vs)
    g = hq // hkv
    for b, L in enumerate(lens):
        for j in range(T):
            visible = list(range(L - T + j + 1))  # positions 0 .. L - T + j
            for h in range(hq):
                kk = [[keys[b][t][h // g][x] for x in range(d)] for t in visible]
                vv = [[vals[b][t][h // g][x] for x in range(d)] for t in visible]
                want = _brute_attention([float(x) for x in q[b, j, h].astype(np.float64)],
                                        kk, vv, sm)
                assert np.max(np.abs(got[b, j, h] - np.array(want))) < 1e-12, (b, j, h)


def test_one_visible_position_and_tokens_before_the_start():
    """L = 1, T = 3: query tokens 0 and 1 sit at positions -2 and -1 (zero
    rows); token 2 sees position 0 only, so it returns V at position 0."""
    rng = np.random.default_rng(9)
    pool, bt, q, keys, vals, ks, vs = _case(rng, "int8", [1], 3, 4, 2, 64)
    got = _run("int8", pool, bt, [1], q, 0.125, 2, 64, ks, vs)
    assert np.all(got[0, :2] == 0)
    for h in range(4):
        assert np.array_equal(got[0, 2, h], np.array(vals[0][0][h // 2]))


def test_single_query_token_is_the_plain_decode():
    rng = np.random.default_rng(10)
    lens = [40, 17]
    pool, bt, q, *_ = _case(rng, "int8", lens, 1, 8, 2, 64)
    a = _run("int8", pool, bt, lens, q, 0.1, 2, 64, None, None)[:, 0]
    b = oracle.decode_int8_from_pool(pool, bt, np.array(lens), q[:, 0], 0.1, 16, 2, 64)
    assert np.array_equal(a, b)


def test_last_query_token_sees_the_whole_context():
    rng = np.random.default_rng(11)
    lens = [50, 23]
    pool, bt, q, *_ = _case(rng, "16bit", lens, 5, 8, 2, 64)
    a = _run("16bit", pool, bt, lens, q, 0.1, 2, 64, None, None)[:, 4]
    b = oracle.decode_16bit_from_pool(pool, bt, np.array(lens), q[:, 4], 0.1, 16, 2, 64, "f16")
    assert np.array_equal(a, b)
