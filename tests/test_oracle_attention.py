"""Pins for the oracle's decode attention (CPU only).

The oracle is compared with an independent pure-Python FP64 brute force
(math.fsum / math.exp on Python floats, no NumPy arithmetic) on tiny inputs
that span several pages and a ragged tail, with closed forms (one token;
a zero query gives the mean of V), and with the GQA == repeated-MHA identity
(MoE-Infinity PR #183, "What landed": MHA/GQA decode over INT8 pages checked
against an FP32-dequantized attention oracle).
"""

import math

import numpy as np
import pytest

import oracle
from oracle import KV_16BIT, KV_INT8_SYM


def _brute_attention(q_row, keys, values, sm_scale):
    """q_row: list of D floats; keys/values: lists of L rows of D floats."""
    if not keys:
        return [0.0] * len(q_row)
    logits = [sm_scale * math.fsum(qd * kd for qd, kd in zip(q_row, k)) for k in keys]
    m = max(logits)
    w = [math.exp(x - m) for x in logits]
    z = math.fsum(w)
    d = len(q_row)
    return [math.fsum(w[t] * values[t][j] for t in range(len(keys))) / z for j in range(d)]


def _make_int8_case(rng, L, hq, hkv, d, bs=16, shuffle=True):
    x_k = rng.standard_normal((L, hkv, d)).astype(np.float32) * rng.uniform(0.1, 5, (L, 1, 1))
    x_v = rng.standard_normal((L, hkv, d)).astype(np.float32)
    x_k = x_k.astype(np.float16).astype(np.float32)
    x_v = x_v.astype(np.float16).astype(np.float32)
    kc, ks = oracle.quantize_rows(x_k)
    vc, vs = oracle.quantize_rows(x_v)
    nblk = max(1, math.ceil(L / bs))
    total = nblk + 3
    perm = rng.permutation(total) if shuffle else np.arange(total)
    bt = perm[:nblk].astype(np.int32)
    pool = oracle.new_pool(KV_INT8_SYM, total, bs, hkv, d, fill=0x7F)
    t = np.arange(L)
    oracle.write_int8_tokens(pool, kc, ks, vc, vs, bt[t // bs] * bs + t % bs, bs)
    q = (rng.standard_normal((1, hq, d)) * 2).astype(np.float16)
    return pool, bt, q, kc, ks, vc, vs


@pytest.mark.parametrize("L", [1, 15, 16, 17, 33])
@pytest.mark.parametrize("hq,hkv,d", [(4, 4, 64), (8, 2, 128), (7, 1, 64)])
def test_int8_decode_matches_pure_python_brute_force(L, hq, hkv, d):
    rng = np.random.default_rng(L * 1000 + hq * 10 + d)
    pool, bt, q, kc, ks, vc, vs = _make_int8_case(rng, L, hq, hkv, d)
    sm = 1.0 / math.sqrt(d)
    got = oracle.decode_int8_from_pool(pool, bt[None], np.array([L]), q, sm, 16, hkv, d)
    g = hq // hkv
    for h in range(hq):
        kvh = h // g
        keys = [[int(kc[t, kvh, j]) * float(ks[t, kvh]) for j in range(d)] for t in range(L)]
        vals = [[int(vc[t, kvh, j]) * float(vs[t, kvh]) for j in range(d)] for t in range(L)]
        want = _brute_attention([float(v) for v in q[0, h].astype(np.float64)], keys, vals, sm)
        assert np.max(np.abs(got[0, h] - np.array(want))) < 1e-12


@pytest.mark.parametrize("kv_dtype", ["f16", "bf16"])
def test_16bit_decode_matches_pure_python_brute_force(kv_dtype):
    import torch
    rng = np.random.default_rng(5)
    L, hq, hkv, d, bs = 37, 6, 2, 64, 16
    xk = torch.from_numpy(rng.standard_normal((L, hkv, d)).astype(np.float32) * 3)
    xv = torch.from_numpy(rng.standard_normal((L, hkv, d)).astype(np.float32))
    tdt = torch.float16 if kv_dtype == "f16" else torch.bfloat16
    kb = xk.to(tdt).view(torch.int16).numpy().view(np.uint16)
    vb = xv.to(tdt).view(torch.int16).numpy().view(np.uint16)
    bt = np.array([4, 0, 2], np.int32)
    pool = oracle.new_pool(KV_16BIT, 5, bs, hkv, d)
    t = np.arange(L)
    oracle.write_16bit_tokens(pool, kb, vb, bt[t // bs] * bs + t % bs, bs)
    q = torch.from_numpy(rng.standard_normal((1, hq, d)).astype(np.float32)).to(tdt)
    sm = 0.125
    got = oracle.decode_16bit_from_pool(pool, bt[None], np.array([L]), q, sm, bs, hkv, d, kv_dtype)
    kf = xk.to(tdt).float().numpy()
    vf = xv.to(tdt).float().numpy()
    qf = q.float().numpy()
    for h in range(hq):
        g = h // (hq // hkv)
        want = _brute_attention([float(x) for x in qf[0, h]], kf[:, g].tolist(), vf[:, g].tolist(), sm)
        assert np.max(np.abs(got[0, h] - np.array(want))) < 1e-12


def test_single_token_returns_its_value():
    rng = np.random.default_rng(1)
    pool, bt, q, kc, ks, vc, vs = _make_int8_case(rng, 1, 8, 2, 128)
    got = oracle.decode_int8_from_pool(pool, bt[None], np.array([1]), q, 0.1, 16, 2, 128)
    v = oracle.dequantize_rows(vc, vs)
    for h in range(8):
        assert np.array_equal(got[0, h], v[0, h // 4].astype(np.float64))


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(2)
    pool, bt, q, kc, ks, vc, vs = _make_int8_case(rng, 45, 4, 2, 64)
    q = np.zeros_like(q)
    got = oracle.decode_int8_from_pool(pool, bt[None], np.array([45]), q, 0.125, 16, 2, 64)
    v = oracle.dequantize_rows(vc, vs).astype(np.float64)
    for h in range(4):
        assert np.allclose(got[0, h], v[:, h // 2].mean(axis=0), rtol=0, atol=1e-12)


def test_context_zero_gives_zero_row():
    rng = np.random.default_rng(3)
    pool, bt, q, *_ = _make_int8_case(rng, 20, 4, 4, 64)
    got = oracle.decode_int8_from_pool(pool, bt[None], np.array([0]), q, 0.125, 16, 4, 64)
    assert np.all(got == 0)


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(4)
    L, hq, hkv, d = 29, 8, 2, 64
    k = rng.standard_normal((L, hkv, d))
    v = rng.standard_normal((L, hkv, d))
    q = rng.standard_normal((hq, d))
    gqa = oracle.attend_one_sequence(q, k, v, 0.2)
    mha = oracle.attend_one_sequence(q, np.repeat(k, hq // hkv, axis=1),
                                     np.repeat(v, hq // hkv, axis=1), 0.2)
    assert np.allclose(gqa, mha, rtol=0, atol=1e-13)


def test_block_table_permutation_invariance():
    """Moving pages to other physical blocks (and updating the table) leaves
    the output unchanged, bit for bit."""
    rng = np.random.default_rng(6)
    pool, bt, q, kc, ks, vc, vs = _make_int8_case(rng, 50, 8, 2, 128, shuffle=False)
    out1 = oracle.decode_int8_from_pool(pool, bt[None], np.array([50]), q, 0.09, 16, 2, 128)
    perm = rng.permutation(pool.shape[0])
    pool2 = np.empty_like(pool)
    pool2[perm] = pool
    out2 = oracle.decode_int8_from_pool(pool2, perm[bt][None].astype(np.int32), np.array([50]),
                                        q, 0.09, 16, 2, 128)
    assert np.array_equal(out1, out2)


def test_sampled_pairs_equal_full_computation():
    rng = np.random.default_rng(7)
    pool, bt, q, *_ = _make_int8_case(rng, 40, 8, 4, 64)
    full = oracle.decode_int8_from_pool(pool, bt[None], np.array([40]), q, 0.125, 16, 4, 64)
    part = oracle.decode_int8_from_pool(pool, bt[None], np.array([40]), q, 0.125, 16, 4, 64,
                                        pairs=[(0, 3), (0, 6)])
    assert np.array_equal(part[0, 3], full[0, 3]) and np.array_equal(part[0, 6], full[0, 6])
    assert np.isnan(part[0, 0]).all()
