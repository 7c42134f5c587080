"""Pins for the oracle's page lifecycle operations (CPU only).

Swap-out / swap-in (MoE-Infinity PR #183, "What landed", serving-lifecycle
bullet) and the front trim that keeps sink tokens (mlxcel PR #717 and its
follow-up: drop the n tokens after the first `keep`, scales moving with their
tokens). Checked against hand-computed byte positions, the untrimmed tail
(keep = 0, as the mlxcel tests do), identities (n = 0, round trips), clamps,
and attention over the token list with the dropped tokens removed.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import KV_16BIT, KV_INT8_STATIC, KV_INT8_SYM


def _pool(rng, kind, lens, hkv=2, d=64, bs=16, spare=3):
    nblk = [max(1, math.ceil(L / bs)) for L in lens]
    total = sum(nblk) + spare
    perm = rng.permutation(total)
    bt = np.zeros((len(lens), max(nblk)), np.int32)
    off = 0
    for b, n in enumerate(nblk):
        bt[b, :n] = perm[off:off + n]
        off += n
    fmt = {"int8": KV_INT8_SYM, "static": KV_INT8_STATIC, "16bit": KV_16BIT}[kind]
    pool = oracle.new_pool(fmt, total, bs, hkv, d)
    pool[:] = rng.integers(0, 256, pool.shape, dtype=np.uint8)  # stale bytes everywhere
    for b, L in enumerate(lens):
        xk = rng.standard_normal((L, hkv, d)).astype(np.float16)
        xv = rng.standard_normal((L, hkv, d)).astype(np.float16)
        t = np.arange(L)
        slots = bt[b, t // bs] * bs + t % bs
        if kind == "int8":
            kc, ks = oracle.quantize_rows(xk.astype(np.float32))
            vc, vs = oracle.quantize_rows(xv.astype(np.float32))
            oracle.write_int8_tokens(pool, kc, ks, vc, vs, slots, bs)
        elif kind == "static":
            oracle.write_int8_static_tokens(pool, oracle.quantize_static(xk.astype(np.float32), 0.03),
                                            oracle.quantize_static(xv.astype(np.float32), 0.03),
                                            slots, bs)
        else:
            oracle.write_16bit_tokens(pool, xk.view(np.uint16), xv.view(np.uint16), slots, bs)
    return fmt, pool, bt


def _tokens(kind, pool, bt_row, L, hkv, d):
    """Everything stored for positions 0..L-1 of one sequence (all heads)."""
    if kind == "int8":
        return oracle.gather_int8_sequence(pool, bt_row, L, 16, hkv, d)
    if kind == "static":
        return oracle.gather_int8_static_sequence(pool, bt_row, L, 16, hkv, d)
    return oracle.gather_16bit_sequence(pool, bt_row, L, 16, hkv, d)


KINDS = ["int8", "static", "16bit"]


@pytest.mark.parametrize("kind", KINDS)
def test_trim_keeps_the_sink_and_the_tail(kind):
    """L = 40, keep = 4, n = 20: new length 20; positions 0..3 are the old
    0..3, positions 4..19 the old 24..39."""
    rng = np.random.default_rng(1)
    fmt, pool, bt = _pool(rng, kind, [40, 23])
    before = [_tokens(kind, pool, bt[b], L, 2, 64) for b, L in enumerate([40, 23])]
    new = oracle.trim_keep_sink(fmt, pool, bt, [40, 23], [20, 0], 4, 16, 2, 64)
    assert new.tolist() == [20, 23]
    after = _tokens(kind, pool, bt[0], 20, 2, 64)
    for a, b_ in zip(after, before[0]):
        assert np.array_equal(a[:4], b_[:4])
        assert np.array_equal(a[4:20], b_[24:40])
    for a, b_ in zip(_tokens(kind, pool, bt[1], 23, 2, 64), before[1]):
        assert np.array_equal(a, b_)  # trim 0: untouched


@pytest.mark.parametrize("kind", KINDS)
def test_trim_without_sink_is_the_untrimmed_tail(kind):
    rng = np.random.default_rng(2)
    lens = [37, 64, 5]
    fmt, pool, bt = _pool(rng, kind, lens)
    before = [_tokens(kind, pool, bt[b], L, 2, 64) for b, L in enumerate(lens)]
    trims = [10, 33, 9]
    new = oracle.trim_keep_sink(fmt, pool, bt, lens, trims, 0, 16, 2, 64)
    assert new.tolist() == [27, 31, 0]  # 9 > 5: clamped
    for b in range(2):
        for a, b_ in zip(_tokens(kind, pool, bt[b], int(new[b]), 2, 64), before[b]):
            assert np.array_equal(a, b_[trims[b]:])


def test_trim_clamps_and_identities():
    rng = np.random.default_rng(3)
    lens = [30, 3, 50]
    fmt, pool, bt = _pool(rng, "int8", lens)
    ref = pool.copy()
    new = oracle.trim_keep_sink(fmt, pool, bt, lens, [0, 0, 0], 4, 16, 2, 64)
    assert new.tolist() == lens and np.array_equal(pool, ref)
    # keep >= L: nothing to drop; n beyond L - keep: everything after the sink goes
    new = oracle.trim_keep_sink(fmt, pool, bt, lens, [5, 2, 999], 4, 16, 2, 64)
    assert new.tolist() == [25, 3, 4]
    with pytest.raises(ValueError):
        oracle.trim_keep_sink(fmt, pool, bt, lens, [1, 1, 1], -1, 16, 2, 64)


def test_trim_byte_positions_by_hand():
    """Per-token INT8, (16, 1 head, D 64): keep 2, n 16 moves old position 21
    (page 1, slot 5) to position 5 (page 0, slot 5). Page = code block
    (2*16*64 = 2048 bytes: K row at 64*slot, V byte of dim d at 1024 +
    (slot//4)*256 + 4*d + slot%4) then 64 bytes of scales (16-byte records per
    four tokens: slot 5's K scale at 2048 + 16 + 2, its V scale at
    2048 + 16 + 8 + 2)."""
    pool = oracle.new_pool(KV_INT8_SYM, 2, 16, 1, 64)
    pool[1, 5 * 64:6 * 64] = np.arange(64, dtype=np.uint8) + 1            # K row of old 21
    pool[1, 1024 + 1 * 256 + 4 * 9 + 1] = 200                           # V dim 9 of old 21
    pool[1, 2066:2068] = [0x11, 0x22]                                   # K scale of old 21
    pool[1, 2074:2076] = [0x33, 0x44]                                   # V scale of old 21
    bt = np.array([[0, 1]], np.int32)
    new = oracle.trim_keep_sink(KV_INT8_SYM, pool, bt, [22], [16], 2, 16, 1, 64)
    assert new.tolist() == [6]
    assert np.array_equal(pool[0, 5 * 64:6 * 64], np.arange(64, dtype=np.uint8) + 1)
    assert pool[0, 1024 + 1 * 256 + 4 * 9 + 1] == 200
    assert pool[0, 2066:2068].tolist() == [0x11, 0x22]
    assert pool[0, 2074:2076].tolist() == [0x33, 0x44]


@pytest.mark.parametrize("kind", KINDS)
def test_attention_after_trim_equals_attention_without_the_dropped_tokens(kind):
    rng = np.random.default_rng(4)
    lens = [77, 40]
    fmt, pool, bt = _pool(rng, kind, lens, hkv=2, d=64)
    q = rng.standard_normal((2, 1, 8, 64)).astype(np.float16)
    full = [_tokens(kind, pool, bt[b], L, 2, 64) for b, L in enumerate(lens)]
    keep, trims = 4, [30, 17]
    new = oracle.trim_keep_sink(fmt, pool, bt, lens, trims, keep, 16, 2, 64)
    got = oracle.decode_multi_from_pool(kind if kind != "16bit" else "16bit", pool, bt, new, q,
                                        0.125, 16, 2, 64, kv_dtype="f16", k_scale=0.03,
                                        v_scale=0.03)
    for b in range(2):
        kept = np.r_[0:keep, keep + trims[b]:lens[b]]
        if kind == "int8":
            kc, ks, vc, vs = full[b]
            k = oracle.dequantize_rows(kc, ks)[kept]
            v = oracle.dequantize_rows(vc, vs)[kept]
        elif kind == "static":
            kc, vc = full[b]
            k, v = oracle.dequantize_static(kc, 0.03)[kept], oracle.dequantize_static(vc, 0.03)[kept]
        else:
            kb, vb = full[b]
            k, v = oracle.bits_to_f32(kb, "f16")[kept], oracle.bits_to_f32(vb, "f16")[kept]
        want = oracle.attend_one_sequence(q[b, 0].astype(np.float32), k, v, 0.125)
        assert np.array_equal(got[b, 0], want)


def test_swap_round_trip_and_relocation():
    rng = np.random.default_rng(5)
    lens = [50, 21]
    fmt, pool, bt = _pool(rng, "int8", lens, spare=8)
    ids = bt[0, :4].copy()
    pages = oracle.swap_out_pages(pool, ids)
    assert pages.shape == (4, pool.shape[1])
    for i, blk in enumerate(ids):
        assert np.array_equal(pages[i], pool[blk])
    # swap back into other (free) pages and remap the table: same tokens, same decode
    used = set(bt[0, :4].tolist()) | set(bt[1, :2].tolist())
    free = np.array([p for p in range(pool.shape[0]) if p not in used][:4], np.int32)
    before = _tokens("int8", pool, bt[0], 50, 2, 64)
    oracle.swap_in_pages(pool, free, pages)
    bt2 = bt.copy()
    bt2[0, :4] = free
    for a, b_ in zip(_tokens("int8", pool, bt2[0], 50, 2, 64), before):
        assert np.array_equal(a, b_)


def test_swap_skips_out_of_range_ids():
    rng = np.random.default_rng(6)
    fmt, pool, bt = _pool(rng, "static", [20])
    pages = oracle.swap_out_pages(pool, [1, -1, pool.shape[0], 0])
    assert np.array_equal(pages[0], pool[1]) and np.array_equal(pages[3], pool[0])
    assert not pages[1].any() and not pages[2].any()
    ref = pool.copy()
    oracle.swap_in_pages(pool, [-3, pool.shape[0] + 2], pages[:2])
    assert np.array_equal(pool, ref)
