"""Pins for the oracle's page layout (CPU only).

The byte totals are the ones printed on MoE-Infinity PR #183 ("Precision &
memory"); the offsets inside a page are the documented layout contract
(INT8: every KV head's codes, then every KV head's scales), checked here at
hand-computed byte positions.
"""

import numpy as np

import oracle
from oracle import KV_16BIT, KV_INT8_SYM


def test_page_bytes_match_the_printed_totals(golden):
    (row,) = golden("page_bytes.txt")
    bs, hkv, d, i8, f16, ratio = row[0].split()
    bs, hkv, d = int(bs), int(hkv), int(d)
    assert oracle.page_bytes(KV_INT8_SYM, bs, hkv, d) == int(i8)
    assert oracle.page_bytes(KV_16BIT, bs, hkv, d) == int(f16)
    assert int(i8) / int(f16) == float(ratio)


def test_small_head_page_bytes():
    # 2 KV heads, head_dim 64: 2 * (2*16*64 + 4*16) = 4224; 16-bit: 2*4*16*64 = 8192
    assert oracle.page_bytes(KV_INT8_SYM, 16, 2, 64) == 4224
    assert oracle.page_bytes(KV_16BIT, 16, 2, 64) == 8192


def test_pool_bytes_equal_blocks_times_page_bytes():
    pool = oracle.new_pool(KV_INT8_SYM, 37, 16, 8, 128)
    assert pool.nbytes == 37 * 33280


def test_int8_byte_offsets_by_hand():
    """One token written to slot 5 of page 2, head 3 of a (16, 8, 128) pool."""
    pool = oracle.new_pool(KV_INT8_SYM, 4, 16, 8, 128)
    kc = np.zeros((1, 8, 128), np.int8)
    vc = np.zeros((1, 8, 128), np.int8)
    ks = np.ones((1, 8), np.float16)
    vs = np.ones((1, 8), np.float16)
    kc[0, 3, 5] = 11
    vc[0, 3, 7] = -13
    ks[0, 3] = np.float16(0.5)       # 0x3800
    vs[0, 3] = np.float16(0.25)      # 0x3400
    oracle.write_int8_tokens(pool, kc, ks, vc, vs, [2 * 16 + 5], 16)
    flat = pool.reshape(-1)
    page = 2 * 33280
    code = page + 3 * 4096                  # head 3's code block (8 blocks of 4096 bytes)
    assert flat[code + 5 * 128 + 5] == 11                               # K[pos 5][d 5]
    assert flat[code + 2048 + (5 // 4) * 512 + 7 * 4 + 5 % 4] == (256 - 13)  # V[pos 5][d 7]
    # scales after the 8 code blocks: head 3's 64 bytes at 32768 + 192; token 5
    # is token 1 of group 1: K scale at 16 + 2, V scale at 16 + 8 + 2
    sc = page + 32768 + 3 * 64
    assert flat[sc + 18] == 0x00 and flat[sc + 19] == 0x38
    assert flat[sc + 26] == 0x00 and flat[sc + 27] == 0x34
    # the other heads' scales of that token are 1.0 = 0x3C00
    assert flat[page + 32768 + 0 * 64 + 19] == 0x3C and flat[page + 32768 + 7 * 64 + 27] == 0x3C
    # nothing else in the page is non-zero except the scales of this token
    nz = np.nonzero(pool[2])[0]
    assert len(nz) == 2 + 8 * 2  # two codes + (one high scale byte) * 8 heads * 2


def test_16bit_byte_offsets_by_hand():
    pool = oracle.new_pool(KV_16BIT, 3, 16, 2, 64)
    k = np.zeros((1, 2, 64), np.uint16)
    v = np.zeros((1, 2, 64), np.uint16)
    k[0, 1, 9] = 0x1234
    v[0, 1, 63] = 0xABCD
    oracle.write_16bit_tokens(pool, k, v, [1 * 16 + 14], 16)
    w = pool.reshape(-1).view(np.uint16)
    head_w = 1 * (8192 // 2) + 1 * (2 * 16 * 64)
    assert w[head_w + 14 * 64 + 9] == 0x1234
    assert w[head_w + 16 * 64 + (14 // 4) * 256 + 63 * 4 + 14 % 4] == 0xABCD
    assert np.count_nonzero(w) == 2


def test_write_then_gather_round_trip_shuffled():
    rng = np.random.default_rng(0)
    L, hkv, d, bs = 70, 3, 64, 16
    nblk = 5
    bt = rng.permutation(8)[:nblk]
    kc = rng.integers(-127, 128, (L, hkv, d)).astype(np.int8)
    vc = rng.integers(-127, 128, (L, hkv, d)).astype(np.int8)
    ks = rng.uniform(0.01, 2, (L, hkv)).astype(np.float16)
    vs = rng.uniform(0.01, 2, (L, hkv)).astype(np.float16)
    pool = oracle.new_pool(KV_INT8_SYM, 8, bs, hkv, d, fill=0xAA)
    t = np.arange(L)
    slots = bt[t // bs] * bs + t % bs
    # write in a random order, and with one padding token that must be skipped
    order = rng.permutation(L)
    oracle.write_int8_tokens(pool, kc[order], ks[order], vc[order], vs[order], slots[order], bs)
    oracle.write_int8_tokens(pool, kc[:1] * 0 + 5, ks[:1], vc[:1], vs[:1], [-1], bs)
    gk, gks, gv, gvs = oracle.gather_int8_sequence(pool, bt, L, bs, hkv, d)
    assert np.array_equal(gk, kc) and np.array_equal(gv, vc)
    assert np.array_equal(gks.view(np.uint16), ks.view(np.uint16))
    assert np.array_equal(gvs.view(np.uint16), vs.view(np.uint16))
    gk1, _, gv1, _ = oracle.gather_int8_sequence(pool, bt, L, bs, hkv, d, heads=[2])
    assert np.array_equal(gk1[:, 0], kc[:, 2]) and np.array_equal(gv1[:, 0], vc[:, 2])

    kb = rng.integers(0, 65536, (L, hkv, d)).astype(np.uint16)
    vb = rng.integers(0, 65536, (L, hkv, d)).astype(np.uint16)
    pool16 = oracle.new_pool(KV_16BIT, 8, bs, hkv, d)
    oracle.write_16bit_tokens(pool16, kb, vb, slots, bs)
    g16k, g16v = oracle.gather_16bit_sequence(pool16, bt, L, bs, hkv, d)
    assert np.array_equal(g16k, kb) and np.array_equal(g16v, vb)
