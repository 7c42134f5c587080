"""Pins for the oracle's static-scale INT8 variant (CPU only).

Static scales: one calibrated scalar for all of K and one for all of V of a
layer (InfiniLM PR #553, "Summary" and "Notes for Reviewers"; TensorRT-LLM
PR #18953, "Summary"). Each test checks the oracle against something other
than itself: hand-derived worked examples, an exact-rational brute force that
rounds the quotient to binary32 from the format's definition, closed forms
(lossless powers of two, saturation, sign symmetry), the equality with the
per-token oracle where both schemes pick the same scale, the cache sizes the
InfiniLM page prints, hand-computed byte offsets, and a pure-Python FP64
attention brute force.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import KV_16BIT, KV_INT8_STATIC, KV_INT8_SYM
from tests.test_oracle_attention import _brute_attention


def _f32(v):
    return float(np.float32(v))


def test_worked_examples(golden):
    rows = golden("static_quant_examples.txt")
    assert len(rows) >= 3
    for name, s, xs, codes in rows:
        s32 = np.float32(float(s))
        assert Fraction(float(s32)) == Fraction(s), name  # the scale is a binary32 value
        x = np.array([float(t) for t in xs.split()], dtype=np.float32)
        assert oracle.quantize_static(x, s32).tolist() == [int(t) for t in codes.split()], name


def _round_binary32(q: Fraction) -> Fraction:
    """Round an exact rational to the nearest binary32 value, ties to even
    (normal range only: 24-bit significand)."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    n = a * (1 << 23)
    whole = n.numerator // n.denominator
    rest = n - whole
    if rest > Fraction(1, 2) or (rest == Fraction(1, 2) and whole % 2 == 1):
        whole += 1
    return sign * Fraction(whole, 1 << 23) * Fraction(2) ** e


def _brute_static(row, s):
    """code = clip(round_half_even(binary32(x / s)), -127, 127), in exact rationals."""
    sf = Fraction(float(np.float32(s)))
    out = []
    for v in row:
        q = _round_binary32(Fraction(float(v)) / sf)
        out.append(max(-127, min(127, round(q))))  # round(): ties to even
    return out


def _rows(kind, n, d, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d)).astype(np.float32)
    x[:, rng.choice(d, 4, replace=False)] *= 20
    x *= np.float32(10.0 ** rng.uniform(-2, 1))
    t = torch.from_numpy(x)
    return (t.half() if kind == "f16" else t.bfloat16()).float().numpy()


@pytest.mark.parametrize("kind", ["f16", "bf16"])
@pytest.mark.parametrize("scale", [1.0, 0.05, 0.0625, 0.0371, 3.7e-3, 2.5])
def test_codes_match_exact_rational_brute_force(kind, scale):
    x = _rows(kind, 12, 64, int(scale * 1e4) + (kind == "bf16"))
    c = oracle.quantize_static(x, scale)
    for i in range(x.shape[0]):
        assert c[i].tolist() == _brute_static(x[i], scale)


def test_lossless_when_values_are_codes_times_scale():
    """x = c * 2^k with |c| <= 127: codes come back exactly."""
    rng = np.random.default_rng(1)
    for k in (-12, -5, 0, 3):
        c = rng.integers(-127, 128, size=(8, 128)).astype(np.int8)
        x = c.astype(np.float32) * np.float32(2.0 ** k)
        got = oracle.quantize_static(x, 2.0 ** k)
        assert np.array_equal(got, c)
        assert np.array_equal(oracle.dequantize_static(got, 2.0 ** k), x.astype(np.float64))


def test_saturation_and_no_minus_128():
    s = np.float32(0.01)
    x = np.array([1.275, 1.2751, 5.0, 1e4, -1.2751, -5.0, -1e4], np.float32)
    c = oracle.quantize_static(x, s)
    assert c.tolist() == [127, 127, 127, 127, -127, -127, -127]


def test_sign_symmetry_and_monotonicity():
    x = np.sort(_rows("f16", 1, 4096, 9)[0])
    for s in (0.05, 0.013, 1.0):
        c = oracle.quantize_static(x, s).astype(np.int32)
        assert np.all(np.diff(c) >= 0)
        assert np.array_equal(oracle.quantize_static(-x, s), (-c).astype(np.int8))


def test_error_within_half_step_inside_the_range():
    """|x - c*s| <= s * (1/2 + 127 * 2^-24) for |x| <= 127 s (the division's
    relative error is at most 2^-24, then the integer rounding adds 1/2)."""
    rng = np.random.default_rng(4)
    for s in (0.05, 0.0371, 1.0):
        x = (rng.uniform(-127, 127, 20000) * s).astype(np.float32)
        c = oracle.quantize_static(x, s).astype(np.float64)
        s64 = float(np.float32(s))
        err = np.abs(x.astype(np.float64) - c * s64)
        assert np.all(err <= s64 * (0.5 + 127 * 2.0 ** -24))


def test_matches_per_token_codes_when_the_scales_agree():
    """A row whose absmax is 127 * s for an FP16 value s gets per-token scale
    s exactly, so both schemes give the same codes."""
    rng = np.random.default_rng(6)
    for s16 in (np.float16(0.0500488), np.float16(1.0), np.float16(0.00390625)):
        s = float(s16)
        x = rng.uniform(-127 * s, 127 * s, (32, 128)).astype(np.float16).astype(np.float32)
        x[:, 0] = 127 * s  # exact in fp16 times 127 (fp32 holds 11 + 7 bits)
        codes_pt, scale_pt = oracle.quantize_rows(x)
        assert np.all(scale_pt == s16)
        assert np.array_equal(oracle.quantize_static(x, s), codes_pt)


def test_scale_validity_and_shared_scale():
    for bad in (0.0, -1.0, float("nan"), float("inf"), -0.0):
        with pytest.raises(ValueError):
            oracle.quantize_static(np.ones(4, np.float32), bad)
    assert oracle.shared_static_scale(0.05, 0.5) == np.float32(0.5)
    assert oracle.shared_static_scale(3.0, 0.25) == np.float32(3.0)
    with pytest.raises(ValueError):
        oracle.shared_static_scale(0.05, 0.0)


def test_cache_bytes_match_the_printed_sizes(golden):
    rows = golden("static_cache_bytes.txt")
    assert len(rows) == 4
    for name, shape, bf16, i8, unit in rows:
        layers, hkv, d, tokens = (int(t) for t in shape.split())
        div = {"MiB": 2.0 ** 20, "MB": 1e6}[unit]
        pages = tokens // 16
        b16 = layers * pages * oracle.page_bytes(KV_16BIT, 16, hkv, d)
        b8 = layers * pages * oracle.page_bytes(KV_INT8_STATIC, 16, hkv, d)
        assert round(b16 / div, 2) == float(bf16), name
        assert round(b8 / div, 2) == float(i8), name
        assert 2 * b8 == b16, name


def test_static_page_bytes_by_hand():
    # (16, 8, 128): 8 * 2 * 16 * 128 = 32768; (16, 2, 64): 2 * 2 * 16 * 64 = 4096
    assert oracle.page_bytes(KV_INT8_STATIC, 16, 8, 128) == 32768
    assert oracle.page_bytes(KV_INT8_STATIC, 16, 2, 64) == 4096


def test_static_byte_offsets_by_hand():
    """One token written to slot 13 of page 1, head 1 of a (16, 2, 64) pool."""
    pool = oracle.new_pool(KV_INT8_STATIC, 3, 16, 2, 64)
    kc = np.zeros((1, 2, 64), np.int8)
    vc = np.zeros((1, 2, 64), np.int8)
    kc[0, 1, 7] = 5
    vc[0, 1, 62] = -9
    oracle.write_int8_static_tokens(pool, kc, vc, [1 * 16 + 13], 16)
    flat = pool.reshape(-1)
    head = 1 * 4096 + 1 * 2048
    assert flat[head + 13 * 64 + 7] == 5                                   # K[13][7]
    assert flat[head + 1024 + (13 // 4) * 256 + 62 * 4 + 13 % 4] == 256 - 9  # V[13][62]
    assert np.count_nonzero(pool) == 2
    kc2, vc2 = oracle.gather_int8_static_sequence(pool, [2, 1], 30, 16, 2, 64)
    assert kc2[29, 1, 7] == 5 and vc2[29, 1, 62] == -9


def _static_case(rng, L, hq, hkv, d, sk, sv):
    xk = rng.standard_normal((L, hkv, d)).astype(np.float16).astype(np.float32)
    xv = rng.standard_normal((L, hkv, d)).astype(np.float16).astype(np.float32)
    kc, vc = oracle.quantize_static(xk, sk), oracle.quantize_static(xv, sv)
    nblk = max(1, math.ceil(L / 16))
    bt = rng.permutation(nblk + 2)[:nblk].astype(np.int32)
    pool = oracle.new_pool(KV_INT8_STATIC, nblk + 2, 16, hkv, d, fill=0x55)
    t = np.arange(L)
    oracle.write_int8_static_tokens(pool, kc, vc, bt[t // 16] * 16 + t % 16, 16)
    q = (rng.standard_normal((1, hq, d)) * 2).astype(np.float16)
    return pool, bt, q, kc, vc


@pytest.mark.parametrize("L", [1, 16, 33])
@pytest.mark.parametrize("hq,hkv,d", [(4, 4, 64), (8, 2, 128), (7, 1, 64)])
def test_static_decode_matches_pure_python_brute_force(L, hq, hkv, d):
    rng = np.random.default_rng(L * 7 + hq + d)
    sk, sv = 0.0371, 0.0229
    pool, bt, q, kc, vc = _static_case(rng, L, hq, hkv, d, sk, sv)
    sm = 1.0 / math.sqrt(d)
    got = oracle.decode_int8_static_from_pool(pool, bt[None], np.array([L]), q, sm, sk, sv,
                                              16, hkv, d)
    g = hq // hkv
    for h in range(hq):
        kvh = h // g
        keys = [[int(kc[t, kvh, j]) * _f32(sk) for j in range(d)] for t in range(L)]
        vals = [[int(vc[t, kvh, j]) * _f32(sv) for j in range(d)] for t in range(L)]
        want = _brute_attention([float(v) for v in q[0, h].astype(np.float64)], keys, vals, sm)
        assert np.max(np.abs(got[0, h] - np.array(want))) < 1e-12


def test_static_decode_equals_per_token_decode_with_equal_scales():
    """A per-token pool whose every scale is the FP16 value s decodes to the
    same result as a static pool with the same codes and k/v scale s."""
    rng = np.random.default_rng(11)
    L, hq, hkv, d = 45, 8, 2, 64
    s = float(np.float16(0.0419))
    pool_s, bt, q, kc, vc = _static_case(rng, L, hq, hkv, d, s, s)
    pool_t = oracle.new_pool(KV_INT8_SYM, pool_s.shape[0], 16, hkv, d)
    sc = np.full((L, hkv), np.float16(s))
    t = np.arange(L)
    oracle.write_int8_tokens(pool_t, kc, sc, vc, sc, bt[t // 16] * 16 + t % 16, 16)
    a = oracle.decode_int8_static_from_pool(pool_s, bt[None], np.array([L]), q, 0.125, s, s,
                                            16, hkv, d)
    b = oracle.decode_int8_from_pool(pool_t, bt[None], np.array([L]), q, 0.125, 16, hkv, d)
    assert np.array_equal(a, b)


def test_static_decode_closed_forms():
    rng = np.random.default_rng(12)
    hq, hkv, d = 4, 2, 64
    sk, sv = 0.03, 0.07
    # one token: the output is its value
    pool, bt, q, kc, vc = _static_case(rng, 1, hq, hkv, d, sk, sv)
    got = oracle.decode_int8_static_from_pool(pool, bt[None], np.array([1]), q, 0.1, sk, sv,
                                              16, hkv, d)
    for h in range(hq):
        assert np.array_equal(got[0, h], vc[0, h // 2].astype(np.float64) * _f32(sv))
    # zero query: the mean of the values; empty context: zeros
    pool, bt, q, kc, vc = _static_case(rng, 21, hq, hkv, d, sk, sv)
    got = oracle.decode_int8_static_from_pool(pool, bt[None], np.array([21]),
                                              np.zeros_like(q), 0.1, sk, sv, 16, hkv, d)
    want = vc.astype(np.float64).mean(axis=0) * _f32(sv)
    for h in range(hq):
        assert np.allclose(got[0, h], want[h // 2], rtol=0, atol=1e-15)
    got = oracle.decode_int8_static_from_pool(pool, bt[None], np.array([0]), q, 0.1, sk, sv,
                                              16, hkv, d)
    assert np.all(got == 0)


@pytest.mark.parametrize("idx,scale", [(1, 1.0), (4, 0.01)])
def test_per_token_scales_are_more_accurate_than_static(idx, scale):
    """The accuracy side of the static vs per-token comparison (InfiniLM PR
    #553, "Notes for Reviewers": a static scale has a precision ceiling that
    per-token scales remove): against attention over the unquantized 16-bit
    K/V, the per-token scheme's RMS error is below the calibrated static
    scheme's on outlier-channel (config 1) and log-magnitude (config 4) rows."""
    from tests.gpu_util import calibrated_scales, oracle_pool, oracle_static_pool
    from workloads import make_config
    wl = make_config(idx, scale)
    ks, vs = calibrated_scales(wl)
    args = (wl.block_tables, wl.context_lens, wl.q, wl.sm_scale)
    shape = (16, wl.num_kv_heads, wl.head_dim)
    ref = oracle.decode_16bit_from_pool(oracle_pool(wl, KV_16BIT), *args, *shape, wl.kv_dtype)
    pt = oracle.decode_int8_from_pool(oracle_pool(wl, KV_INT8_SYM), *args, *shape)
    st = oracle.decode_int8_static_from_pool(oracle_static_pool(wl, ks, vs), *args, ks, vs,
                                             *shape)
    rms = lambda o: float(np.sqrt(np.mean((o - ref) ** 2)))  # noqa: E731
    assert rms(pt) < 0.7 * rms(st)
