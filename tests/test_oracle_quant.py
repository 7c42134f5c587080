"""Pins for the oracle's INT8 quantizer (CPU only).

Each test checks the oracle against something other than itself:
hand-derived worked examples, the invariants the MoE-Infinity page states
("What landed": no -128, exact zero, |x - c*s| <= s/2 + 1e-6), the zero-token
and max-coordinate rules of the mlxcel page ("The Int8 bug and fix"), exact
rational arithmetic, and exhaustive searches over every FP16 value.
"""

import bisect
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle.quant import ru16

# all positive finite fp16 values, ascending, as exact float64 / Fraction
_F16_POS = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
_F16_FRAC = [Fraction(float(v)) for v in _F16_POS]


def _parse_num(tok):
    return float(tok)


def test_worked_examples(golden):
    rows = golden("quant_worked_examples.txt")
    assert len(rows) >= 7
    for name, xs, sbits, codes in rows:
        x = np.array([[_parse_num(t) for t in xs.split()]], dtype=np.float32)
        c, s = oracle.quantize_rows(x)
        assert int(s.view(np.uint16)[0]) == int(sbits, 16), name
        assert c[0].tolist() == [int(t) for t in codes.split()], name


def _rows(kind, n, d, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d)).astype(np.float32)
    if kind == "outlier":
        x[:, rng.choice(d, 4, replace=False)] *= 20
    mag = 10.0 ** rng.uniform(-6, 3, size=(n, 1))
    x = (x * mag).astype(np.float32)
    t = torch.from_numpy(x)
    return (t.half() if kind != "bf16" else t.bfloat16()).float().numpy()


@pytest.mark.parametrize("kind", ["f16", "outlier", "bf16"])
def test_page_invariants(kind):
    """No -128; exact zero kept; |x - c*s| <= s/2 + 1e-6 (checked in FP64)."""
    x = _rows(kind, 4000, 128, 7)
    x[::37, 5] = 0.0
    x[::41, 9] = -0.0
    c, s = oracle.quantize_rows(x)
    assert c.dtype == np.int8 and s.dtype == np.float16
    assert c.min() >= -127 and c.max() <= 127
    assert np.all(c[x == 0] == 0)
    s64 = s.astype(np.float64)[:, None]
    err = np.abs(x.astype(np.float64) - c.astype(np.float64) * s64)
    assert np.all(err <= s64 / 2 + 1e-6)


@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_scale_is_smallest_fp16_at_or_above(kind):
    """prev16(s) * 127 < absmax <= s * 127, exactly (products exact in FP64)."""
    x = _rows(kind, 4000, 64, 11)
    c, s = oracle.quantize_rows(x)
    a = np.abs(x).max(axis=1).astype(np.float64)
    s64 = s.astype(np.float64)
    prev = np.nextafter(s, np.float16(0)).astype(np.float64)
    assert np.all(a <= s64 * 127)
    assert np.all(prev * 127 < a)


def test_scale_exhaustive_over_fp16_absmax():
    """For every positive finite FP16 absmax, the scale is the smallest FP16
    whose product with 127 reaches it (a search over the sorted FP16 table)."""
    a = _F16_POS.astype(np.float32)
    x = np.zeros((a.size, 2), np.float32)
    x[:, 0] = a
    _, s = oracle.quantize_rows(x)
    idx = np.searchsorted(_F16_POS * 127.0, a.astype(np.float64), side="left")
    assert np.array_equal(s.astype(np.float64), _F16_POS[idx])


def test_scale_exhaustive_over_bf16_absmax():
    """Same search for every bf16 absmax in [2^-30, 127 * 65504]."""
    bits = np.arange(0x3080, 0x4B00, dtype=np.uint32)  # 2^-30 .. 2^23
    a = (bits << 16).view(np.float32)
    a = a[a.astype(np.float64) <= 127.0 * 65504.0]  # scale must fit FP16
    x = np.zeros((a.size, 2), np.float32)
    x[:, 1] = -a
    _, s = oracle.quantize_rows(x)
    idx = np.searchsorted(_F16_POS * 127.0, a.astype(np.float64), side="left")
    assert np.array_equal(s.astype(np.float64), _F16_POS[idx])


def _brute_quantize(row):
    """Pure-Python exact-rational quantizer for one row: scale = smallest FP16
    >= absmax/127 exactly, code = round-half-even(x / scale) exactly."""
    xs = [Fraction(float(v)) for v in row]
    a = max(abs(v) for v in xs)
    if a == 0:
        return [0] * len(xs), Fraction(1)
    target = a / 127
    s = _F16_FRAC[bisect.bisect_left(_F16_FRAC, target)]
    codes = [max(-127, min(127, round(v / s))) for v in xs]  # round(): ties to even
    return codes, s


@pytest.mark.parametrize("kind", ["f16", "outlier", "bf16"])
def test_codes_match_exact_rational_brute_force(kind):
    x = _rows(kind, 60, 128, 3)
    c, s = oracle.quantize_rows(x)
    for i in range(x.shape[0]):
        bc, bs = _brute_quantize(x[i])
        assert Fraction(float(s[i])) == bs
        assert c[i].tolist() == bc


def test_exact_ties_round_to_even():
    """Rows built so that x/s lands exactly on k + 1/2 for many k."""
    k = np.arange(-126, 126, dtype=np.float32)
    x = np.concatenate([[127.0], k + 0.5]).astype(np.float32)[None]  # scale 1.0
    c, s = oracle.quantize_rows(x)
    assert float(s[0]) == 1.0
    expect = [127] + [int(round(Fraction(float(v)))) for v in (k + 0.5)]
    assert c[0].tolist() == expect
    assert np.all(c[0, 1:] % 2 == 0)


def test_zero_token_gets_scale_one():
    x = np.zeros((3, 128), np.float32)
    x[1, 7] = -0.0
    c, s = oracle.quantize_rows(x)
    assert np.all(s == np.float16(1.0))
    assert np.all(c == 0)


def test_no_floor_at_one_for_small_rows():
    """The mlxcel fix: a row with absmax well below 127 keeps its true scale
    (a floor of the scale at 1.0 was the bug)."""
    x = np.array([[0.3, -0.1, 0.05]], np.float32)
    c, s = oracle.quantize_rows(x)
    assert float(s[0]) < 1.0
    assert c[0, 0] == 127


@pytest.mark.parametrize("kind", ["f16", "outlier", "bf16"])
def test_max_coordinate_maps_to_127(kind):
    """With a normal FP16 scale (absmax >= 127 * 2^-14) the largest-magnitude
    coordinate maps to +-127 (mlxcel PR #717, "The Int8 bug and fix")."""
    x = _rows(kind, 3000, 128, 5)
    c, s = oracle.quantize_rows(x)
    a = np.abs(x).max(axis=1)
    j = np.abs(x).argmax(axis=1)
    normal = a >= 127 * 2.0 ** -14
    assert normal.sum() > 100
    top = c[np.arange(len(j)), j]
    assert np.all(np.abs(top[normal]) == 127)
    assert np.all(np.sign(top[normal]) == np.sign(x[np.arange(len(j)), j][normal]))


def test_lossless_when_values_are_codes_times_power_of_two():
    rng = np.random.default_rng(9)
    for k in range(-20, 9):
        codes = rng.integers(-127, 128, size=(5, 64))
        codes[:, 0] = 127 * rng.choice([-1, 1], size=5)
        x = (codes * 2.0 ** k).astype(np.float32)
        c, s = oracle.quantize_rows(x)
        assert np.all(s.astype(np.float64) == 2.0 ** k)
        assert np.array_equal(c, codes)


def test_round_trip_within_one_quant_step():
    """Dequantized values recover the inputs within half a scale step
    (mlxcel PR #717 test idea: fetch recovers values within one quant step)."""
    x = _rows("outlier", 500, 128, 13)
    c, s = oracle.quantize_rows(x)
    back = oracle.dequantize_rows(c, s).astype(np.float64)
    assert np.all(np.abs(back - x) <= s.astype(np.float64)[:, None] / 2 + 1e-6)


def test_dequantize_is_exact_in_fp32():
    c = np.array([[127, -127, 93, 1]], np.int8)
    s = np.array([np.float16(0.00788116455078125)])
    got = oracle.dequantize_rows(c, s).astype(np.float64)
    want = c.astype(np.float64) * float(s[0])
    assert np.array_equal(got, want)


def test_ru16_direction_and_fixed_points():
    vals = _F16_POS[::97].astype(np.float32)
    assert np.array_equal(ru16(vals).astype(np.float32), vals)  # representable: unchanged
    up = np.nextafter(vals, np.float32(np.inf))
    r = ru16(up).astype(np.float64)
    nxt = np.nextafter(vals.astype(np.float16), np.float16(np.inf)).astype(np.float64)
    assert np.array_equal(r, nxt)
    assert ru16(np.float32(0.0)) == 0


def test_out_of_contract_inputs_raise():
    with pytest.raises(ValueError):
        oracle.quantize_rows(np.array([[np.nan, 1.0]], np.float32))
    with pytest.raises(ValueError):
        oracle.quantize_rows(np.array([[127.0 * 65504 * 2, 1.0]], np.float32))
