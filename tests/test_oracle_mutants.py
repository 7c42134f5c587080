"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case monkeypatches one plausible mistake into a copy of an oracle
function — a dropped guard, a wrong rounding rule, a swapped operand or
index — and checks that at least one of the pin tests then fails. This shows
the pins constrain every step, not only the happy path.
"""

import numpy as np
import pytest

import oracle
import oracle.attention as oatt
import oracle.pages as opages
import oracle.quant as oquant
from tests.conftest import read_golden
from tests import test_oracle_attention as TA
from tests import test_oracle_pages as TP
from tests import test_oracle_quant as TQ


def _quantizer(scale_fn=None, round_fn=np.rint, divide=True, zero_guard=True, lo=-127):
    def q(x):
        x = oquant.as_f32(x)
        a = np.max(np.abs(x), axis=-1)
        s32 = np.divide(a, np.float32(127.0), dtype=np.float32)
        s16 = scale_fn(s32) if scale_fn else oquant.ru16(s32)
        if zero_guard:
            s16 = np.where(a == 0, np.float16(1.0), s16).astype(np.float16)
        sf = s16.astype(np.float32)[..., None]
        with np.errstate(all="ignore"):
            qq = np.divide(x, sf, dtype=np.float32) if divide else x * (np.float32(1) / sf)
            codes = np.clip(round_fn(qq), lo, 127)
        return np.nan_to_num(codes).astype(np.int8), s16
    return q


QUANT_MUTANTS = {
    "scale floored at 1.0": _quantizer(
        scale_fn=lambda s: np.maximum(oquant.ru16(s), np.float16(1.0))),
    "round half away from zero": _quantizer(
        round_fn=lambda v: np.sign(v) * np.floor(np.abs(v) + 0.5)),
    "reciprocal multiply": _quantizer(divide=False),
    "scale rounded to nearest": _quantizer(scale_fn=lambda s: s.astype(np.float16)),
    "no zero-token guard": _quantizer(zero_guard=False),
    "absmax/128 with -128 allowed": _quantizer(
        scale_fn=lambda s: oquant.ru16(s * np.float32(127.0 / 128.0)), lo=-128),
}

QUANT_PINS = [
    lambda: TQ.test_worked_examples(read_golden),
    lambda: TQ.test_page_invariants("outlier"),
    lambda: TQ.test_scale_exhaustive_over_fp16_absmax(),
    lambda: TQ.test_zero_token_gets_scale_one(),
    lambda: TQ.test_no_floor_at_one_for_small_rows(),
    lambda: TQ.test_max_coordinate_maps_to_127("f16"),
    lambda: TQ.test_exact_ties_round_to_even(),
]


def _caught(pins):
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


@pytest.mark.parametrize("name", sorted(QUANT_MUTANTS))
def test_quantizer_mutant_is_caught(name, monkeypatch):
    monkeypatch.setattr(oracle, "quantize_rows", QUANT_MUTANTS[name])
    assert _caught(QUANT_PINS), name


def test_unmutated_oracle_passes_the_same_pins():
    assert not _caught(QUANT_PINS)


def _v_index_token_major(pos, d, head_dim):
    return pos * head_dim + d


def _scale_offset_swapped(pos, is_v):
    return (pos // 4) * 16 + 8 * (1 - is_v) + 2 * (pos % 4)


def _scale_offset_token_major(pos, is_v):
    return 2 * pos + 2 * 16 * is_v


PAGE_MUTANTS = {
    "V stored token-major": ("_v_index", _v_index_token_major),
    "K and V scale slots swapped": ("_int8_scale_offset", _scale_offset_swapped),
    "scales not grouped by four tokens": ("_int8_scale_offset", _scale_offset_token_major),
}

PAGE_PINS = [
    lambda: TP.test_int8_byte_offsets_by_hand(),
    lambda: TP.test_16bit_byte_offsets_by_hand(),
]


@pytest.mark.parametrize("name", sorted(PAGE_MUTANTS))
def test_page_layout_mutant_is_caught(name, monkeypatch):
    attr, fn = PAGE_MUTANTS[name]
    monkeypatch.setattr(opages, attr, fn)
    assert _caught(PAGE_PINS), name


def _attend(scale_mul=1.0, swap_kv=False, drop_last=False, no_norm=False,
            ignore_sm_scale=False):
    def f(q, k, v, sm_scale):
        q = np.asarray(q, np.float64)
        k = np.asarray(k, np.float64)
        v = np.asarray(v, np.float64)
        if swap_kv:
            k, v = v, k
        if drop_last and k.shape[0] > 1:
            k, v = k[:-1], v[:-1]
        hq, d = q.shape
        hkv = k.shape[1]
        g = hq // hkv
        out = np.zeros((hq, d))
        if k.shape[0] == 0:
            return out
        for h in range(hq):
            lg = (1.0 if ignore_sm_scale else sm_scale) * scale_mul * (k[:, h // g] @ q[h])
            w = np.exp(lg - lg.max())
            out[h] = (w @ v[:, h // g]) / (1.0 if no_norm else w.sum())
        return out
    return f


def _decode_head_map_modulo(pool, block_tables, context_lens, q, sm_scale, block_size,
                            num_kv_heads, head_dim, pairs=None):
    """decode_int8_from_pool with query head h reading KV head h % Hkv."""
    qf = oquant.as_f32(q)
    B, hq, d = qf.shape
    out = np.zeros((B, hq, d))
    for b in range(B):
        kc, ks, vc, vs = opages.gather_int8_sequence(pool, block_tables[b], int(context_lens[b]),
                                                     block_size, num_kv_heads, head_dim)
        k, v = oquant.dequantize_rows(kc, ks), oquant.dequantize_rows(vc, vs)
        for h in range(hq):
            g = h % num_kv_heads
            out[b, h] = oatt.attend_one_sequence(qf[b, h][None], k[:, g:g + 1], v[:, g:g + 1],
                                                 sm_scale)[0]
    return out


ATT_MUTANTS = {
    "sm_scale ignored": ("attend_one_sequence", _attend(ignore_sm_scale=True)),
    "K and V swapped": ("attend_one_sequence", _attend(swap_kv=True)),
    "last token dropped": ("attend_one_sequence", _attend(drop_last=True)),
    "softmax not normalised": ("attend_one_sequence", _attend(no_norm=True)),
    "GQA head map h % Hkv": ("decode_int8_from_pool", _decode_head_map_modulo),
}

ATT_PINS = [
    lambda: TA.test_int8_decode_matches_pure_python_brute_force(17, 8, 2, 128),
    lambda: TA.test_single_token_returns_its_value(),
    lambda: TA.test_zero_query_gives_mean_of_values(),
]


@pytest.mark.parametrize("name", sorted(ATT_MUTANTS))
def test_attention_mutant_is_caught(name, monkeypatch):
    attr, fn = ATT_MUTANTS[name]
    monkeypatch.setattr(oatt, attr, fn)
    if attr == "decode_int8_from_pool":
        monkeypatch.setattr(oracle, attr, fn)
    assert _caught(ATT_PINS), name


def test_unmutated_attention_passes_the_same_pins():
    assert not _caught(ATT_PINS)


# ---- static (per-tensor) scales -------------------------------------------
from tests import test_oracle_static as TS  # noqa: E402


def _static(divide=True, exact_quotient=False, round_fn=np.rint, lo=-127):
    def q(x, s):
        s32 = oquant.check_static_scale(s)
        x = oquant.as_f32(x)
        if exact_quotient:
            qq = x.astype(np.float64) / np.float64(s32)
        elif divide:
            qq = np.divide(x, s32, dtype=np.float32)
        else:
            qq = x * (np.float32(1) / s32)
        return np.clip(round_fn(qq), lo, 127).astype(np.int8)
    return q


STATIC_MUTANTS = {
    "reciprocal multiply": _static(divide=False),
    "quotient rounded exactly, not in binary32": _static(exact_quotient=True),
    "round half away from zero": _static(round_fn=lambda v: np.sign(v) * np.floor(np.abs(v) + 0.5)),
    "truncation": _static(round_fn=np.trunc),
    "-128 allowed": _static(lo=-128),
    "multiply by the scale": lambda x, s: np.clip(np.rint(oquant.as_f32(x) * np.float32(s)),
                                                  -127, 127).astype(np.int8),
}

STATIC_PINS = [
    lambda: TS.test_worked_examples(read_golden),
    lambda: TS.test_codes_match_exact_rational_brute_force("f16", 0.0371),
    lambda: TS.test_saturation_and_no_minus_128(),
]


@pytest.mark.parametrize("name", sorted(STATIC_MUTANTS))
def test_static_quantizer_mutant_is_caught(name, monkeypatch):
    monkeypatch.setattr(oracle, "quantize_static", STATIC_MUTANTS[name])
    assert _caught(STATIC_PINS), name


def test_unmutated_static_quantizer_passes_the_same_pins():
    assert not _caught(STATIC_PINS)


def _dequant_static_v_uses_k_scale():
    calls = []

    def f(codes, s):
        calls.append(s)
        return codes.astype(np.float64) * float(oquant.check_static_scale(calls[0]))
    return f


STATIC_ATT_MUTANTS = {
    "V dequantized with the K scale": ("dequantize_static", _dequant_static_v_uses_k_scale),
    "static V layout token-major": ("_v_index", lambda: _v_index_token_major),
    "shared scale = min": ("shared_static_scale", lambda: lambda k, v: np.float32(min(k, v))),
}

STATIC_ATT_PINS = [
    lambda: TS.test_static_decode_matches_pure_python_brute_force(33, 8, 2, 128),
    lambda: TS.test_static_decode_closed_forms(),
    lambda: TS.test_static_byte_offsets_by_hand(),
    lambda: TS.test_scale_validity_and_shared_scale(),
]


@pytest.mark.parametrize("name", sorted(STATIC_ATT_MUTANTS))
def test_static_attention_mutant_is_caught(name, monkeypatch):
    attr, make = STATIC_ATT_MUTANTS[name]
    fn = make()
    for mod in (oatt, oquant, opages, oracle):
        if hasattr(mod, attr):
            monkeypatch.setattr(mod, attr, fn)
    assert _caught(STATIC_ATT_PINS), name


def test_unmutated_static_attention_passes_the_same_pins():
    assert not _caught(STATIC_ATT_PINS)


# ---- multi-token query ----------------------------------------------------
from tests import test_oracle_multi as TM  # noqa: E402


def _multi(visible):
    """decode_multi_from_pool with the number of visible positions of query
    token j given by visible(L, T, j)."""
    def f(kind, pool, block_tables, context_lens, q, sm_scale, block_size, num_kv_heads,
          head_dim, kv_dtype=None, k_scale=None, v_scale=None, triples=None):
        qf = oquant.as_f32(q)
        B, T, hq, d = qf.shape
        g = hq // num_kv_heads
        out = np.zeros((B, T, hq, d))
        for b in range(B):
            L = int(context_lens[b])
            k, v = oatt._sequence_kv(kind, pool, block_tables[b], L, block_size, num_kv_heads,
                                     head_dim, list(range(num_kv_heads)), kv_dtype, k_scale,
                                     v_scale)
            for j in range(T):
                n = min(L, visible(L, T, j))
                for h in range(hq):
                    if n > 0:
                        out[b, j, h] = oatt.attend_one_sequence(
                            qf[b, j, h][None], k[:n, h // g:h // g + 1],
                            v[:n, h // g:h // g + 1], sm_scale)[0]
        return out
    return f


MULTI_MUTANTS = {
    "no causal mask among the new tokens": _multi(lambda L, T, j: L),
    "causal limit one short": _multi(lambda L, T, j: L - T + j),
    "query tokens in reverse order": _multi(lambda L, T, j: L - j),
}

MULTI_PINS = [
    lambda: TM.test_multi_matches_pure_python_brute_force("int8", 3, 8, 2, 64),
    lambda: TM.test_one_visible_position_and_tokens_before_the_start(),
]


@pytest.mark.parametrize("name", sorted(MULTI_MUTANTS))
def test_multi_mutant_is_caught(name, monkeypatch):
    monkeypatch.setattr(oracle, "decode_multi_from_pool", MULTI_MUTANTS[name])
    assert _caught(MULTI_PINS), name


def test_unmutated_multi_passes_the_same_pins():
    assert not _caught(MULTI_PINS)


# ---- page lifecycle -----------------------------------------------------------
import oracle.lifecycle as olife  # noqa: E402
from tests import test_oracle_lifecycle as TL  # noqa: E402


def _trim(mode):
    real = olife.trim_keep_sink

    def f(kv_format, pool, block_tables, context_lens, trim_lens, keep, block_size,
          num_kv_heads, head_dim):
        if mode == "oldest":       # drops the n oldest tokens (ignores the sink)
            return real(kv_format, pool, block_tables, context_lens, trim_lens, 0, block_size,
                        num_kv_heads, head_dim)
        if mode == "one_less":     # drops one token fewer
            return real(kv_format, pool, block_tables, context_lens,
                        [max(int(t) - 1, 0) for t in trim_lens], keep, block_size, num_kv_heads,
                        head_dim) - np.where(np.asarray(trim_lens) > 0, 1, 0).astype(np.int32)
        raise ValueError(mode)
    return f


def _index_codes_only(kv_format, block_size, head_dim, num_kv_heads, page_len, blk, pos, head):
    """Byte index of a token without its scales (scales left behind)."""
    full = _ORIG_INDEX(kv_format, block_size, head_dim, num_kv_heads, page_len, blk, pos, head)
    return full[:, :2 * head_dim] if kv_format == oracle.KV_INT8_SYM else full


_ORIG_INDEX = olife._token_byte_index

LIFE_MUTANTS = {
    "trim drops the oldest tokens": ("trim_keep_sink", _trim("oldest")),
    "trim drops one token fewer": ("trim_keep_sink", _trim("one_less")),
    "scales do not move with their codes": ("_token_byte_index", _index_codes_only),
    "swap-out ignores the id order": ("swap_out_pages",
                                      lambda pool, ids: _ORIG_SWAP(pool, np.sort(ids))),
}
_ORIG_SWAP = olife.swap_out_pages

LIFE_PINS = [
    lambda: TL.test_trim_keeps_the_sink_and_the_tail("int8"),
    lambda: TL.test_trim_byte_positions_by_hand(),
    lambda: TL.test_swap_round_trip_and_relocation(),
]


@pytest.mark.parametrize("name", sorted(LIFE_MUTANTS))
def test_lifecycle_mutant_is_caught(name, monkeypatch):
    attr, fn = LIFE_MUTANTS[name]
    monkeypatch.setattr(olife, attr, fn)
    if hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, fn)
    assert _caught(LIFE_PINS), name


def test_unmutated_lifecycle_passes_the_same_pins():
    assert not _caught(LIFE_PINS)
