"""GPU parity of the static-scale INT8 variant (one calibrated scalar scale
for all of K and one for all of V; InfiniLM PR #553 "Summary", TensorRT-LLM
PR #18953 "Summary"): pools written by the library are bit-identical to the
oracle's, and the decode matches the oracle's decode over the same pool
within the FP32-output tolerance, on the benchmark configurations (reduced
sizes) and on edge shapes; the fused append + decode step leaves the same
pool and output as a write followed by a decode."""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import (FILL, MAX_ABS_TOL, calibrated_scales, dev_i32, oracle_static_pool,
                            require_gpu, to_dev)
from workloads import build, make_config

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    return require_gpu()


def _say(msg):
    print(msg, flush=True)


def _gpu_static_pool(P, wl, ks, vs, phases=None):
    pb = P.pdakv_page_bytes(P.KV_INT8_STATIC, wl.block_size, wl.num_kv_heads, wl.head_dim)
    pool = torch.full((wl.num_blocks, pb), FILL, dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    for ph in (wl.phases if phases is None else phases):
        if len(ph.slot_mapping):
            P.kv_quant_int8_static_write(to_dev(ph.k), to_dev(ph.v), dev_i32(ph.slot_mapping),
                                         pool, wl.num_blocks, ks, vs, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return pool


def _gpu_static_decode(P, wl, pool, ks, vs, out_dtype=torch.float32):
    out = torch.empty((wl.num_seqs, wl.num_q_heads, wl.head_dim), dtype=out_dtype,
                      device="cuda")
    ws = P.alloc_workspace(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                           wl.max_context_len)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    P.paged_attn_decode_int8_static(out, to_dev(wl.q), pool, wl.num_blocks,
                                    dev_i32(wl.block_tables), dev_i32(wl.context_lens),
                                    wl.num_kv_heads, wl.max_context_len, wl.sm_scale, ks, vs,
                                    ws, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return out


def _oracle_decode(wl, host, ks, vs, pairs=None):
    return oracle.decode_int8_static_from_pool(host, wl.block_tables, wl.context_lens, wl.q,
                                               wl.sm_scale, ks, vs, wl.block_size,
                                               wl.num_kv_heads, wl.head_dim, pairs=pairs)


def _max_diff(out, want):
    got = out.float().cpu().numpy().astype(np.float64)
    m = ~np.isnan(want)
    return float(np.max(np.abs(got[m] - want[m])))


@pytest.mark.parametrize("idx,scale,shrink", [(1, 1.0, 1.0), (1, 1.0, 8.0), (2, 1.0, 1.0),
                                              (3, 0.05, 1.0), (4, 0.03, 1.0), (4, 0.03, 50.0),
                                              (5, 0.1, 1.0), ("s8k", 0.1, 1.0)])
def test_static_pool_and_decode_match_oracle(P, idx, scale, shrink):
    """shrink > 1: the scales are that much below the calibrated ones, so
    many values saturate at +-127."""
    wl = make_config(idx, scale)
    ks, vs = calibrated_scales(wl, shrink)
    _say(f"static config {idx} scale {scale} shrink {shrink}: ks {ks:.4g} vs {vs:.4g}")
    pool = _gpu_static_pool(P, wl, ks, vs)
    host = oracle_static_pool(wl, ks, vs)
    assert np.array_equal(pool.cpu().numpy(), host), "static pool differs from the oracle's"
    out = _gpu_static_decode(P, wl, pool, ks, vs)
    want = _oracle_decode(wl, host, ks, vs)
    d = _max_diff(out, want)
    _say(f"  max abs diff {d:.3e}")
    assert d <= MAX_ABS_TOL


@pytest.mark.parametrize("hq,hkv,d,dt", [(32, 8, 128, "f16"), (8, 8, 64, "bf16"),
                                         (14, 2, 64, "bf16"), (16, 1, 128, "f16")])
def test_static_edge_lengths(P, hq, hkv, d, dt):
    """Context lengths 0, 1, 15, 16, 17, 33 and a long one in one batch;
    MHA, GQA 4 / 7 / 16, head_dim 64 and 128, fp16 and bf16."""
    wl = build("static-edge", 77, [("prefill", [0, 1, 15, 16, 17, 33, 700])], hq, hkv, d, dt,
               "outlier", shuffle=True, spare_blocks=3)
    ks, vs = calibrated_scales(wl)
    _say(f"static edges {hq}/{hkv}/{d} {dt}")
    pool = _gpu_static_pool(P, wl, ks, vs)
    host = oracle_static_pool(wl, ks, vs)
    assert np.array_equal(pool.cpu().numpy(), host)
    out = _gpu_static_decode(P, wl, pool, ks, vs)
    want = _oracle_decode(wl, host, ks, vs)
    assert _max_diff(out, want) <= MAX_ABS_TOL
    assert torch.all(out[0] == 0)  # empty context -> zero rows


def _static_rows(rng, shape, s, dtype):
    """Values at and one step of the input type beside the half-integer
    multiples k + 1/2 of the scale (k in -130 .. 129, so some saturate),
    mixed with values of random sign spread log-uniformly over a wide range
    around the scale."""
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    n = int(np.prod(shape))
    k = rng.integers(-130, 130, n) + 0.5
    near = torch.from_numpy((k * s).astype(np.float32)).to(tdt)
    bits = near.view(torch.int16).numpy().astype(np.int32)
    bits = np.where(bits == 0, 0, bits + rng.integers(-1, 2, n)).astype(np.int16)
    near = torch.from_numpy(bits).view(tdt).float().numpy()
    lo, hi = (-24.0, 15.9) if dtype == "f16" else (-120.0, 120.0)
    wide = np.exp2(rng.uniform(lo, hi, n)) * rng.choice([-1.0, 1.0], n)
    x = np.where(rng.random(n) < 0.7, near, wide).astype(np.float32)
    x = torch.from_numpy(x).to(tdt).float()
    x[~torch.isfinite(x)] = 0.0
    return x.to(tdt).reshape(shape)


@pytest.mark.parametrize("dtype,ks,vs", [
    ("f16", 0.0390625, 0.0123457), ("bf16", 0.0390625, 3.3e-3),
    ("f16", 2.0 ** -64, 2.0 ** 64), ("bf16", 2.0 ** -64, 2.0 ** 64),
    ("f16", 1e-21, 7e19), ("bf16", 3e-30, 1e25)])
def test_static_codes_beside_ties_and_outside_the_scale_window(P, dtype, ks, vs):
    """Static-scale codes at and beside the ties x = (k + 1/2) s, and for
    scales at the ends of and outside [2^-64, 2^64] (where the writer keeps
    one division per element): bit-exact with the oracle."""
    rng = np.random.default_rng(91)
    T, hkv, d = 1024, 2, 128
    _say(f"static codes: {dtype} ks {ks:.4g} vs {vs:.4g}")
    k = _static_rows(rng, (T, hkv, d), ks, dtype)
    v = _static_rows(rng, (T, hkv, d), vs, dtype)
    nb = T // 16
    slots = rng.permutation(nb * 16).astype(np.int32)[:T]
    pb = P.pdakv_page_bytes(P.KV_INT8_STATIC, 16, hkv, d)
    pool = torch.full((nb, pb), FILL, dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    P.kv_quant_int8_static_write(k.cuda(), v.cuda(), dev_i32(slots), pool, nb, ks, vs,
                                 err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    want = oracle.new_pool(oracle.KV_INT8_STATIC, nb, 16, hkv, d, fill=FILL)
    oracle.write_int8_static_tokens(want, oracle.quantize_static(k, ks),
                                    oracle.quantize_static(v, vs), slots, 16)
    got = pool.cpu().numpy()
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, f"{bad[0].size} bytes differ, first at page {bad[0][0]} byte {bad[1][0]}"


@pytest.mark.parametrize("out_dtype", [torch.float16, torch.bfloat16])
def test_static_16bit_outputs_round_the_fp32_output(P, out_dtype):
    wl = make_config(2, 0.5)
    ks, vs = calibrated_scales(wl)
    pool = _gpu_static_pool(P, wl, ks, vs)
    ref = _gpu_static_decode(P, wl, pool, ks, vs)
    low = _gpu_static_decode(P, wl, pool, ks, vs, out_dtype)
    assert torch.equal(low, ref.to(out_dtype))


def test_static_shared_scale(P):
    """One scale for K and V (the larger of the two calibrated scales)."""
    wl = make_config(3, 0.03)
    ks, vs = calibrated_scales(wl)
    s = float(oracle.shared_static_scale(ks, vs))
    pool = _gpu_static_pool(P, wl, s, s)
    host = oracle_static_pool(wl, s, s)
    assert np.array_equal(pool.cpu().numpy(), host)
    out = _gpu_static_decode(P, wl, pool, s, s)
    assert _max_diff(out, _oracle_decode(wl, host, s, s)) <= MAX_ABS_TOL


@pytest.mark.parametrize("idx,scale", [(3, 0.05), (5, 0.2)])
def test_static_fused_append_matches_write_then_decode(P, idx, scale):
    wl = make_config(idx, scale)
    ks, vs = calibrated_scales(wl)
    last = wl.phases[-1]
    assert np.all(last.counts == 1)
    _say(f"static fused append: config {idx} scale {scale}")
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
    assert np.array_equal(pool.cpu().numpy(), host), "pool after the fused step differs"
    d = _max_diff(out, _oracle_decode(wl, host, ks, vs))
    _say(f"  max abs diff {d:.3e}")
    assert d <= MAX_ABS_TOL
    # the pool it leaves decodes to the same rows with the plain call
    again = _gpu_static_decode(P, wl, pool, ks, vs)
    assert torch.equal(out, again)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_static_non_finite_inputs(P, dtype):
    """Infinities saturate to +-127 and a NaN is stored as -127 (the clamp of
    the division rule ignores a NaN operand), in the static writer and in the
    static fused append alike. The oracle takes finite inputs only, so the
    codes of the non-finite elements are pinned here by hand; the finite ones
    come from the oracle."""
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    hq, hkv, d = 8, 2, 128
    ks, vs = 0.0390625, 0.0123457
    wl = build("nonfinite", 61, [("prefill", [5, 37]), ("append", [1, 1])], hq, hkv, d, dtype,
               "normal", shuffle=True, spare_blocks=1)
    last = wl.phases[-1]
    special = {3: float("inf"), 17: float("-inf"), 40: float("nan"), 99: float("nan")}
    want_code = {3: 127, 17: -127, 40: -127, 99: -127}
    for t in (last.k, last.v):
        for pos, val in special.items():
            t[:, :, pos] = val
    # pinned codes of the new rows: the oracle on the finite elements, then
    # the hand-pinned non-finite ones
    def pinned(x, s):
        clean = x.float().clone()
        clean[~torch.isfinite(clean)] = 0.0
        c = oracle.quantize_static(clean.to(tdt), s).copy()
        for pos, code in want_code.items():
            c[..., pos] = code
        return c
    want_k, want_v = pinned(last.k, ks), pinned(last.v, vs)
    for route in ("writer", "fused"):
        _say(f"static non-finite {dtype}: {route}")
        pool = _gpu_static_pool(P, wl, ks, vs, phases=wl.phases[:-1])
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        if route == "writer":
            P.kv_quant_int8_static_write(to_dev(last.k), to_dev(last.v),
                                         dev_i32(last.slot_mapping), pool, wl.num_blocks, ks, vs,
                                         err_flag=err)
        else:
            out = torch.empty((wl.num_seqs, hq, d), dtype=torch.float32, device="cuda")
            ws = P.alloc_workspace(wl.num_seqs, hq, hkv, d, wl.max_context_len)
            P.paged_attn_decode_int8_static_append(
                out, to_dev(wl.q), to_dev(last.k), to_dev(last.v), pool, wl.num_blocks,
                dev_i32(wl.block_tables), dev_i32(wl.context_lens), hkv, wl.max_context_len,
                wl.sm_scale, ks, vs, ws, err_flag=err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0  # saturation is part of the scheme: nothing flagged
        host = pool.cpu().numpy()
        for b in range(wl.num_seqs):
            L = int(wl.context_lens[b])
            kc, vc = oracle.gather_int8_static_sequence(host, wl.block_tables[b], L, 16, hkv, d)
            assert np.array_equal(kc[L - 1], want_k[b]), (route, b)
            assert np.array_equal(vc[L - 1], want_v[b]), (route, b)
