"""GPU parity of the quantize-on-write kernel (and the 16-bit writer): the
pools written through the C ABI must equal, byte for byte, the pools the CPU
oracle writes from the same seeded inputs (codes and FP16 scales bit-exact;
untouched bytes untouched)."""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import (FILL, bits16, dev_i32, gpu_pool, oracle_pool, require_gpu,
                            to_dev)
from workloads import build, make_config

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    return require_gpu()


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("idx,scale", [(1, 1.0), (2, 1.0), (3, 0.1), (4, 0.05), (5, 1.0),
                                       ("s8k", 0.1)])
def test_int8_pool_bit_exact(P, idx, scale):
    wl = make_config(idx, scale)
    _say(f"int8 write: config {idx} scale {scale} blocks {wl.num_blocks}")
    pool, _ = gpu_pool(P, wl, P.KV_INT8_SYM)
    got = pool.cpu().numpy()
    want = oracle_pool(wl, oracle.KV_INT8_SYM)
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, f"{bad[0].size} bytes differ, first at page {bad[0][0]} byte {bad[1][0]}"


@pytest.mark.parametrize("idx,scale", [(1, 1.0), (4, 0.03), (5, 1.0)])
def test_16bit_pool_exact(P, idx, scale):
    wl = make_config(idx, scale)
    _say(f"16-bit write: config {idx} scale {scale}")
    pool, _ = gpu_pool(P, wl, P.KV_16BIT)
    assert np.array_equal(pool.cpu().numpy(), oracle_pool(wl, oracle.KV_16BIT))


def test_writes_stay_inside_the_pool(P):
    wl = make_config(5, 0.1)
    for fmt in (P.KV_INT8_SYM, P.KV_16BIT):
        _, full = gpu_pool(P, wl, fmt, guard_pages=2)
        f = full.cpu().numpy()
        assert np.all(f[:2] == FILL) and np.all(f[-2:] == FILL)


def test_padding_and_out_of_range_slots(P):
    """slot < 0: skipped silently; slot >= num_blocks*16: skipped and flagged."""
    wl = build("slots", 11, [("prefill", [40])], 8, 2, 128, "f16", "outlier")
    ph = wl.phases[0]
    slots = ph.slot_mapping.copy()
    slots[3] = -1
    slots[7] = wl.num_blocks * 16 + 5
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pool = torch.full((wl.num_blocks, P.pdakv_page_bytes(P.KV_INT8_SYM, 16, 2, 128)), FILL,
                      dtype=torch.uint8, device="cuda")
    P.kv_quant_int8_sym_write(to_dev(ph.k), to_dev(ph.v), dev_i32(slots), pool, wl.num_blocks,
                              err_flag=err)
    assert int(err.item()) == P.EFLAG_SLOT_RANGE
    want = oracle.new_pool(oracle.KV_INT8_SYM, wl.num_blocks, 16, 2, 128, fill=FILL)
    keep = np.ones(len(slots), bool)
    keep[[3, 7]] = False
    kc, ks = oracle.quantize_rows(ph.k)
    vc, vs = oracle.quantize_rows(ph.v)
    oracle.write_int8_tokens(want, kc[keep], ks[keep], vc[keep], vs[keep], slots[keep], 16)
    assert np.array_equal(pool.cpu().numpy(), want)


def test_scale_overflow_is_flagged_and_row_left_unwritten(P):
    k = torch.zeros((2, 1, 64), dtype=torch.bfloat16)
    k[0, 0, 5] = 2.0 ** 24  # absmax / 127 > 65504
    k[1, 0, 3] = 1.5
    v = torch.ones((2, 1, 64), dtype=torch.bfloat16)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pb = P.pdakv_page_bytes(P.KV_INT8_SYM, 16, 1, 64)
    pool = torch.full((1, pb), FILL, dtype=torch.uint8, device="cuda")
    P.kv_quant_int8_sym_write(k.cuda(), v.cuda(), dev_i32([0, 1]), pool, 1, err_flag=err)
    assert int(err.item()) == P.EFLAG_SCALE_RANGE
    got = pool.cpu().numpy()
    want = oracle.new_pool(oracle.KV_INT8_SYM, 1, 16, 1, 64, fill=FILL)
    kc, ks = oracle.quantize_rows(k[1:])
    vc, vs = oracle.quantize_rows(v[1:])
    oracle.write_int8_tokens(want, kc, ks, vc, vs, [1], 16)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_non_finite_rows_are_flagged_and_left_unwritten(P, dtype):
    """A K or V row holding a NaN or an infinity: that (token, KV head) is
    flagged and left unwritten; every other row is written as the oracle
    writes it."""
    rng = np.random.default_rng(5)
    T, hkv, d = 32, 2, 128
    k = torch.from_numpy(rng.standard_normal((T, hkv, d)).astype(np.float32)).to(dtype)
    v = torch.from_numpy(rng.standard_normal((T, hkv, d)).astype(np.float32)).to(dtype)
    k[3, 1, 7] = float("nan")
    k[10, 0, 0] = float("inf")
    v[17, 1, 127] = float("-inf")
    v[25, 0, 64] = float("nan")
    bad = {(3, 1), (10, 0), (17, 1), (25, 0)}
    slots = np.arange(T, dtype=np.int32)
    pb = P.pdakv_page_bytes(P.KV_INT8_SYM, 16, hkv, d)
    pool = torch.full((2, pb), FILL, dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    P.kv_quant_int8_sym_write(k.cuda(), v.cuda(), dev_i32(slots), pool, 2, err_flag=err)
    assert int(err.item()) == P.EFLAG_SCALE_RANGE
    # the oracle writes every row (the bad rows as zeros), then the bytes of
    # the bad (token, head) pairs go back to the fill pattern
    kk, vv = k.float().clone(), v.float().clone()
    for t, h in bad:
        kk[t, h] = 0.0
        vv[t, h] = 0.0
    want = oracle.new_pool(oracle.KV_INT8_SYM, 2, 16, hkv, d, fill=FILL)
    kc, ks = oracle.quantize_rows(kk.numpy())
    vc, vs = oracle.quantize_rows(vv.numpy())
    oracle.write_int8_tokens(want, kc, ks, vc, vs, slots, 16)
    for t, h in bad:
        for idx in oracle.int8_token_bytes(16, hkv, d, h, [t % 16]):
            want[t // 16].reshape(-1)[idx.reshape(-1)] = FILL
    assert np.array_equal(pool.cpu().numpy(), want)


def test_subnormal_and_tie_rows(P):
    """Rows whose scales are FP16 subnormals and rows with exact .5 ties."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal((64, 4, 128)).astype(np.float32)
    x[:16] *= 1e-5                     # subnormal scales
    x[16:32] = np.round(x[16:32] * 20) / 2   # many half-integers
    x[16:32, :, 0] = 127.0             # absmax 127 -> scale 1.0 -> ties at .5
    x[32:34] = 0.0                     # all-zero tokens
    x[34, :, 9] = -0.0
    k = torch.from_numpy(x).half()
    v = torch.from_numpy(x[::-1].copy()).half()
    slots = np.arange(64, dtype=np.int32)[::-1].copy()
    pb = P.pdakv_page_bytes(P.KV_INT8_SYM, 16, 4, 128)
    pool = torch.full((4, pb), FILL, dtype=torch.uint8, device="cuda")
    P.kv_quant_int8_sym_write(k.cuda(), v.cuda(), dev_i32(slots), pool, 4)
    want = oracle.new_pool(oracle.KV_INT8_SYM, 4, 16, 4, 128, fill=FILL)
    kc, ks = oracle.quantize_rows(k)
    vc, vs = oracle.quantize_rows(v)
    oracle.write_int8_tokens(want, kc, ks, vc, vs, slots, 16)
    assert np.array_equal(pool.cpu().numpy(), want)


def _near_tie_rows(rng, n_rows, d, dtype):
    """Rows whose absolute maxima cover the FP16 scale range (subnormal
    scales included) and whose other elements sit on the half-integer
    multiples of the row's scale or one step of the input type beside them:
    the values where a code is decided by the last bit of x / s."""
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    top = 15.9 if dtype == "f16" else 22.9                # scale within FP16
    a = np.exp2(rng.uniform(-22.0, top, n_rows)).astype(np.float32)
    a = torch.from_numpy(a).to(tdt).float().numpy()       # representable maxima
    _, s = oracle.quantize_rows(a[:, None])                # the rows' scales
    s = s.astype(np.float32)
    k = rng.integers(-127, 127, (n_rows, d)) + 0.5
    x = torch.from_numpy((k * s[:, None]).astype(np.float32)).to(tdt)
    bits = x.view(torch.int16).numpy().astype(np.int32)
    step = rng.integers(-1, 2, (n_rows, d))                # below, at, above
    bits = np.where(bits == 0, 0, bits + step).astype(np.int16)
    x = torch.from_numpy(bits).view(tdt).float().numpy()
    x = np.where(np.abs(x) <= a[:, None], x, 0.0).astype(np.float32)
    x[:, 0] = a * np.where(rng.random(n_rows) < 0.5, -1, 1)
    return torch.from_numpy(x).to(tdt)


@pytest.mark.parametrize("dtype,d", [("f16", 128), ("bf16", 128), ("f16", 64)])
def test_codes_beside_ties_every_scale_range(P, dtype, d):
    """Per-token codes at and one step beside every half-integer multiple of
    the row scale, over scales from FP16 subnormals to the top of the FP16 range: bit-exact with
    the oracle's IEEE division."""
    rng = np.random.default_rng(77 if dtype == "f16" else 78)
    T, hkv = 2048, 4
    _say(f"near-tie rows: {dtype} D={d} tokens {T} heads {hkv}")
    k = _near_tie_rows(rng, T * hkv, d, dtype).reshape(T, hkv, d)
    v = _near_tie_rows(rng, T * hkv, d, dtype).reshape(T, hkv, d)
    nb = T // 16
    slots = rng.permutation(nb * 16).astype(np.int32)[:T]
    pb = P.pdakv_page_bytes(P.KV_INT8_SYM, 16, hkv, d)
    pool = torch.full((nb, pb), FILL, dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    P.kv_quant_int8_sym_write(k.cuda(), v.cuda(), dev_i32(slots), pool, nb, err_flag=err)
    assert int(err.item()) == 0
    want = oracle.new_pool(oracle.KV_INT8_SYM, nb, 16, hkv, d, fill=FILL)
    kc, ks = oracle.quantize_rows(k)
    vc, vs = oracle.quantize_rows(v)
    oracle.write_int8_tokens(want, kc, ks, vc, vs, slots, 16)
    got = pool.cpu().numpy()
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, f"{bad[0].size} bytes differ, first at page {bad[0][0]} byte {bad[1][0]}"


def _mixed_slots(rng, num_blocks, runs=18):
    """Runs of consecutive slots (lengths 1..23, any start offset inside a
    page, one of them reversed) in disjoint ranges, with padding and
    out-of-range entries sprinkled in: every way the writer's four-token
    spans can meet a V group."""
    starts = rng.permutation(num_blocks * 16 // 32)[:runs] * 32
    runs = []
    for j, st in enumerate(starts):
        n = int(rng.integers(1, 24))
        run = st + int(rng.integers(0, 8)) + np.arange(n)
        runs.append(run[::-1] if j == 5 else run)
    slots = np.concatenate(runs)
    slots[rng.random(len(slots)) < 0.06] = -1
    slots[rng.random(len(slots)) < 0.03] = num_blocks * 16 + 3
    return slots.astype(np.int32)


@pytest.mark.parametrize("kind", ["int8", "static", "16bit"])
@pytest.mark.parametrize("d,hkv,runs", [(64, 2, 18), (64, 3, 18), (128, 2, 18),
                                        (64, 3, 3000), (128, 2, 3000), (64, 2, 3000),
                                        (64, 6, 400), (128, 1, 400), (128, 3, 3000)])
def test_write_spans_mixed_runs(P, kind, d, hkv, runs):
    """Slot runs of every length and page offset, reversed runs, padding and
    out-of-range slots, token count not a multiple of four, and every lane
    map of the INT8 writers: whole waves of heads (D = 128 with an even head
    count), two quads of four tokens side by side in a wave (two or six heads
    at D = 64, one or three at D = 128) and eight elements per lane (three
    heads at D = 64): the whole pool equals the oracle's writes of the tokens
    with valid slots. 3,000 runs (about 36K tokens) make a call large enough
    for several spans per wave; 18 runs keep one."""
    rng = np.random.default_rng(30 + d + hkv + runs)
    nb = 64 if runs <= 32 else 4 * runs
    slots = _mixed_slots(rng, nb, runs)
    T = len(slots)
    k = torch.from_numpy(rng.standard_normal((T, hkv, d)).astype(np.float32)).half()
    v = torch.from_numpy(rng.standard_normal((T, hkv, d)).astype(np.float32) * 3).half()
    k[1] = 0.0  # an all-zero token
    keep = (slots >= 0) & (slots < nb * 16)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    fmt = {"int8": P.KV_INT8_SYM, "static": P.KV_INT8_STATIC, "16bit": P.KV_16BIT}[kind]
    ofmt = {"int8": oracle.KV_INT8_SYM, "static": oracle.KV_INT8_STATIC,
            "16bit": oracle.KV_16BIT}[kind]
    pool = torch.full((nb, P.pdakv_page_bytes(fmt, 16, hkv, d)), FILL, dtype=torch.uint8,
                      device="cuda")
    want = oracle.new_pool(ofmt, nb, 16, hkv, d, fill=FILL)
    ks, vs = 0.03, 0.07
    _say(f"mixed runs {kind} D={d}: {T} tokens")
    if kind == "int8":
        P.kv_quant_int8_sym_write(k.cuda(), v.cuda(), dev_i32(slots), pool, nb, err_flag=err)
        kc, kss = oracle.quantize_rows(k[keep])
        vc, vss = oracle.quantize_rows(v[keep])
        oracle.write_int8_tokens(want, kc, kss, vc, vss, slots[keep], 16)
    elif kind == "static":
        P.kv_quant_int8_static_write(k.cuda(), v.cuda(), dev_i32(slots), pool, nb, ks, vs,
                                     err_flag=err)
        oracle.write_int8_static_tokens(want, oracle.quantize_static(k[keep], ks),
                                        oracle.quantize_static(v[keep], vs), slots[keep], 16)
    else:
        P.kv_write_16bit(k.cuda(), v.cuda(), dev_i32(slots), pool, nb, err_flag=err)
        oracle.write_16bit_tokens(want, bits16(k[keep]), bits16(v[keep]), slots[keep], 16)
    torch.cuda.synchronize()
    assert int(err.item()) == P.EFLAG_SLOT_RANGE
    got = pool.cpu().numpy()
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, f"{bad[0].size} bytes differ, first at page {bad[0][0]} byte {bad[1][0]}"


@pytest.mark.parametrize("kind", ["int8", "static", "16bit"])
@pytest.mark.parametrize("layout,T", [("dim-major", 200), ("dim-major", 9000),
                                      ("offset", 9000)])
def test_write_element_strided_sources(P, kind, layout, T):
    """K/V sources that need element-by-element loads: views with the head
    dimension not innermost (element stride = number of heads), or
    contiguous rows starting one element past a 16-byte boundary; small
    calls and calls large enough for several spans per wave. Pools
    bit-exact with the oracle's writes of the same values."""
    rng = np.random.default_rng(61 + T)
    hkv, d = 2, 128
    if layout == "dim-major":
        kb = torch.from_numpy(rng.standard_normal((T, d, hkv)).astype(np.float32)).half()
        vb = torch.from_numpy(rng.standard_normal((T, d, hkv)).astype(np.float32) * 2).half()
        k, v = kb.cuda().permute(0, 2, 1), vb.cuda().permute(0, 2, 1)
        assert k.stride(2) == hkv
    else:
        flat_k = torch.from_numpy(rng.standard_normal(T * hkv * d + 1).astype(np.float32)).half()
        flat_v = torch.from_numpy(rng.standard_normal(T * hkv * d + 1).astype(np.float32)).half()
        k = flat_k.cuda()[1:].view(T, hkv, d)
        v = flat_v.cuda()[1:].view(T, hkv, d)
    nb = (T + 15) // 16 + 3
    slots = rng.permutation(nb * 16)[:T].astype(np.int32)
    slots[: T // 2] = np.sort(slots[: T // 2])  # runs of consecutive slots too
    fmt = {"int8": P.KV_INT8_SYM, "static": P.KV_INT8_STATIC, "16bit": P.KV_16BIT}[kind]
    ofmt = {"int8": oracle.KV_INT8_SYM, "static": oracle.KV_INT8_STATIC,
            "16bit": oracle.KV_16BIT}[kind]
    pool = torch.full((nb, P.pdakv_page_bytes(fmt, 16, hkv, d)), FILL, dtype=torch.uint8,
                      device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    _say(f"element-strided {kind} {layout}: {T} tokens")
    kh, vh = k.cpu(), v.cpu()
    want = oracle.new_pool(ofmt, nb, 16, hkv, d, fill=FILL)
    ks, vs = 0.02, 0.05
    if kind == "int8":
        P.kv_quant_int8_sym_write(k, v, dev_i32(slots), pool, nb, err_flag=err)
        kc, kss = oracle.quantize_rows(kh)
        vc, vss = oracle.quantize_rows(vh)
        oracle.write_int8_tokens(want, kc, kss, vc, vss, slots, 16)
    elif kind == "static":
        P.kv_quant_int8_static_write(k, v, dev_i32(slots), pool, nb, ks, vs, err_flag=err)
        oracle.write_int8_static_tokens(want, oracle.quantize_static(kh, ks),
                                        oracle.quantize_static(vh, vs), slots, 16)
    else:
        P.kv_write_16bit(k, v, dev_i32(slots), pool, nb, err_flag=err)
        oracle.write_16bit_tokens(want, bits16(kh), bits16(vh), slots, 16)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    got = pool.cpu().numpy()
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, f"{bad[0].size} bytes differ, first at page {bad[0][0]} byte {bad[1][0]}"
