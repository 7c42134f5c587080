"""GPU parity over seeded random shapes: KV-head counts 1-8, GQA ratios 1-16
(MHA included), head_dim 64 and 128, fp16 and bf16 inputs, the three value
distributions, ragged context lengths with empty sequences and exact page
multiples, shuffled pages and spare pages, for INT8 and 16-bit pools. Each
case writes the pool through the library (bit-exact with the oracle's pool)
and decodes it (within 2e-3 of the oracle's decode over its own pool)."""

import numpy as np
import pytest

import oracle
from tests.gpu_util import (MAX_ABS_TOL, gpu_decode, gpu_pool, oracle_decode, oracle_pool,
                            require_gpu)
from workloads import build

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    return require_gpu()


def _case(i):
    rng = np.random.default_rng(4000 + i)
    hkv = int(rng.choice([1, 2, 3, 4, 8]))
    g = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 16]))
    d = int(rng.choice([64, 128]))
    dt = str(rng.choice(["f16", "bf16"]))
    values = str(rng.choice(["outlier", "logmag", "normal"]))
    B = int(rng.integers(1, 11))
    ctx = rng.integers(1, 700, B)
    ctx[rng.random(B) < 0.15] = 0
    pm = rng.random(B) < 0.2
    ctx[pm] = 16 * rng.integers(1, 40, int(pm.sum()))
    if ctx.sum() == 0:
        ctx[0] = 1
    return dict(hq=g * hkv, hkv=hkv, d=d, dt=dt, values=values, ctx=ctx.tolist(),
                spare=int(rng.integers(0, 5)), seed=4000 + i)


@pytest.mark.parametrize("fmt_name", ["int8", "16bit"])
@pytest.mark.parametrize("i", range(12))
def test_random_shape(P, i, fmt_name):
    c = _case(i)
    print(f"random shape {i} {fmt_name}: {c}", flush=True)
    wl = build(f"rand{i}", c["seed"], [("prefill", c["ctx"])], c["hq"], c["hkv"], c["d"],
               c["dt"], c["values"], shuffle=True, spare_blocks=c["spare"])
    fmt = P.KV_INT8_SYM if fmt_name == "int8" else P.KV_16BIT
    ofmt = oracle.KV_INT8_SYM if fmt_name == "int8" else oracle.KV_16BIT
    pool, _ = gpu_pool(P, wl, fmt)
    host = oracle_pool(wl, ofmt)
    assert np.array_equal(pool.cpu().numpy(), host), "pool differs from the oracle's"
    out = gpu_decode(P, wl, pool, fmt).cpu().numpy().astype(np.float64)
    want = oracle_decode(wl, host, ofmt)
    empty = np.asarray(c["ctx"]) == 0
    assert np.all(out[empty] == 0)
    d = float(np.max(np.abs(out[~empty] - want[~empty])))
    print(f"  max abs diff {d:.3e}", flush=True)
    assert d <= MAX_ABS_TOL
