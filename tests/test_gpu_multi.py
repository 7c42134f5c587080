"""GPU parity of the decode with several query tokens per sequence (the last
T positions, causal among them): INT8 and 16-bit pages against the oracle's
multi-token decode over the same pools, across query-column tilings
(T x G from 4 to 32 columns), ragged and short contexts (a query token before
the sequence start gives a zero row), and the equalities with the one-token
decode."""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import MAX_ABS_TOL, dev_i32, gpu_pool, oracle_pool, require_gpu, to_dev
from workloads import build, make_config, multi_query

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    return require_gpu()


def _say(msg):
    print(msg, flush=True)


def _gpu_multi(P, wl, pool, fmt, q, out_dtype=torch.float32):
    B, T, hq, d = q.shape
    out = torch.empty((B, T, hq, d), dtype=out_dtype, device="cuda")
    ws = P.alloc_multi_workspace(B, T, hq, wl.num_kv_heads, d, wl.max_context_len)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    fn = P.paged_attn_decode_int8_multi if fmt == P.KV_INT8_SYM else P.paged_attn_decode_fp16_multi
    fn(out, q, pool, wl.num_blocks, dev_i32(wl.block_tables), dev_i32(wl.context_lens),
       wl.num_kv_heads, wl.max_context_len, wl.sm_scale, ws, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return out


def _oracle_multi(wl, host, fmt_name, q, triples=None):
    kind = "int8" if fmt_name == "int8" else "16bit"
    return oracle.decode_multi_from_pool(kind, host, wl.block_tables, wl.context_lens, q,
                                         wl.sm_scale, wl.block_size, wl.num_kv_heads,
                                         wl.head_dim, kv_dtype=wl.kv_dtype, triples=triples)


def _fmt(P, name):
    return (P.KV_INT8_SYM, oracle.KV_INT8_SYM) if name == "int8" else (P.KV_16BIT,
                                                                       oracle.KV_16BIT)


def _max_diff(out, want):
    got = out.float().cpu().numpy().astype(np.float64)
    m = ~np.isnan(want)
    return float(np.max(np.abs(got[m] - want[m])))


def _check(P, wl, fmt_name, T, seed):
    fmt, ofmt = _fmt(P, fmt_name)
    pool, _ = gpu_pool(P, wl, fmt)
    q = multi_query(wl, T, seed)
    out = _gpu_multi(P, wl, pool, fmt, to_dev(q))
    want = _oracle_multi(wl, oracle_pool(wl, ofmt), fmt_name, q)
    d = _max_diff(out, want)
    _say(f"  max abs diff {d:.3e}")
    assert d <= MAX_ABS_TOL
    return out, pool, q


@pytest.mark.parametrize("fmt_name", ["int8", "16bit"])
@pytest.mark.parametrize("T", [1, 2, 4, 5, 8])
def test_multi_llama_shape(P, fmt_name, T):
    """32 / 8 heads (G = 4): 4 to 32 query columns per KV head (one or two
    tiles), ragged contexts including ones shorter than T."""
    wl = build("multi-llama", 90 + T, [("prefill", [700, 1, 37, 16, 300, 2])], 32, 8, 128,
               "f16", "outlier", shuffle=True, spare_blocks=2)
    _say(f"multi {fmt_name} T={T} lens {wl.context_lens.tolist()}")
    _check(P, wl, fmt_name, T, seed=T)


@pytest.mark.parametrize("fmt_name", ["int8", "16bit"])
@pytest.mark.parametrize("hq,hkv,d,dt,T", [(14, 2, 64, "bf16", 3), (8, 8, 64, "bf16", 16),
                                           (16, 1, 128, "f16", 2), (28, 4, 128, "bf16", 7)])
def test_multi_other_shapes(P, fmt_name, hq, hkv, d, dt, T):
    """G = 7 (21 columns, two tiles), MHA with 16 tokens (one full tile),
    G = 16 (two full tiles), G = 7 with 49 columns (four tiles)."""
    wl = build("multi-shapes", 7 * T + hq, [("prefill", [0, 5, 64, 259, 1030])], hq, hkv, d,
               dt, "normal", shuffle=True, spare_blocks=1)
    _say(f"multi {fmt_name} {hq}/{hkv}/{d} {dt} T={T}")
    out, _, _ = _check(P, wl, fmt_name, T, seed=100 + T)
    assert torch.all(out[0] == 0)  # empty sequence: zero rows


@pytest.mark.parametrize("fmt_name", ["int8", "16bit"])
def test_multi_long_context_many_partials(P, fmt_name):
    """One 20,000-token sequence and a short one, 4 query tokens: each
    16-column unit is split over hundreds of waves, so the merge runs its
    most waves per workgroup and combines them through LDS."""
    wl = build("multi-long", 61, [("prefill", [20000, 40])], 32, 8, 128, "f16", "outlier",
               shuffle=True)
    _say(f"multi {fmt_name} long context")
    _check(P, wl, fmt_name, 4, seed=62)


@pytest.mark.parametrize("fmt_name", ["int8", "16bit"])
def test_multi_many_short_sequences(P, fmt_name):
    """40 sequences of 1 to 60 tokens (1 to 4 pages), 4 query tokens at the
    Llama shape: a wave's items cross several 16-column units, more than the
    two segments a pass holds, so waves run several passes."""
    lens = (np.arange(40) * 37 % 60 + 1).tolist()
    wl = build("multi-short", 63, [("prefill", lens)], 32, 8, 128, "f16", "outlier",
               shuffle=True)
    _say(f"multi {fmt_name} many short sequences")
    _check(P, wl, fmt_name, 4, seed=64)


def test_multi_one_token_equals_the_plain_decode(P):
    wl = make_config(3, 0.05)
    pool, _ = gpu_pool(P, wl, P.KV_INT8_SYM)
    q1 = to_dev(wl.q)
    out = _gpu_multi(P, wl, pool, P.KV_INT8_SYM, q1[:, None].contiguous())
    ref = torch.empty_like(q1, dtype=torch.float32)
    ws = P.alloc_workspace(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                           wl.max_context_len)
    P.paged_attn_decode_int8(ref, q1, pool, wl.num_blocks, dev_i32(wl.block_tables),
                             dev_i32(wl.context_lens), wl.num_kv_heads, wl.max_context_len,
                             wl.sm_scale, ws)
    torch.cuda.synchronize()
    assert torch.equal(out[:, 0], ref)


def test_multi_batched_step_shape(P):
    """The batched step's shape (reduced batch, full-length contexts) with 4
    draft tokens per sequence, in the launch shape of the full step; sampled
    rows against the oracle."""
    wl = make_config(3, 1.0)
    sub = build("multi-batched", 3, [("prefill", wl.context_lens[:6] - 4), ("draft", [4] * 6)],
                32, 8, 128, "f16", "outlier", shuffle=True)
    pool, _ = gpu_pool(P, sub, P.KV_INT8_SYM)
    q = multi_query(sub, 4, seed=7)
    out = _gpu_multi(P, sub, pool, P.KV_INT8_SYM, to_dev(q))
    rng = np.random.default_rng(1)
    triples = [(int(b), int(j), int(h)) for b, j, h in
               zip(rng.integers(0, 6, 24), rng.integers(0, 4, 24), rng.integers(0, 32, 24))]
    want = _oracle_multi(sub, oracle_pool(sub, oracle.KV_INT8_SYM), "int8", q, triples)
    assert _max_diff(out, want) <= MAX_ABS_TOL


@pytest.mark.parametrize("out_dtype", [torch.float16, torch.bfloat16])
def test_multi_16bit_outputs_round_the_fp32_output(P, out_dtype):
    wl = build("multi-out", 5, [("prefill", [90, 400])], 32, 8, 128, "f16", "outlier",
               shuffle=True)
    pool, _ = gpu_pool(P, wl, P.KV_INT8_SYM)
    q = to_dev(multi_query(wl, 3, seed=3))
    ref = _gpu_multi(P, wl, pool, P.KV_INT8_SYM, q)
    low = _gpu_multi(P, wl, pool, P.KV_INT8_SYM, q, out_dtype)
    assert torch.equal(low, ref.to(out_dtype))


@pytest.mark.parametrize("fmt_name", ["int8", "16bit"])
@pytest.mark.parametrize("T", [16, 32, 64, 128])
def test_multi_wide_query_blocks(P, fmt_name, T):
    """Chunked-prefill widths at the Llama shape (G = 4): 64 to 512 query
    columns per KV head, so units hold four 16-column tiles that share every
    page they stream; ragged contexts, some shorter than T (zero rows for
    query tokens before the sequence start)."""
    wl = build("multi-wide", 300 + T, [("prefill", [700, 5, 130, 2 * T + 3, 1100])], 32, 8, 128,
               "f16", "outlier", shuffle=True, spare_blocks=2)
    _say(f"multi wide {fmt_name} T={T} ({T * 4} columns) lens {wl.context_lens.tolist()}")
    out, _, _ = _check(P, wl, fmt_name, T, seed=400 + T)
    assert torch.all(out[1, :T - 5] == 0)  # positions before the start of sequence 1


@pytest.mark.parametrize("fmt_name", ["int8", "16bit"])
@pytest.mark.parametrize("hq,hkv,d,dt", [(32, 8, 128, "f16"), (14, 2, 64, "bf16")])
def test_multi_256_token_chunk(P, fmt_name, hq, hkv, d, dt):
    """A 256-token chunk decoded against the cache it was just written to
    (chunked prefill): each sequence's last 256 positions are the query
    tokens, after prefixes of different lengths (Llama shape: 1,024 columns
    per KV head; small-head GQA 7 at D = 64: 1,792)."""
    T = 256
    wl = build("multi-chunk", 500 + hq, [("prefix", [3000, 40]), ("chunk", [T, T])], hq, hkv, d,
               dt, "outlier" if dt == "f16" else "normal", shuffle=True)
    _say(f"multi chunk {fmt_name} {hq}/{hkv}/{d} {dt}: T={T}, lens {wl.context_lens.tolist()}")
    _check(P, wl, fmt_name, T, seed=600 + hq)
