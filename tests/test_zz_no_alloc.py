"""GPU check of paged_attn_decode_int8_noalloc, the decode entry point that
allocates nothing (its workspace is the library's per-GPU scratch): called
through the C ABI twice in a row -- the batched step (64 sequences, contexts
1K-8K, shuffled pages), then a smaller input -- each output equals, bit for
bit, that of paged_attn_decode_int8 with a workspace of its own on the same
inputs, and is within the 2e-3 bound of the oracle."""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import (MAX_ABS_TOL, dev_i32, gpu_decode, gpu_pool, oracle_decode,
                            oracle_pool, require_gpu, to_dev)
from workloads import make_config

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    return require_gpu()


def _noalloc(P, wl, pool):
    out = torch.full((wl.num_seqs, wl.num_q_heads, wl.head_dim), float("nan"),
                     dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    P.paged_attn_decode_int8_noalloc(out, to_dev(wl.q), pool, wl.num_blocks,
                                     dev_i32(wl.block_tables), dev_i32(wl.context_lens),
                                     wl.num_kv_heads, wl.max_context_len, wl.sm_scale,
                                     err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return out


def test_noalloc_decode_equals_the_workspace_call_twice_in_a_row(P):
    big = make_config(3)        # 64 sequences: ~2.8 MB of scratch
    small = make_config(3, 0.05)  # 3 sequences: the second call uses less of it
    for wl, with_oracle in ((big, False), (small, True)):
        need = P.pdakv_decode_workspace_bytes(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads,
                                              wl.head_dim, wl.max_context_len)
        print(f"noalloc decode: {wl.name} B {wl.num_seqs}, workspace {need} bytes", flush=True)
        assert 0 < need <= P.NOALLOC_SCRATCH_BYTES
        pool, _ = gpu_pool(P, wl, P.KV_INT8_SYM)
        got = _noalloc(P, wl, pool)
        want = gpu_decode(P, wl, pool, P.KV_INT8_SYM)
        assert torch.equal(got, want)
        if with_oracle:
            ref = oracle_decode(wl, oracle_pool(wl, oracle.KV_INT8_SYM), oracle.KV_INT8_SYM)
            d = float(np.max(np.abs(got.cpu().numpy().astype(np.float64) - ref)))
            assert d <= MAX_ABS_TOL
        del pool
        torch.cuda.empty_cache()


def test_noalloc_rejects_a_call_beyond_the_scratch(P):
    """A shape whose workspace exceeds the scratch is refused before any
    launch; nothing is written."""
    B, hq, hkv, d, L = 512, 32, 8, 128, 32768
    assert P.pdakv_decode_workspace_bytes(B, hq, hkv, d, L) > P.NOALLOC_SCRATCH_BYTES
    out = torch.full((B, hq, d), 7.0, device="cuda")
    q = torch.zeros((B, hq, d), dtype=torch.float16, device="cuda")
    pool = torch.zeros((1, P.pdakv_page_bytes(P.KV_INT8_SYM, 16, hkv, d)), dtype=torch.uint8,
                       device="cuda")
    bt = torch.zeros((B, L // 16), dtype=torch.int32, device="cuda")
    ctx = torch.ones(B, dtype=torch.int32, device="cuda")
    with pytest.raises(P.PdakvError) as e:
        P.paged_attn_decode_int8_noalloc(out, q, pool, 1, bt, ctx, hkv, L, 0.088)
    assert e.value.status == P.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
