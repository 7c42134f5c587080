"""GPU parity of the page lifecycle operations: page swap-out / swap-in
(device and pinned host memory on the far side) and the front trim that
keeps sink tokens, for the three page formats, against the oracle byte for
byte, and decodes over the results against the oracle's decode."""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import (FILL, MAX_ABS_TOL, dev_i32, gpu_decode, gpu_pool, oracle_decode,
                            oracle_pool, oracle_static_pool, require_gpu)
from workloads import build, make_config

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    return require_gpu()


def _say(msg):
    print(msg, flush=True)


def _pool(P, wl, kind):
    """(library format, oracle format, device pool, host pool): the pool is
    built by the oracle on the host and copied to the device, so the
    lifecycle kernels and the oracle start from the same bytes."""
    if kind == "int8":
        fmt, ofmt, host = P.KV_INT8_SYM, oracle.KV_INT8_SYM, oracle_pool(wl, oracle.KV_INT8_SYM)
    elif kind == "static":
        fmt, ofmt = P.KV_INT8_STATIC, oracle.KV_INT8_STATIC
        host = oracle_static_pool(wl, 0.05, 0.05)
    else:
        fmt, ofmt, host = P.KV_16BIT, oracle.KV_16BIT, oracle_pool(wl, oracle.KV_16BIT)
    return fmt, ofmt, torch.from_numpy(host).cuda(), host.copy()


@pytest.mark.parametrize("to_host", [False, True])
def test_swap_out_and_in(P, to_host):
    wl = make_config(3, 0.05)
    _, _, pool, host_ref = _pool(P, wl, "int8")
    rng = np.random.default_rng(0)
    ids = rng.permutation(wl.num_blocks)[:9].astype(np.int32)
    ids_bad = np.concatenate([ids[:4], [-1, wl.num_blocks], ids[4:]]).astype(np.int32)
    pb = pool.shape[1]
    dst = torch.full((len(ids_bad), pb), FILL, dtype=torch.uint8,
                     device="cpu" if to_host else "cuda", pin_memory=to_host)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    P.kv_pages_swap_out(pool, wl.num_blocks, dev_i32(ids_bad), dst, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == P.EFLAG_BLOCK_RANGE
    got = dst.cpu().numpy()
    want = oracle.swap_out_pages(host_ref, ids_bad)
    ok = (ids_bad >= 0) & (ids_bad < wl.num_blocks)
    assert np.array_equal(got[ok], want[ok])
    assert np.all(got[~ok] == FILL)  # entries of bad ids are left as they were
    # swap the valid pages back in to free pages, remap, decode: same rows, bitwise
    before = gpu_decode(P, wl, pool, P.KV_INT8_SYM)
    torch.cuda.synchronize()
    pages = dst[torch.from_numpy(np.nonzero(ok)[0])].contiguous()
    if to_host:
        pages = pages.pin_memory()
    extra = torch.full((len(ids), pb), 0, dtype=torch.uint8, device="cuda")
    big = torch.cat([pool, extra])  # room for the relocated pages
    new_ids = np.arange(wl.num_blocks, wl.num_blocks + len(ids), dtype=np.int32)
    P.kv_pages_swap_in(pages, dev_i32(new_ids), big, big.shape[0])
    bt = wl.block_tables.copy()
    for old, new in zip(ids, new_ids):
        bt[bt == old] = new
    after = gpu_decode(P, wl, big, P.KV_INT8_SYM, block_tables=bt)
    torch.cuda.synchronize()
    assert torch.equal(before, after)


KINDS = ["int8", "static", "16bit"]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("keep", [0, 4])
def test_trim_keep_sink_matches_oracle(P, kind, keep):
    """Trims below a round of 128 tokens (one workgroup walks the sequence),
    of 128 and more (windows of 128 residues mod n, several rounds each, n not
    a multiple of 4), page-aligned, clamped, and zero, over shuffled pages;
    the pool after the trim is the oracle's byte for byte."""
    lens = [700, 300, 40, 3, 129, 1030, 2000, 1000, 700]
    trims = [100, 3, 999, 1, 16, 777, 301, 128, 130]
    wl = build("trim", 31 + keep, [("prefill", lens)], 8, 2, 128 if kind != "static" else 64,
               "f16", "outlier", shuffle=True, spare_blocks=2)
    fmt, ofmt, pool, host = _pool(P, wl, kind)
    new = torch.zeros(len(lens), dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    _say(f"trim {kind} keep {keep}")
    P.kv_trim_keep_sink(fmt, pool, wl.num_blocks, wl.num_kv_heads, wl.head_dim,
                        dev_i32(wl.block_tables), dev_i32(wl.context_lens), dev_i32(trims), keep,
                        new, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    want_lens = oracle.trim_keep_sink(ofmt, host, wl.block_tables, wl.context_lens, trims, keep,
                                      16, wl.num_kv_heads, wl.head_dim)
    assert new.cpu().numpy().tolist() == want_lens.tolist()
    assert np.array_equal(pool.cpu().numpy(), host)


@pytest.mark.parametrize("kind", ["int8", "16bit"])
def test_trim_many_sequences(P, kind):
    """1024 (sequence, KV head) pairs: the launch runs one workgroup per pair,
    which then walks every window of a large trim in turn; mixed small and
    large trims, random lengths."""
    rng = np.random.default_rng(77)
    lens = rng.integers(1, 900, size=128).tolist()
    trims = rng.integers(0, 1000, size=128).astype(np.int32)
    wl = build("trim-many", 78, [("prefill", lens)], 8, 8, 64, "f16", "normal", shuffle=True,
               spare_blocks=1)
    fmt, ofmt, pool, host = _pool(P, wl, kind)
    new = torch.zeros(len(lens), dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    _say(f"trim many sequences {kind}")
    P.kv_trim_keep_sink(fmt, pool, wl.num_blocks, wl.num_kv_heads, wl.head_dim,
                        dev_i32(wl.block_tables), dev_i32(wl.context_lens), dev_i32(trims), 4,
                        new, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    want_lens = oracle.trim_keep_sink(ofmt, host, wl.block_tables, wl.context_lens, trims, 4,
                                      16, wl.num_kv_heads, wl.head_dim)
    assert new.cpu().numpy().tolist() == want_lens.tolist()
    assert np.array_equal(pool.cpu().numpy(), host)


def test_decode_after_trim(P):
    wl = make_config(3, 0.1)
    pool, _ = gpu_pool(P, wl, P.KV_INT8_SYM)
    host = oracle_pool(wl, oracle.KV_INT8_SYM)
    trims = (np.arange(wl.num_seqs) * 37 % 300).astype(np.int32)
    new = torch.zeros(wl.num_seqs, dtype=torch.int32, device="cuda")
    P.kv_trim_keep_sink(P.KV_INT8_SYM, pool, wl.num_blocks, wl.num_kv_heads, wl.head_dim,
                        dev_i32(wl.block_tables), dev_i32(wl.context_lens), dev_i32(trims), 4,
                        new)
    new_lens = oracle.trim_keep_sink(oracle.KV_INT8_SYM, host, wl.block_tables, wl.context_lens,
                                     trims, 4, 16, wl.num_kv_heads, wl.head_dim)
    torch.cuda.synchronize()
    assert new.cpu().numpy().tolist() == new_lens.tolist()
    out = gpu_decode(P, wl, pool, P.KV_INT8_SYM, context_lens=new_lens)
    wl.context_lens = new_lens
    want = oracle_decode(wl, host, oracle.KV_INT8_SYM)
    d = float(np.max(np.abs(out.cpu().numpy().astype(np.float64) - want)))
    _say(f"decode after trim: max abs diff {d:.3e}")
    assert d <= MAX_ABS_TOL


def test_trim_flags_a_missing_page(P):
    """A block id outside the pool in the moved range is flagged; the tokens
    on it are not moved and nothing else faults."""
    wl = build("trim-bad", 8, [("prefill", [90])], 8, 2, 64, "f16", "normal", spare_blocks=1)
    pool, _ = gpu_pool(P, wl, P.KV_16BIT)
    bt = wl.block_tables.copy()
    bt[0, 3] = wl.num_blocks + 5
    new = torch.zeros(1, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    P.kv_trim_keep_sink(P.KV_16BIT, pool, wl.num_blocks, 2, 64, dev_i32(bt),
                        dev_i32(wl.context_lens), dev_i32([10]), 4, new, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == P.EFLAG_BLOCK_RANGE
    assert int(new.item()) == 80


def test_trim_flags_a_missing_page_large_trim(P):
    """The same with a trim above 128 tokens (several windows): the missing
    page is flagged and the new length is still the clamped one."""
    wl = build("trim-bad-wide", 9, [("prefill", [900])], 8, 2, 64, "f16", "normal",
               spare_blocks=1)
    pool, _ = gpu_pool(P, wl, P.KV_INT8_SYM)
    bt = wl.block_tables.copy()
    bt[0, 40] = -1
    new = torch.zeros(1, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    P.kv_trim_keep_sink(P.KV_INT8_SYM, pool, wl.num_blocks, 2, 64, dev_i32(bt),
                        dev_i32(wl.context_lens), dev_i32([300]), 4, new, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == P.EFLAG_BLOCK_RANGE
    assert int(new.item()) == 600


@pytest.mark.slow
def test_trim_full_size_sampled(P):
    """The batched step's full pool (64 sequences, 1K-8K tokens, 8 KV heads,
    written by the library) trimmed as the bench times it (1,024 tokens after
    4 sinks, every sequence), then trimmed again by seeded amounts from 0 to
    3,000 on the new lengths. For sampled sequences every kept token's codes
    and scales, all heads, equal the oracle's quantization of the source
    rows at the positions the two trims leave them."""
    wl = make_config(3)
    _say(f"full-size trim: {wl.num_seqs} seqs, max ctx {wl.max_context_len}")
    pool, _ = gpu_pool(P, wl, P.KV_INT8_SYM)
    keep = 4
    first = np.full(wl.num_seqs, 1024, dtype=np.int32)
    second = np.random.default_rng(12).integers(0, 3001, size=wl.num_seqs).astype(np.int32)
    lens0 = wl.context_lens.astype(np.int64)
    mid = torch.zeros(wl.num_seqs, dtype=torch.int32, device="cuda")
    end = torch.zeros(wl.num_seqs, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    bt = dev_i32(wl.block_tables)
    P.kv_trim_keep_sink(P.KV_INT8_SYM, pool, wl.num_blocks, wl.num_kv_heads, wl.head_dim, bt,
                        dev_i32(wl.context_lens), dev_i32(first), keep, mid, err_flag=err)
    P.kv_trim_keep_sink(P.KV_INT8_SYM, pool, wl.num_blocks, wl.num_kv_heads, wl.head_dim, bt,
                        mid, dev_i32(second), keep, end, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0

    def kept(L, n):  # positions a trim keeps, in order (the trim's definition)
        n = min(max(int(n), 0), max(L - keep, 0))
        return np.concatenate([np.arange(min(keep, L)), np.arange(keep + n, L)]).astype(np.int64)

    host = pool.cpu().numpy()
    got_end = end.cpu().numpy()
    for b in np.random.default_rng(13).choice(wl.num_seqs, 6, replace=False):
        L = int(lens0[b])
        idx1 = kept(L, first[b])
        idx = idx1[kept(len(idx1), second[b])]
        assert int(got_end[b]) == len(idx)
        k, v = wl.tokens_of_seq(int(b))
        kc, ks = oracle.quantize_rows(k)
        vc, vs = oracle.quantize_rows(v)
        gk, gks, gv, gvs = oracle.gather_int8_sequence(host, wl.block_tables[b], len(idx), 16,
                                                       wl.num_kv_heads, wl.head_dim)
        assert np.array_equal(gk, kc[idx]) and np.array_equal(gv, vc[idx])
        assert np.array_equal(gks.view(np.uint16), ks[idx].view(np.uint16))
        assert np.array_equal(gvs.view(np.uint16), vs[idx].view(np.uint16))
        _say(f"  seq {b}: {L} -> {len(idx)} tokens, codes and scales exact")
