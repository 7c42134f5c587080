"""CPU checks of the seeded input generator (shapes, structure, determinism)."""

import numpy as np
import pytest
import torch

from workloads import make_config


@pytest.mark.parametrize("idx,scale", [(1, 1.0), (2, 1.0), (3, 0.05), (4, 0.02), (5, 0.05),
                                       ("s8k", 0.05)])
def test_structure(idx, scale):
    wl = make_config(idx, scale)
    B, bs = wl.num_seqs, wl.block_size
    # every sequence's pages are distinct physical blocks inside the pool
    used = []
    for b in range(B):
        n = -(-int(wl.context_lens[b]) // bs)
        row = wl.block_tables[b, :n]
        assert np.all((row >= 0) & (row < wl.num_blocks))
        used.extend(row.tolist())
    assert len(used) == len(set(used))
    # slots: each written token lands at block_table[pos // bs] * bs + pos % bs
    for p in wl.phases:
        assert p.k.shape == p.v.shape == (len(p.slot_mapping), wl.num_kv_heads, wl.head_dim)
        for b in range(B):
            rows = p.seq_rows(b)
            pos = p.first_pos[b] + np.arange(p.counts[b])
            want = wl.block_tables[b, pos // bs] * bs + pos % bs
            assert np.array_equal(p.slot_mapping[rows], want)
    assert np.array_equal(wl.context_lens, sum(p.counts for p in wl.phases))
    assert wl.q.shape == (B, wl.num_q_heads, wl.head_dim)
    if idx not in (1, 2):
        assert B >= 2  # shrunk batched configurations stay multi-sequence


def test_full_size_shapes_without_values():
    """The full configurations' sizes (values are not drawn here)."""
    import math
    rng = np.random.default_rng(1003)
    lens = rng.integers(1024, 8193, size=64)
    assert lens.min() >= 1024 and lens.max() <= 8192
    # config 5: prefix 7 + chunk 4096 + append 1 -> 4104 tokens, 257 pages;
    # the appended token lands at offset 7 of the last page
    assert math.ceil(4104 / 16) == 257 and 4103 % 16 == 7


def test_tiny_config_has_two_zero_tokens_and_outliers():
    wl = make_config(1)
    k = wl.phases[0].k.float()
    zero_rows = torch.nonzero((k == 0).all(dim=2).all(dim=1)).flatten().tolist()
    assert len(zero_rows) == 2 and zero_rows == sorted(wl.zero_tokens[0].tolist())
    assert k.dtype == torch.float32 and wl.phases[0].k.dtype == torch.float16
    # outlier channels: per KV head, 4 columns with ~20x the spread of the rest
    std = k.std(dim=0)  # [Hkv, D]
    for h in range(8):
        big = (std[h] > 8).sum().item()
        assert big == 4


def test_small_head_config_uses_strided_fused_sources():
    wl = make_config(5, 0.05)
    for p in wl.phases:
        assert p.k.stride() == (1152, 64, 1) and p.v.stride() == (1152, 64, 1)
        assert p.k.dtype == torch.bfloat16
    assert wl.q.stride() == (1152, 64, 1)
    chunk = wl.phase("chunk")
    assert chunk.first_pos[0] == 7 and chunk.slot_mapping[0] % 16 == 7
    zeros = (chunk.k.float() == 0).all(dim=2).all(dim=1)
    assert zeros.sum().item() == wl.num_seqs * max(1, chunk.counts[0] // 100)


def test_deterministic():
    a, b = make_config(3, 0.03), make_config(3, 0.03)
    assert np.array_equal(a.block_tables, b.block_tables)
    assert torch.equal(a.phases[0].k, b.phases[0].k) and torch.equal(a.q, b.q)
