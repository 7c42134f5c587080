"""Device-memory helpers: KV pools and decode workspaces as torch tensors.

PyTorch only provides the allocation here; the sizes come from the library
(``pdakv_page_bytes``, ``pdakv_decode_workspace_bytes``).
"""

from __future__ import annotations

from dataclasses import dataclass

import torch

from ._lib import (pdakv_decode_multi_workspace_bytes, pdakv_decode_workspace_bytes,
                   pdakv_page_bytes)


def alloc_pool(kv_format: int, num_blocks: int, num_kv_heads: int, head_dim: int,
               block_size: int = 16, device="cuda") -> torch.Tensor:
    """uint8 [num_blocks, page_bytes] pool (torch allocations are 256-B aligned)."""
    pb = pdakv_page_bytes(kv_format, block_size, num_kv_heads, head_dim)
    if pb == 0:
        raise ValueError("unsupported page shape")
    return torch.empty((num_blocks, pb), dtype=torch.uint8, device=device)


def alloc_workspace(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                    max_context_len: int, device="cuda"):
    """Scratch for the split merge, or None when the plan needs none. One
    workspace serves any number of non-overlapping calls of up to this size."""
    nbytes = pdakv_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                          max_context_len)
    if nbytes == 0:
        return None
    return torch.empty(nbytes // 4, dtype=torch.float32, device=device)


def alloc_multi_workspace(num_seqs: int, num_query_tokens: int, num_q_heads: int,
                          num_kv_heads: int, head_dim: int, max_context_len: int,
                          device="cuda"):
    """Scratch of the several-query-token decode calls (None when none is needed)."""
    nbytes = pdakv_decode_multi_workspace_bytes(num_seqs, num_query_tokens, num_q_heads,
                                                num_kv_heads, head_dim, max_context_len)
    if nbytes == 0:
        return None
    return torch.empty(nbytes // 4, dtype=torch.float32, device=device)


@dataclass
class DecodeBuffers:
    """Output and workspace for repeated decode calls of one shape."""
    out: torch.Tensor
    workspace: torch.Tensor | None

    @classmethod
    def make(cls, num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
             out_dtype=torch.float32, device="cuda"):
        out = torch.empty((num_seqs, num_q_heads, head_dim), dtype=out_dtype, device=device)
        ws = alloc_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                             device)
        return cls(out, ws)
