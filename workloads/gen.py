"""Workload builder: seeded K/V/Q values, write phases, block tables.

A workload is a batch of sequences. Each sequence receives its tokens in
*write phases* (for example: an untimed prefill, then one appended decode
token); after all phases the decode step attends over every written token.
Per phase, the tokens of all sequences are concatenated sequence-major into
one [T, Hkv, D] source tensor with a slot for each token.

Value modes
-----------
``outlier``  N(0,1); per (tensor, head) 4 channels, drawn once and fixed across
             tokens and sequences, are multiplied by 20.
``logmag``   every K row and every V row (per sequence and token, shared by the
             KV heads) is m * N(0,1) with m = 10**U(-3, 1); the query of a
             sequence is scaled the same way with its own m.
``normal``   N(0,1).

Draw order for seed s (rng = default_rng(s)):
  1. outlier channels: K heads, then V heads, then Q heads (``outlier`` only)
  2. zero-token positions, sequence by sequence (when requested)
  3. the block permutation (when shuffled)
  4. per sequence, per phase: K values [n, Hkv, D], then V values, then (for
     ``logmag``) the K magnitudes [n] and V magnitudes [n]
  5. the query [B, Hq, D] (and ``logmag`` query magnitudes [B]), unless the
     query comes from a fused QKV buffer, in which case the Q columns of every
     phase are drawn together with K and V (step 4 draws the whole fused row)
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

_TORCH = {"f16": torch.float16, "bf16": torch.bfloat16}


@dataclass
class WritePhase:
    name: str
    k: torch.Tensor          # [T, Hkv, D] fp16/bf16, possibly a strided view
    v: torch.Tensor          # [T, Hkv, D]
    slot_mapping: np.ndarray  # [T] int32
    counts: np.ndarray        # [B] tokens each sequence receives in this phase
    first_pos: np.ndarray     # [B] position of each sequence's first token

    def seq_rows(self, b: int) -> slice:
        """Rows of sequence b inside this phase's [T, ...] sources."""
        start = int(self.counts[:b].sum())
        return slice(start, start + int(self.counts[b]))


@dataclass
class Workload:
    name: str
    seed: int
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    kv_dtype: str             # "f16" or "bf16" (q, K and V share it)
    q: torch.Tensor           # [B, Hq, D], possibly a strided view
    phases: list = field(default_factory=list)
    block_tables: np.ndarray = None   # [B, max_blocks] int32
    context_lens: np.ndarray = None   # [B] int32 (decode context)
    num_blocks: int = 0
    sm_scale: float = 0.0
    zero_tokens: dict = field(default_factory=dict)  # seq -> positions

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if len(self.context_lens) else 0

    def phase(self, name: str) -> WritePhase:
        for p in self.phases:
            if p.name == name:
                return p
        raise KeyError(name)

    def tokens_of_seq(self, b: int):
        """K, V [L_b, Hkv, D] of sequence b in position order (host tensors)."""
        ks = [p.k[p.seq_rows(b)] for p in self.phases]
        vs = [p.v[p.seq_rows(b)] for p in self.phases]
        return torch.cat(ks), torch.cat(vs)


def _cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(_TORCH[dtype])


def build(name: str, seed: int, phase_tokens: list, num_q_heads: int,
          num_kv_heads: int, head_dim: int, kv_dtype: str, values: str,
          block_size: int = 16, shuffle: bool = False,
          zero_tokens: tuple | None = None, fused_qkv: bool = False,
          spare_blocks: int = 0) -> Workload:
    """Build a workload.

    phase_tokens: list of (phase_name, per-seq token counts [B]); all phases
        must give every sequence the same count except the first.
    zero_tokens: (phase_name, count) — that many seeded positions per sequence
        inside that phase have all-zero K and V rows (all heads).
    fused_qkv: K and V sources are strided views of a fused [T, Hq+2*Hkv, D]
        buffer (token stride (Hq+2*Hkv)*D elements), and the decode query is
        the Q part of the last phase's token.
    """
    rng = np.random.default_rng(seed)
    hq, hkv, d = num_q_heads, num_kv_heads, head_dim
    counts = [np.asarray(c, dtype=np.int64) for _, c in phase_tokens]
    B = len(counts[0])
    ctx = np.sum(counts, axis=0).astype(np.int64)

    # 1. outlier channels
    och = {}
    if values == "outlier":
        och["k"] = [rng.choice(d, 4, replace=False) for _ in range(hkv)]
        och["v"] = [rng.choice(d, 4, replace=False) for _ in range(hkv)]
        och["q"] = [rng.choice(d, 4, replace=False) for _ in range(hq)]

    # 2. zero-token positions (indices inside the named phase)
    zero_idx = {}
    if zero_tokens is not None:
        zname, zcount = zero_tokens
        zphase = [n for n, _ in phase_tokens].index(zname)
        for b in range(B):
            n_b = int(counts[zphase][b])
            zero_idx[b] = np.sort(rng.choice(n_b, zcount, replace=False))

    # 3. block tables
    nblk = [math.ceil(int(c) / block_size) for c in ctx]
    num_blocks = int(sum(nblk)) + spare_blocks
    order = rng.permutation(num_blocks) if shuffle else np.arange(num_blocks)
    max_blocks = max(nblk) if nblk else 0
    bt = np.zeros((B, max(max_blocks, 1)), dtype=np.int32)
    off = 0
    for b in range(B):
        bt[b, :nblk[b]] = order[off:off + nblk[b]]
        off += nblk[b]

    def scale_channels(x, which):
        if values == "outlier":
            for h, chans in enumerate(och[which]):
                x[:, h, chans] *= 20.0
        return x

    # 4. per sequence, per phase values
    width = hq + 2 * hkv
    phases = []
    fused_last_q = None
    for pi, (pname, _) in enumerate(phase_tokens):
        n_seq = counts[pi]
        if pi > 0 and np.any(n_seq != n_seq[0]):
            raise ValueError("only the first phase may have ragged token counts")
        T = int(n_seq.sum())
        if fused_qkv:
            buf = torch.empty((T, width, d), dtype=_TORCH[kv_dtype])
        else:
            kbuf = torch.empty((T, hkv, d), dtype=_TORCH[kv_dtype])
            vbuf = torch.empty((T, hkv, d), dtype=_TORCH[kv_dtype])
        slots = np.empty(T, dtype=np.int32)
        row = 0
        for b in range(B):
            n = int(n_seq[b])
            first = int(np.sum([c[b] for c in counts[:pi]])) if pi else 0
            if fused_qkv:
                x = rng.standard_normal((n, width, d), dtype=np.float32)
                kx, vx = x[:, hq:hq + hkv], x[:, hq + hkv:]
            else:
                kx = rng.standard_normal((n, hkv, d), dtype=np.float32)
                vx = rng.standard_normal((n, hkv, d), dtype=np.float32)
            if values == "logmag":
                mk = 10.0 ** rng.uniform(-3.0, 1.0, n).astype(np.float32)
                mv = 10.0 ** rng.uniform(-3.0, 1.0, n).astype(np.float32)
                kx *= mk[:, None, None]
                vx *= mv[:, None, None]
            scale_channels(kx, "k")
            scale_channels(vx, "v")
            if zero_tokens is not None and pname == zero_tokens[0]:
                kx[zero_idx[b]] = 0.0
                vx[zero_idx[b]] = 0.0
            if fused_qkv:
                buf[row:row + n] = _cast(x, kv_dtype)
            else:
                kbuf[row:row + n] = _cast(kx, kv_dtype)
                vbuf[row:row + n] = _cast(vx, kv_dtype)
            pos = first + np.arange(n)
            slots[row:row + n] = bt[b, pos // block_size] * block_size + pos % block_size
            row += n
        if fused_qkv:
            k_src, v_src = buf[:, hq:hq + hkv, :], buf[:, hq + hkv:, :]
            fused_last_q = buf[:, :hq, :]
        else:
            k_src, v_src = kbuf, vbuf
        first_pos = np.sum(counts[:pi], axis=0) if pi else np.zeros(B, np.int64)
        phases.append(WritePhase(pname, k_src, v_src, slots, n_seq.copy(), first_pos))

    # 5. query
    if fused_qkv:
        last = phases[-1]
        if np.any(last.counts != 1):
            raise ValueError("fused query needs a one-token last phase")
        q = fused_last_q  # [B, Hq, D] strided view (seq stride = width*D)
    else:
        qx = rng.standard_normal((B, hq, d), dtype=np.float32)
        if values == "logmag":
            mq = 10.0 ** rng.uniform(-3.0, 1.0, B).astype(np.float32)
            qx *= mq[:, None, None]
        if values == "outlier":
            for h, chans in enumerate(och["q"]):
                qx[:, h, chans] *= 20.0
        q = _cast(qx, kv_dtype)

    wl = Workload(name=name, seed=seed, num_seqs=B, num_q_heads=hq, num_kv_heads=hkv,
                  head_dim=d, block_size=block_size, kv_dtype=kv_dtype, q=q,
                  phases=phases, block_tables=bt, context_lens=ctx.astype(np.int32),
                  num_blocks=num_blocks, sm_scale=1.0 / math.sqrt(d),
                  zero_tokens={b: v for b, v in zero_idx.items()})
    return wl


CONFIG_NAMES = {
    1: "tiny-L256",
    2: "llama8b-2k-b1",
    3: "llama8b-batched-1k8k-b64",
    4: "llama8b-32k-b8",
    5: "gqa7-d64-chunk4096-b32",
    "s8k": "llama8b-8k-b8",
}


def make_config(idx, scale: float = 1.0) -> Workload:
    """The five benchmark configurations (+ a supplementary 8K point).

    ``scale`` < 1 shrinks the context lengths (and batch where noted) for
    quick checks; 1.0 gives the full sizes. A shrunk multi-sequence
    configuration keeps at least two sequences.
    """
    def sc(n):
        return max(1, int(round(n * scale)))

    if idx == 1:
        # 1 seq, context 256, GQA 4, fp16 outliers, 2 all-zero tokens,
        # quantize-on-write of all tokens then one decode.
        return build(CONFIG_NAMES[1], 1, [("prefill", [256])], 32, 8, 128, "f16",
                     "outlier", zero_tokens=("prefill", 2))
    if idx == 2:
        return build(CONFIG_NAMES[2], 2, [("prefill", [sc(2048)])], 32, 8, 128, "f16",
                     "outlier")
    if idx == 3:
        rng = np.random.default_rng(1003)  # context lengths: separate stream
        B = max(2, sc(64))
        lens = rng.integers(sc(1024), sc(8192) + 1, size=B)
        return build(CONFIG_NAMES[3], 3, [("prefill", lens), ("append", [1] * B)],
                     32, 8, 128, "f16", "outlier", shuffle=True)
    if idx == 4:
        B = max(2, sc(8))
        return build(CONFIG_NAMES[4], 4, [("prefill", [sc(32768)] * B)], 32, 8, 128,
                     "bf16", "logmag", shuffle=True)
    if idx == 5:
        B = max(2, sc(32))
        chunk = sc(4096)
        nzero = max(1, chunk // 100)
        return build(CONFIG_NAMES[5], 5,
                     [("prefix", [7] * B), ("chunk", [chunk] * B), ("append", [1] * B)],
                     14, 2, 64, "bf16", "normal", shuffle=True,
                     zero_tokens=("chunk", nzero), fused_qkv=True)
    if idx == "s8k":
        B = max(2, sc(8))
        return build(CONFIG_NAMES["s8k"], 6, [("prefill", [sc(8192)] * B)], 32, 8, 128,
                     "f16", "outlier", shuffle=True)
    raise KeyError(idx)


def multi_query(wl: Workload, num_tokens: int, seed: int) -> torch.Tensor:
    """Query rows [B, T, Hq, D] for a decode with T query tokens per sequence
    (the sequence's last T positions): N(0, 1) draws from its own seeded
    generator, in the workload's dtype."""
    rng = np.random.default_rng(seed)
    qx = rng.standard_normal((wl.num_seqs, num_tokens, wl.num_q_heads, wl.head_dim),
                             dtype=np.float32)
    return _cast(qx, wl.kv_dtype)
