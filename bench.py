"""Benchmark of the paged INT8-KV decode step on one MI355X.

Default workload: the batched decode step — 64 Llama-3.1-8B-shaped sequences
(32 query / 8 KV heads, head_dim 128, fp16) with contexts drawn uniformly in
[1024, 8192] over shuffled pages; one step quantizes and appends one new token
per sequence (kv_quant_int8_sym_write) and then runs the INT8 paged decode
(paged_attn_decode_int8) over contexts L_b + 1. The FP16-KV control runs the
same step with kv_write_16bit + paged_attn_decode_fp16. Supplementary decode
points at 2K, 8K and 32K context are reported alongside.

Prints ONE JSON line. Timing: W warm-up steps, then K timed steps between
device synchronizations; HIP events on the launch stream time each decode call
for the roofline figure. Pool replicas are rotated so that more than 2 GB is
touched between reuses (beyond the 256 MB Infinity Cache).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-points", action="store_true", help="skip the 2K/8K/32K points")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rotate-gb", type=float, default=2.2)
    return ap.parse_args()


def decode_bytes(wl, fmt_int8: bool) -> int:
    """Algorithmic HBM bytes of one decode call: K/V payload (+ scales),
    block-table entries, context lengths, q, FP32 output."""
    hkv, d = wl.num_kv_heads, wl.head_dim
    per_tok = hkv * (2 * d + 4) if fmt_int8 else hkv * 4 * d
    total = 0
    for L in wl.context_lens.tolist():
        total += L * per_tok + math.ceil(L / 16) * 4 + 4
    total += wl.num_seqs * wl.num_q_heads * d * (2 + 4)
    return total


def write_bytes(T: int, hkv: int, d: int, fmt_int8: bool) -> int:
    """Read 16-bit K and V, write codes + scales (or 16-bit values), read slots."""
    written = T * hkv * (2 * d + 4) if fmt_int8 else T * hkv * 4 * d
    return T * 4 * hkv * d + written + T * 4


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported "
              "(this library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_decode_attention_kv_amd as P
    from workloads import make_config

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.init()
    stream = torch.cuda.current_stream()

    def to_dev(t):
        if t.is_contiguous():
            return t.to("cuda")
        base = t._base if t._base is not None else t
        return torch.as_strided(base.to("cuda"), t.size(), t.stride(), t.storage_offset())

    def dev_i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda")

    def setup(wl, fmt_int8, append_phase):
        fmt = P.KV_INT8_SYM if fmt_int8 else P.KV_16BIT
        write = P.kv_quant_int8_sym_write if fmt_int8 else P.kv_write_16bit
        pb = P.pdakv_page_bytes(fmt, 16, wl.num_kv_heads, wl.head_dim)
        pool = torch.empty((wl.num_blocks, pb), dtype=torch.uint8, device="cuda")
        for ph in wl.phases:
            if ph.name != append_phase:
                write(to_dev(ph.k), to_dev(ph.v), dev_i32(ph.slot_mapping), pool, wl.num_blocks)
        nrep = max(1, math.ceil(args.rotate_gb * 1e9 / pool.numel()))
        pools = [pool] + [pool.clone() for _ in range(nrep - 1)]
        st = dict(fmt_int8=fmt_int8, write=write, pools=pools,
                  decode=P.paged_attn_decode_int8 if fmt_int8 else P.paged_attn_decode_fp16,
                  q=to_dev(wl.q), bt=dev_i32(wl.block_tables), ctx=dev_i32(wl.context_lens),
                  out=torch.empty((wl.num_seqs, wl.num_q_heads, wl.head_dim),
                                  dtype=torch.float32, device="cuda"),
                  ws=P.alloc_workspace(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads,
                                       wl.head_dim, wl.max_context_len))
        if append_phase:
            ph = wl.phase(append_phase)
            st["ak"], st["av"], st["aslots"] = to_dev(ph.k), to_dev(ph.v), dev_i32(ph.slot_mapping)
        torch.cuda.synchronize()
        return st

    def run(wl, st, steps, warmup, with_write):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        pools = st["pools"]

        def one(i, timed):
            pool = pools[i % len(pools)]
            if with_write:
                st["write"](st["ak"], st["av"], st["aslots"], pool, wl.num_blocks, stream=stream)
            if timed:
                ev[i][0].record(stream)
            st["decode"](st["out"], st["q"], pool, wl.num_blocks, st["bt"], st["ctx"],
                         wl.num_kv_heads, wl.max_context_len, wl.sm_scale, st["ws"],
                         stream=stream)
            if timed:
                ev[i][1].record(stream)

        for i in range(warmup):
            one(i, False)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            one(i, True)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        dec_ms = [a.elapsed_time(b) for a, b in ev]
        return (t1 - t0) / steps * 1e3, float(np.mean(dec_ms)), float(np.median(dec_ms))

    # ---- headline: batched decode step (append + decode) ------------------
    wl = make_config(3)
    res = {}
    for fmt_int8 in (True, False):
        st = setup(wl, fmt_int8, "append")
        step_ms, dec_ms, dec_med = run(wl, st, args.steps, args.warmup, with_write=True)
        res["int8" if fmt_int8 else "fp16"] = dict(
            step_ms=step_ms, decode_ms=dec_ms, decode_ms_median=dec_med,
            tokens_per_s=wl.num_seqs / (step_ms * 1e-3),
            decode_gbs=decode_bytes(wl, fmt_int8) / (dec_ms * 1e-3) / 1e9,
            rotate_replicas=len(st["pools"]))
        del st
        torch.cuda.empty_cache()
    pps, nsplit = P.pdakv_decode_plan(wl.num_seqs, wl.num_kv_heads, wl.max_context_len)
    i8 = res["int8"]
    dec_b = decode_bytes(wl, True)
    step_b = dec_b + write_bytes(wl.num_seqs, wl.num_kv_heads, wl.head_dim, True)

    # ---- supplementary decode-only points at 2K / 8K / 32K -------------------
    points = {}
    if not args.no_points:
        for key, idx in (("2k", 2), ("8k", "s8k"), ("32k", 4)):
            pwl = make_config(idx)
            entry = {"config": pwl.name, "batch": pwl.num_seqs,
                     "context": int(pwl.max_context_len)}
            for fmt_int8 in (True, False):
                st = setup(pwl, fmt_int8, None)
                _, dms, _ = run(pwl, st, max(10, args.steps), args.warmup, with_write=False)
                b = decode_bytes(pwl, fmt_int8)
                entry["int8" if fmt_int8 else "fp16"] = {
                    "decode_us": round(dms * 1e3, 2),
                    "tokens_per_s": round(pwl.num_seqs / (dms * 1e-3), 1),
                    "gbs": round(b / (dms * 1e-3) / 1e9, 1),
                    "hbm_frac": round(b / (dms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
                del st
                torch.cuda.empty_cache()
            entry["int8_over_fp16"] = round(entry["int8"]["tokens_per_s"] /
                                            entry["fp16"]["tokens_per_s"], 3)
            points[key] = entry

    # ---- CPU baseline: the oracle on a bounded sample ------------------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl)

    achieved = dec_b / (i8["decode_ms"] * 1e-3) / 1e9
    line = {
        "metric": "INT8-KV paged decode attention: tokens/s and achieved HBM GB/s at 2K/8K/32K",
        "value": round(i8["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(i8["step_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8-kv/fp16-q/fp32-acc",
        "data": "synthetic (seeded N(0,1) fp16 with x20 outlier channels; no model weights)",
        "config": {"workload": wl.name, "batch": wl.num_seqs,
                   "context": "uniform [1024, 8192] + 1 appended token",
                   "mean_context": round(float(wl.context_lens.mean()), 1),
                   "heads_q_kv": [wl.num_q_heads, wl.num_kv_heads], "head_dim": wl.head_dim,
                   "block_size": 16, "step": "kv_quant_int8_sym_write(64 tokens) + "
                   "paged_attn_decode_int8", "pages_per_split": pps, "max_splits": nsplit},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None,
                     "kernel": "paged_attn_decode_int8 (decode + split merge)",
                     "bytes_per_launch": dec_b, "launch_us": round(i8["decode_ms"] * 1e3, 2)},
        "step_bytes": step_b,
        "step_gbs": round(step_b / (i8["step_ms"] * 1e-3) / 1e9, 1),
        "fp16_control": {k: (round(v, 4) if isinstance(v, float) else v)
                         for k, v in res["fp16"].items()},
        "int8_over_fp16_tokens": round(i8["tokens_per_s"] / res["fp16"]["tokens_per_s"], 3),
        "points": points,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(wl, budget_s: float = 15.0):
    """Time the oracle (as it stands) on a bounded sample of the same step.

    Per sampled sequence: its prefill K/V are quantized untimed (that is the
    cache the step starts from); the timed part is the step itself for that
    sequence — quantize the appended token, dequantize the cache, run the
    oracle's FP64 decode for all 32 query heads. Sequences are processed until
    ``budget_s`` of timed work is spent; the rate is sequences (= decoded
    tokens) per second.
    """
    import numpy as np
    import torch
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
    pre, app = wl.phase("prefill"), wl.phase("append")
    done, spent = 0, 0.0
    for b in np.random.default_rng(0).permutation(wl.num_seqs):
        rows = pre.seq_rows(int(b))
        kc, ks = oracle.quantize_rows(pre.k[rows])
        vc, vs = oracle.quantize_rows(pre.v[rows])
        arow = app.seq_rows(int(b))
        t0 = time.perf_counter()
        akc, aks = oracle.quantize_rows(app.k[arow])
        avc, avs = oracle.quantize_rows(app.v[arow])
        kf = oracle.dequantize_rows(np.concatenate([kc, akc]), np.concatenate([ks, aks]))
        vf = oracle.dequantize_rows(np.concatenate([vc, avc]), np.concatenate([vs, avs]))
        oracle.attend_one_sequence(oracle.as_f32(wl.q[int(b)]), kf, vf, wl.sm_scale)
        spent += time.perf_counter() - t0
        done += 1
        if spent >= budget_s:
            break
    del torch
    return {"value": round(done / spent, 3), "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{done} of {wl.num_seqs} sequences of the batched step (append-token "
                      f"quantize + dequantize + FP64 decode of 32 heads), {spent:.1f} s timed"}


if __name__ == "__main__":
    main()
