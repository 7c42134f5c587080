"""Benchmark of the paged INT8-KV decode step on one MI355X.

Default workload: the batched decode step — 64 Llama-3.1-8B-shaped sequences
(32 query / 8 KV heads, head_dim 128, fp16) with contexts drawn uniformly in
[1024, 8192] over shuffled pages; one step quantizes and appends one new token
per sequence and decodes over contexts L_b + 1, in one call
(paged_attn_decode_int8_append). Alongside: the FP16-KV control of the same
step (paged_attn_decode_fp16_append), the unfused form of both (write kernel,
then decode), the static-scale INT8 variant of the step, and decode-only
points at 2K, 8K and 32K context for the three page formats.

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


def _affinity_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# The oracle's host threads: the cores this process may run on, set before
# NumPy (and its BLAS) is imported. A thread count the environment already
# fixes is kept (the GPU machines set one), and the JSON line records both.
AFFINITY_CORES = _affinity_cores()
for _var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_var, str(AFFINITY_CORES))

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-points", action="store_true", help="skip the 2K/8K/32K points")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rotate-gb", type=float, default=2.2)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only copy a 1 GiB buffer 3 times (reference kernel of known size for "
                         "calibrating the FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--profile", metavar="WORKLOAD:CALL",
                    help="only run one call on one workload --steps times after --warmup "
                         "(for profiler runs) and print its mean time; WORKLOAD is one of "
                         "c1 c2 c3 c4 c5 s8k, CALL one of int8 fp16 static int8_append "
                         "fp16_append static_append int8_multiT fp16_multiT (T query tokens)")
    return ap.parse_args()


WORKLOADS = {"c1": 1, "c2": 2, "c3": 3, "c4": 4, "c5": 5, "s8k": "s8k"}


ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles",
                               "decode_int8_append_llama8b-batched-1k8k-b64_traffic.txt")
# the sources that decide what the decode call reads and writes
DECODE_SOURCES = [os.path.join(ROOT, "paged_decode_attention_kv_amd", "csrc", f)
                  for f in ("decode.hip", "launch.h", "device_util.h", "quant_row.h", "abi.cpp")]


def source_hash() -> str:
    """Hash of the decode sources' code: comments, blank lines and trailing
    spaces are left out, so that only a change of the code itself invalidates
    the committed counter summary."""
    import hashlib
    import re
    h = hashlib.sha256()
    for path in DECODE_SOURCES:
        with open(path) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = "\n".join(line.rstrip() for line in text.split("\n") if line.strip())
        h.update(code.encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per decode launch from the committed counter summary, or None
    when the decode source changed since the counters were taken."""
    try:
        fields = {}
        with open(TRAFFIC_PROFILE) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        if fields.get("decode_source_sha256") != source_hash():
            return None
        return int(fields["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def decode_bytes(wl, fmt: str) -> int:
    """Algorithmic HBM bytes of one decode call: K/V payload (+ scales),
    block-table entries, context lengths, q, FP32 output. fmt: "int8"
    (per-token scales), "static" (codes only) or "fp16"."""
    hkv, d = wl.num_kv_heads, wl.head_dim
    per_tok = hkv * {"int8": 2 * d + 4, "static": 2 * d, "fp16": 4 * d}[fmt]
    total = 0
    for L in wl.context_lens.tolist():
        total += L * per_tok + math.ceil(L / 16) * 4 + 4
    total += wl.num_seqs * wl.num_q_heads * d * (2 + 4)
    return total


def append_bytes(wl, fmt: str) -> int:
    """Algorithmic bytes of the fused append: read each sequence's new 16-bit
    K and V rows, write their codes (+ scales) or 16-bit values."""
    d = wl.head_dim
    written = {"int8": 2 * d + 4, "static": 2 * d, "fp16": 4 * d}[fmt]
    return wl.num_seqs * wl.num_kv_heads * (4 * d + written)


def write_bytes(wl, fmt: str) -> int:
    """Algorithmic bytes of writing one token: its 16-bit K and V rows read,
    codes (+ scales) or 16-bit values written, and its slot."""
    d = wl.head_dim
    written = {"int8": 2 * d + 4, "static": 2 * d, "fp16": 4 * d}[fmt]
    return wl.num_kv_heads * (4 * d + written) + 4


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported "
              "(this library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_decode_attention_kv_amd as P
    from workloads import make_config, multi_query

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.init()
    stream = torch.cuda.current_stream()

    if args.calibrate_copy:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": src.numel(), "copies": 3}))
        return

    def to_dev(t):
        if t.is_contiguous():
            return t.to("cuda")
        base = t._base if t._base is not None else t
        return torch.as_strided(base.to("cuda"), t.size(), t.stride(), t.storage_offset())

    def dev_i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda")

    def static_scales(wl):
        """The layer's K and V scales for the static-scale format: an input
        of that format (calibrated outside the path; here the absolute
        maximum of all K or V values of the workload over 127)."""
        ak = max(float(ph.k.float().abs().max()) for ph in wl.phases)
        av = max(float(ph.v.float().abs().max()) for ph in wl.phases)
        return float(np.float32(ak / 127.0)), float(np.float32(av / 127.0))

    def setup(wl, fmt_name, append_phase):
        if fmt_name == "static":
            ks, vs = static_scales(wl)

            def write(k, v, slots, pool, nb, stream=None):
                P.kv_quant_int8_static_write(k, v, slots, pool, nb, ks, vs, stream=stream)

            def decode(*a, **kw):
                P.paged_attn_decode_int8_static(*a[:9], ks, vs, *a[9:], **kw)

            def fused(*a, **kw):
                P.paged_attn_decode_int8_static_append(*a[:11], ks, vs, *a[11:], **kw)
            fmt = P.KV_INT8_STATIC
        elif fmt_name == "int8":
            fmt, write = P.KV_INT8_SYM, P.kv_quant_int8_sym_write
            decode, fused = P.paged_attn_decode_int8, P.paged_attn_decode_int8_append
        else:
            fmt, write = P.KV_16BIT, P.kv_write_16bit
            decode, fused = P.paged_attn_decode_fp16, P.paged_attn_decode_fp16_append
        pb = P.pdakv_page_bytes(fmt, 16, wl.num_kv_heads, wl.head_dim)
        pool = torch.empty((wl.num_blocks, pb), dtype=torch.uint8, device="cuda")
        for ph in wl.phases:
            if ph.name != append_phase:
                write(to_dev(ph.k), to_dev(ph.v), dev_i32(ph.slot_mapping), pool, wl.num_blocks)
        nrep = max(1, math.ceil(args.rotate_gb * 1e9 / pool.numel()))
        pools = [pool] + [pool.clone() for _ in range(nrep - 1)]
        st = dict(write=write, pools=pools, decode=decode, fused=fused,
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

    def run(wl, st, steps, warmup, mode):
        """mode "decode": decode calls only; "unfused": write the appended
        tokens, then decode; "fused": the fused append + decode call.
        Returns (ms per step over `steps` steps with nothing else on the
        stream, mean and median ms of the decode (or fused) call from HIP
        events around it in a second run of `steps` steps)."""
        pools = st["pools"]

        def one(i, ev=None):
            pool = pools[i % len(pools)]
            if mode == "unfused":
                st["write"](st["ak"], st["av"], st["aslots"], pool, wl.num_blocks, stream=stream)
            if ev is not None:
                ev[0].record(stream)
            if mode == "fused":
                st["fused"](st["out"], st["q"], st["ak"], st["av"], pool, wl.num_blocks, st["bt"],
                            st["ctx"], wl.num_kv_heads, wl.max_context_len, wl.sm_scale,
                            st["ws"], stream=stream)
            elif mode == "multi":
                st["multi"](st["mout"], st["mq"], pool, wl.num_blocks, st["bt"], st["ctx"],
                            wl.num_kv_heads, wl.max_context_len, wl.sm_scale, st["mws"],
                            stream=stream)
            else:
                st["decode"](st["out"], st["q"], pool, wl.num_blocks, st["bt"], st["ctx"],
                             wl.num_kv_heads, wl.max_context_len, wl.sm_scale, st["ws"],
                             stream=stream)
            if ev is not None:
                ev[1].record(stream)

        for i in range(warmup):
            one(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            one(i)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for i in range(steps):
            one(i, evs[i])
        torch.cuda.synchronize()
        dec_ms = [a.elapsed_time(b) for a, b in evs]
        return (t1 - t0) / steps * 1e3, float(np.mean(dec_ms)), float(np.median(dec_ms))

    if args.profile:
        wname, call = args.profile.split(":")
        pwl = make_config(WORKLOADS[wname])
        key = call.split("_")[0]
        append = call.endswith("_append")
        st = setup(pwl, key, "append" if append else None)
        mode = "fused" if append else "decode"
        if "_multi" in call:
            T = int(call.split("_multi")[1])
            st["multi"] = (P.paged_attn_decode_int8_multi if key == "int8"
                           else P.paged_attn_decode_fp16_multi)
            st["mq"] = to_dev(multi_query(pwl, T, seed=2024))
            st["mout"] = torch.empty((pwl.num_seqs, T, pwl.num_q_heads, pwl.head_dim),
                                     dtype=torch.float32, device="cuda")
            st["mws"] = P.alloc_multi_workspace(pwl.num_seqs, T, pwl.num_q_heads,
                                                pwl.num_kv_heads, pwl.head_dim,
                                                pwl.max_context_len)
            mode = "multi"
        step, ms, med = run(pwl, st, args.steps, args.warmup, mode)
        # step_us: back-to-back calls (as the headline's step loop runs them);
        # call_us: each call between its own pair of events
        print(json.dumps({"profile": args.profile, "workload": pwl.name,
                          "dispatches": args.warmup + 2 * args.steps,
                          "step_us": round(step * 1e3, 2),
                          "call_us": round(ms * 1e3, 2), "call_us_median": round(med * 1e3, 2)}),
              flush=True)
        return

    # ---- headline: batched decode step (append + decode) ------------------
    # fused: one call appends the 64 new tokens and decodes; unfused: the
    # separate quantize-on-write call, then the decode call
    wl = make_config(3)
    res, unfused = {}, {}
    for key in ("int8", "fp16", "static"):
        st = setup(wl, key, "append")
        step_ms, dec_ms, dec_med = run(wl, st, args.steps, args.warmup, "fused")
        res[key] = dict(
            step_ms=step_ms, call_ms=dec_ms, call_ms_median=dec_med,
            tokens_per_s=wl.num_seqs / (step_ms * 1e-3),
            call_gbs=(decode_bytes(wl, key) + append_bytes(wl, key)) / (dec_ms * 1e-3) / 1e9,
            rotate_replicas=len(st["pools"]))
        if key != "static":
            step_ms, dec_ms, dec_med = run(wl, st, args.steps, args.warmup, "unfused")
            unfused[key] = dict(step_ms=round(step_ms, 5), decode_ms=round(dec_ms, 5),
                                tokens_per_s=round(wl.num_seqs / (step_ms * 1e-3), 1),
                                decode_gbs=round(decode_bytes(wl, key) / (dec_ms * 1e-3) / 1e9,
                                                 1))
        del st
        torch.cuda.empty_cache()
    waves, ppw = P.pdakv_decode_plan(P.KV_INT8_SYM, wl.num_seqs, wl.num_kv_heads,
                                     wl.head_dim, wl.max_context_len)
    i8 = res["int8"]
    dec_b = decode_bytes(wl, "int8")
    call_b = dec_b + append_bytes(wl, "int8")

    # ---- supplementary decode-only points at 2K / 8K / 32K -------------------
    points = {}
    if not args.no_points:
        for pname, idx, bound in (("c1", 1, "latency-bound (0.56 MB per call)"),
                                  ("2k", 2, "latency-bound (4.3 MB per call)"),
                                  ("8k", "s8k", "hbm"), ("32k", 4, "hbm"),
                                  ("c5", 5, "latency/Infinity-Cache-bound (35 MB per call)")):
            pwl = make_config(idx)
            entry = {"config": pwl.name, "batch": pwl.num_seqs,
                     "context": int(pwl.max_context_len), "bound": bound,
                     "heads_q_kv": [pwl.num_q_heads, pwl.num_kv_heads],
                     "head_dim": pwl.head_dim, "dtype": pwl.kv_dtype}
            for key in ("int8", "fp16", "static"):
                st = setup(pwl, key, None)
                sms, dms, _ = run(pwl, st, max(10, args.steps), args.warmup, "decode")
                b = decode_bytes(pwl, key)
                # decode_us: one call between its own pair of events (a
                # latency, with the events' own cost); step_us: calls back to
                # back, host-timed between synchronizations like the headline
                entry[key] = {
                    "decode_us": round(dms * 1e3, 2),
                    "tokens_per_s": round(pwl.num_seqs / (dms * 1e-3), 1),
                    "gbs": round(b / (dms * 1e-3) / 1e9, 1),
                    "hbm_frac": round(b / (dms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "step_us": round(sms * 1e3, 2),
                    "step_gbs": round(b / (sms * 1e-3) / 1e9, 1)}
                del st
                torch.cuda.empty_cache()
            entry["int8_over_fp16"] = round(entry["int8"]["tokens_per_s"] /
                                            entry["fp16"]["tokens_per_s"], 3)
            if not args.no_cpu_baseline:
                entry["oracle"] = oracle_decode_rate(pwl)
            points[pname] = entry

    # ---- several query tokens: verify 4 draft tokens per sequence -----------
    # the batched step's pool (contexts L_b + 1); the last 4 positions of every
    # sequence are the query tokens (causal among them)
    # T = 4 and 8 draft tokens (16 and 32 query columns per KV head: one and
    # two 16-column tiles, both streamed once) and a 64-token block (256
    # columns, 16 tiles in units of 4)
    multi = None
    if not args.no_points:
        multi = {"config": wl.name}
        for key in ("int8", "fp16"):
            st = setup(wl, key, None)
            st["multi"] = (P.paged_attn_decode_int8_multi if key == "int8"
                           else P.paged_attn_decode_fp16_multi)
            _, dms, _ = run(wl, st, args.steps, args.warmup, "decode")
            multi[key] = {"one_token_call_us": round(dms * 1e3, 2)}
            for T in (4, 8, 64):
                st["mq"] = to_dev(multi_query(wl, T, seed=2024))
                st["mout"] = torch.empty((wl.num_seqs, T, wl.num_q_heads, wl.head_dim),
                                         dtype=torch.float32, device="cuda")
                st["mws"] = P.alloc_multi_workspace(wl.num_seqs, T, wl.num_q_heads,
                                                    wl.num_kv_heads, wl.head_dim,
                                                    wl.max_context_len)
                _, mms, _ = run(wl, st, args.steps, args.warmup, "multi")
                b = (decode_bytes(wl, key) +
                     wl.num_seqs * (T - 1) * wl.num_q_heads * wl.head_dim * 6)
                multi[key][f"T{T}"] = {
                    "call_us": round(mms * 1e3, 2),
                    "query_tokens_per_s": round(wl.num_seqs * T / (mms * 1e-3), 1),
                    "gbs": round(b / (mms * 1e-3) / 1e9, 1),
                    "vs_T_one_token_calls": round(T * dms / mms, 3)}
            multi[key]["T8_over_T4"] = round(multi[key]["T8"]["call_us"] /
                                             multi[key]["T4"]["call_us"], 3)
            del st
            torch.cuda.empty_cache()
        multi["int8_over_fp16_T4"] = round(multi["fp16"]["T4"]["call_us"] /
                                           multi["int8"]["T4"]["call_us"], 3)

    def timed(fn, reps):
        """Seconds per call of fn, from HIP events on the launch stream."""
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    # ---- page lifecycle: swap-out / swap-in and the sink-keeping trim -----------
    lifecycle = None
    if not args.no_points:
        st = setup(wl, "int8", None)
        pool = st["pools"][0]
        pb = pool.shape[1]
        # device side: every page of the pool, in a shuffled order (far more
        # than the caches hold); pinned host side: 2048 pages (PCIe-bound)
        perm = np.random.default_rng(5).permutation(wl.num_blocks)
        all_ids = dev_i32(perm)
        dev_buf = torch.empty((wl.num_blocks, pb), dtype=torch.uint8, device="cuda")
        dev_bytes = wl.num_blocks * pb
        t_dev = timed(lambda: P.kv_pages_swap_out(pool, wl.num_blocks, all_ids, dev_buf,
                                                  stream=stream), 10)
        # a plain device-to-device copy of the same bytes: the practical
        # ceiling of a read-and-write pass
        with torch.cuda.stream(stream):
            t_copy = timed(lambda: dev_buf.copy_(pool), 10)
        del dev_buf
        npages = 2048
        ids = dev_i32(perm[:npages])
        host_buf = torch.empty((npages, pb), dtype=torch.uint8, pin_memory=True)
        nbytes = npages * pb
        t_out = timed(lambda: P.kv_pages_swap_out(pool, wl.num_blocks, ids, host_buf,
                                                  stream=stream), 5)
        t_in = timed(lambda: P.kv_pages_swap_in(host_buf, ids, pool, wl.num_blocks,
                                                stream=stream), 5)
        keep, ntrim = 4, 1024
        trims = dev_i32(np.full(wl.num_seqs, ntrim))
        new_lens = torch.empty(wl.num_seqs, dtype=torch.int32, device="cuda")
        t_trim = timed(lambda: P.kv_trim_keep_sink(P.KV_INT8_SYM, pool, wl.num_blocks,
                                                   wl.num_kv_heads, wl.head_dim, st["bt"],
                                                   st["ctx"], trims, keep, new_lens,
                                                   stream=stream), 5)
        moved = int(np.maximum(wl.context_lens.astype(np.int64) - keep - ntrim, 0).sum())
        trim_bytes = 2 * moved * wl.num_kv_heads * (2 * wl.head_dim + 4)
        copy_gbs = 2 * dev_bytes / t_copy / 1e9
        lifecycle = {
            "page_bytes": pb,
            "device_copy_ref": {"bytes": dev_bytes, "us": round(t_copy * 1e6, 2),
                                "gbs": round(copy_gbs, 1)},
            "swap_out_to_device": {"pages": wl.num_blocks, "us": round(t_dev * 1e6, 2),
                                   "gbs": round(2 * dev_bytes / t_dev / 1e9, 1),
                                   "hbm_frac": round(2 * dev_bytes / t_dev / 1e9 / HBM_PEAK_GBS, 4),
                                   "of_copy": round(2 * dev_bytes / t_dev / 1e9 / copy_gbs, 3)},
            "swap_out_to_pinned_host": {"pages": npages, "us": round(t_out * 1e6, 2),
                                        "gbs": round(nbytes / t_out / 1e9, 1)},
            "swap_in_from_pinned_host": {"pages": npages, "us": round(t_in * 1e6, 2),
                                         "gbs": round(nbytes / t_in / 1e9, 1)},
            "trim_keep_sink": {"keep": keep, "trim": ntrim, "tokens_moved": moved,
                               "us": round(t_trim * 1e6, 2),
                               "gbs": round(trim_bytes / t_trim / 1e9, 1),
                               "hbm_frac": round(trim_bytes / t_trim / 1e9 / HBM_PEAK_GBS, 4),
                               "of_copy": round(trim_bytes / t_trim / 1e9 / copy_gbs, 3)},
        }
        del st, host_buf
        torch.cuda.empty_cache()

    # ---- bulk quantize-on-write: the small-head chunk and the batched prefill -
    # the 32 x 4,096-token chunk of the small-head configuration (strided bf16
    # views of a fused QKV buffer, chunk starting at page offset 7), and the
    # 296K-token prefill of the batched step's pool
    writes = None
    if not args.no_points:
        writes = {}
        for wname, wwl, phase in (("chunk_b32x4096_gqa7_d64", make_config(5), "chunk"),
                                  ("prefill_" + wl.name, wl, "prefill")):
            ph = wwl.phase(phase)
            k, v, sl = to_dev(ph.k), to_dev(ph.v), dev_i32(ph.slot_mapping)
            ntok = int(ph.k.shape[0])
            entry = {"tokens": ntok, "kv_heads": wwl.num_kv_heads, "head_dim": wwl.head_dim}
            wstatic = static_scales(wwl)
            for key, fmt, fn in (
                    ("int8", P.KV_INT8_SYM, P.kv_quant_int8_sym_write),
                    ("static", P.KV_INT8_STATIC,
                     lambda *x, **kw: P.kv_quant_int8_static_write(*x, *wstatic, **kw)),
                    ("fp16", P.KV_16BIT, P.kv_write_16bit)):
                pb = P.pdakv_page_bytes(fmt, 16, wwl.num_kv_heads, wwl.head_dim)
                wpool = torch.empty((wwl.num_blocks, pb), dtype=torch.uint8, device="cuda")
                reps = 50 if ntok < 200000 else 10
                t_w = timed(lambda: fn(k, v, sl, wpool, wwl.num_blocks, stream=stream), reps)
                wb = ntok * write_bytes(wwl, key)
                entry[key] = {"us": round(t_w * 1e6, 2), "gbs": round(wb / t_w / 1e9, 1),
                              "hbm_frac": round(wb / t_w / 1e9 / HBM_PEAK_GBS, 4)}
                del wpool
            writes[wname] = entry
            del k, v, sl
            torch.cuda.empty_cache()

    # ---- CPU baseline: the oracle on a bounded sample ------------------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl)

    achieved = call_b / (i8["call_ms"] * 1e-3) / 1e9
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
                   "block_size": 16, "step": "paged_attn_decode_int8_append (quantize-on-write "
                   "of the 64 new tokens fused into the decode launch)", "decode_waves": waves},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(),
                     "kernel": "paged_attn_decode_int8_append (decode with fused append + "
                               "partial merge)",
                     "bytes_per_launch": call_b, "launch_us": round(i8["call_ms"] * 1e3, 2)},
        "fp16_control": {k: (round(v, 4) if isinstance(v, float) else v)
                         for k, v in res["fp16"].items()},
        "int8_over_fp16_tokens": round(i8["tokens_per_s"] / res["fp16"]["tokens_per_s"], 3),
        "static_scale_step": {k: (round(v, 4) if isinstance(v, float) else v)
                              for k, v in res["static"].items()},
        "unfused_step": unfused,
        "multi_token": multi,
        "lifecycle": lifecycle,
        "bulk_write": writes,
        "points": points,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_threads() -> int:
    """Threads of the BLAS pools NumPy uses (the oracle's host threads)."""
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return 1


def host_info() -> dict:
    return {"cpu_model": cpu_model(), "affinity_cores": AFFINITY_CORES,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def stratified_sample(lens, n: int):
    """n sequences at evenly spaced ranks of the context lengths (ranks
    (i + 1/2) * B / n): the sample's length distribution follows the batch's,
    so its rate is that of the whole batch."""
    import numpy as np
    order = np.argsort(np.asarray(lens), kind="stable")
    B = len(order)
    if n >= B:
        return sorted(order.tolist())
    ranks = ((np.arange(n) + 0.5) * B / n).astype(int)
    return sorted(int(order[r]) for r in ranks)


def _oracle_pool_for(wl, seqs):
    """An oracle pool holding every written token of the sampled sequences
    (pages renumbered compactly, each sequence keeping its page order), with
    its block table and context lengths. Untimed set-up."""
    import numpy as np
    import oracle
    tables, ctx, total = [], [], 0
    for b in seqs:
        n = -(-int(wl.context_lens[b]) // 16)
        tables.append(np.arange(total, total + n, dtype=np.int32))
        ctx.append(int(wl.context_lens[b]))
        total += n
    bt = np.zeros((len(seqs), max(len(t) for t in tables)), np.int32)
    for i, t in enumerate(tables):
        bt[i, :len(t)] = t
    pool = oracle.new_pool(oracle.KV_INT8_SYM, total, 16, wl.num_kv_heads, wl.head_dim)
    for i, b in enumerate(seqs):
        k, v = wl.tokens_of_seq(int(b))
        pos = np.arange(k.shape[0])
        kc, ks = oracle.quantize_rows(k)
        vc, vs = oracle.quantize_rows(v)
        oracle.write_int8_tokens(pool, kc, ks, vc, vs, bt[i, pos // 16] * 16 + pos % 16, 16)
    return pool, bt, np.array(ctx, np.int32)


def oracle_decode_rate(wl, budget_s: float = 4.0, max_seqs: int = 4) -> dict:
    """The oracle's INT8 paged decode (FP64) on a bounded, length-stratified
    sample of the workload's sequences, repeated for about budget_s seconds
    (at least once). Returns decoded sequences (= tokens) per second and the
    attended context tokens per second."""
    import numpy as np
    import oracle
    import torch
    seqs = stratified_sample(wl.context_lens, min(max_seqs, wl.num_seqs))
    pool, bt, ctx = _oracle_pool_for(wl, seqs)
    q = torch.stack([wl.q[b] for b in seqs])
    reps, spent = 0, 0.0
    while spent < budget_s or reps == 0:
        t0 = time.perf_counter()
        oracle.decode_int8_from_pool(pool, bt, ctx, q, wl.sm_scale, 16, wl.num_kv_heads,
                                     wl.head_dim)
        spent += time.perf_counter() - t0
        reps += 1
    return {"tokens_per_s": round(reps * len(seqs) / spent, 3),
            "context_tokens_per_s": round(reps * float(np.sum(ctx)) / spent, 1),
            "sample": f"{len(seqs)} of {wl.num_seqs} sequences (mean context "
                      f"{float(ctx.mean()):.0f}, batch mean {float(wl.context_lens.mean()):.0f}), "
                      f"{reps} oracle decodes in {spent:.1f} s",
            "threads": blas_threads()}


def cpu_baseline(wl, budget_s: float = 15.0, sample_seqs: int = 8):
    """Time the oracle (as it stands, untuned) on a bounded sample of the step.

    Sample: ``sample_seqs`` sequences at evenly spaced ranks of the batch's
    context lengths, so that the sample's mean context matches the batch's.
    Setup (untimed): an oracle pool holding their prefill, quantized and
    written by the oracle. Timed: the step for those sequences with the
    oracle's own functions -- quantize the appended tokens, write them into
    the pool, decode all query heads from the pool -- repeated until
    ``budget_s`` is spent. The rate is decoded tokens (one per sequence per
    step) per second; the attended context tokens per second are given too.
    """
    import numpy as np
    import oracle
    import torch
    pre, app = wl.phase("prefill"), wl.phase("append")
    seqs = stratified_sample(wl.context_lens, sample_seqs)
    # compact pool for the sample: each sampled sequence keeps its page order
    tables, ctx, total = [], [], 0
    for b in seqs:
        n = -(-int(wl.context_lens[b]) // 16)
        tables.append(np.arange(total, total + n, dtype=np.int32))
        ctx.append(int(wl.context_lens[b]))
        total += n
    bt = np.zeros((len(seqs), max(len(t) for t in tables)), np.int32)
    for i, t in enumerate(tables):
        bt[i, :len(t)] = t
    ctx = np.array(ctx, np.int32)
    pool = oracle.new_pool(oracle.KV_INT8_SYM, total, 16, wl.num_kv_heads, wl.head_dim)
    a_k, a_v, a_slots, qs = [], [], [], []
    for i, b in enumerate(seqs):
        rows = pre.seq_rows(int(b))
        n_pre = rows.stop - rows.start
        pos = np.arange(n_pre)
        kc, ks = oracle.quantize_rows(pre.k[rows])
        vc, vs = oracle.quantize_rows(pre.v[rows])
        oracle.write_int8_tokens(pool, kc, ks, vc, vs, bt[i, pos // 16] * 16 + pos % 16, 16)
        arow = app.seq_rows(int(b))
        a_k.append(app.k[arow])
        a_v.append(app.v[arow])
        a_slots.append(bt[i, n_pre // 16] * 16 + n_pre % 16)
        qs.append(wl.q[int(b)])
    ak, av, q = torch.cat(a_k), torch.cat(a_v), torch.stack(qs)
    slots = np.array(a_slots, np.int32)
    steps, spent = 0, 0.0
    while spent < budget_s:
        t0 = time.perf_counter()
        kc, ks = oracle.quantize_rows(ak)
        vc, vs = oracle.quantize_rows(av)
        oracle.write_int8_tokens(pool, kc, ks, vc, vs, slots, 16)
        oracle.decode_int8_from_pool(pool, bt, ctx, q, wl.sm_scale, 16, wl.num_kv_heads,
                                     wl.head_dim)
        spent += time.perf_counter() - t0
        steps += 1
    info = host_info()
    return {"value": round(steps * len(seqs) / spent, 3), "unit": "tokens/s",
            "cores": blas_threads(), "kind": "oracle",
            "sample": f"{len(seqs)} of {wl.num_seqs} sequences of the batched step at evenly "
                      f"spaced context-length ranks (mean context {float(ctx.mean()):.0f}, "
                      f"batch mean {float(wl.context_lens.mean()):.0f}); oracle quantize + "
                      f"page write of the appended tokens and FP64 paged decode of all "
                      f"{wl.num_q_heads} query heads, {steps} steps in {spent:.1f} s",
            "context_tokens_per_s": round(steps * float(ctx.sum()) / spent, 1),
            "cpu_model": info["cpu_model"], "affinity_cores": info["affinity_cores"],
            "omp_num_threads": info["omp_num_threads"]}


if __name__ == "__main__":
    main()
