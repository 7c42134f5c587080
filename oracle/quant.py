"""Per-token symmetric INT8 quantizer — CPU oracle (test infrastructure only).

What it computes (MoE-Infinity PR #183, "What landed", format-contract bullet,
and "Precision & memory"; mlxcel PR #717, "The Int8 bug and fix"):

* one FP16 scale per row, where a row is the D values of one token of one KV
  head of K, or of V (K and V are quantized separately);
* the scale is the row's absolute maximum divided by 127, rounded *upward* to
  FP16;
* codes are limited to [-127, 127] (no -128), and an exact zero stays zero;
* every element satisfies |x - code * scale| <= scale / 2 + 1e-6;
* only an all-zero row (absmax exactly 0) gets the substitute scale 1.0; any
  other row keeps its true scale, so its largest-magnitude coordinate maps to
  +-127 (the fix on the mlxcel page replaced a floor of the scale at 1.0).

Readings of points the pages leave open (each is also listed in the design doc):

* "absmax / 127" is evaluated as an IEEE binary32 division (round to nearest
  even); "rounded upward" then takes the smallest FP16 value that is >= that
  binary32 quotient.  For 16-bit inputs this equals the smallest FP16 >= the
  exact quotient (checked exhaustively in the tests).
* code = round-half-to-even(x / scale) with x / scale an IEEE binary32
  division — not a multiplication by a reciprocal.
* FP16 subnormal scales are kept (no flush to zero).
* -0.0 gives code 0.
* Rows whose scale would exceed the FP16 range (absmax > 127 * 65504, reachable
  only from bf16 inputs) and rows with NaN/Inf are outside the contract; this
  oracle raises on them.
"""

from __future__ import annotations

import numpy as np

_F16_MAX = np.float32(65504.0)


def as_f32(x) -> np.ndarray:
    """Return ``x`` (NumPy array or torch tensor of fp16/bf16/fp32) as float32.

    Widening fp16 or bf16 to fp32 is exact, so nothing is rounded here.
    """
    if isinstance(x, np.ndarray):
        return x.astype(np.float32, copy=False)
    # torch tensor (lazy import so the oracle does not require torch)
    return x.detach().to("cpu").float().numpy()


def ru16(s32: np.ndarray) -> np.ndarray:
    """Round binary32 values upward (toward +inf) to binary16.

    Returns the smallest FP16 value that is >= each input. Written from the
    definition: round to nearest, and if that landed below the input, step to
    the next representable FP16 value above it. Inputs must be finite and
    >= 0 and at most 65504.
    """
    s32 = np.asarray(s32, dtype=np.float32)
    if np.any(~np.isfinite(s32)) or np.any(s32 < 0) or np.any(s32 > _F16_MAX):
        raise ValueError("ru16: input outside [0, 65504]")
    h = s32.astype(np.float16)  # IEEE round-to-nearest-even
    below = h.astype(np.float32) < s32
    if np.any(below):
        h = np.where(below, np.nextafter(h, np.float16(np.inf)), h)
    return h.astype(np.float16)


def quantize_rows(x) -> tuple[np.ndarray, np.ndarray]:
    """Quantize each row (last axis) of ``x``; returns (codes int8, scales f16).

    Steps (MoE-Infinity PR #183 "What landed"; mlxcel PR #717 "The Int8 bug
    and fix"):

    1. a = max_d |x_d|                          (exact in binary32)
    2. a == 0  ->  scale 1.0, all codes 0        (all-zero token guard)
    3. otherwise s = ru16(fl32(a / 127))         (upward-rounded FP16 scale)
    4. code_d = clip(rint(x_d / s), -127, 127)   (binary32 division, RNE)
    """
    x = as_f32(x)
    if not np.all(np.isfinite(x)):
        raise ValueError("quantize_rows: NaN/Inf input is outside the contract")
    a = np.max(np.abs(x), axis=-1)
    zero = a == 0
    s32 = np.divide(a, np.float32(127.0), dtype=np.float32)
    if np.any(s32 > _F16_MAX):
        raise ValueError("quantize_rows: scale exceeds the FP16 range")
    s16 = ru16(s32)
    s16 = np.where(zero, np.float16(1.0), s16).astype(np.float16)
    q = np.divide(x, s16.astype(np.float32)[..., None], dtype=np.float32)
    codes = np.clip(np.rint(q), -127, 127).astype(np.int8)
    return codes, s16


def dequantize_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """code * scale, evaluated in binary32.

    A code has at most 7 significant bits and an FP16 scale 11, so the product
    is exact in binary32 (this is the "FP32 dequantized" value of the
    MoE-Infinity page's oracle, "What landed", runtime-integration bullet).
    """
    return codes.astype(np.float32) * scales.astype(np.float32)[..., None]


# ---------------------------------------------------------------------------
# Static (per-tensor) scales
# ---------------------------------------------------------------------------
#
# The other scheme on the pages: one calibrated scalar scale for all of K and
# one for all of V of a layer (InfiniLM PR #553, "Summary", bullets on the
# kv_cache_k_scale / kv_cache_v_scale parameters and "Notes for Reviewers";
# TensorRT-LLM PR #18953, "Summary": paired positive finite scalar k_scale /
# v_scale in float32, whose maximum serves as one shared K/V scale). The pages
# give the scales and their validity (finite, positive) but not the element
# formula; the reading taken is the per-token scheme's formula with the given
# scale: code = clip(rint(fl32(x / s)), -127, 127), x / s an IEEE binary32
# division, round half to even, symmetric range (no -128; zero point 0). Values
# beyond 127.5 * s saturate: that clipping is part of the static scheme.


def check_static_scale(s) -> np.float32:
    """The scale as binary32; raises unless it is finite and > 0 (the
    validity rule of TensorRT-LLM PR #18953, "Summary")."""
    s32 = np.float32(s)
    if not np.isfinite(s32) or not s32 > 0:
        raise ValueError("static scale must be finite and positive")
    return s32


def shared_static_scale(k_scale, v_scale) -> np.float32:
    """One scale for both K and V: the larger of the two (TensorRT-LLM
    PR #18953, "Summary": the maximum of the paired scales feeds the shared
    K/V scale)."""
    return np.float32(max(check_static_scale(k_scale), check_static_scale(v_scale)))


def quantize_static(x, s) -> np.ndarray:
    """Codes of ``x`` (any shape) under the static scale ``s``:
    clip(rint(fl32(x / s)), -127, 127) as int8."""
    s32 = check_static_scale(s)
    x = as_f32(x)
    if not np.all(np.isfinite(x)):
        raise ValueError("quantize_static: NaN/Inf input is outside the contract")
    q = np.divide(x, s32, dtype=np.float32)
    return np.clip(np.rint(q), -127, 127).astype(np.int8)


def dequantize_static(codes: np.ndarray, s) -> np.ndarray:
    """code * s in FP64 (exact: 8 bits times a 24-bit significand)."""
    return codes.astype(np.float64) * float(check_static_scale(s))
