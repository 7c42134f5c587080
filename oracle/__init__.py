"""CPU oracle for paged INT8-KV decode attention — test infrastructure only.

This package is a plain, slow, deliberately unoptimised NumPy implementation
of what the GPU path computes. It exists to check the GPU path; it is never
part of it. Only the test suite, the smoke check in ``__graft_entry__`` and the
CPU-baseline leg of ``bench.py`` may import it. It shares no code, header,
table or constant with the HIP library, and it imports nothing from it.

Modules
-------
quant      per-token symmetric INT8 quantizer (one FP16 scale per row), and
           the static variant (one given FP32 scale per tensor)
pages      the paged byte layout of INT8 and 16-bit KV pools, written from
           the layout contract, plus page write / gather helpers
attention  decode attention over dequantized K/V with FP64 accumulation, for
           one query token per sequence or several (causal among them)
lifecycle  page swap-out / swap-in and the front trim that keeps sink tokens

Every function cites the passage it follows. Sources are four pull-request
pages; they are cited by project, PR number and section:

* MoE-Infinity PR #183 "feat: opt-in INT8 KV-cache quantization"
  (sections "What landed", "Precision & memory", "Scope & fallback").
* mlxcel PR #717 "fix(cuda/kv): correct Int8 KV per-token scale and document
  CUDA KV mode status" (sections "The Int8 bug and fix", "Int8 vs Fp16 decode
  benchmark (warmed)").
* InfiniLM PR #553 "fix: #552 int8 kv cache quantization cannot be enabled"
  ("Summary").
* TensorRT-LLM PR #18953 "Add calibrated INT8 KV cache to PyTorch backend".

Parity status: every function here is pinned by CPU tests against values
derived by hand from the definitions, closed forms, invariants stated on the
pages, exhaustive searches and an independent pure-Python FP64 brute force
(``tests/test_oracle_*.py``). No function is "parity unpinned".
"""

from .quant import (  # noqa: F401
    as_f32,
    ru16,
    quantize_rows,
    dequantize_rows,
    check_static_scale,
    shared_static_scale,
    quantize_static,
    dequantize_static,
)
from .pages import (  # noqa: F401
    KV_INT8_SYM,
    KV_16BIT,
    KV_INT8_STATIC,
    page_bytes,
    int8_layout,
    int8_token_bytes,
    new_pool,
    write_int8_tokens,
    write_16bit_tokens,
    gather_int8_sequence,
    gather_16bit_sequence,
    write_int8_static_tokens,
    gather_int8_static_sequence,
)
from .attention import (  # noqa: F401
    bits_to_f32,
    attend_one_sequence,
    decode_int8_from_pool,
    decode_16bit_from_pool,
    decode_int8_static_from_pool,
    decode_multi_from_pool,
)
from .lifecycle import (  # noqa: F401
    swap_out_pages,
    swap_in_pages,
    trim_keep_sink,
)
