"""Seeded synthetic inputs for paged decode attention.

This module only draws random numbers and lays out block tables; it holds none
of the method's arithmetic (no quantization, no attention). It is the one
piece shared by the CPU oracle's tests and the GPU path's tests and bench, so
that both sides see identical inputs.

Random draws use NumPy's PCG64 generator (``numpy.random.default_rng(seed)``)
in float32 and are cast round-to-nearest-even to fp16 or bf16 (torch's CPU
casts). The draw order is fixed by the code below and documented in the design doc.

Shapes are those of a Llama-3.1-8B attention layer (32 query heads, 8 KV heads,
head_dim 128) and of a small-head GQA layer (14 / 2 heads, head_dim 64); the
pages measure decode at 2K/8K/32K context on a llama-3.1-8b model (mlxcel PR
#717, "Int8 vs Fp16 decode benchmark (warmed)"), and these synthetic shapes
stand in for that model, which is not available here.
"""

from .gen import (  # noqa: F401
    Workload,
    WritePhase,
    build,
    make_config,
    multi_query,
    CONFIG_NAMES,
)
