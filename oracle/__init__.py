"""CPU oracle for the UltraSketchLLM sketch encoder and the sketch-decoded product.

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product (the HIP library and its
binding) never imports this package, and this package imports nothing from it.

The arithmetic lives in plain C (``sketch_oracle.c``); ``oracle.py`` loads it
with ctypes and adapts NumPy arrays.  ``build.py`` compiles it with gcc.
"""
from .oracle import (  # noqa: F401
    ABSMAX,
    ABSMIN,
    BF16,
    F16,
    F32,
    OracleError,
    alloc_plan,
    block_importance,
    bucket,
    bucket_map,
    decode,
    decode_alloc,
    decode_q4,
    encode,
    encode_alloc,
    encode_q4,
    f16_to_f64,
    f32_to_f16,
    f32_to_f16_array,
    hash32,
    layout,
    layout_q4,
    matmul,
    matmul_alloc,
    matmul_q4,
    matmul_sampled,
    matmul_sampled_alloc,
    matmul_sampled_q4,
    max_threads,
)
