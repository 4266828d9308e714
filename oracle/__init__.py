"""CPU oracle for C = act(s * A.B [+ bias]) [+ r] and for scaled dot-product
attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library and its Python binding never import,
load or call it; the two share no code.  See ``oracle.c`` for the definition
it computes and the passages it follows.
"""
from .oracle import (  # noqa: F401
    FORMATS,
    attention,
    LAYOUTS,
    EPILOGUES,
    build,
    lib_path,
    decode,
    decode_array,
    encode,
    encode_array,
    gelu,
    gemm_epi,
    gemm_epi_points,
    max_threads,
    silu,
)
