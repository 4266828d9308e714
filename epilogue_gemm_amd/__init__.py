"""MI355X (gfx950) GEMM with a fused epilogue: C = act(A.B [+ bias]).

The computation lives in the HIP library ``libgemm_epi.so`` (C ABI in
``include/gemm_epi.h``); ``binding`` is its ctypes front end and ``inputs``
the seeded synthetic-input generator.  Importing this package loads nothing:
the library is loaded on first use and its absence is an error.
"""
