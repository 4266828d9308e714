"""ctypes front end of the C oracle -- TEST INFRASTRUCTURE ONLY.

Argument marshalling only: every value is computed by ``oracle.c``.  Inputs
are the raw bit patterns the GPU side also sees (numpy ``uint16`` arrays for
fp16/bf16), so both sides start from identical bytes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# Codes understood by oracle.c (its own numbering; nothing is shared with the
# GPU library's header).
FORMATS = {"f16": 0, "bf16": 1, "f32": 2, "fp8": 3}
LAYOUTS = {"row": 0, "col": 1}
EPILOGUES = {"none": 0, "relu": 1, "bias_relu": 2, "bias_gelu": 3, "bias": 4, "silu": 5, "bias_silu": 6}

_lib = None


def lib_path() -> str:
    return _LIB


def build() -> str:
    """Compile oracle.c with the host C compiler (no HIP involved)."""
    cmd = [
        "gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-Wall",
        "-shared", "-fPIC", _SRC, "-o", _LIB, "-lm",
    ]
    subprocess.run(cmd, check=True)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    i64, i32, u32, vp, dp = ctypes.c_int64, ctypes.c_int, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_double
    lib.oracle_decode.argtypes = [i32, u32]
    lib.oracle_decode.restype = dp
    lib.oracle_encode.argtypes = [i32, dp]
    lib.oracle_encode.restype = u32
    lib.oracle_decode_n.argtypes = [i32, vp, vp, i64]
    lib.oracle_decode_n.restype = None
    lib.oracle_encode_n.argtypes = [i32, vp, vp, i64]
    lib.oracle_encode_n.restype = None
    lib.oracle_gelu.argtypes = [dp]
    lib.oracle_gelu.restype = dp
    lib.oracle_silu.argtypes = [dp]
    lib.oracle_silu.restype = dp
    lib.oracle_gemm_epi_ex.argtypes = [i64, i64, i64, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, i32]
    lib.oracle_gemm_epi_ex.restype = i32
    lib.oracle_gemm_epi_points_ex.argtypes = [i64, i64, i64, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                              i64, vp, vp, vp, vp, i32]
    lib.oracle_gemm_epi_points_ex.restype = i32
    lib.oracle_attention.argtypes = [i64, i64, i64, i64, i32, i32, vp, vp, vp, i64, vp, vp, vp, vp, vp, i32]
    lib.oracle_attention.restype = i32
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = i32
    _lib = lib
    return lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def decode(fmt: str, bits: int) -> float:
    return float(_load().oracle_decode(FORMATS[fmt], int(bits)))


def encode(fmt: str, x: float) -> int:
    return int(_load().oracle_encode(FORMATS[fmt], float(x)))


def decode_array(fmt: str, bits) -> np.ndarray:
    """Values (fp64) of an array of bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint32)
    out = np.empty(b.shape, np.float64)
    _load().oracle_decode_n(FORMATS[fmt], _ptr(b), _ptr(out), b.size)
    return out


def encode_array(fmt: str, x) -> np.ndarray:
    """Bit patterns (uint32) of an fp64 array rounded once to the format."""
    v = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(v.shape, np.uint32)
    _load().oracle_encode_n(FORMATS[fmt], _ptr(v), _ptr(out), v.size)
    return out


def gelu(x: float) -> float:
    return float(_load().oracle_gelu(float(x)))


def silu(x: float) -> float:
    return float(_load().oracle_silu(float(x)))


def _ptr(a):
    return None if a is None else a.ctypes.data


def _bits16(a, name):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"{name}: expected uint16 bit patterns, got {a.dtype}")
    return a


_OUT_NP = {"f16": np.uint16, "bf16": np.uint16, "f32": np.uint32, "fp8": np.uint8}


def _extras(scale, residual, M, N, out_dtype, out_scale=None):
    """Optional epilogue operands as the arrays oracle.c reads: the fp32 column
    scale as uint32 bit patterns (N), the residual as output-format bit
    patterns (M x N row-major), the fp32 output scale as one bit pattern."""
    if out_scale is not None:
        out_scale = np.array([out_scale], np.float32).view(np.uint32)
    if scale is not None:
        scale = np.ascontiguousarray(scale)
        if scale.dtype == np.float32:
            scale = scale.view(np.uint32)
        if scale.dtype != np.uint32 or scale.size != N:
            raise ValueError("scale: expected N float32 values (or their uint32 bit patterns)")
    if residual is not None:
        if out_dtype == "fp8":
            raise ValueError("residual: not defined for fp8 output")
        residual = np.ascontiguousarray(residual)
        want = np.uint32 if out_dtype == "f32" else np.uint16
        if residual.dtype == np.float32 and out_dtype == "f32":
            residual = residual.view(np.uint32)
        if residual.dtype != want or residual.size != M * N:
            raise ValueError(f"residual: expected M*N {want.__name__} bit patterns of the output format")
    return scale, residual, out_scale


def gemm_epi(A, B, bias, M, N, K, in_dtype, out_dtype, layout_a, layout_b, epilogue,
             want_y=True, want_c=True, nthreads=0, scale=None, residual=None, out_scale=None):
    """Full M x N product.  Returns (y, c): y is fp64 q * (act(s * A.B [+ bias])
    [+ r]) (row-major M x N), the value that is rounded; c the output bit
    patterns (uint16; uint32 for f32; uint8 for fp8).  scale (N fp32),
    residual (M x N, output format; not for fp8) and out_scale (q, an fp32
    scalar) are optional."""
    A, B, bias = _bits16(A, "A"), _bits16(B, "B"), _bits16(bias, "bias")
    if A.size != M * K or B.size != K * N or (bias is not None and bias.size != N):
        raise ValueError("operand sizes do not match M, N, K")
    scale, residual, out_scale = _extras(scale, residual, M, N, out_dtype, out_scale)
    y = np.empty((M, N), np.float64) if want_y else None
    c = np.empty((M, N), _OUT_NP[out_dtype]) if want_c else None
    rc = _load().oracle_gemm_epi_ex(M, N, K, FORMATS[in_dtype], FORMATS[out_dtype], LAYOUTS[layout_a],
                                    LAYOUTS[layout_b], EPILOGUES[epilogue], _ptr(A), _ptr(B), _ptr(bias),
                                    _ptr(scale), _ptr(residual), _ptr(out_scale), _ptr(y), _ptr(c), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_gemm_epi rejected its arguments (rc={rc})")
    return y, c


def gemm_epi_points(A, B, bias, M, N, K, in_dtype, out_dtype, layout_a, layout_b, epilogue,
                    rows, cols, nthreads=0, scale=None, residual=None, out_scale=None):
    """Selected elements (rows[p], cols[p]).  Returns (y, bits) as 1-D arrays."""
    A, B, bias = _bits16(A, "A"), _bits16(B, "B"), _bits16(bias, "bias")
    if A.size != M * K or B.size != K * N or (bias is not None and bias.size != N):
        raise ValueError("operand sizes do not match M, N, K")
    scale, residual, out_scale = _extras(scale, residual, M, N, out_dtype, out_scale)
    rows = np.ascontiguousarray(rows, np.int64)
    cols = np.ascontiguousarray(cols, np.int64)
    if rows.shape != cols.shape:
        raise ValueError("rows and cols differ in length")
    y = np.empty(rows.size, np.float64)
    bits = np.empty(rows.size, np.uint32)
    rc = _load().oracle_gemm_epi_points_ex(M, N, K, FORMATS[in_dtype], FORMATS[out_dtype], LAYOUTS[layout_a],
                                           LAYOUTS[layout_b], EPILOGUES[epilogue], _ptr(A), _ptr(B), _ptr(bias),
                                           _ptr(scale), _ptr(residual), _ptr(out_scale), rows.size, _ptr(rows),
                                           _ptr(cols), _ptr(y), _ptr(bits), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_gemm_epi_points rejected its arguments (rc={rc})")
    return y, bits


def attention(Q, K, V, B, S, H, D, dtype, causal, rows=None, want_y=True, want_o=True, nthreads=0):
    """Scaled dot-product attention, fp64.  Q, K, V: uint16 bit patterns laid
    out [B, S, H, D].  rows: None for every query row (outputs [B, S, H, D]),
    or a tuple of index arrays (b, i, h) (outputs [len, D]).  Returns (y, o):
    fp64 values and their RNE bit patterns in `dtype`."""
    Q, K, V = _bits16(Q, "Q"), _bits16(K, "K"), _bits16(V, "V")
    n = B * S * H * D
    if Q.size != n or K.size != n or V.size != n:
        raise ValueError("Q, K, V must each hold B*S*H*D elements")
    if rows is None:
        count, rb, ri, rh, shape = -1, None, None, None, (B, S, H, D)
    else:
        rb, ri, rh = (np.ascontiguousarray(x, np.int64) for x in rows)
        if not (rb.shape == ri.shape == rh.shape):
            raise ValueError("row index arrays differ in length")
        count, shape = rb.size, (rb.size, D)
    y = np.empty(shape, np.float64) if want_y else None
    o = np.empty(shape, np.uint16) if want_o else None
    rc = _load().oracle_attention(B, S, H, D, FORMATS[dtype], int(bool(causal)), _ptr(Q), _ptr(K), _ptr(V), count,
                                  _ptr(rb), _ptr(ri), _ptr(rh), _ptr(y), _ptr(o), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_attention rejected its arguments (rc={rc})")
    return y, o
