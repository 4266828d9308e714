"""Helpers for comparing the HIP library's output with the oracle.

Tolerance (stated for this path): relative Frobenius error <= 1e-3 and
max elementwise error <= 2e-2, both measured between the GPU output and the
oracle's output rounded to the same format.  An element whose error exceeds
2e-2 is still accepted when the GPU value is the other of the two
output-format neighbours that bracket the oracle's exact fp64 value: near a
rounding tie, fp32 accumulation noise may legitimately pick either
neighbour, and in bf16 one ulp is 0.03125 for |y| in [4, 8).  Such accepted
flips are counted, and at most max(1, 1e-3 n) of n outputs may take one: a
systematic one-ulp bias (truncation, say) flips a large share of them.  The
same rule holds for every output format; the relative error is always taken
over the outputs as the GPU wrote them.
"""
from __future__ import annotations

import numpy as np
import torch

REL_FRO_TOL = 1e-3
MAX_ABS_TOL = 2e-2

_TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32, "fp8": torch.float8_e4m3fn}
# largest fraction of outputs (at least one) allowed to take the other
# rounding at a near-tie with an error above the max-abs bound
MAX_TIE_FLIP_FRACTION = 1e-3


def to_device(bits: np.ndarray, dtype: str, device="cuda"):
    """uint16 bit patterns -> contiguous device tensor of the 16-bit format."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).reshape(-1).copy())
    return t.view(_TORCH_DT[dtype]).to(device)


def to_device_out(bits: np.ndarray, dtype: str, device="cuda"):
    """Output-format bit patterns (uint16; uint32 for f32; uint8 for fp8) -> device tensor."""
    if dtype == "fp8":
        t = torch.from_numpy(np.ascontiguousarray(bits).astype(np.uint8).reshape(-1).copy())
        return t.view(torch.float8_e4m3fn).to(device)
    if dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(bits).astype(np.uint32).view(np.int32).reshape(-1).copy())
        return t.view(torch.float32).to(device)
    return to_device(np.asarray(bits).astype(np.uint16), dtype, device)


def empty_out(n: int, dtype: str, device="cuda"):
    return torch.empty(n, dtype=_TORCH_DT[dtype], device=device)


def out_bits(t: torch.Tensor) -> np.ndarray:
    """Device output tensor -> numpy bit patterns (uint16, or uint32 for f32)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy().copy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32).copy()
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def values(bits: np.ndarray, dtype: str) -> np.ndarray:
    bits = np.asarray(bits)
    if dtype == "fp8":
        t = torch.from_numpy(bits.astype(np.uint8).copy()).view(torch.float8_e4m3fn)
        return t.to(torch.float64).numpy()
    if dtype == "f32":
        return bits.astype(np.uint32).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    t = torch.from_numpy(bits.astype(np.uint16).view(np.int16).copy()).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def _neighbour(bits: np.ndarray, dtype: str, up: bool) -> np.ndarray:
    """Bit pattern of the next representable value toward +inf (up) or -inf."""
    nbits = {"f32": 32, "fp8": 8}.get(dtype, 16)
    sign = np.uint64(1) << np.uint64(nbits - 1)
    b = bits.astype(np.uint64)
    neg = (b & sign) != 0
    mag = b & (sign - np.uint64(1))
    out = np.empty_like(b)
    # toward +inf: positive magnitude grows, negative magnitude shrinks
    grow = neg != up
    zero = mag == 0
    out[grow] = b[grow] + np.uint64(1)
    out[~grow & ~zero] = b[~grow & ~zero] - np.uint64(1)
    # stepping through zero: from +-0 toward the other sign's smallest value
    zs = ~grow & zero
    out[zs] = (sign if up is False else np.uint64(0)) | np.uint64(1)
    return out.astype({32: np.uint32, 16: np.uint16, 8: np.uint8}[nbits])


def compare(gpu_bits, oracle_bits, oracle_y, dtype: str, rel_tol=REL_FRO_TOL, abs_tol=MAX_ABS_TOL):
    """Returns a dict of metrics and 'ok' (bool) for one comparison."""
    gpu_bits = np.asarray(gpu_bits).reshape(-1)
    oracle_bits = np.asarray(oracle_bits).reshape(-1)
    y = np.asarray(oracle_y, np.float64).reshape(-1)
    g = values(gpu_bits, dtype)
    o = values(oracle_bits, dtype)
    finite = bool(np.all(np.isfinite(g)))
    err = np.abs(g - o)
    rel = float(np.linalg.norm(g - o) / max(float(np.linalg.norm(o)), 1e-12))
    over = np.nonzero(err > abs_tol)[0]
    rejected = []
    for idx in over:
        ob = oracle_bits[idx:idx + 1]
        other = _neighbour(ob, dtype, up=bool(y[idx] > o[idx]))
        if y[idx] == o[idx] or gpu_bits[idx] != other[0]:
            rejected.append(int(idx))
    max_abs = float(err.max()) if err.size else 0.0
    n_accepted = int(over.size) - len(rejected)
    max_flips = max(1, int(MAX_TIE_FLIP_FRACTION * g.size))
    ok = finite and rel <= rel_tol and not rejected and n_accepted <= max_flips
    return {
        "ok": ok,
        "rel_fro": rel,
        "max_abs": max_abs,
        "n": int(g.size),
        "n_over_abs_tol": int(over.size),
        "n_rejected": len(rejected),
        "n_accepted": n_accepted,
        "n_mismatch_bits": int(np.count_nonzero(gpu_bits != oracle_bits)),
        "finite": finite,
    }
