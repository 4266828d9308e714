"""Seeded synthetic inputs for C = act(A.B [+ bias]).

This module only draws random numbers and lays them out; it holds none of the
product's arithmetic.  The GPU tests, the benchmark and the CPU oracle all
start from the bit patterns it returns, so both sides see identical bytes.

Recipe (the pages draw operands with ``torch.randn``, e.g. the GEMM+ReLU
example in atlascloud.ai "Writing high-performance kernels in TileLang",
section "Écrivons un GEMM", and the bias+GELU example in ainew.jp
"TileLang で GPU カーネル設計を解説", section 4):

  1. ``g = torch.Generator('cpu').manual_seed(seed)``;
  2. draw, in this order, A (M x K), B (logical K x N) and, when the epilogue
     has a bias, bias (N), each with ``torch.randn(..., generator=g)`` in fp32;
  3. scale in fp32: ``B /= b_div``, ``bias *= bias_std``;
  4. round each to the input format with ``Tensor.to`` (round to nearest even);
  5. lay out: a column-major operand is the transpose made contiguous.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

_TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One GEMM+epilogue problem: shapes, formats, layouts, value recipe."""

    name: str
    M: int
    N: int
    K: int
    in_dtype: str  # "f16" | "bf16"
    out_dtype: str  # "f16" | "bf16" | "f32"
    layout_a: str  # "row" | "col"
    layout_b: str  # "row" | "col"
    epilogue: str  # "none" | "relu" | "bias_relu" | "bias_gelu" | "bias" | "silu" | "bias_silu"
    b_div: float  # B ~ N(0,1) / b_div
    bias_std: float  # bias ~ N(0, bias_std^2)
    seed: int

    @property
    def has_bias(self) -> bool:
        return self.epilogue.startswith("bias")

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    def compulsory_bytes(self) -> int:
        isz = 2
        osz = 4 if self.out_dtype == "f32" else 2
        b = (self.M * self.K + self.K * self.N) * isz + self.M * self.N * osz
        if self.has_bias:
            b += self.N * isz
        return b


# The five workloads the library is measured and checked on.
WORKLOADS = {
    w.name: w
    for w in [
        # TileFusion global->register GEMM example: A 128x256 row-major,
        # B 256x64 column-major, fp32 result.
        Workload("gemm_f16_f32out_128x64x256_rm_cm", 128, 64, 256, "f16", "f32", "row", "col", "none",
                 16.0, 0.0, 0),
        Workload("gemm_relu_f16_1024x1024x1024_rm_rm", 1024, 1024, 1024, "f16", "f16", "row", "row", "relu",
                 32.0, 0.0, 1),
        Workload("gemm_relu_f16_4096x4096x4096_rm_rm", 4096, 4096, 4096, "f16", "f16", "row", "row", "relu",
                 64.0, 0.0, 2),
        Workload("gemm_bias_gelu_bf16_8192x8192x8192_rm_cm", 8192, 8192, 8192, "bf16", "bf16", "row", "col",
                 "bias_gelu", math.sqrt(8192.0), 0.1, 3),
        Workload("skinny_gemm_bias_bf16_32x8192x8192_rm_cm", 32, 8192, 8192, "bf16", "bf16", "row", "col", "bias",
                 math.sqrt(8192.0), 0.1, 4),
    ]
}
WORKLOAD_LIST = list(WORKLOADS.values())


def to_bits(t: torch.Tensor) -> np.ndarray:
    """Bit patterns of a CPU fp16/bf16 tensor as a numpy uint16 array."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16).copy()


def make_inputs(M: int, N: int, K: int, in_dtype: str, layout_a: str, layout_b: str, with_bias: bool,
                b_div: float, bias_std: float, seed: int):
    """Returns dict(A=..., B=..., bias=...) of uint16 bit arrays laid out as asked.

    A is M x K (row-major: shape (M, K); column-major: shape (K, M)), B is the
    logical K x N matrix (row-major: shape (K, N); column-major: shape (N, K)),
    bias has length N or is None.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    a = torch.randn(M, K, generator=g, dtype=torch.float32)
    b = torch.randn(K, N, generator=g, dtype=torch.float32)
    bias = torch.randn(N, generator=g, dtype=torch.float32) if with_bias else None
    b = b / float(b_div)
    if bias is not None:
        bias = bias * float(bias_std)
    dt = _TORCH_DT[in_dtype]
    a, b = a.to(dt), b.to(dt)
    if layout_a == "col":
        a = a.t().contiguous()
    if layout_b == "col":
        b = b.t().contiguous()
    return {
        "A": to_bits(a),
        "B": to_bits(b),
        "bias": to_bits(bias.to(dt)) if bias is not None else None,
    }


def workload_inputs(w: Workload):
    return make_inputs(w.M, w.N, w.K, w.in_dtype, w.layout_a, w.layout_b, w.has_bias, w.b_div, w.bias_std, w.seed)


def integer_inputs(M: int, N: int, K: int, in_dtype: str, layout_a: str, layout_b: str, with_bias: bool,
                   seed: int, lo: int = -2, hi: int = 2):
    """Integer-valued operands in [lo, hi] (exact in fp16 and bf16), laid out
    as in make_inputs.  Every product and partial sum is a small integer, so
    any accumulation order in fp32 gives the same exact result."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    a = torch.randint(lo, hi + 1, (M, K), generator=g).to(torch.float32)
    b = torch.randint(lo, hi + 1, (K, N), generator=g).to(torch.float32)
    bias = torch.randint(lo, hi + 1, (N,), generator=g).to(torch.float32) if with_bias else None
    dt = _TORCH_DT[in_dtype]
    a, b = a.to(dt), b.to(dt)
    if layout_a == "col":
        a = a.t().contiguous()
    if layout_b == "col":
        b = b.t().contiguous()
    return {
        "A": to_bits(a),
        "B": to_bits(b),
        "bias": to_bits(bias.to(dt)) if bias is not None else None,
    }


def integer_bits(rows: int, cols: int, in_dtype: str, seed: int, lo: int = -2, hi: int = 2,
                 chunk_rows: int = 4096):
    """rows x cols uint16 bit patterns of integers drawn uniformly from
    [lo, hi] (numpy PCG64 seeded with `seed`), generated chunk by chunk so
    that operands of 2^31 elements need no wider temporary than a chunk.
    The integers are exact in fp16 and bf16."""
    vals = np.arange(lo, hi + 1, dtype=np.float32)
    table = to_bits(torch.from_numpy(vals).to(_TORCH_DT[in_dtype])).astype(np.uint16)
    rng = np.random.default_rng(int(seed))
    out = np.empty((rows, cols), np.uint16)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        out[r0:r1] = table[rng.integers(0, hi - lo + 1, size=(r1 - r0, cols), dtype=np.int8)]
    return out


def extras_inputs(M: int, N: int, out_dtype: str, seed: int, integer: bool = False):
    """Optional epilogue operands: dict(scale=float32 array of N, residual=bit
    patterns of an M x N row-major array in the output format (uint16 for
    f16/bf16, uint32 for f32; None for fp8, which takes no residual),
    out_scale=a float).

    Random (integer=False): scale ~ U(0.5, 1.5), residual ~ N(0, 1),
    out_scale 2^u with u ~ U(-1, 3) rounded to an integer.
    Integer (integer=True): scale from {-2, -1, -0.5, 0.5, 1, 2}, residual
    integers in [-8, 8] and out_scale from {0.25, 0.5, 1, 2}, so that with
    integer operands every fp32 step of the epilogue is exact."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) + 7919)
    if integer:
        choices = torch.tensor([-2.0, -1.0, -0.5, 0.5, 1.0, 2.0])
        scale = choices[torch.randint(0, 6, (N,), generator=g)]
        resid = torch.randint(-8, 9, (M, N), generator=g).to(torch.float32)
        out_scale = float([0.25, 0.5, 1.0, 2.0][int(torch.randint(0, 4, (1,), generator=g))])
    else:
        scale = torch.rand(N, generator=g, dtype=torch.float32) + 0.5
        resid = torch.randn(M, N, generator=g, dtype=torch.float32)
        out_scale = float(2.0 ** int(torch.randint(-1, 4, (1,), generator=g)))
    if out_dtype == "fp8":
        rbits = None
    elif out_dtype == "f32":
        rbits = resid.contiguous().view(torch.int32).numpy().view(np.uint32).copy().reshape(-1)
    else:
        rbits = to_bits(resid.to(_TORCH_DT[out_dtype])).reshape(-1)
    return {"scale": scale.numpy().astype(np.float32), "residual": rbits, "out_scale": out_scale}


# ---------------------------------------------------------------------------
# attention forward (the second workload)
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class AttentionWorkload:
    """Scaled dot-product attention, Q, K, V, O laid out [B, S, H, D]."""
    name: str
    B: int
    S: int
    H: int
    D: int
    dtype: str  # "f16" | "bf16"
    causal: bool
    seed: int

    @property
    def flops(self) -> float:
        # two products of 2 S^2 D per (batch, head); half of them when causal
        return 4.0 * self.B * self.H * self.S * self.S * self.D * (0.5 if self.causal else 1.0)

    def compulsory_bytes(self) -> int:
        return 4 * self.B * self.S * self.H * self.D * 2


# The ainew.jp page's section-6 example: B, H, S, D = 4, 8, 1024, 64, fp16,
# full and causal.
ATTENTION_WORKLOADS = {
    w.name: w
    for w in [
        AttentionWorkload("attn_fwd_f16_b4_s1024_h8_d64_full", 4, 1024, 8, 64, "f16", False, 5),
        AttentionWorkload("attn_fwd_f16_b4_s1024_h8_d64_causal", 4, 1024, 8, 64, "f16", True, 6),
    ]
}


def attention_inputs(B: int, S: int, H: int, D: int, dtype: str, seed: int):
    """dict(Q=..., K=..., V=...) of uint16 bit arrays laid out [B, S, H, D]:
    torch.randn in fp32 in the order Q, K, V from one seeded generator,
    rounded to `dtype` (the page draws q, k, v with torch.randn)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    dt = _TORCH_DT[dtype]
    out = {}
    for name in ("Q", "K", "V"):
        out[name] = to_bits(torch.randn(B, S, H, D, generator=g, dtype=torch.float32).to(dt)).reshape(-1)
    return out
