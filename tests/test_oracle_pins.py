"""Pins of the CPU oracle against things other than itself.

Every check here compares the oracle with an independent source: numpy's and
torch's own format conversions, exact rational arithmetic (fractions), closed
forms (identity, all-ones), torch's float64 matmul and tanh-GELU, and the
constants the pages print (tests/golden/page_constants.json).  The set is
chosen so that a dropped term, a wrong sign, a wrong index or a transposed
operand in the oracle fails at least one test.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from epilogue_gemm_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _np_f16_values(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def _torch_bf16_values(bits):
    t = torch.from_numpy(np.asarray(bits, np.uint16).view(np.int16).copy()).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


# --------------------------------------------------------------------------
# format decoding: exhaustive over every 16-bit pattern
# --------------------------------------------------------------------------

def test_decode_f16_exhaustive_vs_numpy():
    bits = np.arange(65536, dtype=np.uint32)
    got = oracle.decode_array("f16", bits)
    ref = _np_f16_values(bits.astype(np.uint16))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_decode_bf16_exhaustive_vs_torch():
    bits = np.arange(65536, dtype=np.uint32)
    got = oracle.decode_array("bf16", bits)
    ref = _torch_bf16_values(bits.astype(np.uint16))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_decode_f32_sample_vs_numpy():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    bits[:8] = [0, 0x80000000, 1, 0x007FFFFF, 0x00800000, 0x7F7FFFFF, 0x7F800000, 0xFF800000]
    got = oracle.decode_array("f32", bits)
    ref = bits.view(np.float32).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# --------------------------------------------------------------------------
# format encoding: one round-to-nearest-even step from fp64
# --------------------------------------------------------------------------

def _random_doubles(rng, n, lo_exp, hi_exp):
    mant = rng.uniform(1.0, 2.0, n)
    ex = rng.integers(lo_exp, hi_exp, n)
    sign = rng.choice([-1.0, 1.0], n)
    return sign * np.ldexp(mant, ex)


def test_encode_f16_vs_numpy_random():
    rng = np.random.default_rng(11)
    # normal, subnormal, underflow-to-zero and overflow ranges
    x = np.concatenate([_random_doubles(rng, 300_000, -30, 17), rng.standard_normal(100_000)])
    got = oracle.encode_array("f16", x).astype(np.uint16)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_encode_f16_constructed_ties():
    # ties between neighbours go to the even one; overflow edge at 65520
    cases = {
        1.0 + 2.0**-11: 0x3C00,  # halfway 1 and 1+2^-10 -> even (1.0)
        1.0 + 3 * 2.0**-11: 0x3C02,  # halfway 1+2^-10 and 1+2^-9 -> even (1+2^-9)
        1.0 + 2.0**-11 + 2.0**-40: 0x3C01,  # just above the tie -> up
        65504.0: 0x7BFF,
        65519.99: 0x7BFF,
        65520.0: 0x7C00,  # tie with 65536 -> even -> overflow to inf
        -65520.0: 0xFC00,
        2.0**-24: 0x0001,  # smallest subnormal
        2.0**-25: 0x0000,  # tie between 0 and 2^-24 -> even (0)
        3 * 2.0**-25: 0x0002,  # tie between 2^-24 and 2^-23 -> even
        -0.0: 0x8000,
    }
    for x, want in cases.items():
        assert oracle.encode("f16", x) == want, (x, hex(oracle.encode("f16", x)), hex(want))
        with np.errstate(over="ignore"):
            assert int(np.float16(x).view(np.uint16)) == want


def test_encode_f32_vs_numpy_random():
    rng = np.random.default_rng(12)
    x = np.concatenate([_random_doubles(rng, 300_000, -150, 129), rng.standard_normal(50_000)])
    got = oracle.encode_array("f32", x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float32).view(np.uint32)
    assert np.array_equal(got, ref)


def test_encode_bf16_vs_torch_on_f32_values():
    # torch rounds fp32 -> bf16 to nearest even; on fp32-representable inputs
    # that is a single rounding, so it must match the oracle's fp64 -> bf16.
    rng = np.random.default_rng(13)
    x32 = np.concatenate([_random_doubles(rng, 300_000, -133, 128), rng.standard_normal(50_000)]).astype(np.float32)
    x32 = x32[np.isfinite(x32)]
    got = oracle.encode_array("bf16", x32.astype(np.float64)).astype(np.uint16)
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_encode_bf16_single_rounding_from_f64():
    # values that an fp64 -> fp32 -> bf16 double rounding would get wrong
    cases = {
        1.0 + 2.0**-8: 0x3F80,  # exact tie -> even (1.0)
        1.0 + 3 * 2.0**-8: 0x3F82,  # exact tie -> even (1 + 2^-6)
        1.0 + 2.0**-8 + 2.0**-40: 0x3F81,  # above the tie: up (fp32 would have made it a tie)
        1.0 + 2.0**-8 - 2.0**-40: 0x3F80,  # below the tie: down
        -(1.0 + 2.0**-8 + 2.0**-40): 0xBF81,
        3.3895313892515355e38: 0x7F7F,  # largest finite bf16
        3.3961775292304718e38: 0x7F80,  # halfway to 2^128: tie -> even -> inf
    }
    for x, want in cases.items():
        assert oracle.encode("bf16", x) == want, (x, hex(oracle.encode("bf16", x)), hex(want))


def test_encode_decode_round_trip_all_patterns():
    for fmt in ("f16", "bf16"):
        bits = np.arange(65536, dtype=np.uint32)
        vals = oracle.decode_array(fmt, bits)
        finite = np.isfinite(vals)
        back = oracle.encode_array(fmt, vals)
        assert np.array_equal(back[finite], bits[finite])


# --------------------------------------------------------------------------
# GELU and the constants the pages print
# --------------------------------------------------------------------------

def test_page_constants_golden():
    g = json.load(open(os.path.join(GOLDEN, "page_constants.json")))
    c1, c2 = g["gelu_logistic_c1"]["value"], g["gelu_cubic_c2"]["value"]
    # the logistic constant is 2*sqrt(2/pi) to the printed 10 decimals
    assert abs(c1 - 2.0 * math.sqrt(2.0 / math.pi)) < 1e-10
    assert g["gelu_reference_mode"]["value"] == "tanh"
    # the oracle uses exactly the printed constants: at x where the cubic term
    # dominates, a changed c2 moves the value by far more than rounding
    for x in (-3.0, -1.7, -0.5, 0.25, 1.3, 2.9):
        want = x / (1.0 + math.exp(-c1 * (x + c2 * x * x * x)))
        assert oracle.gelu(x) == pytest.approx(want, rel=1e-15, abs=1e-300)


def test_gelu_vs_torch_tanh_gelu_f64():
    x = np.linspace(-12.0, 12.0, 20001)
    got = np.array([oracle.gelu(v) for v in x[::7]])
    ref = torch.nn.functional.gelu(torch.from_numpy(x[::7]), approximate="tanh").numpy()
    # constants agree to ~4e-12 relative; allow 1e-9 relative
    assert np.allclose(got, ref, rtol=1e-9, atol=1e-12)
    # and it is not the erf form (they differ by up to ~5e-4 near 2.7)
    erf_form = torch.nn.functional.gelu(torch.tensor([2.7], dtype=torch.float64)).item()
    assert abs(oracle.gelu(2.7) - erf_form) > 1e-5


def test_gelu_special_values():
    assert oracle.gelu(0.0) == 0.0
    assert oracle.gelu(40.0) == 40.0  # logistic factor rounds to 1
    assert oracle.gelu(-40.0) == 0.0 or abs(oracle.gelu(-40.0)) < 1e-300
    assert oracle.gelu(1.0) > 0.84 and oracle.gelu(-1.0) < 0.0


# --------------------------------------------------------------------------
# the contraction and the epilogues
# --------------------------------------------------------------------------

def _bits_of(vals, fmt):
    return oracle.encode_array(fmt, np.asarray(vals, np.float64)).astype(np.uint16)


def _values(bits, fmt):
    return oracle.decode_array(fmt, np.asarray(bits).astype(np.uint32))


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_identity_gives_b(fmt):
    # A = I (K x K), C = round(B) exactly, both layouts of B
    K, N = 48, 40
    rng = np.random.default_rng(3)
    b = rng.standard_normal((K, N))
    b_bits = _bits_of(b, fmt)
    a_bits = _bits_of(np.eye(K), fmt)
    for lb in ("row", "col"):
        B = b_bits if lb == "row" else np.ascontiguousarray(b_bits.T)
        y, c = oracle.gemm_epi(a_bits, B, None, K, N, K, fmt, fmt, "row", lb, "none")
        assert np.array_equal(c, b_bits)
        assert np.array_equal(y, _values(b_bits, fmt))


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("K", [1, 7, 256, 1024, 4096, 8192])
def test_all_ones_gives_k(fmt, K):
    M, N = 3, 5
    one, minus_one = _bits_of([1.0], fmt)[0], _bits_of([-1.0], fmt)[0]
    A = np.full(M * K, one, np.uint16)
    B = np.full(K * N, one, np.uint16)
    y, c = oracle.gemm_epi(A, B, None, M, N, K, fmt, "f32", "row", "col", "none")
    assert np.all(y == K)
    # ReLU of -K is 0; ReLU of +K is K
    An = np.full(M * K, minus_one, np.uint16)
    y, _ = oracle.gemm_epi(An, B, None, M, N, K, fmt, fmt, "row", "row", "relu")
    assert np.all(y == 0.0)
    y, _ = oracle.gemm_epi(A, B, None, M, N, K, fmt, fmt, "row", "row", "relu")
    assert np.all(y == K)
    # bias is added per column, before the activation
    bias_vals = np.array([0.5, -0.25, 2.0, -K - 1.0, 0.0])
    bias = _bits_of(bias_vals, fmt)
    bv = _values(bias, fmt)
    y, _ = oracle.gemm_epi(A, B, bias, M, N, K, fmt, "f32", "row", "col", "bias")
    assert np.array_equal(y, np.broadcast_to(K + bv, (M, N)))
    y, _ = oracle.gemm_epi(A, B, bias, M, N, K, fmt, "f32", "row", "col", "bias_relu")
    assert np.array_equal(y, np.broadcast_to(np.maximum(K + bv, 0.0), (M, N)))
    # bias before GELU: GELU(K + b), which differs from GELU(K) + b
    y, _ = oracle.gemm_epi(A, B, bias, M, N, K, fmt, "f32", "row", "col", "bias_gelu")
    want = np.array([oracle.gelu(K + v) for v in bv])
    assert np.array_equal(y, np.broadcast_to(want, (M, N)))
    # and with A = -1 the bias decides the sign under ReLU
    y, _ = oracle.gemm_epi(An, B, bias, M, N, K, fmt, "f32", "row", "col", "bias_relu")
    assert np.array_equal(y, np.broadcast_to(np.maximum(-K + bv, 0.0), (M, N)))


def _exact_reference(a_vals, b_vals, bias_vals, epilogue):
    """Exact rational z = A.B [+ bias] and, for the piecewise-linear epilogues,
    the exact activation."""
    M, K = a_vals.shape
    N = b_vals.shape[1]
    fa = [[Fraction(float(a_vals[i, k])) for k in range(K)] for i in range(M)]
    fb = [[Fraction(float(b_vals[k, j])) for j in range(N)] for k in range(K)]
    out = []
    for i in range(M):
        row = []
        for j in range(N):
            z = sum((fa[i][k] * fb[k][j] for k in range(K)), Fraction(0))
            if epilogue in ("bias", "bias_relu", "bias_gelu"):
                z += Fraction(float(bias_vals[j]))
            if epilogue in ("relu", "bias_relu"):
                z = max(z, Fraction(0))
            row.append(z)
        out.append(row)
    return out


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(2, 8, 4), (1, 1, 1), (3, 5, 7), (4, 2, 16), (5, 7, 3), (8, 16, 8), (16, 3, 2)])
@pytest.mark.parametrize("epilogue", ["none", "relu", "bias", "bias_relu"])
def test_brute_force_exact(fmt, shape, epilogue):
    M, N, K = shape
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    a = _values(_bits_of(rng.standard_normal((M, K)) * 3, fmt), fmt).reshape(M, K)
    b = _values(_bits_of(rng.standard_normal((K, N)), fmt), fmt).reshape(K, N)
    bias = _values(_bits_of(rng.standard_normal(N), fmt), fmt)
    exact = _exact_reference(a, b, bias, epilogue)
    a_bits, b_bits = _bits_of(a, fmt).reshape(M, K), _bits_of(b, fmt).reshape(K, N)
    bias_bits = _bits_of(bias, fmt) if epilogue.startswith("bias") else None
    for la in ("row", "col"):
        for lb in ("row", "col"):
            A = a_bits if la == "row" else np.ascontiguousarray(a_bits.T)
            B = b_bits if lb == "row" else np.ascontiguousarray(b_bits.T)
            y, c = oracle.gemm_epi(A, B, bias_bits, M, N, K, fmt, fmt, la, lb, epilogue)
            for i in range(M):
                for j in range(N):
                    e = exact[i][j]
                    # fp64 sum of at most 16 exact products: within a few ulp of exact
                    scale = float(sum(abs(Fraction(float(a[i, k])) * Fraction(float(b[k, j]))) for k in range(K)))
                    scale += abs(float(bias[j])) if bias_bits is not None else 0.0
                    assert abs(y[i, j] - float(e)) <= 4 * 2.0**-52 * max(scale, 1e-300), (i, j)
                    # the output is the correctly rounded exact value, unless the
                    # exact value sits within fp64 noise of a rounding tie
                    want = int(np.float16(float(e)).view(np.uint16)) if fmt == "f16" else None
                    if fmt == "bf16":
                        want = oracle.encode("bf16", float(e))
                    got = int(c[i, j])
                    if got != want:
                        lo_v, hi_v = sorted([oracle.decode(fmt, got), oracle.decode(fmt, want)])
                        mid = (Fraction(lo_v) + Fraction(hi_v)) / 2
                        assert abs(e - mid) <= Fraction(scale) * Fraction(2) ** -50, (i, j, got, want)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_matches_torch_matmul_f64(fmt):
    M, N, K = 37, 53, 129
    rng = np.random.default_rng(5)
    a_bits = _bits_of(rng.standard_normal((M, K)), fmt).reshape(M, K)
    b_bits = _bits_of(rng.standard_normal((K, N)) / 8, fmt).reshape(K, N)
    bias_bits = _bits_of(rng.standard_normal(N) * 0.1, fmt)
    a = torch.from_numpy(_values(a_bits, fmt).reshape(M, K))
    b = torch.from_numpy(_values(b_bits, fmt).reshape(K, N))
    bias = torch.from_numpy(_values(bias_bits, fmt))
    ref = a @ b
    y, _ = oracle.gemm_epi(a_bits, np.ascontiguousarray(b_bits.T), None, M, N, K, fmt, "f32", "row", "col", "none")
    assert np.allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)
    y, _ = oracle.gemm_epi(a_bits, b_bits, bias_bits, M, N, K, fmt, "f32", "row", "row", "bias_gelu")
    ref_g = torch.nn.functional.gelu(ref + bias, approximate="tanh")
    assert np.allclose(y, ref_g.numpy(), rtol=1e-9, atol=1e-12)
    y, _ = oracle.gemm_epi(a_bits, b_bits, bias_bits, M, N, K, fmt, "f32", "row", "row", "bias_relu")
    assert np.allclose(y, torch.relu(ref + bias).numpy(), rtol=1e-12, atol=1e-12)


def test_layouts_are_bitwise_equivalent():
    M, N, K = 19, 23, 31
    d = inputs.make_inputs(M, N, K, "bf16", "row", "row", True, 4.0, 0.1, 9)
    A, B, bias = d["A"].reshape(M, K), d["B"].reshape(K, N), d["bias"]
    ref_y, ref_c = oracle.gemm_epi(A, B, bias, M, N, K, "bf16", "bf16", "row", "row", "bias_gelu")
    for la in ("row", "col"):
        for lb in ("row", "col"):
            Aa = A if la == "row" else np.ascontiguousarray(A.T)
            Bb = B if lb == "row" else np.ascontiguousarray(B.T)
            y, c = oracle.gemm_epi(Aa, Bb, bias, M, N, K, "bf16", "bf16", la, lb, "bias_gelu")
            assert np.array_equal(y, ref_y) and np.array_equal(c, ref_c)


def test_points_match_full_product():
    M, N, K = 33, 65, 70
    d = inputs.make_inputs(M, N, K, "f16", "row", "col", True, 8.0, 0.1, 10)
    y, c = oracle.gemm_epi(d["A"], d["B"], d["bias"], M, N, K, "f16", "f16", "row", "col", "bias_gelu")
    rng = np.random.default_rng(0)
    rows, cols = rng.integers(0, M, 300), rng.integers(0, N, 300)
    py, pb = oracle.gemm_epi_points(d["A"], d["B"], d["bias"], M, N, K, "f16", "f16", "row", "col", "bias_gelu",
                                    rows, cols)
    assert np.array_equal(py, y[rows, cols])
    assert np.array_equal(pb.astype(np.uint16), c[rows, cols])


def test_output_rounding_is_single_rne_of_y():
    M, N, K = 16, 24, 40
    d = inputs.make_inputs(M, N, K, "bf16", "row", "col", True, 4.0, 0.1, 21)
    y, c = oracle.gemm_epi(d["A"], d["B"], d["bias"], M, N, K, "bf16", "bf16", "row", "col", "bias_gelu")
    # torch's fp64 -> bf16 goes through fp32 (two roundings); compare where the
    # two agree by construction: values already exact in fp32
    y32 = y.astype(np.float32).astype(np.float64)
    exact32 = y32 == y
    ref = torch.from_numpy(y.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(c[exact32], ref[exact32])
    # and f16 output against numpy's direct fp64 -> fp16
    d = inputs.make_inputs(M, N, K, "f16", "row", "col", False, 4.0, 0.0, 22)
    y, c = oracle.gemm_epi(d["A"], d["B"], None, M, N, K, "f16", "f16", "row", "col", "relu")
    assert np.array_equal(c, y.astype(np.float16).view(np.uint16))


def test_rejects_bad_arguments():
    A = np.zeros(4, np.uint16)
    with pytest.raises(ValueError):
        oracle.gemm_epi(A, A, None, 2, 2, 2, "f16", "bf16", "row", "row", "none")  # mixed out format
    with pytest.raises(ValueError):
        oracle.gemm_epi(A, A, None, 2, 2, 2, "f16", "f16", "row", "row", "bias")  # missing bias
    with pytest.raises(ValueError):
        oracle.gemm_epi(A, A, None, 2, 3, 2, "f16", "f16", "row", "row", "none")  # size mismatch


# K = 0: the sum over k is empty, so the product is zero and the output is the
# epilogue of zero -- act(bias), scaled zero, the residual added, the output
# scale applied -- for every layout (A and B are empty arrays).
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_k_zero_is_the_epilogue_of_an_empty_sum(fmt):
    M, N = 3, 11
    e = np.zeros(0, np.uint16)
    vals = np.array([-3.0, -1.0, -0.5, 0.0, 0.25, 0.5, 1.0, 2.0, 3.0, 6.0, -6.0])
    bias = oracle.encode_array(fmt, vals).astype(np.uint16)
    bd = np.array([oracle.decode(fmt, int(b)) for b in bias])
    t = torch.from_numpy(bd)
    want = {"none": np.zeros(N), "relu": np.zeros(N), "silu": np.zeros(N), "bias": bd,
            "bias_relu": np.maximum(bd, 0.0),
            "bias_gelu": torch.nn.functional.gelu(t, approximate="tanh").numpy(),
            "bias_silu": torch.nn.functional.silu(t).numpy()}
    for la, lb in (("row", "col"), ("col", "row")):
        for epi, w in want.items():
            y, c = oracle.gemm_epi(e, e, bias if epi.startswith("bias") else None, M, N, 0, fmt, "f32", la, lb, epi)
            # (the page constants of GELU agree with the tanh form to ~4e-12)
            assert np.allclose(y, np.broadcast_to(w, (M, N)), rtol=1e-9, atol=1e-12), (la, lb, epi)
            if epi in ("none", "relu", "bias", "bias_relu"):
                assert np.array_equal(y, np.broadcast_to(w, (M, N)))
    # with the extras: act(s * 0 + bias) + r, times q
    scale = np.full(N, 7.0, np.float32)
    res = np.arange(M * N, dtype=np.float32)
    y, _ = oracle.gemm_epi(e, e, bias, M, N, 0, fmt, "f32", "row", "col", "bias_relu", scale=scale, residual=res,
                           out_scale=0.5)
    assert np.array_equal(y, 0.5 * (np.maximum(bd, 0.0)[None, :] + np.arange(M * N).reshape(M, N)))


# --------------------------------------------------------------------------
# further epilogues: SiLU, per-column scale, residual
# --------------------------------------------------------------------------

def test_silu_vs_torch_and_closed_forms():
    x = np.linspace(-30.0, 30.0, 6001)
    got = np.array([oracle.silu(v) for v in x])
    # torch's float64 SiLU (a library routine)
    ref = torch.nn.functional.silu(torch.from_numpy(x)).numpy()
    assert np.allclose(got, ref, rtol=1e-14, atol=1e-300)
    # x * sigmoid(x) = (x / 2) (1 + tanh(x / 2)): a different transcendental
    # (which cancels for x << 0, hence the absolute term)
    alt = 0.5 * x * (1.0 + np.tanh(0.5 * x))
    assert np.allclose(got, alt, rtol=1e-13, atol=1e-13)
    # silu(x) - silu(-x) = x (sigmoid(x) + sigmoid(-x) = 1); slope 1/2 at 0
    neg = np.array([oracle.silu(-v) for v in x])
    assert np.allclose(got - neg, x, rtol=1e-14, atol=1e-14)
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(1e-8) == pytest.approx(0.5e-8, rel=1e-7)
    assert oracle.silu(40.0) == 40.0
    assert oracle.silu(-800.0) == 0.0
    # its minimum is at x = -1.2784645 with value -0.2784645 (the root of
    # 1 + x (1 - sigmoid(x)) = 0, where silu(x) = -(1 + x))
    xs = np.linspace(-1.3, -1.25, 5001)
    v = np.array([oracle.silu(t) for t in xs])
    assert xs[np.argmin(v)] == pytest.approx(-1.2784645, abs=2e-5)
    assert v.min() == pytest.approx(-0.2784645, abs=1e-6)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("K", [1, 64, 4096])
def test_all_ones_with_scale_and_residual(fmt, K):
    M, N = 3, 5
    one = _bits_of([1.0], fmt)[0]
    A = np.full(M * K, one, np.uint16)
    B = np.full(K * N, one, np.uint16)
    s = np.array([0.5, -2.0, 0.25, 3.0, 1.0], np.float32)
    bias = _bits_of([1.0, 0.5, -3.0, -1.0, 0.0], fmt)
    bv = _values(bias, fmt)
    r_vals = np.arange(M * N, dtype=np.float64).reshape(M, N) - 6.0
    r = oracle.encode_array("f32", r_vals)
    # the scale multiplies the product, then the bias is added
    y, _ = oracle.gemm_epi(A, B, bias, M, N, K, fmt, "f32", "row", "col", "bias", scale=s)
    assert np.array_equal(y, np.broadcast_to(s * K + bv, (M, N)))
    # ...then the activation, then the residual
    y, _ = oracle.gemm_epi(A, B, bias, M, N, K, fmt, "f32", "row", "col", "bias_relu", scale=s, residual=r)
    assert np.array_equal(y, np.maximum(s * K + bv, 0.0) + r_vals)
    y, _ = oracle.gemm_epi(A, B, None, M, N, K, fmt, "f32", "row", "col", "relu", residual=r)
    assert np.array_equal(y, K + r_vals)
    y, _ = oracle.gemm_epi(A, B, bias, M, N, K, fmt, "f32", "row", "row", "bias_silu", scale=s)
    want = np.array([oracle.silu(s[j] * K + bv[j]) for j in range(N)])
    assert np.array_equal(y, np.broadcast_to(want, (M, N)))
    y, _ = oracle.gemm_epi(A, B, None, M, N, K, fmt, "f32", "row", "row", "silu")
    assert np.all(y == oracle.silu(float(K)))
    # residual in a 16-bit output format
    r16 = _bits_of(r_vals.reshape(-1), fmt)
    y, c = oracle.gemm_epi(A, B, None, M, N, K, fmt, fmt, "row", "col", "none", residual=r16)
    assert np.array_equal(y, K + _values(r16, fmt).reshape(M, N))
    assert np.array_equal(c.reshape(-1), oracle.encode_array(fmt, y.reshape(-1)).astype(np.uint16))


def _exact_reference_ex(a_vals, b_vals, bias_vals, scale, resid, epilogue):
    """Exact rational act(s * A.B + bias) + r for the piecewise-linear epilogues."""
    z = _exact_reference(a_vals, b_vals, None, "none")
    M, N = len(z), len(z[0])
    out = []
    for i in range(M):
        row = []
        for j in range(N):
            v = z[i][j] * Fraction(float(scale[j]))
            if epilogue in ("bias", "bias_relu"):
                v += Fraction(float(bias_vals[j]))
            if epilogue in ("relu", "bias_relu"):
                v = max(v, Fraction(0))
            row.append(v + Fraction(float(resid[i, j])))
        out.append(row)
    return out


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(2, 8, 4), (3, 5, 7), (5, 7, 3)])
@pytest.mark.parametrize("epilogue", ["none", "relu", "bias", "bias_relu"])
def test_brute_force_exact_scale_residual(fmt, shape, epilogue):
    M, N, K = shape
    rng = np.random.default_rng(M * 1000 + N * 10 + K)
    a = _values(_bits_of(rng.standard_normal((M, K)) * 3, fmt), fmt).reshape(M, K)
    b = _values(_bits_of(rng.standard_normal((K, N)), fmt), fmt).reshape(K, N)
    bias = _values(_bits_of(rng.standard_normal(N), fmt), fmt)
    scale = rng.standard_normal(N).astype(np.float32)
    resid = _values(_bits_of(rng.standard_normal(M * N), "f32").astype(np.uint32), "f32").reshape(M, N)
    exact = _exact_reference_ex(a, b, bias, scale, resid, epilogue)
    bias_bits = _bits_of(bias, fmt) if epilogue.startswith("bias") else None
    y, c = oracle.gemm_epi(_bits_of(a, fmt), np.ascontiguousarray(_bits_of(b, fmt).reshape(K, N).T), bias_bits,
                           M, N, K, fmt, "f32", "row", "col", epilogue, scale=scale,
                           residual=oracle.encode_array("f32", resid.reshape(-1)))
    for i in range(M):
        for j in range(N):
            mag = float(sum(abs(Fraction(float(a[i, k])) * Fraction(float(b[k, j]))) for k in range(K)))
            mag = mag * abs(float(scale[j])) + abs(float(bias[j])) + abs(float(resid[i, j]))
            assert abs(y[i, j] - float(exact[i][j])) <= 8 * 2.0**-52 * max(mag, 1e-300), (i, j)


def test_silu_matches_torch_on_a_product():
    fmt, M, N, K = "bf16", 29, 41, 96
    rng = np.random.default_rng(12)
    a_bits = _bits_of(rng.standard_normal((M, K)), fmt).reshape(M, K)
    b_bits = _bits_of(rng.standard_normal((K, N)) / 8, fmt).reshape(K, N)
    bias_bits = _bits_of(rng.standard_normal(N) * 0.1, fmt)
    scale = (rng.random(N) + 0.5).astype(np.float32)
    r_bits = _bits_of(rng.standard_normal(M * N), fmt)
    a = torch.from_numpy(_values(a_bits, fmt).reshape(M, K))
    b = torch.from_numpy(_values(b_bits, fmt).reshape(K, N))
    ref = torch.nn.functional.silu((a @ b) * torch.from_numpy(scale.astype(np.float64))
                                   + torch.from_numpy(_values(bias_bits, fmt)))
    ref = ref + torch.from_numpy(_values(r_bits, fmt).reshape(M, N))
    y, _ = oracle.gemm_epi(a_bits, b_bits, bias_bits, M, N, K, fmt, fmt, "row", "row", "bias_silu", scale=scale,
                           residual=r_bits)
    assert np.allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)
    # the points entry computes the same values
    rows, cols = rng.integers(0, M, 50), rng.integers(0, N, 50)
    py, _ = oracle.gemm_epi_points(a_bits, b_bits, bias_bits, M, N, K, fmt, fmt, "row", "row", "bias_silu", rows,
                                   cols, scale=scale, residual=r_bits)
    assert np.array_equal(py, y[rows, cols])


def test_rejects_bad_extras():
    A = np.zeros(4, np.uint16)
    with pytest.raises(ValueError):
        oracle.gemm_epi(A, A, None, 2, 2, 2, "f16", "f16", "row", "row", "none", scale=np.ones(3, np.float32))
    with pytest.raises(ValueError):
        oracle.gemm_epi(A, A, None, 2, 2, 2, "f16", "f16", "row", "row", "none", residual=np.zeros(4, np.uint32))
    with pytest.raises(ValueError):
        oracle.gemm_epi(A, A, None, 2, 2, 2, "f16", "f16", "row", "row", "bias_silu")  # missing bias


# --------------------------------------------------------------------------
# FP8 E4M3 output (OCP 8-bit floating point, E4M3 variant) and output scale
# --------------------------------------------------------------------------

def _torch_e4m3_values(codes):
    t = torch.from_numpy(np.asarray(codes, np.uint8).copy()).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def test_decode_fp8_exhaustive_vs_torch():
    codes = np.arange(256, dtype=np.uint32)
    got = oracle.decode_array("fp8", codes)
    ref = _torch_e4m3_values(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2  # S.1111.111 only
    assert np.array_equal(got[~nan], ref[~nan])
    assert oracle.decode("fp8", 0x7E) == 448.0 and oracle.decode("fp8", 0x01) == 2.0**-9
    assert oracle.decode("fp8", 0x08) == 2.0**-6 and oracle.decode("fp8", 0xB8) == -1.0


def test_encode_fp8_vs_torch_in_range():
    # torch's fp32 -> e4m3fn conversion is round-to-nearest-even; inside the
    # finite range it must agree with the oracle on fp32-representable values
    rng = np.random.default_rng(17)
    x = np.concatenate([rng.standard_normal(200000) * 40, rng.standard_normal(50000) * 0.01,
                        np.ldexp(rng.random(20000), rng.integers(-12, 9, 20000))])
    x = x.astype(np.float32)
    x = x[np.abs(x) < 448]
    got = oracle.encode_array("fp8", x.astype(np.float64)).astype(np.uint8)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_encode_fp8_ties_and_saturation():
    enc = lambda v: oracle.encode("fp8", v)  # noqa: E731
    # ties to even in the normal range: 1 + 1/16 between 1 and 1.125 -> 1;
    # 1 + 3/16 between 1.125 and 1.25 -> 1.25
    assert enc(1.0 + 1 / 16) == 0x38 and enc(1.0 + 3 / 16) == 0x3A
    assert enc(1.0 + 1 / 16 + 2.0**-30) == 0x39  # just above the tie
    # subnormal ties: half the smallest step rounds to 0, 1.5 steps to 2 steps
    assert enc(2.0**-10) == 0x00 and enc(3 * 2.0**-10) == 0x02 and enc(-(2.0**-10)) == 0x80
    # carry out of the subnormal range into the first normal binade
    assert enc(7.5 * 2.0**-9) == 0x08
    # saturation at +-448 (no infinities in E4M3), NaN stays NaN
    for v, code in ((448.0, 0x7E), (460.0, 0x7E), (464.0, 0x7E), (1e30, 0x7E), (math.inf, 0x7E),
                    (-500.0, 0xFE), (-math.inf, 0xFE), (416.0, 0x7D), (432.0, 0x7E)):
        assert enc(v) == code, (v, hex(enc(v)))
    assert enc(math.nan) == 0x7F
    # every finite code is its own encoding
    for c in range(256):
        v = oracle.decode("fp8", c)
        if not math.isnan(v):
            assert enc(v) == c, c


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_fp8_output_all_ones_and_out_scale(fmt):
    M, N = 2, 3
    one = _bits_of([1.0], fmt)[0]
    for K, q, want in ((64, None, 64.0), (256, None, 256.0), (1024, None, 448.0), (1024, 0.25, 256.0),
                       (96, 1.0, 96.0), (100, 1.0, 96.0), (104, 1.0, 104.0), (9, 0.5, 4.5)):
        A = np.full(M * K, one, np.uint16)
        B = np.full(K * N, one, np.uint16)
        y, c = oracle.gemm_epi(A, B, None, M, N, K, fmt, "fp8", "row", "col", "none", out_scale=q)
        assert c.dtype == np.uint8
        assert np.all(oracle.decode_array("fp8", c.reshape(-1).astype(np.uint32)) == want), (K, q)
        assert np.all(y == K * (q if q is not None else 1.0))
    # 100 lies between the codes for 96 and 104 (spacing 8): ties to even -> 96;
    # and the output scale multiplies after the activation, for any format
    A = np.full(M * 8, one, np.uint16)
    B = np.full(8 * N, one, np.uint16)
    bias = _bits_of([1.0, -20.0, 0.5], fmt)
    y, c = oracle.gemm_epi(A, B, bias, M, N, 8, fmt, "f32", "row", "col", "bias_relu", out_scale=-2.0)
    assert np.array_equal(y, np.broadcast_to(-2.0 * np.maximum(8.0 + _values(bias, fmt), 0.0), (M, N)))


def _e4m3_brute_force(x):
    """Nearest E4M3 code of each fp64 value by exhaustive search over the
    finite codes (decoded by torch), ties to the code with an even last
    fraction bit, saturating at +-448 -- no frexp/ldexp arithmetic, so it
    shares nothing with the oracle's encoder."""
    codes = np.arange(256, dtype=np.uint8)
    vals = _torch_e4m3_values(codes)
    fin = ~np.isnan(vals)
    codes, vals = codes[fin], vals[fin]
    out = np.empty(len(x), np.uint8)
    for i, v in enumerate(x):
        if np.isnan(v):
            out[i] = 0x7F
            continue
        c = min(max(v, -448.0), 448.0)
        d = np.abs(vals - c)
        best = np.nonzero(d == d.min())[0]
        if len(best) > 1:  # a tie (or +-0): the even code, positive zero's sign from v
            even = [b for b in best if codes[b] & 1 == 0]
            best = [b for b in even if (codes[b] >> 7) == (1 if np.signbit(v) else 0)] or even
        out[i] = codes[best[0]]
    return out


def test_encode_fp8_single_rounding_from_fp64_brute_force():
    # values that are not fp32-representable (so a rounding through fp32 would
    # show), against an exhaustive nearest-code search
    rng = np.random.default_rng(23)
    x = np.concatenate([rng.standard_normal(4000) * 40, rng.standard_normal(1000) * 0.02,
                        np.ldexp(rng.random(2000) + 1.0, rng.integers(-11, 9, 2000)),
                        [500.0, -1e9, 0.0, -0.0, np.nan]])
    # push a quarter of them onto near-ties: a midpoint between two codes plus
    # or minus a few fp64 ulps (below fp32 resolution)
    codes = np.arange(0, 0x7E, dtype=np.uint8)
    v = _torch_e4m3_values(codes)
    mids = (v[:-1] + v[1:]) / 2
    pick = mids[rng.integers(0, len(mids), 3000)]
    off = rng.choice([-1.0, 1.0], 3000) * np.ldexp(1.0, rng.integers(-45, -30, 3000)) * np.maximum(pick, 2.0**-9)
    sgn = rng.choice([-1.0, 1.0], 3000)
    x = np.concatenate([x, sgn * (pick + off), sgn * pick])
    got = oracle.encode_array("fp8", x.astype(np.float64)).astype(np.uint8)
    assert np.array_equal(got, _e4m3_brute_force(x))


def test_fp8_output_rounded_once_from_fp64():
    # A value just above (or below) an E4M3 tie by less than half an fp32 ulp
    # goes to the nearer code: the output is rounded once, from the fp64
    # value, like every other output format.
    fmt, M, N, K = "f16", 1, 1, 2
    a = _bits_of([1.0, 1.0], fmt)
    # 1 + 1/16 lies halfway between the codes 1 (0x38) and 1.125 (0x39)
    b = _bits_of([1.0 + 1 / 16, 2.0**-20], fmt)
    y, c = oracle.gemm_epi(a, b, None, M, N, K, fmt, "fp8", "row", "row", "none")
    assert y[0, 0] == 1.0 + 1 / 16 + 2.0**-20 and c[0, 0] == 0x39
    # 1 + 1/16 + 2^-24 (the smallest fp16 subnormal as the second product):
    # fp32 would round this onto the tie, which goes to even (0x38); one
    # rounding from fp64 gives the upper neighbour
    b = _bits_of([1.0 + 1 / 16, 2.0**-24], fmt)
    y, c = oracle.gemm_epi(a, b, None, M, N, K, fmt, "fp8", "row", "row", "none")
    assert y[0, 0] == 1.0 + 1 / 16 + 2.0**-24 and c[0, 0] == 0x39
    # and just below the tie, by the same amount: the lower neighbour
    b = _bits_of([1.0 + 1 / 16, -(2.0**-24)], fmt)
    y, c = oracle.gemm_epi(a, b, None, M, N, K, fmt, "fp8", "row", "row", "none")
    assert y[0, 0] == 1.0 + 1 / 16 - 2.0**-24 and c[0, 0] == 0x38
    # bf16: 2^-30 above the tie between 1.125 and 1.25 (1 + 3/16, which goes
    # to the even 1.25 = 0x3A when exact) is still the upper code; 2^-30
    # below is the lower one
    abf = _bits_of([1.0, 1.0], "bf16")
    for extra, want in ((2.0**-30, 0x3A), (-(2.0**-30), 0x39), (0.0, 0x3A)):
        bf = _bits_of([1.0 + 3 / 16, extra], "bf16")
        y, c = oracle.gemm_epi(abf, bf, None, M, N, K, "bf16", "fp8", "row", "row", "none")
        assert y[0, 0] == 1.0 + 3 / 16 + extra and c[0, 0] == want, (extra, hex(c[0, 0]))
    # the exact tie 1 + 1/16 goes to even (0x38), as torch's fp32 -> e4m3fn does
    ref = torch.tensor([1.0 + 1 / 16], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).item()
    b = _bits_of([1.0 + 1 / 16, 0.0], fmt)
    y, c = oracle.gemm_epi(a, b, None, M, N, K, fmt, "fp8", "row", "row", "none")
    assert c[0, 0] == ref == 0x38


def test_fp8_rejects_residual():
    A = np.zeros(4, np.uint16)
    with pytest.raises(ValueError):
        oracle.gemm_epi(A, A, None, 2, 2, 2, "f16", "fp8", "row", "row", "none", residual=np.zeros(4, np.uint8))
