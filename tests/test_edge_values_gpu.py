"""Edge values through the C ABI, in every kernel family, against the oracle:

  * fp16 output overflow: exact integer sums at and around the largest fp16
    value (65504; 65519 rounds down to it, 65520 is the tie that rounds to
    +inf, 65536 and up overflow), both signs -- round to nearest even with
    overflow to +-inf, subnormals kept;
  * negative zero: a row of zeros times an output scale of -1 gives -0 on
    both sides, and ReLU of negative sums gives zero;
  * non-finite inputs: +inf, -inf and NaN in A spread to their rows as IEEE
    arithmetic says (inf * 0 = NaN, ReLU of NaN is 0 as max(x, 0) takes it,
    GELU of -inf is NaN in the logistic form);
  * subnormal inputs: fp16 operands below 2^-14 (multiples of 2^-24), whose
    products and sums are exact in fp32, must come out bit for bit.

Integer-valued sums keep every fp32 step exact, so the comparisons are bit
for bit (NaN compared as NaN)."""
import numpy as np
import pytest
import torch

import oracle
from epilogue_gemm_amd import binding as gb
from epilogue_gemm_amd import inputs
from tests import parity

pytestmark = pytest.mark.gpu

# (family, config, M, N, K, layout_a, layout_b): the 64 x 64 tile (any layout),
# the 16x16x32 256 x 256 tile, the 32x32x16 256 x 256 tile, the skinny ring and
# the generic kernel
CASES = [
    ("tile", 2, 128, 192, 128, "row", "row"),
    ("tile", 4, 256, 256, 128, "row", "col"),
    ("tile", 0, 256, 256, 192, "col", "row"),
    ("skinny", 0, 24, 96, 1536, "row", "col"),
    ("generic", 0, 40, 50, 36, "row", "col"),
]

OVERFLOW_TARGETS = [65504, 65519, 65520, 65536, 131072, 65503, 1000, 0, 70000, 65535, 65488, 2**20]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gb.load_library()


def _bits(vals, fmt):
    return oracle.encode_array(fmt, np.asarray(vals, np.float64)).astype(np.uint16)


def _layout(x, layout):
    """Row-major logical R x C array -> bit array in the given layout."""
    return np.ascontiguousarray(x if layout == "row" else x.T)


def _run(A, B, bias, M, N, K, in_dt, out_dt, la, lb, epi, kernel, config, out_scale=None):
    dA, dB = parity.to_device(A, in_dt), parity.to_device(B, in_dt)
    dbias = parity.to_device(bias, in_dt) if bias is not None else None
    C = parity.empty_out(M * N, out_dt)
    C.fill_(12345.0 if out_dt != "f16" else 1234.0)
    osc = torch.tensor([out_scale], dtype=torch.float32, device="cuda") if out_scale is not None else None
    plan = gb.Plan(M, N, K, in_dt, out_dt, la, lb, epi, kernel, config)
    plan.run(dA, dB, dbias, C, out_scale=osc)
    torch.cuda.synchronize()
    name = plan.name
    plan.close()
    return parity.out_bits(C).reshape(M, N), name


def _same(got, want, fmt):
    """Bit-equal, except that NaNs need only both be NaN."""
    g, w = parity.values(got, fmt), parity.values(want, fmt)
    nan = np.isnan(w)
    return np.array_equal(np.isnan(g), nan) and np.array_equal(got[~nan], want[~nan].astype(got.dtype))


@pytest.mark.parametrize("kernel,config,M,N,K,la,lb", CASES)
@pytest.mark.parametrize("epi", ["none", "relu"])
def test_fp16_overflow_to_inf(kernel, config, M, N, K, la, lb, epi):
    # row i sums to +-target[i % len]: A holds the target's binary digits
    # (powers of two up to 2^15, exact in fp16) and B a column sign
    a = np.zeros((M, K))
    for i in range(M):
        t, k = OVERFLOW_TARGETS[i % len(OVERFLOW_TARGETS)], 0
        while t >= 32768:
            a[i, k], t, k = 32768.0, t - 32768, k + 1
        for bit in range(15, -1, -1):
            if t >> bit & 1:
                a[i, k], k = float(1 << bit), k + 1
        assert k <= K
    sign = np.where(np.arange(N) % 3 == 1, -1.0, 1.0)
    b = np.broadcast_to(sign, (K, N)).copy()
    A, B = _layout(_bits(a, "f16").reshape(M, K), la), _layout(_bits(b, "f16").reshape(K, N), lb)
    got, name = _run(A, B, None, M, N, K, "f16", "f16", la, lb, epi, kernel, config)
    _, want = oracle.gemm_epi(A, B, None, M, N, K, "f16", "f16", la, lb, epi)
    assert name.startswith(kernel if kernel != "generic" else "generic")
    assert _same(got, want, "f16"), f"{name}: {np.count_nonzero(got != want)} outputs differ"
    v = parity.values(got, "f16")
    # against numpy's correctly rounded fp64 -> fp16 conversion of the exact
    # sum: 65519 -> 65504, the 65520 tie and beyond -> +-inf, 65488 (a tie
    # between 65472 and 65504) -> 65472
    for i, t in enumerate(OVERFLOW_TARGETS[:min(M, len(OVERFLOW_TARGETS))]):
        with np.errstate(over="ignore"):
            expect = float(np.float16(float(t)))
        pos = v[i, sign > 0]
        assert np.all(pos == expect), (name, t, pos[:4])
        neg = v[i, sign < 0]
        assert np.all(neg == (0.0 if epi == "relu" else -expect)), (name, t, neg[:4])


@pytest.mark.parametrize("kernel,config,M,N,K,la,lb", CASES)
def test_negative_zero_and_relu_of_negatives(kernel, config, M, N, K, la, lb):
    bits = inputs.integer_inputs(M, N, K, "bf16", la, lb, True, seed=M + N)
    A = bits["A"].reshape(M, K) if la == "row" else bits["A"].reshape(K, M)
    A = A.copy()
    # row 1 of A all zeros: its sums are +0, its bias -0 keeps z = +0, and the
    # output scale -1 turns relu(+0) = +0 into -0 on both sides
    if la == "row":
        A[1, :] = 0
    else:
        A[:, 1] = 0
    bias = bits["bias"].copy()
    bias[:] = 0x8000  # -0 in bf16
    got, name = _run(A.reshape(-1), bits["B"], bias, M, N, K, "bf16", "bf16", la, lb, "bias_relu", kernel, config,
                     out_scale=-1.0)
    _, want = oracle.gemm_epi(A.reshape(-1), bits["B"], bias, M, N, K, "bf16", "bf16", la, lb, "bias_relu",
                              out_scale=-1.0)
    assert np.array_equal(got, want.astype(np.uint16)), f"{name}: {np.count_nonzero(got != want)} differ"
    assert np.all(got[1] == 0x8000)  # -0
    v = parity.values(got, "bf16")
    assert np.all(v <= 0) and np.count_nonzero(v == 0) > 0


@pytest.mark.parametrize("kernel,config,M,N,K,la,lb", CASES)
@pytest.mark.parametrize("epi", ["none", "relu", "bias_gelu"])
def test_nonfinite_inputs_propagate(kernel, config, M, N, K, la, lb, epi):
    bits = inputs.integer_inputs(M, N, K, "bf16", la, lb, epi.startswith("bias"), seed=K + len(epi))
    A = (bits["A"].reshape(M, K) if la == "row" else bits["A"].reshape(K, M).T).copy()
    A[3, 5], A[7, 9], A[11, 0] = 0x7F80, 0xFF80, 0x7FC0  # +inf, -inf, NaN
    A = _layout(A, la)
    got, name = _run(A.reshape(-1), bits["B"], bits["bias"], M, N, K, "bf16", "bf16", la, lb, epi, kernel, config)
    y, want = oracle.gemm_epi(A.reshape(-1), bits["B"], bits["bias"], M, N, K, "bf16", "bf16", la, lb, epi)
    g, w = parity.values(got, "bf16"), parity.values(want, "bf16")
    assert np.array_equal(np.isnan(g), np.isnan(w)), f"{name}: NaN positions differ"
    inf = np.isinf(w)
    assert np.array_equal(g[inf], w[inf]), f"{name}: infinities differ"
    fin = np.isfinite(w)
    assert np.count_nonzero(~fin) > 0
    if epi == "bias_gelu":
        r = parity.compare(got[fin], want[fin], y[fin], "bf16")
        assert r["ok"], f"{name}: {r}"
    else:
        assert np.array_equal(got[fin], want[fin].astype(np.uint16)), f"{name}: finite outputs differ"
    # rows 3, 7 and 11 are the only non-finite ones before the activation
    if epi == "none":
        bad = np.nonzero(~np.isfinite(g).all(axis=1))[0]
        assert set(bad.tolist()) <= {3, 7, 11}


@pytest.mark.parametrize("kernel,config,M,N,K,la,lb", CASES)
def test_fp16_subnormal_inputs(kernel, config, M, N, K, la, lb):
    # A: integer multiples of 2^-24 below 2^-14 (fp16 subnormals), B: integers
    # in [-2, 2]; every product and sum is exact in fp32
    g = torch.Generator().manual_seed(M * K)
    a = torch.randint(-1023, 1024, (M, K), generator=g).double().numpy() * 2.0**-24
    b = torch.randint(-2, 3, (K, N), generator=g).double().numpy()
    A, B = _layout(_bits(a, "f16").reshape(M, K), la), _layout(_bits(b, "f16").reshape(K, N), lb)
    for out_dt in ("f16", "f32"):
        got, name = _run(A.reshape(-1), B.reshape(-1), None, M, N, K, "f16", out_dt, la, lb, "none", kernel, config)
        _, want = oracle.gemm_epi(A.reshape(-1), B.reshape(-1), None, M, N, K, "f16", out_dt, la, lb, "none")
        mism = np.count_nonzero(got != want.astype(got.dtype))
        assert mism == 0, f"{name} -> {out_dt}: {mism} of {got.size} outputs differ"


def test_generic_launch_beyond_2_30_columns():
    # M = K = 1 runs on the generic kernel; N = 2^30 + 64 columns would need
    # more than 2^32 work-items along x with 256-thread rows of workgroups
    M, K, N = 1, 1, 2**30 + 64
    plan = gb.Plan(M, N, K, "bf16", "bf16", "row", "row", "none")
    assert plan.name == "generic"
    A = torch.tensor([2.0], dtype=torch.bfloat16, device="cuda")
    B = torch.arange(N, device="cuda", dtype=torch.int32).remainder_(7).sub_(3).to(torch.bfloat16)
    C = torch.full((N,), float("nan"), dtype=torch.bfloat16, device="cuda")
    plan.run(A, B, None, C)
    torch.cuda.synchronize()
    plan.close()
    cols = np.concatenate([np.arange(64), np.arange(N - 64, N), np.random.default_rng(0).integers(0, N, 256)])
    got = parity.out_bits(C[torch.from_numpy(cols).cuda()])
    # each output depends on its own column only: the oracle on those columns
    bsel = parity.out_bits(B[torch.from_numpy(cols).cuda()])
    _, want = oracle.gemm_epi(parity.out_bits(A), bsel, None, 1, cols.size, 1, "bf16", "bf16", "row", "row", "none")
    assert np.array_equal(got, want.reshape(-1).astype(np.uint16))
    del B, C


# K = 0, the degenerate product: the sum over k is empty, so C is the
# epilogue of zero -- act(bias), with the optional scale, residual and output
# scale -- on the generic kernel, with A and B passed as NULL.  Integer bias
# values keep the exact epilogues bit for bit; GELU and SiLU within the
# tolerance.
@pytest.mark.parametrize("in_dt,out_dt", [("bf16", "bf16"), ("f16", "f32"), ("f16", "f16"), ("bf16", "fp8")])
@pytest.mark.parametrize("la,lb", [("row", "col"), ("col", "row")])
def test_k_zero_is_the_epilogue_of_an_empty_sum(in_dt, out_dt, la, lb):
    M, N = 37, 200
    empty = np.zeros(0, np.uint16)
    for epi in ("none", "relu", "silu", "bias", "bias_relu", "bias_gelu", "bias_silu"):
        bits = inputs.integer_inputs(M, N, 8, in_dt, la, lb, epi.startswith("bias"), seed=len(epi))
        bias = bits["bias"]
        plan = gb.Plan(M, N, 0, in_dt, out_dt, la, lb, epi)
        assert plan.name == "generic"
        C = parity.empty_out(M * N, out_dt)
        C.fill_(float("nan"))
        plan.run(None, None, parity.to_device(bias, in_dt) if bias is not None else None, C)
        torch.cuda.synchronize()
        plan.close()
        got = parity.out_bits(C)
        y, c = oracle.gemm_epi(empty, empty, bias, M, N, 0, in_dt, out_dt, la, lb, epi)
        if epi in ("none", "relu", "bias", "bias_relu"):
            assert np.array_equal(got.reshape(-1), c.reshape(-1).astype(got.dtype)), epi
        else:
            r = parity.compare(got.reshape(-1), c.reshape(-1), y.reshape(-1), out_dt)
            assert r["ok"], f"{epi}: {r}"
    if out_dt in ("bf16", "f32"):
        # with the extras: act(s * 0 + bias) + r, times q
        bits = inputs.integer_inputs(M, N, 8, in_dt, la, lb, True, seed=11)
        ex = inputs.extras_inputs(M, N, out_dt, seed=11, integer=True)
        plan = gb.Plan(M, N, 0, in_dt, out_dt, la, lb, "bias_relu")
        C = parity.empty_out(M * N, out_dt)
        q = torch.tensor([0.5], dtype=torch.float32, device="cuda")
        plan.run(None, None, parity.to_device(bits["bias"], in_dt), C, scale=torch.from_numpy(ex["scale"]).cuda(),
                 residual=parity.to_device_out(ex["residual"], out_dt), out_scale=q)
        torch.cuda.synchronize()
        plan.close()
        got = parity.out_bits(C)
        y, c = oracle.gemm_epi(empty, empty, bits["bias"], M, N, 0, in_dt, out_dt, la, lb, "bias_relu",
                               scale=ex["scale"], residual=ex["residual"], out_scale=0.5)
        assert np.array_equal(got.reshape(-1), c.reshape(-1).astype(got.dtype))
