"""Leading dimensions (gemm_epi_plan_set_ld): every kernel family computes
the product of sub-matrices of larger arrays.  The padding between rows of
A and B holds NaN bit patterns (a read of it would poison the result) and
the padding of C holds a sentinel that must survive; integer operands make
the comparison with the oracle (on packed copies) bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from epilogue_gemm_amd import binding as gb
from epilogue_gemm_amd import inputs
from tests import parity

pytestmark = pytest.mark.gpu

NAN16 = {"f16": 0x7E00, "bf16": 0x7FC0}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gb.load_library()


def _pad(mat, ld, fill):
    """rows x cols bit array -> rows x ld with `fill` in the padding."""
    rows, cols = mat.shape
    out = np.full((rows, ld), fill, mat.dtype)
    out[:, :cols] = mat
    return out


def run_strided(M, N, K, in_dt, out_dt, la, lb, epi, pads, kernel="auto", config=-1, extras=False, extra_rows=0):
    """Run with leading dimensions padded by pads = (A, B, C), NaN in A's and
    B's padding, a sentinel in C's padding and in extra_rows rows of C past
    row M; check C's M x N outputs bit for bit and that no padding changed."""
    bits = inputs.integer_inputs(M, N, K, in_dt, la, lb, epi.startswith("bias"), seed=M + N + K)
    a_shape = (M, K) if la == "row" else (K, M)
    b_shape = (K, N) if lb == "row" else (N, K)
    lda, ldb, ldc = a_shape[1] + pads[0], b_shape[1] + pads[1], N + pads[2]
    A = parity.to_device(_pad(bits["A"].reshape(a_shape), lda, NAN16[in_dt]), in_dt)
    B = parity.to_device(_pad(bits["B"].reshape(b_shape), ldb, NAN16[in_dt]), in_dt)
    bias = parity.to_device(bits["bias"], in_dt) if bits["bias"] is not None else None
    sentinel = {"f16": 0x3C01, "bf16": 0x3F81, "f32": 0x3F800001, "fp8": 0x39}[out_dt]
    np_out = {"f32": np.uint32, "fp8": np.uint8}.get(out_dt, np.uint16)
    C = parity.to_device_out(np.full((M + extra_rows) * ldc, sentinel, np_out), out_dt)
    plan = gb.Plan(M, N, K, in_dt, out_dt, la, lb, epi, kernel, config, lda=lda, ldb=ldb, ldc=ldc)
    ex = inputs.extras_inputs(M, N, out_dt, seed=3, integer=True) if extras else None
    res = None
    if extras and ex["residual"] is not None:
        res = parity.to_device_out(_pad(ex["residual"].reshape(M, N), ldc, 0).reshape(-1), out_dt)
    sc = torch.from_numpy(ex["scale"]).cuda() if extras else None
    plan.run(A, B, bias, C, scale=sc, residual=res)
    torch.cuda.synchronize()
    got_all = parity.out_bits(C).reshape(M + extra_rows, ldc)
    got = got_all[:M]
    name = plan.name
    plan.close()
    y, c = oracle.gemm_epi(bits["A"], bits["B"], bits["bias"], M, N, K, in_dt, out_dt, la, lb, epi,
                           scale=ex["scale"] if extras else None,
                           residual=ex["residual"] if extras and ex["residual"] is not None else None)
    mism = np.count_nonzero(got[:, :N] != c.reshape(M, N).astype(got.dtype))
    assert mism == 0, f"{name}: {mism} of {M * N} outputs differ"
    assert np.all(got[:, N:] == sentinel), f"{name}: padding of C was written"
    assert np.all(got_all[M:] == sentinel), f"{name}: rows of C past M were written"
    return name


@pytest.mark.parametrize("config", [0, 1, 2, 3])
@pytest.mark.parametrize("la,lb", [("row", "col"), ("row", "row"), ("col", "col"), ("col", "row")])
def test_tile_strided_integer_bitexact(config, la, lb):
    M, N, K = {0: (512, 512, 192), 1: (256, 384, 128), 2: (200, 144, 256), 3: (520, 272, 128)}[config]
    for in_dt, out_dt, epi, pads, extras in (("bf16", "bf16", "bias_relu", (8, 16, 24), False),
                                             ("f16", "f32", "relu", (64, 8, 8), True),
                                             ("bf16", "fp8", "bias", (16, 8, 16), False)):
        name = run_strided(M, N, K, in_dt, out_dt, la, lb, epi, pads, "tile", config, extras)
        assert name.startswith("tile_")


@pytest.mark.parametrize("config", [0, 3])
@pytest.mark.parametrize("M,N", [(1, 96), (32, 200)])
def test_skinny_strided_integer_bitexact(config, M, N):
    K = 1536  # whole chunks for both rings (256 x 6, 128 x 12)
    for in_dt, out_dt, epi, pads, extras in (("bf16", "bf16", "bias", (8, 64, 40), True),
                                             ("f16", "f32", "none", (128, 8, 8), False)):
        name = run_strided(M, N, K, in_dt, out_dt, "row", "col", epi, pads, "skinny", config, extras)
        assert name.startswith("skinny_")


@pytest.mark.parametrize("config", [0, 3, 5])
def test_skinny_strided_k_tail_integer_bitexact(config):
    # K not a whole number of chunks, and row padding of at least a chunk:
    # the positions before k = 0 of the shifted first chunk lie in the
    # previous row's NaN padding, so a load that is not masked poisons C
    M, N = 32, 96
    kc = {0: 256, 3: 128, 5: 128}[config]
    K = {0: 1288, 3: 1160, 5: 264}[config]
    for in_dt, out_dt, epi, pads in (("bf16", "bf16", "bias", (kc, kc + 8, 8)), ("f16", "f32", "none", (kc + 64, kc, 0))):
        name = run_strided(M, N, K, in_dt, out_dt, "row", "col", epi, pads, "skinny", config)
        assert name.startswith("skinny_")


@pytest.mark.parametrize("config", [6, 7, 8, 9])
def test_skinny_rowb_strided_integer_bitexact(config):
    # row-major B with padded rows (and K tails): the NaN padding past
    # column N, and the rows before k = 0 of the shifted first chunk, must
    # never reach a product
    K = {6: 1288, 7: 1160, 8: 264, 9: 1160}[config]
    for M, N, in_dt, out_dt, epi, pads in ((32, 96, "bf16", "bf16", "bias", (8, 24, 8)),
                                           (5, 200, "f16", "f32", "none", (64, 8, 0))):
        name = run_strided(M, N, K, in_dt, out_dt, "row", "row", epi, pads, "skinny", config)
        assert name.startswith("skinny_rowb_")


@pytest.mark.parametrize("la,lb", [("row", "col"), ("col", "row")])
def test_generic_strided_integer_bitexact(la, lb):
    # odd leading dimensions: only the generic kernel can take them
    name = run_strided(37, 53, 29, "f16", "f16", la, lb, "bias_relu", (3, 5, 7))
    assert name == "generic"
    name = run_strided(256, 256, 128, "bf16", "bf16", la, lb, "relu", (1, 0, 0))
    assert name == "generic"
