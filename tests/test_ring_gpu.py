"""Parity of the deep-ring 64 x 64 tile configurations (8, 4 or 2 LDS slots;
A row-major, or column-major through transposing LDS reads (the last tile
row masked, M any with lda a multiple of 8); B row-major through
transposing LDS reads or column-major) with
the oracle: bit-exact on integer operands for every exact epilogue, every
K padding (the first chunk partial), chunk counts of one to several ring
turns, shifted edge tiles, leading dimensions, the optional scale, residual
and FP8 output; problems smaller than the tile (M or N below 64, masked)
and odd chunk counts through two slots; within the tolerance on random
operands and on the two workloads the ring serves (1024^3 row-major ReLU
and 128 x 64 x 256)."""
import numpy as np
import pytest
import torch

from epilogue_gemm_amd import binding as gb
from epilogue_gemm_amd import inputs
from tests.test_parity_epilogues_gpu import EXTRA_CASES, check_ex
from tests.test_parity_gpu import BITWISE_EPIS, EPIS, check_case
from tests.test_strides_gpu import run_strided

pytestmark = pytest.mark.gpu

RINGS = {5: ("tile_64x64_ring8", 8), 6: ("tile_64x64_ring4", 4), 7: ("tile_64x64_ring2", 2)}
LBS = ["row", "col"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gb.load_library()
    torch.cuda.init()


def _k(P, turns, kpad=0):
    """K of `turns` ring turns of P 64-deep chunks, the first chunk short by kpad."""
    return 64 * P * turns - kpad


@pytest.mark.parametrize("config", list(RINGS))
@pytest.mark.parametrize("lb", LBS)
@pytest.mark.parametrize("in_dt,out_dt", [("f16", "f16"), ("bf16", "bf16"), ("f16", "f32")])
def test_ring_integer_bitexact(config, lb, in_dt, out_dt):
    name, P = RINGS[config]
    M, N, K = 192, 256, _k(P, 2)
    for epi in EPIS:
        bits = inputs.integer_inputs(M, N, K, in_dt, "row", lb, epi.startswith("bias"), seed=len(epi) + config)
        got = check_case(bits, M, N, K, in_dt, out_dt, "row", lb, epi, "tile", config, epi in BITWISE_EPIS)
        assert got == name


# every K padding (a multiple of 8 below 64) and one to three ring turns;
# M and N not multiples of 64 shift the last tile row and column back
@pytest.mark.parametrize("config", list(RINGS))
@pytest.mark.parametrize("lb", LBS)
@pytest.mark.parametrize("kpad,turns", [(0, 1), (8, 1), (16, 2), (24, 1), (32, 3), (40, 2), (48, 1), (56, 2)])
def test_ring_ktails_and_edges_bitexact(config, lb, kpad, turns):
    name, P = RINGS[config]
    M, N, K = 200, 136, _k(P, turns, kpad)
    for in_dt, out_dt, epi in (("bf16", "bf16", "bias_relu"), ("f16", "f32", "none")):
        bits = inputs.integer_inputs(M, N, K, in_dt, "row", lb, epi.startswith("bias"), seed=K + kpad)
        got = check_case(bits, M, N, K, in_dt, out_dt, "row", lb, epi, "tile", config, True)
        assert got == name


@pytest.mark.parametrize("config", list(RINGS))
@pytest.mark.parametrize("lb", LBS)
def test_ring_random_tolerance(config, lb):
    name, P = RINGS[config]
    M, N, K = 320, 384, _k(P, 2, 16)
    for in_dt in ("bf16", "f16"):
        for epi in ("bias_gelu", "relu"):
            bits = inputs.make_inputs(M, N, K, in_dt, "row", lb, epi.startswith("bias"), float(np.sqrt(K)), 0.1,
                                      seed=M + K)
            assert check_case(bits, M, N, K, in_dt, in_dt, "row", lb, epi, "tile", config, False) == name


@pytest.mark.parametrize("config", list(RINGS))
@pytest.mark.parametrize("lb", LBS)
def test_ring_extras_fp8_and_strides(config, lb):
    name, P = RINGS[config]
    M, N, K = 136, 200, _k(P, 1, 24)
    for in_dt, out_dt in (("bf16", "bf16"), ("f16", "f32")):
        for epi, use_s, use_r in EXTRA_CASES:
            assert check_ex(M, N, K, in_dt, out_dt, "row", lb, epi, "tile", config, use_s, use_r, True,
                            seed=13 + len(epi)) == name
    # FP8 output (N a multiple of 16), with the output scale
    assert check_ex(M, 208, K, "bf16", "fp8", "row", lb, "bias_relu", "tile", config, True, False, True, seed=5,
                    use_oscale=True) == name
    # leading dimensions with NaN padding in A and B, a sentinel in C's
    for in_dt, out_dt, epi, pads, extras in (("bf16", "bf16", "bias_relu", (8, 16, 24), False),
                                             ("f16", "f32", "relu", (64, 8, 8), True)):
        assert run_strided(M, N, K, in_dt, out_dt, "row", lb, epi, pads, "tile", config, extras) == name


# Problems smaller than the tile: M or N below 64 take one tile row or
# column, masked past the end (C carries a sentinel in 64 rows past row M
# and in its row padding; no output there may change).  K of one chunk, of
# an odd number of chunks (two slots only) and with a partial first chunk.
SMALL = [(1, 8, 8), (33, 40, 64), (48, 56, 200), (63, 8, 320), (17, 136, 64), (200, 24, 136), (40, 264, 128),
         (64, 48, 72), (7, 16, 1000)]


@pytest.mark.parametrize("lb", LBS)
@pytest.mark.parametrize("M,N,K", SMALL)
def test_ring_small_problems_bitexact(lb, M, N, K):
    for in_dt, out_dt, epi, pads, extras in (("bf16", "bf16", "bias_relu", (8, 16, 24), False),
                                             ("f16", "f32", "relu", (64, 8, 8), True),
                                             ("f16", "f16", "bias", (0, 0, 0), True)):
        assert run_strided(M, N, K, in_dt, out_dt, "row", lb, epi, pads, "tile", 7, extras,
                           extra_rows=64) == "tile_64x64_ring2"
    if N % 16 == 0:
        assert run_strided(M, N, K, "bf16", "fp8", "row", lb, "bias", (8, 8, 16), "tile", 7, False,
                           extra_rows=64) == "tile_64x64_ring2"
    # the automatic plan takes the same kernel where no other fits
    bits = inputs.integer_inputs(M, N, K, "bf16", "row", lb, True, seed=M * N + K)
    name = check_case(bits, M, N, K, "bf16", "bf16", "row", lb, "bias_gelu", "auto", -1, False)
    assert name.startswith("tile_64x64_ring") or name.startswith("skinny_"), name


@pytest.mark.parametrize("config", [5, 6])
@pytest.mark.parametrize("lb", LBS)
def test_ring_small_problems_deep_rings_bitexact(config, lb):
    name, P = RINGS[config]
    for M, N in ((33, 40), (63, 8), (5, 200)):
        K = _k(P, 1, 24)
        assert run_strided(M, N, K, "bf16", "bf16", "row", lb, "bias_relu", (8, 16, 24), "tile", config, True,
                           extra_rows=64) == name


@pytest.mark.parametrize("lb", LBS)
def test_ring_small_problems_random_tolerance(lb):
    for M, N, K in ((48, 56, 200), (33, 264, 1000)):
        for in_dt in ("bf16", "f16"):
            bits = inputs.make_inputs(M, N, K, in_dt, "row", lb, True, float(np.sqrt(K)), 0.1, seed=M + K)
            assert check_case(bits, M, N, K, in_dt, in_dt, "row", lb, "bias_gelu", "tile", 7, False) == \
                "tile_64x64_ring2"


# ---------------------------------------------------------------------------
# A column-major: 64 k-rows of the tile's rows in LDS, read through
# transposing reads like a row-major B; the last tile row is not shifted
# back but masked past M, so M need not be a multiple of 8 (with lda one)
# ---------------------------------------------------------------------------

def _pads_cola(M, pb=16, pc=24):
    """Padding of A, B and C: A's leading dimension (M + pad) a multiple of 8."""
    return ((-M) % 8 + 8, pb, pc)


@pytest.mark.parametrize("config", list(RINGS))
@pytest.mark.parametrize("lb", LBS)
@pytest.mark.parametrize("in_dt,out_dt", [("f16", "f16"), ("bf16", "bf16"), ("f16", "f32")])
def test_ring_col_a_integer_bitexact(config, lb, in_dt, out_dt):
    name, P = RINGS[config]
    M, N, K = 192, 256, _k(P, 2)
    for epi in EPIS:
        bits = inputs.integer_inputs(M, N, K, in_dt, "col", lb, epi.startswith("bias"), seed=len(epi) + 3 * config)
        assert check_case(bits, M, N, K, in_dt, out_dt, "col", lb, epi, "tile", config, epi in BITWISE_EPIS) == name


# K paddings and ring turns; M past a multiple of 64 by a ragged amount (the
# unshifted last tile row, masked), N shifted back as before
@pytest.mark.parametrize("config", list(RINGS))
@pytest.mark.parametrize("lb", LBS)
@pytest.mark.parametrize("M,kpad,turns", [(200, 0, 1), (203, 8, 2), (129, 24, 1), (77, 40, 2), (250, 56, 1)])
def test_ring_col_a_edges_bitexact(config, lb, M, kpad, turns):
    name, P = RINGS[config]
    N, K = 136, _k(P, turns, kpad)
    for in_dt, out_dt, epi, extras in (("bf16", "bf16", "bias_relu", False), ("f16", "f32", "none", True)):
        assert run_strided(M, N, K, in_dt, out_dt, "col", lb, epi, _pads_cola(M), "tile", config, extras,
                           extra_rows=64) == name


@pytest.mark.parametrize("lb", LBS)
@pytest.mark.parametrize("M,N,K", [(1, 8, 8), (33, 40, 64), (63, 8, 320), (17, 136, 64), (200, 24, 136),
                                   (61, 264, 128), (7, 16, 1000), (100, 72, 200)])
def test_ring_col_a_small_problems_bitexact(lb, M, N, K):
    for in_dt, out_dt, epi, extras in (("bf16", "bf16", "bias_relu", False), ("f16", "f32", "relu", True),
                                       ("f16", "f16", "bias", True)):
        assert run_strided(M, N, K, in_dt, out_dt, "col", lb, epi, _pads_cola(M), "tile", 7, extras,
                           extra_rows=64) == "tile_64x64_ring2"
    if N % 16 == 0:
        assert run_strided(M, N, K, "bf16", "fp8", "col", lb, "bias", _pads_cola(M, 8, 16), "tile", 7, False,
                           extra_rows=64) == "tile_64x64_ring2"
    # the automatic plan takes a ring where no other kernel fits (packed
    # operands: M a multiple of 8 keeps A's columns 16-byte aligned)
    if M % 8 == 0:
        bits = inputs.integer_inputs(M, N, K, "bf16", "col", lb, True, seed=M * N + K)
        name = check_case(bits, M, N, K, "bf16", "bf16", "col", lb, "bias_gelu", "auto", -1, False)
        assert name.startswith("tile_64x64_ring"), name


@pytest.mark.parametrize("config", list(RINGS))
@pytest.mark.parametrize("lb", LBS)
def test_ring_col_a_random_tolerance(config, lb):
    name, P = RINGS[config]
    M, N, K = 320, 384, _k(P, 2, 16)
    for in_dt in ("bf16", "f16"):
        for epi in ("bias_gelu", "relu"):
            bits = inputs.make_inputs(M, N, K, in_dt, "col", lb, epi.startswith("bias"), float(np.sqrt(K)), 0.1,
                                      seed=M + K + 1)
            assert check_case(bits, M, N, K, in_dt, in_dt, "col", lb, epi, "tile", config, False) == name


# ---------------------------------------------------------------------------
# N off the 16-byte output chunks (or a row-major B's 8-column chunks), or
# rows of C not 16-byte aligned: the ring kernels (two and four slots) mask
# their last tile column instead of shifting it back, and the epilogue
# reads bias, scale and residual and stores C element by element where a
# group reaches past N or a row is unaligned
# ---------------------------------------------------------------------------

def _pads_ragged(M, N, K, la, lb, pc):
    """Paddings that keep A's and B's leading dimensions multiples of 8."""
    pa = ((-M) % 8 + 8) if la == "col" else 8
    pb = ((-N) % 8 + 8) if lb == "row" else 16
    return (pa, pb, pc)


@pytest.mark.parametrize("config", [6, 7])
@pytest.mark.parametrize("la", ["row", "col"])
@pytest.mark.parametrize("lb", LBS)
@pytest.mark.parametrize("M,N,ldc_pad", [(100, 77, 3), (130, 1004, 0), (33, 13, 0), (70, 200, 4), (64, 129, 15)])
def test_ring_ragged_n_bitexact(config, la, lb, M, N, ldc_pad):
    name, P = RINGS[config]
    K = _k(P, 1, 24)
    for in_dt, out_dt, epi, extras in (("bf16", "bf16", "bias_relu", False), ("f16", "f32", "relu", True),
                                       ("f16", "f16", "bias", True)):
        assert run_strided(M, N, K, in_dt, out_dt, la, lb, epi, _pads_ragged(M, N, K, la, lb, ldc_pad), "tile",
                           config, extras, extra_rows=64) == name
    # FP8 output: rows of C in 16-byte chunks of 16 outputs
    assert run_strided(M, N, K, "bf16", "fp8", la, lb, "bias_relu", _pads_ragged(M, N, K, la, lb, ldc_pad), "tile",
                       config, True, extra_rows=64) == name


@pytest.mark.parametrize("M,N,K", [(300, 1001, 512), (512, 5003, 256), (48, 77, 1000)])
def test_ring_ragged_n_packed_auto(M, N, K):
    # packed C of odd width: the automatic plan takes a masked ring
    for in_dt, out_dt, epi in (("bf16", "bf16", "bias_gelu"), ("f16", "f32", "bias")):
        bits = inputs.integer_inputs(M, N, K, in_dt, "row", "col", True, seed=N + M)
        name = check_case(bits, M, N, K, in_dt, out_dt, "row", "col", epi, "auto", -1, epi != "bias_gelu")
        assert name.startswith("tile_64x64_ring"), name
    # a row-major B of odd width needs a padded ldb: through the strided path
    assert run_strided(M, N, K, "bf16", "bf16", "row", "row", "bias_relu", (8, (-N) % 8 + 8, 0), "auto", -1,
                       False).startswith("tile_64x64_ring")
