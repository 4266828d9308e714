"""Parity of the 16x16x32-MFMA tile configurations (four waves, 256 x 256
tiles; A row-major, B column-major or -- through transposing LDS reads --
row-major) with the oracle: bit-exact on integer operands for every
epilogue that is exact, K tails of every padding, shifted edge tiles,
leading dimensions, the optional scale, residual and FP8 output; within the
tolerance on random operands."""
import numpy as np
import pytest
import torch

from epilogue_gemm_amd import binding as gb
from epilogue_gemm_amd import inputs
from tests.test_parity_gpu import BITWISE_EPIS, EPIS, check_case
from tests.test_parity_epilogues_gpu import EXTRA_CASES, check_ex
from tests.test_strides_gpu import run_strided

pytestmark = pytest.mark.gpu

NAMES = {4: "tile_256x256x64_m16", 8: "tile_256x256x64_m16_rowb"}
LB = {4: "col", 8: "row"}
CFGS = list(NAMES)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gb.load_library()
    torch.cuda.init()


@pytest.mark.parametrize("config", CFGS)
@pytest.mark.parametrize("in_dt,out_dt", [("f16", "f16"), ("bf16", "bf16"), ("f16", "f32"), ("bf16", "f32")])
def test_tile16_integer_bitexact(config, in_dt, out_dt):
    M, N, K = 512, 768, 640
    for epi in EPIS:
        bits = inputs.integer_inputs(M, N, K, in_dt, "row", LB[config], epi.startswith("bias"), seed=len(epi))
        name = check_case(bits, M, N, K, in_dt, out_dt, "row", LB[config], epi, "tile", config, epi in BITWISE_EPIS)
        assert name == NAMES[config]


# K % 64 != 0 shifts the k axis (the first k-step partial, its leading
# k-values zeros); odd and even k-step counts start in either stage; M and N
# that are not multiples of 256 shift the last tile row and column back.
@pytest.mark.parametrize("config", CFGS)
@pytest.mark.parametrize("K", [72, 104, 136, 168, 200, 232, 248, 128, 192, 256, 264, 296, 328, 360, 376,
                               384, 1000, 4104])
def test_tile16_ktails_and_edges_bitexact(config, K):
    M, N = 264, 520
    for in_dt, out_dt, epi in (("bf16", "bf16", "bias_relu"), ("f16", "f32", "none")):
        bits = inputs.integer_inputs(M, N, K, in_dt, "row", LB[config], epi.startswith("bias"), seed=K)
        name = check_case(bits, M, N, K, in_dt, out_dt, "row", LB[config], epi, "tile", config, True)
        assert name == NAMES[config]


@pytest.mark.parametrize("config", CFGS)
@pytest.mark.parametrize("M,N,K", [(1024, 1024, 1024), (768, 512, 2056)])
def test_tile16_random_bias_gelu(config, M, N, K):
    for in_dt in ("bf16", "f16"):
        bits = inputs.make_inputs(M, N, K, in_dt, "row", LB[config], True, float(np.sqrt(K)), 0.1, seed=M + K)
        check_case(bits, M, N, K, in_dt, in_dt, "row", LB[config], "bias_gelu", "tile", config, False)


@pytest.mark.parametrize("config", CFGS)
@pytest.mark.parametrize("edge", [False, True])
def test_tile16_extras_integer_bitexact(config, edge):
    M, N, K = (264, 520, 328) if edge else (512, 512, 320)
    for in_dt, out_dt in (("bf16", "bf16"), ("f16", "f32")):
        for epi, use_s, use_r in EXTRA_CASES:
            name = check_ex(M, N, K, in_dt, out_dt, "row", LB[config], epi, "tile", config, use_s, use_r, True,
                            seed=13 + len(epi))
            assert name == NAMES[config]


@pytest.mark.parametrize("config", CFGS)
def test_tile16_silu_and_fp8_output(config):
    M, N, K = 512, 528, 352
    for integer in (True, False):
        name = check_ex(M, N, K, "bf16", "fp8", "row", LB[config], "bias_gelu" if not integer else "bias", "tile",
                        config, False, False, integer, seed=40 + integer, use_oscale=True)
        assert name == NAMES[config]
    for epi in ("silu", "bias_silu"):
        check_ex(M, N, K, "bf16", "bf16", "row", LB[config], epi, "tile", config, True, True, False, seed=len(epi))


@pytest.mark.parametrize("config", CFGS)
def test_tile16_strided_integer_bitexact(config):
    M, N, K = 520, 272, 328
    for in_dt, out_dt, epi, pads, extras in (("bf16", "bf16", "bias_relu", (8, 16, 24), False),
                                             ("f16", "f32", "relu", (64, 8, 8), True),
                                             ("bf16", "fp8", "bias", (16, 8, 16), False)):
        name = run_strided(M, N, K, in_dt, out_dt, "row", LB[config], epi, pads, "tile", config, extras)
        assert name == NAMES[config]


# N or ldc off the 16-byte output chunks (B column-major): the last tile
# column stays in place, masked past N, and its edge is read and stored
# element by element; C carries a sentinel in its padding and in 64 rows
# past M, and packed rows of odd width are all unaligned
@pytest.mark.parametrize("M,N,K,ldc_pad", [(512, 300, 256, 0), (300, 777, 200, 0), (256, 1003, 136, 5),
                                           (264, 520, 264, 4), (256, 264, 192, 3)])
def test_tile16_ragged_n_bitexact(M, N, K, ldc_pad):
    for in_dt, out_dt, epi, extras in (("bf16", "bf16", "bias_relu", False), ("f16", "f32", "relu", True),
                                       ("f16", "f16", "bias", True), ("bf16", "fp8", "bias", True)):
        assert run_strided(M, N, K, in_dt, out_dt, "row", "col", epi, (8, 16, ldc_pad), "tile", 4, extras,
                           extra_rows=64) == NAMES[4]


def test_tile16_ragged_n_random_tolerance():
    M, N, K = 512, 777, 1000
    for in_dt in ("bf16", "f16"):
        bits = inputs.make_inputs(M, N, K, in_dt, "row", "col", True, float(np.sqrt(K)), 0.1, seed=777)
        assert check_case(bits, M, N, K, in_dt, in_dt, "row", "col", "bias_gelu", "tile", 4, False) == NAMES[4]
