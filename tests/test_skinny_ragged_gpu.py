"""Parity of the decode-shape kernel (M <= 32, B column-major) with N not a
multiple of 8 or below the workgroup's 32 columns, and with rows of C that
are not 4-element aligned (packed C of odd width): the last workgroup is
then not shifted back but masked past N (B's rows past N load as zeros; no
output, bias, scale or residual past N is touched), and a quad of outputs
reaching past N, or every quad when C's rows are unaligned, is stored
element by element.  Bit-exact on integer operands for every column-major
configuration, the extras, FP8 and fp32 outputs and split K; within the
tolerance on random operands at a vocabulary-sized N."""
import numpy as np
import pytest
import torch

from epilogue_gemm_amd import binding as gb
from epilogue_gemm_amd import inputs
from tests import parity
from tests.test_parity_gpu import check_case, oracle_full
from tests.test_strides_gpu import run_strided

pytestmark = pytest.mark.gpu

# column-major B configurations and a K that gives each of them enough chunks
CM_CONFIGS = {0: "skinny_32n_8w_5x256k", 1: "skinny_32n_8w_4x256k", 2: "skinny_32n_4w_4x256k",
              3: "skinny_32n_4w_8x128k", 4: "skinny_32n_4w_2x256k", 5: "skinny_32n_2w_2x128k"}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gb.load_library()


@pytest.mark.parametrize("M", [1, 7, 32])
@pytest.mark.parametrize("N", [1, 13, 77, 1001, 4103])
def test_ragged_n_packed_bitexact(M, N):
    # packed C: ldc = N, rows not 4-element aligned unless N % 4 == 0
    K = 1280
    for in_dt, out_dt, epi in (("bf16", "bf16", "bias_relu"), ("f16", "f32", "bias"), ("bf16", "fp8", "bias"),
                               ("f16", "f16", "none")):
        bits = inputs.integer_inputs(M, N, K, in_dt, "row", "col", epi.startswith("bias"), seed=M * 7 + N)
        name = check_case(bits, M, N, K, in_dt, out_dt, "row", "col", epi, "auto", -1, True)
        assert name.startswith("skinny_32n_"), name


@pytest.mark.parametrize("config", list(CM_CONFIGS))
@pytest.mark.parametrize("N,ldc_pad", [(77, 3), (77, 11), (100, 4), (13, 0)])
def test_ragged_n_strided_extras_bitexact(config, N, ldc_pad):
    # every column-major configuration; C's padding (and 8 rows past M)
    # carries a sentinel that must survive; column scale and residual
    M, K = 19, 2048
    for in_dt, out_dt, epi in (("bf16", "bf16", "bias_relu"), ("f16", "f32", "relu")):
        name = run_strided(M, N, K, in_dt, out_dt, "row", "col", epi, (8, 16, ldc_pad), "skinny", config, True,
                           extra_rows=8)
        assert name == CM_CONFIGS[config]


@pytest.mark.parametrize("M,N,K", [(7, 77, 4096), (32, 1001, 8192), (3, 13, 8192)])
def test_ragged_n_split_bitexact(M, N, K):
    for in_dt, out_dt, epi in (("bf16", "bf16", "bias_relu"), ("f16", "f32", "none")):
        bits = inputs.integer_inputs(M, N, K, in_dt, "row", "col", epi.startswith("bias"), seed=N + K + M)
        plan = gb.Plan(M, N, K, in_dt, out_dt, "row", "col", epi)
        assert plan.kernel == "skinny" and plan.workspace_size > 0
        ws = torch.zeros(plan.workspace_size, dtype=torch.uint8, device="cuda")
        A = parity.to_device(bits["A"], in_dt)
        B = parity.to_device(bits["B"], in_dt)
        bias = parity.to_device(bits["bias"], in_dt) if bits["bias"] is not None else None
        c = oracle_full(bits, M, N, K, in_dt, out_dt, "row", "col", epi)[1]
        for rep in range(2):
            C = parity.empty_out(M * N, out_dt)
            C.fill_(float("nan"))
            plan.run(A, B, bias, C, workspace=ws)
            torch.cuda.synchronize()
            got = parity.out_bits(C)
            mism = np.count_nonzero(got.reshape(-1) != c.reshape(-1).astype(got.dtype))
            assert mism == 0, (rep, epi, mism)
        assert not ws.cpu().numpy().any()
        plan.close()


def test_vocabulary_sized_n_random_tolerance():
    # a decode step's output projection over an odd vocabulary size
    M, N, K = 4, 50257, 1280
    bits = inputs.make_inputs(M, N, K, "bf16", "row", "col", True, float(np.sqrt(K)), 0.1, seed=50257)
    assert check_case(bits, M, N, K, "bf16", "bf16", "row", "col", "bias", "auto", -1, False) == \
        "skinny_32n_8w_5x256k"
