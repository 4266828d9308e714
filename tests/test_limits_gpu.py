"""The largest operands the boundary accepts (fewer than 2^31 elements, 4 GiB
in bf16), whose buffer extents and offsets sit just inside the kernels'
32-bit range: A of 262143 x 8192 for the tile kernel, and a weight of
8192 x 261888 for the skinny kernel.  Integer operands make the comparison
with the oracle bit-exact on whole sampled rows or columns (for the tile
kernel the last 257 rows, where the last tile row is shifted back)."""
import sys

import numpy as np
import pytest
import torch

import oracle
from epilogue_gemm_amd import binding as gb
from epilogue_gemm_amd import inputs
from tests import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gb.load_library()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("epi", ["bias_relu", "none"])
def test_largest_accepted_a_operand(epi):
    M, N, K = 262143, 256, 8192
    assert M * K < 2**31 <= (M + 1) * K  # one more row of A would be refused
    _say(f"[limits] generating A {M}x{K} bf16 ({epi})")
    A = inputs.integer_bits(M, K, "bf16", seed=31)
    B = inputs.integer_bits(N, K, "bf16", seed=32)  # column-major B: N x K
    bias = inputs.integer_bits(1, N, "bf16", seed=33).reshape(-1) if epi.startswith("bias") else None
    dA, dB = parity.to_device(A, "bf16"), parity.to_device(B, "bf16")
    dbias = parity.to_device(bias, "bf16") if bias is not None else None
    C = parity.empty_out(M * N, "bf16")
    C.fill_(float("nan"))
    plan = gb.Plan(M, N, K, "bf16", "bf16", "row", "col", epi)
    _say(f"[limits] running {plan.name}")
    plan.run(dA, dB, dbias, C)
    torch.cuda.synchronize()
    name = plan.name
    plan.close()
    del dA, dB
    rows = np.concatenate([[0, M // 2], np.arange(M - 257, M)])
    rr = np.repeat(rows, N)
    cc = np.tile(np.arange(N), rows.size)
    got = parity.out_bits(C.view(M, N)[torch.from_numpy(rows).cuda()]).reshape(-1)
    _say(f"[limits] oracle on {rr.size} outputs")
    _, bits = oracle.gemm_epi_points(A, B, bias, M, N, K, "bf16", "bf16", "row", "col", epi, rr, cc)
    mism = np.count_nonzero(got != bits.astype(np.uint16))
    assert name.startswith("tile_")
    assert mism == 0, f"{name}: {mism} of {got.size} sampled outputs differ"
    assert bool(torch.isfinite(C.float()).all())


def test_largest_accepted_weight_skinny():
    # the decode shape with a weight of 8192 x 261888 = 2^31 - 2^21 elements
    # (K whole 256-deep chunks), its buffer extent within 2 MiB of 4 GiB
    M, N, K = 32, 8192, 261888
    assert K * N < 2**31 and K % 256 == 0
    _say("[limits] generating the skinny operands")
    A = inputs.integer_bits(M, K, "bf16", seed=41)
    B = inputs.integer_bits(N, K, "bf16", seed=42)  # column-major B: N x K
    bias = inputs.integer_bits(1, N, "bf16", seed=43).reshape(-1)
    dA, dB, dbias = parity.to_device(A, "bf16"), parity.to_device(B, "bf16"), parity.to_device(bias, "bf16")
    C = parity.empty_out(M * N, "bf16")
    C.fill_(float("nan"))
    plan = gb.Plan(M, N, K, "bf16", "bf16", "row", "col", "bias")
    _say(f"[limits] running {plan.name}")
    plan.run(dA, dB, dbias, C)
    torch.cuda.synchronize()
    name = plan.name
    plan.close()
    got = parity.out_bits(C).reshape(-1)
    # every row at the first, a middle and the last 40 columns
    cols = np.concatenate([[0, N // 2 + 3], np.arange(N - 40, N)])
    rr = np.repeat(np.arange(M), cols.size)
    cc = np.tile(cols, M)
    _say(f"[limits] oracle on {rr.size} outputs")
    _, bits = oracle.gemm_epi_points(A, B, bias, M, N, K, "bf16", "bf16", "row", "col", "bias", rr, cc)
    mism = np.count_nonzero(got.reshape(M, N)[rr, cc] != bits.astype(np.uint16))
    assert name.startswith("skinny_")
    assert mism == 0, f"{name}: {mism} of {rr.size} sampled outputs differ"
