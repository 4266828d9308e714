"""gemm_epi_tune on the GPU: it measures every configuration that can run a
problem, keeps the fastest, records it in the tuning table, and the result of
the tuned plan still matches the oracle."""
import numpy as np
import pytest
import torch

import oracle
from epilogue_gemm_amd import binding as gb
from epilogue_gemm_amd import inputs
from tests import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu_and_clean_table():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gb.load_library()
    gb.gemm_epi_tuning_clear()
    yield
    gb.gemm_epi_tuning_clear()


def _supported(plan_args):
    out = set()
    for fam in ("tile", "skinny"):
        for c in range(gb.gemm_epi_num_configs(fam)):
            h = gb.gemm_epi_plan(*plan_args)
            try:
                if gb.gemm_epi_plan_select(h, fam, c) == 0:
                    out.add((fam, c))
            finally:
                gb.gemm_epi_destroy(h)
    return out


@pytest.mark.parametrize("M,N,K,in_dt,out_dt,la,lb,epi,cold", [
    (1024, 1024, 1024, "f16", "f16", "row", "row", "relu", False),
    (2048, 1024, 512, "bf16", "bf16", "row", "col", "bias_gelu", True),
    (32, 4096, 4096, "bf16", "bf16", "row", "col", "bias", True),
    (512, 512, 256, "bf16", "fp8", "row", "col", "bias_silu", False),
])
def test_tune_picks_a_supported_config_and_stays_correct(tmp_path, M, N, K, in_dt, out_dt, la, lb, epi, cold):
    args = (M, N, K, in_dt, out_dt, la, lb, epi)
    bits = inputs.make_inputs(M, N, K, in_dt, la, lb, epi.startswith("bias"), float(np.sqrt(K)), 0.1, seed=M + N)
    A, B = parity.to_device(bits["A"], in_dt), parity.to_device(bits["B"], in_dt)
    bias = parity.to_device(bits["bias"], in_dt) if bits["bias"] is not None else None
    C = parity.empty_out(M * N, out_dt)
    plan = gb.Plan(*args)
    us = plan.tune(A, B, bias, C, iters=5, cold=cold)
    assert us > 0.0
    assert (plan.kernel, plan.config) in _supported(args)
    assert gb.gemm_epi_tuning_size() == 1
    # the tuned plan computes the right thing
    C2 = parity.empty_out(M * N, out_dt)
    plan.run(A, B, bias, C2)
    torch.cuda.synchronize()
    y, c = oracle.gemm_epi(bits["A"], bits["B"], bits["bias"], M, N, K, in_dt, out_dt, la, lb, epi)
    r = parity.compare(parity.out_bits(C2), c, y, out_dt)
    assert r["ok"], r
    # a new plan of the same problem takes the recorded choice, also after a
    # save / clear / load round trip
    assert gb.Plan(*args).config == plan.config
    f = tmp_path / "tuned.txt"
    assert gb.gemm_epi_tuning_save(f) == 0
    gb.gemm_epi_tuning_clear()
    assert gb.gemm_epi_tuning_load(f) == 0
    again = gb.Plan(*args)
    assert (again.kernel, again.config) == (plan.kernel, plan.config)
    again.close()
    plan.close()
