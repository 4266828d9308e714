"""gemm_epi_run_noalloc (through the C ABI): the entry point that allocates
nothing, for callers that cannot call hipMalloc.  Its output must equal
gemm_epi_run_ws's with a caller-allocated workspace, bit for bit (the same
kernels, the same split order), on consecutive calls that share the static
scratch array -- the second one smaller -- and, for a plan that does not
split, gemm_epi_run's."""
import numpy as np
import pytest
import torch

from epilogue_gemm_amd import binding as gb
from epilogue_gemm_amd import inputs
from tests import parity

SCRATCH = 4194304 + 4096  # GEMM_EPI_NOALLOC_SCRATCH_BYTES


def test_noalloc_scratch_covers_every_workspace():
    # host only: the largest workspace any skinny plan asks for fits the
    # static array (N below 256 column blocks at any width, K long enough to
    # split 16 ways)
    gb.load_library()
    worst = 0
    for in_dt in ("bf16", "f16"):
        for lb in ("col", "row"):
            for N in list(range(32, 16384 + 1, 32)):
                for M in (1, 32):
                    h = gb.gemm_epi_plan(M, N, 65536, in_dt, in_dt, "row", lb, "bias")
                    worst = max(worst, gb.gemm_epi_workspace_size(h))
                    gb.gemm_epi_destroy(h)
    assert 0 < worst <= SCRATCH, worst


def _case(M, N, K, in_dt, out_dt, epi, seed):
    bits = inputs.make_inputs(M, N, K, in_dt, "row", "col", epi.startswith("bias"), float(np.sqrt(K)), 0.1, seed)
    A, B = parity.to_device(bits["A"], in_dt), parity.to_device(bits["B"], in_dt)
    bias = parity.to_device(bits["bias"], in_dt) if bits["bias"] is not None else None
    return A, B, bias


def _ptr(t):
    return None if t is None else t.data_ptr()


@pytest.mark.gpu
def test_noalloc_matches_workspace_run_twice():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gb.load_library()
    s = torch.cuda.current_stream().cuda_stream
    # two calls in a row on the shared scratch: the second plan is smaller
    # (fewer column blocks and splits), and its region of the array is the
    # one the first left behind
    for M, N, K, in_dt, out_dt, epi, seed in ((32, 2048, 8192, "bf16", "bf16", "bias", 1),
                                              (17, 512, 4096, "f16", "f32", "bias_relu", 2)):
        plan = gb.Plan(M, N, K, in_dt, out_dt, "row", "col", epi)
        need = plan.workspace_size
        assert 0 < need <= SCRATCH, (plan.name, need)
        A, B, bias = _case(M, N, K, in_dt, out_dt, epi, seed)
        ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
        C_ws = parity.empty_out(M * N, out_dt)
        C_na = parity.empty_out(M * N, out_dt)
        C_ws.fill_(float("nan"))
        C_na.fill_(float("nan"))
        assert gb.gemm_epi_run_ws(plan.handle, A.data_ptr(), B.data_ptr(), _ptr(bias), C_ws.data_ptr(),
                                  ws.data_ptr(), need, s) == 0
        assert gb.gemm_epi_run_noalloc(plan.handle, A.data_ptr(), B.data_ptr(), _ptr(bias), C_na.data_ptr(), s) == 0
        torch.cuda.synchronize()
        print(f"noalloc {plan.name} M{M} N{N} K{K} {in_dt}->{out_dt} {epi}: workspace {need} B", flush=True)
        plan.close()
        got, want = parity.out_bits(C_na), parity.out_bits(C_ws)
        assert bool(torch.isfinite(C_na.float()).all())
        assert np.array_equal(got, want), f"{np.count_nonzero(got != want)} of {got.size} outputs differ"


@pytest.mark.gpu
def test_noalloc_without_split_is_run():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gb.load_library()
    s = torch.cuda.current_stream().cuda_stream
    M, N, K = 256, 256, 512  # a tile plan: no workspace
    plan = gb.Plan(M, N, K, "bf16", "bf16", "row", "col", "bias_gelu")
    assert plan.workspace_size == 0
    A, B, bias = _case(M, N, K, "bf16", "bf16", "bias_gelu", 3)
    C1, C2 = parity.empty_out(M * N, "bf16"), parity.empty_out(M * N, "bf16")
    assert gb.gemm_epi_run(plan.handle, A.data_ptr(), B.data_ptr(), bias.data_ptr(), C1.data_ptr(), s) == 0
    assert gb.gemm_epi_run_noalloc(plan.handle, A.data_ptr(), B.data_ptr(), bias.data_ptr(), C2.data_ptr(), s) == 0
    # argument errors before anything is enqueued
    assert gb.gemm_epi_run_noalloc(plan.handle, A.data_ptr(), B.data_ptr(), None, C2.data_ptr(), s) == 1
    assert gb.gemm_epi_run_noalloc(None, A.data_ptr(), B.data_ptr(), bias.data_ptr(), C2.data_ptr(), s) == 1
    torch.cuda.synchronize()
    plan.close()
    assert np.array_equal(parity.out_bits(C1), parity.out_bits(C2))
