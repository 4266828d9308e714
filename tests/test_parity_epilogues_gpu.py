"""Parity of the further epilogues with the CPU oracle, through the C ABI:
SiLU (with and without bias), the optional fp32 column scale, residual and
output scale of gemm_epi_run_ex, and the FP8 E4M3 output, in every kernel
family.

  * integer operands, integer residuals and scales in {+-0.5, +-1, +-2}:
    every fp32 step is exact, so none/ReLU/bias/bias+ReLU must match the
    oracle bit for bit, with the extras applied in the stated order
    (scale before bias, residual after the activation);
  * random operands: the tolerance of tests/parity.py (SiLU is
    transcendental);
  * FP8 E4M3 output with integer operands: the exact value is rounded once
    on both sides, so every code (ties to even, saturation at 448 included)
    must match the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle
from epilogue_gemm_amd import binding as gb
from epilogue_gemm_amd import inputs
from tests import parity

pytestmark = pytest.mark.gpu

LAYOUTS = [("row", "col"), ("row", "row"), ("col", "col"), ("col", "row")]
TILE_SHAPES = {0: (512, 512, 192), 1: (256, 384, 128), 2: (192, 128, 320), 3: (768, 512, 256)}
TILE_EDGE_SHAPES = {0: (264, 520, 192), 1: (200, 136, 128), 2: (72, 200, 256), 3: (304, 264, 128)}
# (epilogue, use the scale, use the residual)
EXTRA_CASES = [("bias_relu", True, True), ("none", True, False), ("relu", False, True), ("bias", True, True)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gb.load_library()
    torch.cuda.init()


def run_ex(bits, ex, M, N, K, in_dt, out_dt, la, lb, epi, kernel="auto", config=-1, use_scale=True, use_res=True,
           workspace=None, scale_offset=0, use_oscale=False):
    A, B = parity.to_device(bits["A"], in_dt), parity.to_device(bits["B"], in_dt)
    bias = parity.to_device(bits["bias"], in_dt) if bits["bias"] is not None else None
    scale = None
    if use_scale:
        full = torch.zeros(N + scale_offset, dtype=torch.float32, device="cuda")
        full[scale_offset:] = torch.from_numpy(ex["scale"]).cuda()
        scale = full[scale_offset:]
    res = parity.to_device_out(ex["residual"], out_dt) if use_res else None
    osc = torch.tensor([ex["out_scale"]], dtype=torch.float32, device="cuda") if use_oscale else None
    C = parity.empty_out(M * N, out_dt)
    if out_dt == "fp8":
        C.view(torch.uint8).fill_(0x7F)  # NaN
    else:
        C.fill_(float("nan"))
    plan = gb.Plan(M, N, K, in_dt, out_dt, la, lb, epi, kernel, config)
    plan.run(A, B, bias, C, workspace=workspace, scale=scale, residual=res, out_scale=osc)
    torch.cuda.synchronize()
    name = plan.name
    plan.close()
    return parity.out_bits(C), name


def oracle_ex(bits, ex, M, N, K, in_dt, out_dt, la, lb, epi, use_scale=True, use_res=True, use_oscale=False):
    return oracle.gemm_epi(bits["A"], bits["B"], bits["bias"], M, N, K, in_dt, out_dt, la, lb, epi,
                           scale=ex["scale"] if use_scale else None, residual=ex["residual"] if use_res else None,
                           out_scale=ex["out_scale"] if use_oscale else None)


def check_ex(M, N, K, in_dt, out_dt, la, lb, epi, kernel, config, use_scale, use_res, integer, seed, **kw):
    if integer:
        bits = inputs.integer_inputs(M, N, K, in_dt, la, lb, epi.startswith("bias"), seed=seed)
    else:
        bits = inputs.make_inputs(M, N, K, in_dt, la, lb, epi.startswith("bias"), float(np.sqrt(K)), 0.1, seed)
    ex = inputs.extras_inputs(M, N, out_dt, seed, integer=integer)
    got, name = run_ex(bits, ex, M, N, K, in_dt, out_dt, la, lb, epi, kernel, config, use_scale, use_res, **kw)
    y, c = oracle_ex(bits, ex, M, N, K, in_dt, out_dt, la, lb, epi, use_scale, use_res, kw.get("use_oscale", False))
    if integer:
        mism = np.count_nonzero(got.reshape(-1) != c.reshape(-1).astype(got.dtype))
        assert mism == 0, f"{name} {epi} scale={use_scale} res={use_res}: {mism} of {got.size} outputs differ"
    else:
        r = parity.compare(got, c, y, out_dt)
        assert r["ok"], f"{name} {epi} scale={use_scale} res={use_res}: {r}"
    return name


@pytest.mark.parametrize("config", [0, 1, 2, 3])
@pytest.mark.parametrize("la,lb", LAYOUTS)
@pytest.mark.parametrize("edge", [False, True])
def test_tile_extras_integer_bitexact(config, la, lb, edge):
    M, N, K = (TILE_EDGE_SHAPES if edge else TILE_SHAPES)[config]
    for in_dt, out_dt in (("bf16", "bf16"), ("f16", "f32")):
        for epi, use_s, use_r in EXTRA_CASES:
            name = check_ex(M, N, K, in_dt, out_dt, la, lb, epi, "tile", config, use_s, use_r, True,
                            seed=config * 13 + len(epi))
            assert name.startswith("tile_")


@pytest.mark.parametrize("config", [0, 3, 4, 5])
@pytest.mark.parametrize("M,N", [(1, 96), (32, 96), (17, 40)])
def test_skinny_extras_integer_bitexact(config, M, N):
    kc, slots = [(256, 5), (256, 4), (256, 4), (128, 8), (256, 2), (128, 2)][config]
    K = kc * (slots + 1)
    for in_dt, out_dt in (("bf16", "bf16"), ("f16", "f32")):
        for epi, use_s, use_r in EXTRA_CASES:
            name = check_ex(M, N, K, in_dt, out_dt, "row", "col", epi, "skinny", config, use_s, use_r, True,
                            seed=M + N + config)
            assert name.startswith("skinny_")


@pytest.mark.parametrize("M,N,K", [(32, 1024, 8192), (5, 96, 4096)])
def test_skinny_split_extras_integer_bitexact(M, N, K):
    plan = gb.Plan(M, N, K, "bf16", "bf16", "row", "col", "bias_relu")
    ws = torch.zeros(plan.workspace_size, dtype=torch.uint8, device="cuda")
    assert plan.workspace_size > 0
    plan.close()
    for rep in range(2):  # the split path leaves its counters at zero for the next run
        check_ex(M, N, K, "bf16", "bf16", "row", "col", "bias_relu", "auto", -1, True, True, True, seed=N + rep,
                 workspace=ws)
    assert not ws.cpu().numpy().any()  # the whole workspace is left zero-filled


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (37, 53, 29), (65, 130, 200)])
@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_generic_extras_integer_bitexact(M, N, K, la, lb):
    for in_dt, out_dt in (("f16", "f16"), ("bf16", "f32")):
        for epi, use_s, use_r in EXTRA_CASES:
            check_ex(M, N, K, in_dt, out_dt, la, lb, epi, "generic", 0, use_s, use_r, True, seed=M * N + K)


@pytest.mark.parametrize("kernel,config,M,N,K,la,lb", [
    ("tile", 0, 768, 1024, 512, "row", "col"),
    ("tile", 0, 512, 768, 640, "row", "row"),
    ("tile", 1, 384, 256, 1024, "col", "row"),
    ("tile", 2, 320, 192, 448, "col", "col"),
    ("tile", 3, 1000, 1000, 1024, "row", "col"),
    ("skinny", 0, 32, 512, 4096, "row", "col"),
    ("skinny", 5, 5, 160, 768, "row", "col"),
    ("generic", 0, 97, 61, 333, "row", "row"),
])
@pytest.mark.parametrize("in_dt,out_dt,epi", [("bf16", "bf16", "bias_silu"), ("f16", "f16", "silu"),
                                              ("bf16", "f32", "bias_silu"), ("bf16", "bf16", "bias_gelu")])
@pytest.mark.parametrize("use_s,use_r", [(False, False), (True, True)])
def test_silu_and_extras_random_tolerance(kernel, config, M, N, K, la, lb, in_dt, out_dt, epi, use_s, use_r):
    check_ex(M, N, K, in_dt, out_dt, la, lb, epi, kernel, config, use_s, use_r, False, seed=M + N + K)


def test_unaligned_scale_or_residual_uses_generic():
    # a column scale 4 bytes off 16-byte alignment sends the call to the
    # generic kernel, which must still be correct
    M, N, K = 256, 256, 128
    name = check_ex(M, N, K, "bf16", "bf16", "row", "col", "bias_relu", "auto", -1, True, True, True, seed=3,
                    scale_offset=1)
    assert name.startswith("tile_")  # the plan's choice; the run itself went to the generic kernel


def test_extras_none_equals_plain_run():
    # run_ex with a NULL extras pointer is gemm_epi_run
    M, N, K = 512, 512, 256
    bits = inputs.make_inputs(M, N, K, "bf16", "row", "col", True, 16.0, 0.1, seed=4)
    A, B = parity.to_device(bits["A"], "bf16"), parity.to_device(bits["B"], "bf16")
    bias = parity.to_device(bits["bias"], "bf16")
    plan = gb.Plan(M, N, K, "bf16", "bf16", "row", "col", "bias_silu")
    outs = []
    for use_ex in (False, True):
        C = parity.empty_out(M * N, "bf16")
        s = torch.cuda.current_stream().cuda_stream
        if use_ex:
            st = gb.gemm_epi_run_ex(plan.handle, A.data_ptr(), B.data_ptr(), bias.data_ptr(), None, None,
                                    C.data_ptr(), None, 0, s, extras_null=True)
        else:
            st = gb.gemm_epi_run(plan.handle, A.data_ptr(), B.data_ptr(), bias.data_ptr(), C.data_ptr(), s)
        assert st == 0
        torch.cuda.synchronize()
        outs.append(parity.out_bits(C))
    plan.close()
    assert np.array_equal(outs[0], outs[1])


# ---------------------------------------------------------------------------
# FP8 E4M3 output (and the output scale)
# ---------------------------------------------------------------------------

# N a multiple of 16 (1-byte rows of C stay 16-byte aligned in the tile kernel)
FP8_TILE_SHAPES = {0: (512, 512, 192), 1: (256, 384, 128), 2: (192, 128, 320), 3: (768, 512, 256)}
FP8_TILE_EDGE_SHAPES = {0: (264, 528, 192), 1: (200, 144, 128), 2: (72, 208, 256), 3: (304, 272, 128)}
# (epilogue, column scale, output scale)
FP8_CASES = [("none", False, False), ("bias_relu", False, True), ("bias", True, True), ("relu", True, False)]


@pytest.mark.parametrize("config", [0, 1, 2, 3])
@pytest.mark.parametrize("la,lb", LAYOUTS)
@pytest.mark.parametrize("edge", [False, True])
def test_tile_fp8_integer_bitexact(config, la, lb, edge):
    M, N, K = (FP8_TILE_EDGE_SHAPES if edge else FP8_TILE_SHAPES)[config]
    for in_dt in ("bf16", "f16"):
        for epi, use_s, use_q in FP8_CASES:
            # operands in [-2, 2]: sums reach past 448, so saturation is exercised
            name = check_ex(M, N, K, in_dt, "fp8", la, lb, epi, "tile", config, use_s, False, True,
                            seed=config * 5 + len(epi), use_oscale=use_q)
            assert name.startswith("tile_")


@pytest.mark.parametrize("config", [0, 3, 5])
@pytest.mark.parametrize("M,N", [(1, 96), (32, 96), (9, 40)])
def test_skinny_fp8_integer_bitexact(config, M, N):
    kc, slots = [(256, 5), (256, 4), (256, 4), (128, 8), (256, 2), (128, 2)][config]
    K = kc * (slots + 1)
    for epi, use_s, use_q in FP8_CASES:
        name = check_ex(M, N, K, "bf16", "fp8", "row", "col", epi, "skinny", config, use_s, False, True,
                        seed=M + N + config, use_oscale=use_q)
        assert name.startswith("skinny_")


def test_skinny_split_fp8_integer_bitexact():
    M, N, K = 32, 1024, 8192
    plan = gb.Plan(M, N, K, "bf16", "fp8", "row", "col", "bias")
    ws = torch.zeros(plan.workspace_size, dtype=torch.uint8, device="cuda")
    plan.close()
    for rep in range(2):
        check_ex(M, N, K, "bf16", "fp8", "row", "col", "bias", "auto", -1, True, False, True, seed=rep,
                 workspace=ws, use_oscale=True)
    assert not ws.cpu().numpy().any()  # the whole workspace is left zero-filled


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (37, 53, 29), (65, 130, 200)])
@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_generic_fp8_integer_bitexact(M, N, K, la, lb):
    for epi, use_s, use_q in FP8_CASES:
        check_ex(M, N, K, "f16", "fp8", la, lb, epi, "generic", 0, use_s, False, True, seed=M + K, use_oscale=use_q)


@pytest.mark.parametrize("kernel,config,M,N,K,la,lb", [
    ("tile", 0, 768, 1024, 512, "row", "col"),
    ("tile", 1, 384, 256, 1024, "col", "row"),
    ("tile", 3, 1008, 1008, 1024, "row", "col"),
    ("skinny", 0, 32, 512, 4096, "row", "col"),
    ("generic", 0, 97, 61, 333, "row", "row"),
])
@pytest.mark.parametrize("epi", ["bias_gelu", "bias_silu", "none"])
def test_fp8_random_tolerance(kernel, config, M, N, K, la, lb, epi):
    check_ex(M, N, K, "bf16", "fp8", la, lb, epi, kernel, config, True, False, False, seed=M + K,
             use_oscale=True)


def test_fp8_rejects_residual():
    M, N, K = 256, 256, 128
    plan = gb.Plan(M, N, K, "bf16", "fp8", "row", "col", "none")
    A = torch.zeros(M * K, dtype=torch.bfloat16, device="cuda")
    B = torch.zeros(K * N, dtype=torch.bfloat16, device="cuda")
    C = torch.empty(M * N, dtype=torch.float8_e4m3fn, device="cuda")
    R = torch.zeros(M * N, dtype=torch.float8_e4m3fn, device="cuda")
    st = gb.gemm_epi_run_ex(plan.handle, A.data_ptr(), B.data_ptr(), None, None, R.data_ptr(), C.data_ptr(), None, 0,
                            torch.cuda.current_stream().cuda_stream)
    plan.close()
    assert st == 1
