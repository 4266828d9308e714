"""Parity of the HIP library (through its C ABI) with the CPU oracle.

  * integer-valued operands: every product and partial sum is an exact
    small integer in fp32, so for none/ReLU/bias/bias+ReLU the GPU output
    must equal the oracle's bit for bit, whatever the accumulation order;
    this pins indexing, layouts, swizzles, pipelining and rasterisation;
  * N(0,1)-type operands at sizes that span several tiles, and the five
    workloads at full size in the launch configuration the benchmark
    times (outputs sampled where the full oracle would take too long):
    relative Frobenius error <= 1e-3 and max error <= 2e-2 after output
    rounding (tests/parity.py states the one-ulp tie rule).
"""
import numpy as np
import pytest
import torch

import oracle
from epilogue_gemm_amd import binding as gb
from epilogue_gemm_amd import inputs
from tests import parity

pytestmark = pytest.mark.gpu

EPIS = ["none", "relu", "bias", "bias_relu", "bias_gelu"]
BITWISE_EPIS = {"none", "relu", "bias", "bias_relu"}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gb.load_library()
    torch.cuda.init()


def run_gpu(bits, M, N, K, in_dt, out_dt, la, lb, epi, kernel="auto", config=-1, offset=0):
    """Runs one problem through the library; `offset` shifts every device
    pointer by that many elements (to test unaligned pointers)."""
    def dev(b):
        if b is None:
            return None
        t = parity.to_device(np.concatenate([np.zeros(offset, np.uint16), b.reshape(-1)]), in_dt)
        return t[offset:]

    A, B, bias = dev(bits["A"]), dev(bits["B"]), dev(bits["bias"])
    Cfull = parity.empty_out(M * N + offset, out_dt)
    C = Cfull[offset:]
    C.fill_(float("nan"))
    plan = gb.Plan(M, N, K, in_dt, out_dt, la, lb, epi, kernel, config)
    st = gb.gemm_epi_run(plan.handle, A.data_ptr(), B.data_ptr(), bias.data_ptr() if bias is not None else None,
                         C.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, gb.gemm_epi_status_string(st)
    torch.cuda.synchronize()
    name = plan.name
    plan.close()
    return parity.out_bits(C), name


def oracle_full(bits, M, N, K, in_dt, out_dt, la, lb, epi):
    return oracle.gemm_epi(bits["A"], bits["B"], bits["bias"], M, N, K, in_dt, out_dt, la, lb, epi)


def check_case(bits, M, N, K, in_dt, out_dt, la, lb, epi, kernel, config, bitwise, offset=0):
    got, name = run_gpu(bits, M, N, K, in_dt, out_dt, la, lb, epi, kernel, config, offset)
    y, c = oracle_full(bits, M, N, K, in_dt, out_dt, la, lb, epi)
    if bitwise:
        mism = np.count_nonzero(got.reshape(-1) != c.reshape(-1).astype(got.dtype))
        assert mism == 0, f"{name}: {mism} of {got.size} outputs differ from the oracle bit pattern"
    else:
        r = parity.compare(got, c, y, out_dt)
        assert r["ok"], f"{name}: {r}"
    return name


# ---------------------------------------------------------------------------
# integer operands: bit-exact
# ---------------------------------------------------------------------------

TILE_SHAPES = {0: (512, 512, 192), 1: (256, 384, 128), 2: (192, 128, 320), 3: (768, 512, 256)}


@pytest.mark.parametrize("config", [0, 1, 2, 3])
@pytest.mark.parametrize("la,lb", [("row", "col"), ("row", "row"), ("col", "col"), ("col", "row")])
@pytest.mark.parametrize("in_dt,out_dt", [("f16", "f16"), ("bf16", "bf16"), ("f16", "f32"), ("bf16", "f32")])
def test_tile_integer_bitexact(config, la, lb, in_dt, out_dt):
    M, N, K = TILE_SHAPES[config]
    epis = EPIS if (la, lb) in (("row", "col"), ("row", "row")) else ["bias_relu", "bias_gelu"]
    for epi in epis:
        bits = inputs.integer_inputs(M, N, K, in_dt, la, lb, epi.startswith("bias"), seed=config * 7 + len(epi))
        name = check_case(bits, M, N, K, in_dt, out_dt, la, lb, epi, "tile", config, epi in BITWISE_EPIS)
        assert name.startswith("tile_")


# M and N that are not tile multiples: the last tile row and column are
# shifted back to end at M and N and overlap their neighbours
TILE_EDGE_SHAPES = {0: (264, 520, 192), 1: (200, 136, 128), 2: (72, 200, 256), 3: (304, 264, 128)}


@pytest.mark.parametrize("config", [0, 1, 2, 3])
@pytest.mark.parametrize("la,lb", [("row", "col"), ("row", "row"), ("col", "col"), ("col", "row")])
@pytest.mark.parametrize("in_dt,out_dt", [("bf16", "bf16"), ("f16", "f32")])
def test_tile_edge_integer_bitexact(config, la, lb, in_dt, out_dt):
    M, N, K = TILE_EDGE_SHAPES[config]
    for epi in ("relu", "bias_relu"):
        bits = inputs.integer_inputs(M, N, K, in_dt, la, lb, epi.startswith("bias"), seed=config * 11 + len(epi))
        name = check_case(bits, M, N, K, in_dt, out_dt, la, lb, epi, "tile", config, True)
        assert name.startswith("tile_")


# K a multiple of 8 but not of 64: the first k-step is partial, its leading
# 64 - K % 64 k-values loaded as zeros
@pytest.mark.parametrize("config", [0, 1, 2, 3])
@pytest.mark.parametrize("la,lb", [("row", "col"), ("row", "row"), ("col", "col"), ("col", "row")])
def test_tile_ktail_integer_bitexact(config, la, lb):
    M, N = {0: (264, 520), 1: (256, 136), 2: (72, 200), 3: (304, 264)}[config]
    for K in (72, 104, 1000):
        for in_dt, out_dt, epi in (("bf16", "bf16", "bias_relu"), ("f16", "f32", "none")):
            bits = inputs.integer_inputs(M, N, K, in_dt, la, lb, epi.startswith("bias"), seed=K + config)
            name = check_case(bits, M, N, K, in_dt, out_dt, la, lb, epi, "tile", config, True)
            assert name.startswith("tile_")


@pytest.mark.parametrize("kpad", [8, 16, 24, 32, 40, 48, 56])
def test_tile_ktail_every_padding(kpad):
    M, N, K = 128, 128, 128 - kpad
    for la, lb in (("row", "col"), ("col", "row")):
        bits = inputs.integer_inputs(M, N, K, "bf16", la, lb, True, seed=kpad)
        check_case(bits, M, N, K, "bf16", "bf16", la, lb, "bias", "tile", 2, True)


@pytest.mark.parametrize("M", [1, 32])
@pytest.mark.parametrize("N", [40, 1000])
def test_skinny_edge_integer_bitexact(M, N):
    # N % 32 != 0: the last workgroup's columns are shifted back to end at N
    K = 1280
    for in_dt, out_dt, epi in (("bf16", "bf16", "bias_relu"), ("f16", "f32", "bias")):
        bits = inputs.integer_inputs(M, N, K, in_dt, "row", "col", True, seed=M + N)
        name = check_case(bits, M, N, K, in_dt, out_dt, "row", "col", epi, "auto", -1, True)
        assert name.startswith("skinny_")


# split K: narrow N with a workspace; the last workgroup of each column
# block sums the partials in split order
@pytest.mark.parametrize("M,N,K", [(32, 1024, 8192), (7, 96, 4096), (1, 40, 2560)])
def test_skinny_split_integer_bitexact(M, N, K):
    for in_dt, out_dt, epi in (("bf16", "bf16", "bias_relu"), ("f16", "f32", "none")):
        bits = inputs.integer_inputs(M, N, K, in_dt, "row", "col", epi.startswith("bias"), seed=N + K)
        plan = gb.Plan(M, N, K, in_dt, out_dt, "row", "col", epi)
        assert plan.kernel == "skinny" and plan.workspace_size > 0
        ws = torch.zeros(plan.workspace_size, dtype=torch.uint8, device="cuda")
        A = parity.to_device(bits["A"], in_dt)
        B = parity.to_device(bits["B"], in_dt)
        bias = parity.to_device(bits["bias"], in_dt) if bits["bias"] is not None else None
        y, c = oracle_full(bits, M, N, K, in_dt, out_dt, "row", "col", epi)
        for rep in range(2):  # the second run relies on the first leaving the counters at zero
            C = parity.empty_out(M * N, out_dt)
            C.fill_(float("nan"))
            plan.run(A, B, bias, C, workspace=ws)
            torch.cuda.synchronize()
            got = parity.out_bits(C)
            mism = np.count_nonzero(got.reshape(-1) != c.reshape(-1).astype(got.dtype))
            assert mism == 0, (rep, epi, mism)
        # every completed run leaves the whole workspace zero-filled
        # (partials cleared by the summing workgroup, counters re-armed)
        assert not ws.cpu().numpy().any()
        plan.close()


def test_skinny_split_shared_workspace():
    # two split plans on one workspace: the narrower plan's counters lie
    # inside the wider plan's partial area, so each run must leave the
    # whole workspace zero-filled for the other's next run
    M, K = 32, 8192
    plans, data = [], []
    for N in (2048, 1024):
        bits = inputs.integer_inputs(M, N, K, "bf16", "row", "col", True, seed=N)
        plan = gb.Plan(M, N, K, "bf16", "bf16", "row", "col", "bias_relu")
        assert plan.kernel == "skinny" and plan.workspace_size > 0
        A, B = parity.to_device(bits["A"], "bf16"), parity.to_device(bits["B"], "bf16")
        bias = parity.to_device(bits["bias"], "bf16")
        c = oracle_full(bits, M, N, K, "bf16", "bf16", "row", "col", "bias_relu")[1]
        plans.append(plan)
        data.append((A, B, bias, c, N))
    assert plans[0].workspace_size > plans[1].workspace_size
    ws = torch.zeros(plans[0].workspace_size, dtype=torch.uint8, device="cuda")
    for rep in range(3):
        for plan, (A, B, bias, c, N) in zip(plans, data):
            C = parity.empty_out(M * N, "bf16")
            plan.run(A, B, bias, C, workspace=ws)
            torch.cuda.synchronize()
            mism = np.count_nonzero(parity.out_bits(C).reshape(-1) != c.reshape(-1).astype(np.uint16))
            assert mism == 0, (rep, N, mism)
    assert not ws.cpu().numpy().any()
    for plan in plans:
        plan.close()


def test_skinny_split_random_and_fallback():
    M, N, K = 32, 1024, 8192
    bits = inputs.make_inputs(M, N, K, "bf16", "row", "col", True, float(np.sqrt(K)), 0.1, seed=12)
    plan = gb.Plan(M, N, K, "bf16", "bf16", "row", "col", "bias")
    A, B = parity.to_device(bits["A"], "bf16"), parity.to_device(bits["B"], "bf16")
    bias = parity.to_device(bits["bias"], "bf16")
    y, c = oracle_full(bits, M, N, K, "bf16", "bf16", "row", "col", "bias")
    outs = []
    for ws in (torch.zeros(plan.workspace_size, dtype=torch.uint8, device="cuda"),
               torch.zeros(plan.workspace_size - 16, dtype=torch.uint8, device="cuda"),  # too small: no split
               None):
        C = parity.empty_out(M * N, "bf16")
        plan.run(A, B, bias, C, workspace=ws)
        torch.cuda.synchronize()
        r = parity.compare(parity.out_bits(C), c, y, "bf16")
        assert r["ok"], r
        outs.append(parity.out_bits(C))
    assert np.array_equal(outs[1], outs[2])  # the fallback is the unsplit kernel
    plan.close()


# (k per chunk, ring slots) of each skinny configuration, in order
SKINNY_CHUNKS = [(256, 5), (256, 4), (256, 4), (128, 8), (256, 2), (128, 2)]


@pytest.mark.parametrize("config", range(len(SKINNY_CHUNKS)))
@pytest.mark.parametrize("M", [1, 7, 31, 32])
@pytest.mark.parametrize("in_dt,out_dt", [("bf16", "bf16"), ("f16", "f16"), ("bf16", "f32")])
def test_skinny_integer_bitexact(config, M, in_dt, out_dt):
    # one ring turn; then chunk counts that leave a head of one and of
    # P - 1 chunks before the whole turns
    N = 96
    kc, slots = SKINNY_CHUNKS[config]
    cases = [(kc * slots, epi) for epi in EPIS] + [(kc * (2 * slots + 1), "bias_relu"), (kc * (2 * slots - 1), "bias")]
    for K, epi in cases:
        bits = inputs.integer_inputs(M, N, K, in_dt, "row", "col", epi.startswith("bias"), seed=M + config)
        name = check_case(bits, M, N, K, in_dt, out_dt, "row", "col", epi, "skinny", config, epi in BITWISE_EPIS)
        assert name.startswith("skinny_")


@pytest.mark.parametrize("config", range(len(SKINNY_CHUNKS)))
@pytest.mark.parametrize("M", [1, 32])
def test_skinny_k_tail_integer_bitexact(config, M):
    # K not a whole number of chunks: the axis is shifted so that the first
    # chunk is the partial one, its positions before k = 0 loaded as zeros;
    # the largest pad (K % kc = 8), a middle one and the smallest (kc - 8),
    # with chunk counts that leave different heads before the ring turns
    N = 96
    kc, slots = SKINNY_CHUNKS[config]
    for K, epi in ((kc * (slots - 1) + 8, "bias_relu"), (kc * slots + kc // 2 + 8, "bias"),
                   (kc * 2 * slots - 8, "none")):
        for in_dt, out_dt in (("bf16", "bf16"), ("f16", "f32")):
            bits = inputs.integer_inputs(M, N, K, in_dt, "row", "col", epi.startswith("bias"), seed=K + M)
            name = check_case(bits, M, N, K, in_dt, out_dt, "row", "col", epi, "skinny", config, True)
            assert name.startswith("skinny_")


def test_skinny_k_tail_split_and_auto():
    # the automatic plan for a padded K is the skinny kernel; with a
    # workspace it splits K (the padded chunk belongs to split 0)
    for M, N, K in ((32, 1024, 7944), (5, 200, 3336)):  # 32 chunks in 4 splits, 14 in 2
        bits = inputs.integer_inputs(M, N, K, "bf16", "row", "col", True, seed=K)
        plan = gb.Plan(M, N, K, "bf16", "bf16", "row", "col", "bias_relu")
        assert plan.kernel == "skinny" and plan.workspace_size > 0, plan.name
        A, B = parity.to_device(bits["A"], "bf16"), parity.to_device(bits["B"], "bf16")
        bias = parity.to_device(bits["bias"], "bf16")
        y, c = oracle_full(bits, M, N, K, "bf16", "bf16", "row", "col", "bias_relu")
        ws = torch.zeros(plan.workspace_size, dtype=torch.uint8, device="cuda")
        for w in (ws, ws, None):
            C = parity.empty_out(M * N, "bf16")
            C.fill_(float("nan"))
            plan.run(A, B, bias, C, workspace=w)
            torch.cuda.synchronize()
            mism = np.count_nonzero(parity.out_bits(C).reshape(-1) != c.reshape(-1).astype(np.uint16))
            assert mism == 0, (M, N, K, w is None, mism)
        assert not ws.cpu().numpy().any()
        plan.close()


def test_skinny_k_tail_random_decode_shape():
    # 32 x 8192 x 8200, random operands, automatic plan
    M, N, K = 32, 8192, 8200
    bits = inputs.make_inputs(M, N, K, "bf16", "row", "col", True, float(np.sqrt(K)), 0.1, seed=21)
    got, name = run_gpu(bits, M, N, K, "bf16", "bf16", "row", "col", "bias_gelu")
    assert name == "skinny_32n_8w_5x256k"
    y, c = oracle_full(bits, M, N, K, "bf16", "bf16", "row", "col", "bias_gelu")
    r = parity.compare(got, c, y, "bf16")
    assert r["ok"], r


# row-major B (K x N, n contiguous): configurations 6-9, whose B fragments
# come from transposing LDS reads (9: 64 columns per workgroup)
SKINNY_ROWB = {6: (256, 5), 7: (128, 8), 8: (128, 2), 9: (128, 6)}


@pytest.mark.parametrize("config", sorted(SKINNY_ROWB))
@pytest.mark.parametrize("M", [1, 7, 32])
@pytest.mark.parametrize("in_dt,out_dt", [("bf16", "bf16"), ("f16", "f32")])
def test_skinny_rowb_integer_bitexact(config, M, in_dt, out_dt):
    # one ring turn, heads of one and of P - 1 chunks before the whole turns,
    # K tails (the largest and a middle pad); N = 1000 shifts the last
    # column block back to end at N
    kc, slots = SKINNY_ROWB[config]
    cases = [(kc * slots, "bias_relu", 96), (kc * (2 * slots + 1), "bias", 1000), (kc * (2 * slots - 1), "none", 96),
             (kc * (slots - 1) + 8, "relu", 40 if config != 9 else 72), (kc * slots + kc // 2 + 8, "bias", 96)]
    for K, epi, N in cases:
        bits = inputs.integer_inputs(M, N, K, in_dt, "row", "row", epi.startswith("bias"), seed=M + K)
        name = check_case(bits, M, N, K, in_dt, out_dt, "row", "row", epi, "skinny", config, True)
        assert name.startswith("skinny_rowb_"), name


def test_skinny_rowb_split_and_random():
    # split K with a workspace (bit-exact on two runs, workspace left
    # zero-filled), then the 32 x 8192 x 8192 decode shape with random
    # operands through the automatic plan
    M, N, K = 32, 1024, 7928  # 62 chunks of 128 (the first padded) in 2 splits
    bits = inputs.integer_inputs(M, N, K, "bf16", "row", "row", True, seed=5)
    plan = gb.Plan(M, N, K, "bf16", "bf16", "row", "row", "bias_relu")
    assert plan.name == "skinny_rowb_64n_8w_6x128k" and plan.workspace_size > 0
    A, B = parity.to_device(bits["A"], "bf16"), parity.to_device(bits["B"], "bf16")
    bias = parity.to_device(bits["bias"], "bf16")
    c = oracle_full(bits, M, N, K, "bf16", "bf16", "row", "row", "bias_relu")[1]
    ws = torch.zeros(plan.workspace_size, dtype=torch.uint8, device="cuda")
    for w in (ws, ws, None):
        C = parity.empty_out(M * N, "bf16")
        C.fill_(float("nan"))
        plan.run(A, B, bias, C, workspace=w)
        torch.cuda.synchronize()
        mism = np.count_nonzero(parity.out_bits(C).reshape(-1) != c.reshape(-1).astype(np.uint16))
        assert mism == 0, (w is None, mism)
    assert not ws.cpu().numpy().any()
    plan.close()
    M, N, K = 32, 8192, 8192
    bits = inputs.make_inputs(M, N, K, "bf16", "row", "row", True, float(np.sqrt(K)), 0.1, seed=22)
    got, name = run_gpu(bits, M, N, K, "bf16", "bf16", "row", "row", "bias_gelu")
    assert name == "skinny_rowb_64n_8w_6x128k"
    y, c = oracle_full(bits, M, N, K, "bf16", "bf16", "row", "row", "bias_gelu")
    r = parity.compare(got, c, y, "bf16")
    assert r["ok"], r


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (2, 8, 4), (37, 53, 29), (65, 130, 200), (3, 700, 5)])
@pytest.mark.parametrize("la,lb", [("row", "col"), ("row", "row"), ("col", "col"), ("col", "row")])
def test_generic_integer_bitexact(M, N, K, la, lb):
    for in_dt, out_dt in [("f16", "f16"), ("bf16", "bf16"), ("bf16", "f32")]:
        for epi in EPIS:
            bits = inputs.integer_inputs(M, N, K, in_dt, la, lb, epi.startswith("bias"), seed=M * N + K)
            check_case(bits, M, N, K, in_dt, out_dt, la, lb, epi, "generic", 0, epi in BITWISE_EPIS)


# The generic kernel's tiling: 64 x 64 outputs per workgroup, K through LDS
# 16 at a time (the last step stopping at K), so shapes straddling those
# steps and tiles, and every layout, keep the bits of a per-output loop.
@pytest.mark.parametrize("M,N,K", [(64, 64, 16), (129, 63, 17), (130, 200, 15), (200, 130, 33), (70, 300, 1001)])
@pytest.mark.parametrize("la,lb", [("row", "col"), ("col", "row")])
def test_generic_tiles_and_k_steps_bitexact(M, N, K, la, lb):
    for in_dt, out_dt, epi in (("bf16", "bf16", "bias_relu"), ("f16", "f32", "none"), ("f16", "fp8", "bias")):
        bits = inputs.integer_inputs(M, N, K, in_dt, la, lb, epi.startswith("bias"), seed=M + N + K)
        assert check_case(bits, M, N, K, in_dt, out_dt, la, lb, epi, "generic", 0, True) == "generic"


def test_generic_random_tolerance_large_odd_k():
    M, N, K = 300, 520, 1001
    for la, lb in (("row", "col"), ("col", "col")):
        bits = inputs.make_inputs(M, N, K, "bf16", la, lb, True, float(np.sqrt(K)), 0.1, seed=K)
        got, name = run_gpu(bits, M, N, K, "bf16", "bf16", la, lb, "bias_gelu")
        assert name == "generic"  # K % 8 != 0: the fast kernels do not apply
        y, c = oracle_full(bits, M, N, K, "bf16", "bf16", la, lb, "bias_gelu")
        r = parity.compare(got, c, y, "bf16")
        assert r["ok"], r


# More than 65535 row tiles of 64: the grid's y extent stops at 65535 and
# each workgroup loops over the row tiles past it.
def test_generic_rows_past_the_grid_y_extent():
    M, N, K = 64 * 65535 + 100, 3, 8
    bits = inputs.integer_inputs(M, N, K, "bf16", "row", "col", True, seed=5)
    assert check_case(bits, M, N, K, "bf16", "bf16", "row", "col", "bias_relu", "generic", 0, True) == "generic"


# ---------------------------------------------------------------------------
# random operands: tolerance
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kernel,config,M,N,K,la,lb", [
    ("tile", 0, 768, 1024, 512, "row", "col"),
    ("tile", 0, 512, 768, 640, "row", "row"),
    ("tile", 3, 512, 1024, 704, "row", "col"),
    ("tile", 3, 768, 512, 384, "row", "row"),
    ("tile", 3, 1000, 1000, 1024, "row", "col"),
    ("tile", 3, 1000, 1000, 1000, "row", "col"),
    ("tile", 0, 512, 768, 584, "row", "row"),
    ("tile", 1, 384, 256, 968, "col", "col"),
    ("tile", 2, 1000, 1000, 1024, "col", "row"),
    ("tile", 1, 384, 256, 1024, "row", "row"),
    ("tile", 2, 320, 192, 448, "col", "col"),
    ("skinny", 0, 32, 512, 4096, "row", "col"),
    ("skinny", 5, 5, 160, 768, "row", "col"),
    ("skinny", 0, 17, 256, 6144, "row", "col"),
    ("skinny", 3, 32, 96, 3072, "row", "col"),
    ("skinny", 1, 3, 64, 6144, "row", "col"),
    ("skinny", 0, 32, 256, 8192, "row", "col"),
    ("skinny", 2, 11, 128, 4352, "row", "col"),
    ("skinny", 4, 29, 64, 1792, "row", "col"),
    ("generic", 0, 97, 61, 333, "row", "row"),
    ("generic", 0, 64, 64, 4096, "col", "col"),
])
@pytest.mark.parametrize("in_dt,out_dt,epi", [("bf16", "bf16", "bias_gelu"), ("f16", "f16", "relu"),
                                              ("f16", "f32", "none"), ("bf16", "bf16", "bias")])
def test_random_tolerance(kernel, config, M, N, K, la, lb, in_dt, out_dt, epi):
    bits = inputs.make_inputs(M, N, K, in_dt, la, lb, epi.startswith("bias"), float(np.sqrt(K)), 0.1, seed=M + N)
    check_case(bits, M, N, K, in_dt, out_dt, la, lb, epi, kernel, config, bitwise=False)


def test_unaligned_pointers_use_generic_and_stay_correct():
    M, N, K = 256, 256, 128
    bits = inputs.make_inputs(M, N, K, "bf16", "row", "col", True, 11.0, 0.1, seed=5)
    got_a, name_a = run_gpu(bits, M, N, K, "bf16", "bf16", "row", "col", "bias_gelu")
    got_u, name_u = run_gpu(bits, M, N, K, "bf16", "bf16", "row", "col", "bias_gelu", offset=1)
    assert name_a.startswith("tile_")
    y, c = oracle_full(bits, M, N, K, "bf16", "bf16", "row", "col", "bias_gelu")
    for got in (got_a, got_u):
        r = parity.compare(got, c, y, "bf16")
        assert r["ok"], r


def test_run_is_deterministic():
    M, N, K = 1024, 1024, 512
    bits = inputs.make_inputs(M, N, K, "bf16", "row", "col", True, 22.0, 0.1, seed=6)
    a, _ = run_gpu(bits, M, N, K, "bf16", "bf16", "row", "col", "bias_gelu", "tile", 0)
    b, _ = run_gpu(bits, M, N, K, "bf16", "bf16", "row", "col", "bias_gelu", "tile", 0)
    assert np.array_equal(a, b)


def test_all_tile_configs_agree_on_integers():
    # every tile configuration and the generic kernel give identical bits
    # (the 16x16x32 configuration takes A row-major and B column-major only)
    M, N, K = 512, 512, 320
    bits = inputs.integer_inputs(M, N, K, "f16", "row", "row", True, seed=8)
    ref, _ = run_gpu(bits, M, N, K, "f16", "f16", "row", "row", "bias_relu", "generic", 0)
    for cfg in range(4):
        got, _ = run_gpu(bits, M, N, K, "f16", "f16", "row", "row", "bias_relu", "tile", cfg)
        assert np.array_equal(got, ref), cfg
    # K = 384 (6 chunks of 64) also suits the rings of 2 slots; K = 512 those
    # of 4 and 8
    for K in (384, 512):
        bits = inputs.integer_inputs(M, N, K, "bf16", "row", "col", True, seed=9)
        ref, _ = run_gpu(bits, M, N, K, "bf16", "bf16", "row", "col", "bias_relu", "generic", 0)
        ran = 0
        for cfg in range(gb.gemm_epi_num_configs("tile")):
            h = gb.gemm_epi_plan(M, N, K, "bf16", "bf16", "row", "col", "bias_relu")
            ok = gb.gemm_epi_plan_select(h, "tile", cfg) == 0
            gb.gemm_epi_destroy(h)
            if not ok:
                continue
            got, _ = run_gpu(bits, M, N, K, "bf16", "bf16", "row", "col", "bias_relu", "tile", cfg)
            assert np.array_equal(got, ref), (K, cfg)
            ran += 1
        assert ran >= 6, K


# ---------------------------------------------------------------------------
# the five workloads at full size, auto-selected plan (what the benchmark runs)
# ---------------------------------------------------------------------------

def _sample_points(M, N, n, seed):
    rng = np.random.default_rng(seed)
    rows = rng.integers(0, M, n)
    cols = rng.integers(0, N, n)
    # plus one full row and one full column
    rows = np.concatenate([rows, np.full(N, M // 3), np.arange(M)])
    cols = np.concatenate([cols, np.arange(N), np.full(M, N // 5)])
    return rows, cols


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_workload_full_size(name):
    w = inputs.WORKLOADS[name]
    bits = inputs.workload_inputs(w)
    print(f"[workload] {w.name}", flush=True)
    got, kname = run_gpu(bits, w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.layout_a, w.layout_b, w.epilogue)
    got = got.reshape(w.M, w.N)
    assert kname != "generic"
    assert np.all(np.isfinite(parity.values(got.reshape(-1), w.out_dtype)))
    if w.M * w.N * w.K <= 2**31:
        y, c = oracle_full(bits, w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.layout_a, w.layout_b, w.epilogue)
        r = parity.compare(got, c, y, w.out_dtype)
    else:
        rows, cols = _sample_points(w.M, w.N, 8192, seed=w.seed)
        y, c = oracle.gemm_epi_points(bits["A"], bits["B"], bits["bias"], w.M, w.N, w.K, w.in_dtype, w.out_dtype,
                                      w.layout_a, w.layout_b, w.epilogue, rows, cols)
        c = c.astype(np.uint16 if w.out_dtype != "f32" else np.uint32)
        r = parity.compare(got[rows, cols], c, y, w.out_dtype)
    print(f"[workload] {w.name} kernel={kname} {r}", flush=True)
    assert r["ok"], r


# The same workloads, shapes and automatic plans on integer operands, where
# every fp32 sum is exact: the whole output against the oracle, bit for bit
# for the exact epilogues; for 8192^3 the first and the last band of 256
# rows (a tile row each, both edges of the raster) in full, and bias+GELU
# under the tolerance rule.
@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_workload_integer_outputs(name):
    w = inputs.WORKLOADS[name]
    bits = inputs.integer_inputs(w.M, w.N, w.K, w.in_dtype, w.layout_a, w.layout_b, w.epilogue.startswith("bias"),
                                 seed=w.seed + 1)
    print(f"[workload-int] {w.name}", flush=True)
    got, kname = run_gpu(bits, w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.layout_a, w.layout_b, w.epilogue)
    got = got.reshape(w.M, w.N)
    assert kname != "generic"
    exact = w.epilogue in BITWISE_EPIS
    if w.M * w.N * w.K <= 2**37:
        y, c = oracle_full(bits, w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.layout_a, w.layout_b, w.epilogue)
        got_s, c, y = got.reshape(-1), c.reshape(-1), y.reshape(-1)
    else:
        band = np.concatenate([np.arange(256), np.arange(w.M - 256, w.M)])
        rows = np.repeat(band, w.N)
        cols = np.tile(np.arange(w.N), band.size)
        y, c = oracle.gemm_epi_points(bits["A"], bits["B"], bits["bias"], w.M, w.N, w.K, w.in_dtype, w.out_dtype,
                                      w.layout_a, w.layout_b, w.epilogue, rows, cols)
        got_s = got[rows, cols]
    c = c.astype(got_s.dtype)
    if exact:
        mism = np.count_nonzero(got_s != c)
        assert mism == 0, f"{w.name} {kname}: {mism} of {got_s.size} outputs differ"
    else:
        r = parity.compare(got_s, c, y, w.out_dtype)
        assert r["ok"], r
    print(f"[workload-int] {w.name} kernel={kname} {got_s.size} outputs", flush=True)
