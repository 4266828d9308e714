"""Parity of the attention forward kernel (gemm_epi_attention_fwd, through
the C ABI) with the fp64 oracle, on seeded N(0, 1) inputs laid out
[B, S, H, D]: small shapes in full, the B, H, S, D = 4, 8, 1024, 64
workloads in full, and closed-form cases."""
import numpy as np
import pytest
import torch

import oracle
from epilogue_gemm_amd import binding as gb
from epilogue_gemm_amd import inputs
from tests import parity

pytestmark = pytest.mark.gpu

# Tolerance: the GEMM's bar for both formats, rel-Fro 1e-3 and max-abs 2e-2
# after output rounding (with the tie rule of tests/parity.py).  The kernel
# carries the probabilities into the second product with about 11
# significant bits in fp16 (one rounding, relative error <= 2^-11 per
# weight) and about 16 in bf16 (a rounded part plus its rounded remainder);
# since the weights of the row sum are the same rounded values, O is a
# weighted mean with perturbed weights and its error relative to O is of the
# order of that per-weight error, well under 1e-3.
TOL = {"f16": (parity.REL_FRO_TOL, parity.MAX_ABS_TOL), "bf16": (parity.REL_FRO_TOL, parity.MAX_ABS_TOL)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gb.load_library()


def run_gpu(d, B, S, H, D, dtype, causal):
    q, k, v = (parity.to_device(d[n], dtype).view(B, S, H, D) for n in ("Q", "K", "V"))
    o = torch.full_like(q, float("nan"))
    gb.attention_fwd(q, k, v, o, causal=causal)
    torch.cuda.synchronize()
    return parity.out_bits(o).reshape(B, S, H, D)


def check(got, y, o, dtype, what):
    rel, ab = TOL[dtype]
    r = parity.compare(got.reshape(-1), o.reshape(-1), y.reshape(-1), dtype, rel_tol=rel, abs_tol=ab)
    assert r["ok"], f"{what}: {r}"
    return r


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
# (2, 512, 2) and (3, 256, 4): workgroup counts 16 and 24, which the kernel
# renumbers across the XCDs (the others keep the launch order)
@pytest.mark.parametrize("B,S,H", [(1, 128, 1), (2, 384, 3), (1, 640, 2), (2, 512, 2), (3, 256, 4)])
def test_attention_small_full_parity(dtype, causal, B, S, H):
    D = 64
    d = inputs.attention_inputs(B, S, H, D, dtype, seed=S + H)
    got = run_gpu(d, B, S, H, D, dtype, causal)
    y, o = oracle.attention(d["Q"], d["K"], d["V"], B, S, H, D, dtype, causal)
    r = check(got, y, o, dtype, f"B{B} S{S} H{H} {dtype} causal={causal}")
    print(f"attention {dtype} causal={causal} B{B} S{S} H{H}: rel_fro={r['rel_fro']:.2e} max_abs={r['max_abs']:.2e}")


# S not a multiple of 128: the last query block reaches past S (those rows
# are not stored), the last key block is masked past S (its rows there load
# as zeros); S <= 64 leaves the second key parity without a block.  A guard
# of NaN past the output tensor must stay untouched.
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,S,H", [(1, 1, 1), (2, 50, 3), (1, 64, 1), (1, 77, 2), (2, 130, 1), (3, 200, 2),
                                   (1, 1000, 2)])
def test_attention_ragged_s_parity(dtype, causal, B, S, H):
    D = 64
    d = inputs.attention_inputs(B, S, H, D, dtype, seed=S + 7 * H)
    q, k, v = (parity.to_device(d[n], dtype).view(B, S, H, D) for n in ("Q", "K", "V"))
    n, guard = B * S * H * D, 4096
    o_all = torch.full((n + guard,), float("nan"), dtype=q.dtype, device="cuda")
    gb.attention_fwd(q, k, v, o_all[:n].view(B, S, H, D), causal=causal)
    torch.cuda.synchronize()
    bits = parity.out_bits(o_all)
    assert np.all(bits[n:] == bits[n + guard - 1]), "output written past the tensor"
    y, o = oracle.attention(d["Q"], d["K"], d["V"], B, S, H, D, dtype, causal)
    r = check(bits[:n].reshape(B, S, H, D), y, o, dtype, f"B{B} S{S} H{H} {dtype} causal={causal}")
    print(f"attention ragged {dtype} causal={causal} B{B} S{S} H{H}: rel_fro={r['rel_fro']:.2e}")


@pytest.mark.parametrize("name", list(inputs.ATTENTION_WORKLOADS))
def test_attention_workload_full_output(name):
    # the whole output of the workload (B, H, S, D = 4, 8, 1024, 64)
    w = inputs.ATTENTION_WORKLOADS[name]
    d = inputs.attention_inputs(w.B, w.S, w.H, w.D, w.dtype, w.seed)
    got = run_gpu(d, w.B, w.S, w.H, w.D, w.dtype, w.causal)
    y, o = oracle.attention(d["Q"], d["K"], d["V"], w.B, w.S, w.H, w.D, w.dtype, w.causal)
    r = check(got, y, o, w.dtype, name)
    print(f"{name}: rel_fro={r['rel_fro']:.2e} max_abs={r['max_abs']:.2e} on {got.size} outputs")


def test_attention_closed_forms():
    B, S, H, D, dtype = 1, 256, 2, 64, "f16"
    d = inputs.attention_inputs(B, S, H, D, dtype, seed=1)
    # every value row the same vector: O is that vector (exactly, up to the
    # sum of the rounded weights)
    row = np.linspace(-2.0, 2.0, D)
    vconst = oracle.encode_array(dtype, np.broadcast_to(row, (B, S, H, D)).reshape(-1)).astype(np.uint16)
    for causal in (False, True):
        got = run_gpu({**d, "V": vconst}, B, S, H, D, dtype, causal)
        y, o = oracle.attention(d["Q"], d["K"], vconst, B, S, H, D, dtype, causal)
        check(got, y, o, dtype, f"constant V causal={causal}")
    # causal query 0 sees key 0 only: O[0] = V[0] bit for bit
    got = run_gpu(d, B, S, H, D, dtype, True)
    assert np.array_equal(got[:, 0], d["V"].reshape(B, S, H, D)[:, 0])
    # Q = 0: uniform weights (the mean of the visible values)
    zq = np.zeros_like(d["Q"])
    for causal in (False, True):
        got = run_gpu({**d, "Q": zq}, B, S, H, D, dtype, causal)
        y, o = oracle.attention(zq, d["K"], d["V"], B, S, H, D, dtype, causal)
        check(got, y, o, dtype, f"Q = 0 causal={causal}")


def test_attention_rejects_unsupported():
    B, S, H = 1, 128, 1
    t = torch.zeros(B * S * H * 64 + 8, dtype=torch.float16, device="cuda")
    p = t.data_ptr()
    st = torch.cuda.current_stream().cuda_stream
    assert gb.gemm_epi_attention_fwd(p, p, p, p, B, S, H, 32, "f16", 0, st) == 2  # D != 64
    assert gb.gemm_epi_attention_fwd(p, p, p, p, B, 128 * 65535 + 1, H, 64, "f16", 0, st) == 2  # query blocks
    assert gb.gemm_epi_attention_fwd(p + 2, p, p, p, B, S, H, 64, "f16", 0, st) == 2  # unaligned
    assert gb.gemm_epi_attention_fwd(None, p, p, p, B, S, H, 64, "f16", 0, st) == 1
    assert gb.gemm_epi_attention_fwd(p, p, p, p, B, S, H, 64, "f32", 0, st) == 1
