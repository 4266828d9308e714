"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/gemm_epi.h declares, and gemm_epi_plan's validation
and kernel selection behave as the header documents.  gemm_epi_plan makes
no HIP call, so all of this runs on a machine without a GPU."""
import ctypes
import os
import subprocess

import pytest

from epilogue_gemm_amd import binding as gb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gb.LIB_PATH):
        pytest.fail("libgemm_epi.so is not built (run __graft_entry__.build())")
    return gb.load_library()


def test_exports_every_declared_function(lib):
    declared = gb.header_functions()
    assert len(declared) >= 8
    out = subprocess.run(["nm", "-D", "--defined-only", gb.LIB_PATH], capture_output=True, text=True, check=True)
    exported = {line.split()[-1] for line in out.stdout.splitlines() if line.strip()}
    missing = [f for f in declared if f not in exported]
    assert not missing, missing
    for f in declared:
        assert hasattr(lib, f)


def test_header_is_plain_c():
    # every header must compile as C with no HIP or C++ headers
    srcs = gb.headers()
    assert os.path.join(ROOT, "include", "gemm_epi.h") in srcs and len(srcs) >= 2
    for src in srcs:
        r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-x", "c", src],
                           capture_output=True, text=True)
        assert r.returncode == 0, (src, r.stderr)


def test_probe_argument_checks(lib):
    # argument validation happens before any HIP call
    assert gb.gemm_epi_probe_hbm_read(None, 1024, None, None) == 1
    assert gb.gemm_epi_probe_mfma(0, 1, None, None) == 1
    assert gb.gemm_epi_probe_mfma_flops(10, 4) == 4 * 4 * 10 * 8 * 16 * 16 * 32 * 2


def test_status_strings(lib):
    for code, name in gb.STATUS.items():
        assert gb.gemm_epi_status_string(code) == "GEMM_EPI_" + name
    assert gb.gemm_epi_status_string(99) == "GEMM_EPI_ERR_UNKNOWN"
    assert gb.gemm_epi_last_hip_error() == 0


def test_plan_rejects_invalid_arguments(lib):
    ok = dict(M=64, N=64, K=64, in_dtype="f16", out_dtype="f16", layout_a="row", layout_b="row", epilogue="none")
    assert gb.gemm_epi_plan_status(**ok) == 0
    for k, v in [("M", 0), ("N", -1), ("K", -1)]:
        assert gb.gemm_epi_plan_status(**{**ok, k: v}) == 1
    assert gb.gemm_epi_plan_status(**{**ok, "in_dtype": "f32", "out_dtype": "f32"}) == 1  # f32 input
    assert gb.gemm_epi_plan_status(**{**ok, "out_dtype": "bf16"}) == 1  # mixed 16-bit formats
    assert gb.gemm_epi_plan_status(**{**ok, "out_dtype": "fp8"}) == 0  # quantised output
    assert gb.gemm_epi_plan_status(**{**ok, "in_dtype": "fp8", "out_dtype": "fp8"}) == 1  # fp8 input
    raw = [0, 0, 0, 0, 0]
    for pos, bad in [(0, 7), (0, 3), (1, 9), (2, 2), (3, -1), (4, 7), (4, -1)]:
        args = list(raw)
        args[pos] = bad
        assert gb.gemm_epi_plan_status(64, 64, 64, *args, raw=True) == 1
    # null out pointer
    assert lib.gemm_epi_plan(None, 64, 64, 64, 0, 0, 0, 0, 0) == 1


def test_k_zero_is_the_degenerate_product_on_the_generic_kernel(lib):
    # K = 0: C = act(bias) (+ extras) from an empty sum; only the generic
    # kernel takes it, and A and B may be NULL
    for la, lb, epi in (("row", "col", "bias_gelu"), ("col", "row", "none"), ("row", "row", "bias")):
        h = gb.gemm_epi_plan(32, 8192, 0, "bf16", "bf16", la, lb, epi)
        try:
            assert gb.gemm_epi_plan_describe(h)[0] == "generic"
            assert gb.gemm_epi_workspace_size(h) == 0
            for fam in ("tile", "skinny"):
                assert gb.gemm_epi_plan_select(h, fam, 0) == 2
                assert gb.gemm_epi_plan_select(h, fam, -1) == 2
            assert gb.gemm_epi_plan_select(h, "auto", -1) == 0
            assert gb.gemm_epi_plan_describe(h)[0] == "generic"
            bias = 0x1000 if epi.startswith("bias") else None
            assert gb.gemm_epi_run(h, None, None, bias, None, None) == 1  # C is still required
            assert gb.gemm_epi_run(h, None, None, None if bias else 0x1000, 0x1000, None) == 1  # bias rule
        finally:
            gb.gemm_epi_destroy(h)


def test_plan_rejects_oversized(lib):
    big = 1 << 31
    assert gb.gemm_epi_plan_status(big, 1, 1, "f16", "f16", "row", "row", "none") == 2
    assert gb.gemm_epi_plan_status(65536, 32768, 1, "f16", "f16", "row", "row", "none") == 2  # M*N = 2^31
    assert gb.gemm_epi_plan_status(46340, 46340, 1, "f16", "f16", "row", "row", "none") == 0


def test_run_rejects_invalid_arguments_without_touching_the_device(lib):
    h = gb.gemm_epi_plan(64, 64, 64, "bf16", "bf16", "row", "col", "bias_gelu")
    try:
        p = 0x1000
        assert gb.gemm_epi_run(None, p, p, p, p, None) == 1  # null plan
        assert gb.gemm_epi_run(h, None, p, p, p, None) == 1  # null A
        assert gb.gemm_epi_run(h, p, p, None, p, None) == 1  # bias epilogue without bias
        assert gb.gemm_epi_run(h, p, p, p, None, None) == 1  # null C
    finally:
        gb.gemm_epi_destroy(h)
    h = gb.gemm_epi_plan(64, 64, 64, "f16", "f16", "row", "row", "relu")
    try:
        assert gb.gemm_epi_run(h, 0x1000, 0x1000, 0x1000, 0x1000, None) == 1  # bias without a bias epilogue
    finally:
        gb.gemm_epi_destroy(h)
    assert gb.gemm_epi_destroy(None) == 0


def test_run_ex_rejects_invalid_arguments_without_touching_the_device(lib):
    M, N = 64, 64
    h = gb.gemm_epi_plan(M, N, 64, "bf16", "bf16", "row", "col", "bias_silu")
    try:
        p, c = 0x10000, 0x100000
        nbytes = M * N * 2
        # no plan / missing bias / bias without a bias epilogue
        assert gb.gemm_epi_run_ex(None, p, p, p, 0, 0, c, None, 0, None) == 1
        assert gb.gemm_epi_run_ex(h, p, p, None, 0, 0, c, None, 0, None) == 1
        # a residual overlapping C (same start, inside, straddling the end)
        for r in (c, c + 64, c + nbytes - 2, c - nbytes + 2):
            assert gb.gemm_epi_run_ex(h, p, p, p, None, r, c, None, 0, None) == 1, hex(r)
    finally:
        gb.gemm_epi_destroy(h)
    h = gb.gemm_epi_plan(M, N, 64, "f16", "f32", "row", "row", "silu")
    try:
        c = 0x100000
        # fp32 output: the residual spans 4 bytes per element
        assert gb.gemm_epi_run_ex(h, 0x1000, 0x1000, None, None, c + M * N * 4 - 4, c, None, 0, None) == 1
        assert gb.gemm_epi_run_ex(h, 0x1000, 0x1000, 0x1000, None, None, c, None, 0, None) == 1  # bias given
    finally:
        gb.gemm_epi_destroy(h)
    h = gb.gemm_epi_plan(M, N, 64, "bf16", "fp8", "row", "col", "none")
    try:
        # no residual for a quantised output, wherever it lies
        assert gb.gemm_epi_run_ex(h, 0x1000, 0x1000, None, None, 0x900000, 0x100000, None, 0, None) == 1
    finally:
        gb.gemm_epi_destroy(h)


def test_fp8_output_off_16_columns_takes_the_masked_ring(lib):
    # FP8 rows of C in 16-byte chunks: with N % 16 != 0 the ring kernel
    # masks its last tile column (both take the ring here: 16 x 9 tiles
    # of 64)
    for N, want in ((528, "tile_64x64_ring4"), (520, "tile_64x64_ring4")):
        h = gb.gemm_epi_plan(1024, N, 256, "bf16", "fp8", "row", "col", "none")
        try:
            assert gb.gemm_epi_plan_describe(h)[2] == want, N
        finally:
            gb.gemm_epi_destroy(h)


@pytest.mark.parametrize("M,N,K,la,lb,want_kernel,want_name", [
    (8192, 8192, 8192, "row", "col", "tile", "tile_256x256x64_m16"),
    (4096, 4096, 4096, "row", "row", "tile", "tile_256x256x64_m16_rowb"),  # B through transposing LDS reads
    (8192, 8192, 8192, "row", "row", "tile", "tile_256x256x64_m16_rowb"),
    (4096, 4096, 4096, "col", "row", "tile", "tile_256x256x64"),  # column-major A: register-staged
    (4096, 4096, 4096, "row", "col", "tile", "tile_256x256x64_m16"),
    (1024, 1024, 1024, "row", "row", "tile", "tile_64x64_ring4"),  # 16 chunks of 64 through 4 slots
    (128, 64, 256, "row", "col", "tile", "tile_64x64_ring4"),  # 4 chunks of 64
    (32, 8192, 8192, "row", "col", "skinny", "skinny_32n_8w_5x256k"),
    (1, 4096, 4096, "row", "col", "skinny", "skinny_32n_8w_5x256k"),
    (32, 4096, 768, "row", "col", "skinny", "skinny_32n_4w_2x256k"),  # three chunks of 256
    (32, 4096, 192, "row", "col", "skinny", "skinny_32n_2w_2x128k"),  # two chunks of 128, the first padded
    (32, 4096, 128, "row", "col", "tile", "tile_64x64_ring2"),  # K too short for a skinny ring: one masked tile row
    (32, 8192, 8200, "row", "col", "skinny", "skinny_32n_8w_5x256k"),  # 33 chunks of 256, the first padded
    (32, 8192, 8320, "row", "col", "skinny", "skinny_32n_4w_8x128k"),  # whole chunks of 128 come first
    (32, 8192, 8196, "row", "col", "generic", "generic"),  # K not a multiple of 8
    (32, 50257, 4096, "row", "col", "skinny", "skinny_32n_8w_5x256k"),  # N % 8 != 0: last workgroup masked
    (8, 13, 256, "row", "col", "skinny", "skinny_32n_2w_2x128k"),  # N below the workgroup's 32 columns
    (32, 50257, 4096, "row", "row", "generic", "generic"),  # packed row-major B: ldb = 50257, unaligned rows
    (32, 8192, 8192, "row", "row", "skinny", "skinny_rowb_64n_8w_6x128k"),  # N-contiguous B: transposing LDS reads
    (32, 4096, 1152, "row", "row", "skinny", "skinny_rowb_64n_8w_6x128k"),  # nine chunks of 128
    (32, 40, 1152, "row", "row", "skinny", "skinny_rowb_32n_4w_8x128k"),  # N < 64: 32-column workgroups
    (32, 4096, 200, "row", "row", "skinny", "skinny_rowb_32n_2w_2x128k"),  # two chunks of 128, the first padded
    (32, 8192, 8192, "col", "row", "tile", "tile_64x64_ring4"),  # column-major A: no decode-shape kernel; ring
    (2000, 8200, 4096, "row", "col", "tile", "tile_256x256x64_m16"),  # last tile row and column shifted back
    (1000, 1000, 1024, "row", "col", "tile", "tile_64x64_ring4"),  # 16 x 16 edge-tiled 64 x 64 tiles
    (3000, 2000, 4096, "row", "row", "tile", "tile_128x128x64"),  # 24 x 16 tiles of 128
    (1000, 1000, 1024, "col", "col", "tile", "tile_64x64_ring4"),  # column-major A through transposing reads
    (1001, 1000, 1024, "col", "col", "generic", "generic"),  # packed column-major A: lda = 1001, unaligned
    (1000, 1004, 1024, "row", "col", "tile", "tile_64x64_ring4"),  # N % 8 != 0: last tile column masked
    (4096, 50257, 4096, "row", "col", "tile", "tile_256x256x64_m16"),  # odd N, packed C: masked 256-wide tiles
    (4096, 50257, 4096, "row", "row", "generic", "generic"),  # packed row-major B of odd width: unaligned
    (37, 53, 29, "row", "row", "generic", "generic"),
    (256, 256, 100, "col", "row", "generic", "generic"),  # K not a multiple of 8
    (1024, 1024, 1000, "row", "col", "tile", "tile_64x64_ring4"),  # K % 64 = 40: a partial first chunk
    (1024, 1024, 1536, "row", "row", "tile", "tile_64x64_ring4"),  # 24 chunks: 4 divides (as does 8)
    (1024, 1024, 1152, "row", "row", "tile", "tile_64x64_ring2"),  # 18 chunks
    (1024, 1024, 320, "row", "row", "tile", "tile_64x64_ring2"),  # 5 chunks: two slots take an odd count
    (1024, 1024, 384, "row", "col", "tile", "tile_64x64_ring2"),  # 6 chunks
    (4096, 4096, 4040, "row", "col", "tile", "tile_256x256x64_m16"),
    (256, 256, 72, "col", "row", "tile", "tile_64x64_ring2"),  # two chunks
    (256, 256, 64, "row", "row", "tile", "tile_64x64_ring2"),  # one chunk
    (256, 256, 64, "col", "row", "tile", "tile_64x64_ring2"),  # one chunk
    (8, 8, 8, "col", "col", "tile", "tile_64x64_ring2"),
    (4096, 4096, 4096, "col", "col", "tile", "tile_256x256x64"),  # two-stage, register-staged A
    (48, 40, 64, "row", "row", "tile", "tile_64x64_ring2"),  # M and N below the tile: masked
    (63, 1000, 320, "row", "col", "tile", "tile_64x64_ring2"),
    (1, 8, 8, "row", "row", "tile", "tile_64x64_ring2"),
    (40, 4096, 4096, "row", "col", "tile", "tile_64x64_ring4"),  # M just past the skinny kernels
])
def test_auto_selection(lib, M, N, K, la, lb, want_kernel, want_name):
    h = gb.gemm_epi_plan(M, N, K, "bf16", "bf16", la, lb, "none")
    try:
        kern, cfg, name = gb.gemm_epi_plan_describe(h)
        assert (kern, name) == (want_kernel, want_name)
    finally:
        gb.gemm_epi_destroy(h)


def test_eight_slot_ring_refuses_ragged_columns(lib):
    # the masked ring instance exists for two and four slots only
    for N, ldc in ((77, 0), (256, 260)):
        h = gb.gemm_epi_plan(256, N, 512, "bf16", "bf16", "row", "col", "none")
        try:
            if ldc:
                assert gb.gemm_epi_plan_set_ld(h, 0, 0, ldc) == 0
            assert gb.gemm_epi_plan_select(h, "tile", 5) == 2
            assert gb.gemm_epi_plan_select(h, "tile", 6) == 0
            assert gb.gemm_epi_plan_select(h, "tile", 7) == 0
        finally:
            gb.gemm_epi_destroy(h)
    h = gb.gemm_epi_plan(256, 256, 512, "bf16", "bf16", "row", "col", "none")
    try:
        assert gb.gemm_epi_plan_select(h, "tile", 5) == 0
    finally:
        gb.gemm_epi_destroy(h)


def test_select_forces_and_validates(lib):
    h = gb.gemm_epi_plan(512, 512, 256, "f16", "f32", "row", "col", "none")
    try:
        assert gb.gemm_epi_num_configs("tile") == 9
        assert gb.gemm_epi_num_configs("skinny") == 10
        assert gb.gemm_epi_num_configs("generic") == 1
        assert gb.gemm_epi_num_configs("auto") == 0
        for cfg in range(4):
            assert gb.gemm_epi_plan_select(h, "tile", cfg) == 0
            assert gb.gemm_epi_plan_describe(h)[:2] == ("tile", cfg)
        assert gb.gemm_epi_plan_select(h, "tile", 4) == 0  # 16x16x32, k-contiguous operands
        assert gb.gemm_epi_plan_select(h, "generic", 0) == 0
        assert gb.gemm_epi_plan_describe(h)[0] == "generic"
        assert gb.gemm_epi_plan_select(h, "skinny", -1) == 2  # M = 512 > 32: unsupported, plan unchanged
        assert gb.gemm_epi_plan_describe(h)[0] == "generic"
        assert gb.gemm_epi_plan_select(h, "tile", 9) == 1  # no such config
        assert gb.gemm_epi_plan_select(h, "tile", 8) == 2  # 16x16x32 with row-major B only
        assert gb.gemm_epi_plan_select(h, "tile", 5) == 2  # ring of 8: 4 chunks are too few
        assert gb.gemm_epi_plan_select(h, "tile", 6) == 0  # ring of 4
        assert lib.gemm_epi_plan_select(ctypes.c_void_p(h), 9, 0) == 1  # bad enum
        assert gb.gemm_epi_plan_select(h, "auto", -1) == 0
        assert gb.gemm_epi_plan_describe(h) == ("tile", 6, "tile_64x64_ring4")  # 64 workgroups beats 16
    finally:
        gb.gemm_epi_destroy(h)
    h = gb.gemm_epi_plan(32, 128, 1024, "bf16", "bf16", "row", "col", "bias")
    try:
        assert gb.gemm_epi_plan_describe(h)[:2] == ("skinny", 1)  # first config that fits
        assert gb.gemm_epi_plan_select(h, "skinny", 0) == 2  # four chunks of 256 do not fill five slots
        assert gb.gemm_epi_plan_select(h, "skinny", 3) == 0
        assert gb.gemm_epi_plan_select(h, "tile", -1) == 0  # one masked 64 x 64 tile row
        assert gb.gemm_epi_plan_describe(h) == ("tile", 6, "tile_64x64_ring4")  # 16 chunks
        assert gb.gemm_epi_plan_select(h, "tile", 0) == 2  # M = 32 holds no 256 x 256 tile
    finally:
        gb.gemm_epi_destroy(h)
    h = gb.gemm_epi_plan(512, 512, 320, "bf16", "bf16", "row", "row", "bias")
    try:
        assert gb.gemm_epi_plan_select(h, "tile", 4) != 0  # k-contiguous operands only
    finally:
        gb.gemm_epi_destroy(h)


# (k per chunk, ring slots) of each skinny configuration, in order: K must
# be a multiple of 8 that makes at least one chunk per slot, the first chunk
# padded with zeros when K is not a whole number of chunks
# (configurations 0-5 take a column-major B, 6-9 a row-major one)
SKINNY_CHUNKS = [(256, 5), (256, 4), (256, 4), (128, 8), (256, 2), (128, 2), (256, 5), (128, 8), (128, 2), (128, 6)]


def test_skinny_k_granularity(lib):
    assert gb.gemm_epi_num_configs("skinny") == len(SKINNY_CHUNKS)
    for cfg, (kc, slots) in enumerate(SKINNY_CHUNKS):
        lb, other = ("col", "row") if cfg < 6 else ("row", "col")
        for K, ok in ((kc * slots, True), (kc * (slots + 1), True), (kc * (slots - 1), False),
                      (kc * slots + 64, True), (kc * (slots - 1) + 8, True), (kc * slots + 4, False)):
            for layout, want in ((lb, ok), (other, False)):
                h = gb.gemm_epi_plan(32, 64, K, "bf16", "bf16", "row", layout, "none")
                try:
                    assert (gb.gemm_epi_plan_select(h, "skinny", cfg) == 0) == want, (cfg, K, layout)
                finally:
                    gb.gemm_epi_destroy(h)


def test_workspace_size(lib):
    # skinny plans with fewer than 256 column blocks of 32 split K when given
    # a workspace: one 4 KiB fp32 partial per (block, split), then one
    # counter per block (rounded to 256 bytes)
    h = gb.gemm_epi_plan(32, 1024, 8192, "bf16", "bf16", "row", "col", "bias")
    try:
        assert gb.gemm_epi_plan_describe(h)[:2] == ("skinny", 0)
        assert gb.gemm_epi_workspace_size(h) == 32 * 4 * 4096 + 256  # 32 chunks of 256, 4 splits of 8
    finally:
        gb.gemm_epi_destroy(h)
    for args in ((32, 8192, 8192, "bf16", "bf16", "row", "col", "bias"),   # 256 blocks already
                 (8192, 8192, 8192, "bf16", "bf16", "row", "col", "bias_gelu"),
                 (37, 53, 29, "f16", "f16", "row", "row", "none")):
        h = gb.gemm_epi_plan(*args)
        try:
            assert gb.gemm_epi_workspace_size(h) == 0, args
        finally:
            gb.gemm_epi_destroy(h)
    assert lib.gemm_epi_workspace_size(None) == 0
    assert lib.gemm_epi_run_ws(None, None, None, None, None, None, 0, None) == 1  # INVALID_ARG


# --------------------------------------------------------------------------
# tuning table: file format, merge, and the plan's use of it (host only)
# --------------------------------------------------------------------------

def _describe(*args):
    h = gb.gemm_epi_plan(*args)
    try:
        return gb.gemm_epi_plan_describe(h)
    finally:
        gb.gemm_epi_destroy(h)


def test_tuning_table_drives_the_plan(lib, tmp_path):
    gb.gemm_epi_tuning_clear()
    args = (1024, 1024, 1024, "f16", "f16", "row", "row", "relu")
    assert _describe(*args)[:2] == ("tile", 6)  # static rule: 64 x 64 fills the CUs, 16 chunks ring through 4 slots
    f = tmp_path / "t.txt"
    f.write_text("# a comment\n\n1024 1024 1024 0 0 0 0 1 2 1 12.5  # tile config 1\n")
    assert gb.gemm_epi_tuning_load(f) == 0 and gb.gemm_epi_tuning_size() == 1
    assert _describe(*args)[:2] == ("tile", 1)
    assert _describe(1024, 1024, 1024, "f16", "f16", "row", "row", "none")[:2] == ("tile", 6)  # other epilogue
    # plan_select(AUTO) restores the tuned choice
    h = gb.gemm_epi_plan(*args)
    try:
        assert gb.gemm_epi_plan_select(h, "generic", 0) == 0
        assert gb.gemm_epi_plan_select(h, "auto", -1) == 0
        assert gb.gemm_epi_plan_describe(h)[:2] == ("tile", 1)
    finally:
        gb.gemm_epi_destroy(h)
    # save -> clear -> load round trip
    g = tmp_path / "saved.txt"
    assert gb.gemm_epi_tuning_save(g) == 0
    gb.gemm_epi_tuning_clear()
    assert gb.gemm_epi_tuning_size() == 0 and _describe(*args)[:2] == ("tile", 6)
    assert gb.gemm_epi_tuning_load(g) == 0 and _describe(*args)[:2] == ("tile", 1)
    lines = [l for l in g.read_text().splitlines() if l and not l.startswith("#")]
    assert lines == ["1024 1024 1024 0 0 0 0 1 2 1 12.500"]
    gb.gemm_epi_tuning_clear()


def test_tuning_entry_that_cannot_run_is_ignored(lib, tmp_path):
    gb.gemm_epi_tuning_clear()
    f = tmp_path / "t.txt"
    # skinny for M = 1024, and tile config 0 (256 x 256) for a 64 x 64 problem
    f.write_text("1024 1024 1024 0 0 0 1 0 3 0 1.0\n64 64 256 1 1 0 1 0 2 0 1.0\n")
    assert gb.gemm_epi_tuning_load(f) == 0 and gb.gemm_epi_tuning_size() == 2
    assert _describe(1024, 1024, 1024, "f16", "f16", "row", "col", "none")[0] == "tile"
    assert _describe(64, 64, 256, "bf16", "bf16", "row", "col", "none")[:2] == ("tile", 6)  # the static rule: ring of 4
    gb.gemm_epi_tuning_clear()


@pytest.mark.parametrize("text", [
    "1024 1024 1024 0 0 0 0 1 2 1\n",             # missing field
    "1024 1024 1024 0 0 0 0 1 2 1 3.0 7\n",       # extra field
    "1024 1024 0 0 0 0 0 1 2 1 3.0\n",            # K = 0
    "1024 1024 1024 0 5 0 0 1 2 1 3.0\n",         # bad format
    "1024 1024 1024 0 0 0 0 9 2 1 3.0\n",         # bad epilogue
    "1024 1024 1024 0 0 0 0 1 0 1 3.0\n",         # kernel AUTO is not a choice
    "1024 1024 1024 0 0 0 0 1 2 -1 3.0\n",        # negative config
    "garbage\n",
])
def test_tuning_load_rejects_malformed_files(lib, tmp_path, text):
    gb.gemm_epi_tuning_clear()
    ok = tmp_path / "ok.txt"
    ok.write_text("512 512 512 1 1 0 1 3 2 3 9.0\n")
    assert gb.gemm_epi_tuning_load(ok) == 0
    f = tmp_path / "bad.txt"
    f.write_text("256 256 256 0 0 0 0 0 2 2 1.0\n" + text)
    assert gb.gemm_epi_tuning_load(f) == 1
    assert gb.gemm_epi_tuning_size() == 1  # unchanged: nothing from the bad file
    assert gb.gemm_epi_tuning_load(tmp_path / "missing.txt") == 1
    assert gb.gemm_epi_tuning_load(None) == 1 and gb.gemm_epi_tuning_save(None) == 1
    gb.gemm_epi_tuning_clear()


def test_tune_rejects_invalid_arguments_without_touching_the_device(lib):
    h = gb.gemm_epi_plan(256, 256, 128, "bf16", "bf16", "row", "col", "bias")
    try:
        p = 0x10000
        assert gb.gemm_epi_tune(None, p, p, p, p, 5, None)[0] == 1
        assert gb.gemm_epi_tune(h, p, p, None, p, 5, None)[0] == 1  # bias missing
        assert gb.gemm_epi_tune(h, p, p, p, p, 0, None)[0] == 1  # iters
        assert gb.gemm_epi_tune(h, p + 2, p, p, p, 5, None)[0] == 1  # unaligned
        assert gb.gemm_epi_tune(h, p, p, p, p, 5, None, flags=2)[0] == 1  # unknown flag
    finally:
        gb.gemm_epi_destroy(h)
    assert gb.gemm_epi_tuning_size() == 0


def test_plan_set_ld_validates_and_reselects(lib):
    h = gb.gemm_epi_plan(512, 512, 256, "bf16", "bf16", "row", "col", "none")
    try:
        kern0 = gb.gemm_epi_plan_describe(h)
        assert gb.gemm_epi_plan_set_ld(None, 0, 0, 0) == 1
        assert gb.gemm_epi_plan_set_ld(h, 255, 0, 0) == 1  # A row-major: lda >= K
        assert gb.gemm_epi_plan_set_ld(h, 0, 255, 0) == 1  # B column-major: ldb >= K
        assert gb.gemm_epi_plan_set_ld(h, 0, 0, 511) == 1  # ldc >= N
        assert gb.gemm_epi_plan_describe(h) == kern0  # unchanged on error
        assert gb.gemm_epi_plan_set_ld(h, 264, 320, 520) == 0
        assert gb.gemm_epi_plan_describe(h)[0] == "tile"
        assert gb.gemm_epi_plan_set_ld(h, 260, 0, 0) == 0  # rows no longer 16-byte aligned
        assert gb.gemm_epi_plan_describe(h)[0] == "generic"
        assert gb.gemm_epi_plan_set_ld(h, 0, 0, 0) == 0  # packed again
        assert gb.gemm_epi_plan_describe(h) == kern0
        assert gb.gemm_epi_plan_set_ld(h, 1 << 31, 0, 0) == 2
        assert gb.gemm_epi_plan_set_ld(h, 1 << 24, 0, 0) == 2  # 511 rows of 2^24: past 2^31 elements
    finally:
        gb.gemm_epi_destroy(h)
    h = gb.gemm_epi_plan(32, 1024, 4096, "bf16", "bf16", "row", "col", "bias")
    try:
        assert gb.gemm_epi_plan_describe(h)[0] == "skinny"
        assert gb.gemm_epi_plan_set_ld(h, 4096 + 64, 4096 + 8, 2048) == 0
        assert gb.gemm_epi_plan_describe(h)[0] == "skinny"
        assert gb.gemm_epi_plan_set_ld(h, 0, 4100, 0) == 0
        assert gb.gemm_epi_plan_describe(h)[0] == "generic"
    finally:
        gb.gemm_epi_destroy(h)
    # column-major A: lda >= M
    h = gb.gemm_epi_plan(256, 256, 128, "f16", "f16", "col", "row", "none")
    try:
        assert gb.gemm_epi_plan_set_ld(h, 255, 0, 0) == 1
        assert gb.gemm_epi_plan_set_ld(h, 264, 264, 0) == 0
        assert gb.gemm_epi_plan_describe(h)[0] == "tile"
    finally:
        gb.gemm_epi_destroy(h)


def test_attention_validates_without_touching_the_device(lib):
    p = 0x10000
    assert gb.gemm_epi_attention_fwd(None, p, p, p, 1, 128, 1, 64, "f16", 0, None) == 1
    assert gb.gemm_epi_attention_fwd(p, p, p, p, 0, 128, 1, 64, "f16", 0, None) == 1
    assert gb.gemm_epi_attention_fwd(p, p, p, p, 1, 128, 1, 64, "fp8", 0, None) == 1
    assert gb.gemm_epi_attention_fwd(p, p, p, p, 1, 128, 1, 128, "bf16", 1, None) == 2  # D = 128
    # more than 65535 query blocks of 128 (any S is taken: the last block masked)
    assert gb.gemm_epi_attention_fwd(p, p, p, p, 1, 128 * 65535 + 1, 1, 64, "bf16", 1, None) == 2
    assert gb.gemm_epi_attention_fwd(p + 8, p, p, p, 1, 128, 1, 64, "bf16", 1, None) == 2  # alignment
    assert gb.gemm_epi_attention_fwd(p, p, p, p, 1 << 12, 1 << 12, 1 << 4, 64, "bf16", 0, None) == 2  # 2^34 elements


def test_skinny_rowb_64_columns(lib):
    # configuration 9 gives a workgroup 64 columns of a row-major B: it needs
    # N >= 64, and its split-K partial blocks are 32 x 64 fp32 (8 KiB)
    for N, ok in ((40, False), (64, True), (72, True)):
        h = gb.gemm_epi_plan(32, N, 1152, "bf16", "bf16", "row", "row", "none")
        try:
            assert (gb.gemm_epi_plan_select(h, "skinny", 9) == 0) == ok, N
        finally:
            gb.gemm_epi_destroy(h)
    h = gb.gemm_epi_plan(32, 1024, 7928, "bf16", "bf16", "row", "row", "bias")
    try:
        assert gb.gemm_epi_plan_describe(h)[:3] == ("skinny", 9, "skinny_rowb_64n_8w_6x128k")
        # 16 column blocks x 2 splits of 31 chunks of 128, then 16 counters (256 bytes)
        assert gb.gemm_epi_workspace_size(h) == 16 * 2 * 8192 + 256
    finally:
        gb.gemm_epi_destroy(h)
