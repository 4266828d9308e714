"""Python binding of libgemm_epi.so (include/gemm_epi.h) -- argument
marshalling only.

The functions below carry the C names and call straight into the library;
every step of the computation runs in its HIP kernels.  ``Plan`` is a thin
convenience over them that takes torch CUDA tensors (used only as device
memory) and torch's current stream.  There is no fallback: if the library
is missing, loading fails with an error that says how to build it.
"""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgemm_epi.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "gemm_epi.h")

# Enum values of include/gemm_epi.h
DTYPES = {"f16": 0, "bf16": 1, "f32": 2, "fp8": 3}
LAYOUTS = {"row": 0, "col": 1}
EPILOGUES = {"none": 0, "relu": 1, "bias_relu": 2, "bias_gelu": 3, "bias": 4, "silu": 5, "bias_silu": 6}
KERNELS = {"auto": 0, "generic": 1, "tile": 2, "skinny": 3}
KERNEL_NAMES = {v: k for k, v in KERNELS.items()}
STATUS = {0: "OK", 1: "ERR_INVALID_ARG", 2: "ERR_UNSUPPORTED", 3: "ERR_HIP", 4: "ERR_NO_MEMORY"}
OK = 0


class Extras(ctypes.Structure):
    """struct gemm_epi_extras: optional column scale, residual and output
    scale pointers."""
    _fields_ = [("col_scale", ctypes.c_void_p), ("residual", ctypes.c_void_p), ("out_scale", ctypes.c_void_p)]


class GemmEpiError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = f"{fn} returned {gemm_epi_status_string(status)}"
        if status == 3:
            msg += f" (hipError_t {gemm_epi_last_hip_error()})"
        super().__init__(msg)


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libgemm_epi.so once.  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: the HIP library has not been built. "
            "Run `python -c 'import __graft_entry__ as g; g.build()'` or "
            "`python epilogue_gemm_amd/build.py` first.")
    lib = ctypes.CDLL(path)
    i64, i32, vp, cp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_char_p
    lib.gemm_epi_plan.argtypes = [ctypes.POINTER(vp), i64, i64, i64, i32, i32, i32, i32, i32]
    lib.gemm_epi_plan.restype = i32
    lib.gemm_epi_plan_set_ld.argtypes = [vp, i64, i64, i64]
    lib.gemm_epi_plan_set_ld.restype = i32
    lib.gemm_epi_run.argtypes = [vp, vp, vp, vp, vp, vp]
    lib.gemm_epi_run.restype = i32
    lib.gemm_epi_workspace_size.argtypes = [vp]
    lib.gemm_epi_workspace_size.restype = ctypes.c_size_t
    lib.gemm_epi_run_ws.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.gemm_epi_run_ws.restype = i32
    lib.gemm_epi_run_noalloc.argtypes = [vp, vp, vp, vp, vp, vp]
    lib.gemm_epi_run_noalloc.restype = i32
    lib.gemm_epi_run_ex.argtypes = [vp, vp, vp, vp, ctypes.POINTER(Extras), vp, vp, ctypes.c_size_t, vp]
    lib.gemm_epi_run_ex.restype = i32
    lib.gemm_epi_tune.argtypes = [vp, vp, vp, vp, vp, i32, i32, vp, ctypes.POINTER(ctypes.c_float)]
    lib.gemm_epi_tune.restype = i32
    lib.gemm_epi_tuning_save.argtypes = [cp]
    lib.gemm_epi_tuning_save.restype = i32
    lib.gemm_epi_tuning_load.argtypes = [cp]
    lib.gemm_epi_tuning_load.restype = i32
    lib.gemm_epi_tuning_clear.argtypes = []
    lib.gemm_epi_tuning_clear.restype = None
    lib.gemm_epi_tuning_size.argtypes = []
    lib.gemm_epi_tuning_size.restype = i32
    lib.gemm_epi_attention_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, vp]
    lib.gemm_epi_attention_fwd.restype = i32
    lib.gemm_epi_destroy.argtypes = [vp]
    lib.gemm_epi_destroy.restype = i32
    lib.gemm_epi_status_string.argtypes = [i32]
    lib.gemm_epi_status_string.restype = cp
    lib.gemm_epi_last_hip_error.argtypes = []
    lib.gemm_epi_last_hip_error.restype = i32
    lib.gemm_epi_plan_select.argtypes = [vp, i32, i32]
    lib.gemm_epi_plan_select.restype = i32
    lib.gemm_epi_num_configs.argtypes = [i32]
    lib.gemm_epi_num_configs.restype = i32
    lib.gemm_epi_plan_describe.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.gemm_epi_plan_describe.restype = cp
    # measurement helpers (include/gemm_epi_probes.h)
    lib.gemm_epi_probe_hbm_read.argtypes = [vp, ctypes.c_size_t, vp, vp]
    lib.gemm_epi_probe_hbm_read.restype = i32
    lib.gemm_epi_probe_mfma.argtypes = [i32, i32, vp, vp]
    lib.gemm_epi_probe_mfma.restype = i32
    lib.gemm_epi_probe_mfma_flops.argtypes = [i32, i32]
    lib.gemm_epi_probe_mfma_flops.restype = ctypes.c_double
    _lib = lib
    return lib


def headers():
    """Every header of the C ABI (include/*.h)."""
    d = os.path.dirname(HEADER)
    return sorted(os.path.join(d, f) for f in os.listdir(d) if f.endswith(".h"))


def header_functions(header: str | None = None):
    """Names of the functions the C ABI headers declare (all of include/*.h,
    or the one given)."""
    names = set()
    for h in [header] if header else headers():
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"\b(gemm_epi_\w+)\s*\(", text))
    return sorted(names)


# ---- the C entry points, same names ----------------------------------------

def gemm_epi_plan(M, N, K, in_dtype, out_dtype, layout_a, layout_b, epilogue) -> int:
    """Returns the plan handle (an int); raises GemmEpiError on failure."""
    h = ctypes.c_void_p()
    st = load_library().gemm_epi_plan(ctypes.byref(h), int(M), int(N), int(K), DTYPES[in_dtype], DTYPES[out_dtype],
                                      LAYOUTS[layout_a], LAYOUTS[layout_b], EPILOGUES[epilogue])
    if st != OK:
        raise GemmEpiError("gemm_epi_plan", st)
    return h.value


def gemm_epi_plan_status(M, N, K, in_dtype, out_dtype, layout_a, layout_b, epilogue, raw=False) -> int:
    """Status code of gemm_epi_plan for raw (possibly invalid) enum values;
    destroys the plan if one was made.  For tests of argument validation."""
    h = ctypes.c_void_p()
    lib = load_library()
    if raw:
        args = (in_dtype, out_dtype, layout_a, layout_b, epilogue)
    else:
        args = (DTYPES[in_dtype], DTYPES[out_dtype], LAYOUTS[layout_a], LAYOUTS[layout_b], EPILOGUES[epilogue])
    st = lib.gemm_epi_plan(ctypes.byref(h), int(M), int(N), int(K), *args)
    if st == OK:
        lib.gemm_epi_destroy(h)
    return st


def gemm_epi_plan_set_ld(plan, lda=0, ldb=0, ldc=0) -> int:
    return load_library().gemm_epi_plan_set_ld(plan, int(lda), int(ldb), int(ldc))


def gemm_epi_run(plan, A_ptr, B_ptr, bias_ptr, C_ptr, stream) -> int:
    return load_library().gemm_epi_run(plan, A_ptr, B_ptr, bias_ptr, C_ptr, stream)


def gemm_epi_run_noalloc(plan, A_ptr, B_ptr, bias_ptr, C_ptr, stream) -> int:
    return load_library().gemm_epi_run_noalloc(plan, A_ptr, B_ptr, bias_ptr, C_ptr, stream)


def gemm_epi_workspace_size(plan) -> int:
    return int(load_library().gemm_epi_workspace_size(plan))


def gemm_epi_run_ws(plan, A_ptr, B_ptr, bias_ptr, C_ptr, ws_ptr, ws_bytes, stream) -> int:
    return load_library().gemm_epi_run_ws(plan, A_ptr, B_ptr, bias_ptr, C_ptr, ws_ptr, int(ws_bytes), stream)


def gemm_epi_run_ex(plan, A_ptr, B_ptr, bias_ptr, scale_ptr, residual_ptr, C_ptr, ws_ptr, ws_bytes, stream,
                    extras_null=False, out_scale_ptr=None) -> int:
    """extras_null passes a NULL gemm_epi_extras pointer (the three extras
    pointers are then ignored)."""
    ex = None if extras_null else ctypes.byref(Extras(scale_ptr, residual_ptr, out_scale_ptr))
    return load_library().gemm_epi_run_ex(plan, A_ptr, B_ptr, bias_ptr, ex, C_ptr, ws_ptr, int(ws_bytes), stream)


TUNE_COLD = 1


def gemm_epi_tune(plan, A_ptr, B_ptr, bias_ptr, C_ptr, iters, stream, flags=0):
    """Returns (status, best microseconds per launch)."""
    us = ctypes.c_float(0.0)
    st = load_library().gemm_epi_tune(plan, A_ptr, B_ptr, bias_ptr, C_ptr, int(iters), int(flags), stream,
                                      ctypes.byref(us))
    return st, float(us.value)


def gemm_epi_tuning_save(path: str) -> int:
    return load_library().gemm_epi_tuning_save(None if path is None else str(path).encode())


def gemm_epi_tuning_load(path: str) -> int:
    return load_library().gemm_epi_tuning_load(None if path is None else str(path).encode())


def gemm_epi_tuning_clear() -> None:
    load_library().gemm_epi_tuning_clear()


def gemm_epi_tuning_size() -> int:
    return int(load_library().gemm_epi_tuning_size())


def gemm_epi_attention_fwd(Q_ptr, K_ptr, V_ptr, O_ptr, B, S, H, D, dtype, causal, stream) -> int:
    return load_library().gemm_epi_attention_fwd(Q_ptr, K_ptr, V_ptr, O_ptr, int(B), int(S), int(H), int(D),
                                                 DTYPES[dtype], int(bool(causal)), stream)


def attention_fwd(q, k, v, o, causal=False, stream=None):
    """Scaled dot-product attention on torch CUDA tensors [B, S, H, D]
    (contiguous, fp16 or bf16): fills `o`; enqueued on torch's current
    stream (or `stream`), not synchronised."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError(f"{name}: expected a contiguous 4-d CUDA tensor [B, S, H, D]")
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{name}: shape/dtype differ from q")
    B, S, H, D = q.shape
    if _dtype_name(q) not in ("f16", "bf16"):
        raise ValueError(f"q: dtype {q.dtype}; expected float16 or bfloat16")
    s = stream.cuda_stream if stream is not None else _current_stream_handle(torch)
    st = gemm_epi_attention_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, S, H, D,
                                _dtype_name(q), causal, s)
    if st != OK:
        raise GemmEpiError("gemm_epi_attention_fwd", st)


# ---- measurement helpers (include/gemm_epi_probes.h) -------------------------

def gemm_epi_probe_hbm_read(buf_ptr, nbytes, sink_ptr, stream) -> int:
    return load_library().gemm_epi_probe_hbm_read(buf_ptr, int(nbytes), sink_ptr, stream)


def gemm_epi_probe_mfma(iters, workgroups, out_ptr, stream) -> int:
    return load_library().gemm_epi_probe_mfma(int(iters), int(workgroups), out_ptr, stream)


def gemm_epi_probe_mfma_flops(iters, workgroups) -> float:
    return float(load_library().gemm_epi_probe_mfma_flops(int(iters), int(workgroups)))


def gemm_epi_destroy(plan) -> int:
    return load_library().gemm_epi_destroy(plan)


def gemm_epi_status_string(status: int) -> str:
    return load_library().gemm_epi_status_string(int(status)).decode()


def gemm_epi_last_hip_error() -> int:
    return int(load_library().gemm_epi_last_hip_error())


def gemm_epi_plan_select(plan, kernel: str, config: int = -1) -> int:
    return load_library().gemm_epi_plan_select(plan, KERNELS[kernel], int(config))


def gemm_epi_num_configs(kernel: str) -> int:
    return int(load_library().gemm_epi_num_configs(KERNELS[kernel]))


def gemm_epi_plan_describe(plan):
    """(kernel family name, config index, config name)."""
    k, c = ctypes.c_int(), ctypes.c_int()
    name = load_library().gemm_epi_plan_describe(plan, ctypes.byref(k), ctypes.byref(c))
    if name is None:
        raise ValueError("NULL plan")
    return KERNEL_NAMES[k.value], c.value, name.decode()


# ---- convenience over torch tensors (device memory + stream only) ----------

_TORCH_DTYPE_NAMES = {"float16": "f16", "bfloat16": "bf16", "float32": "f32", "float8_e4m3fn": "fp8"}
_NAME_OF_DTYPE = {}  # torch.dtype -> format name (None: not a format of the library), filled on use


def _dtype_name(t):
    d = t.dtype
    try:
        return _NAME_OF_DTYPE[d]
    except KeyError:
        n = _NAME_OF_DTYPE[d] = _TORCH_DTYPE_NAMES.get(str(d).replace("torch.", ""))
        return n


def _current_stream_handle(torch) -> int:
    """hipStream_t of torch's current stream on the current device (the raw
    handle without building a Stream object, where torch offers it)."""
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


class Plan:
    """A planned problem.  ``run(A, B, bias, C)`` enqueues on torch's current
    CUDA stream (or the given one) and returns without synchronising."""

    def __init__(self, M, N, K, in_dtype, out_dtype, layout_a="row", layout_b="row", epilogue="none",
                 kernel: str = "auto", config: int = -1, lda: int = 0, ldb: int = 0, ldc: int = 0):
        self.M, self.N, self.K = int(M), int(N), int(K)
        self.in_dtype, self.out_dtype = in_dtype, out_dtype
        self.layout_a, self.layout_b, self.epilogue = layout_a, layout_b, epilogue
        self.handle = gemm_epi_plan(M, N, K, in_dtype, out_dtype, layout_a, layout_b, epilogue)
        # stored extents (elements) of A, B and C: (rows - 1) * ld + row length
        a_rows, a_cols = (self.M, self.K) if layout_a == "row" else (self.K, self.M)
        b_rows, b_cols = (self.K, self.N) if layout_b == "row" else (self.N, self.K)
        self.lda, self.ldb, self.ldc = int(lda) or a_cols, int(ldb) or b_cols, int(ldc) or self.N
        self._extent = {"A": (a_rows - 1) * self.lda + a_cols, "B": (b_rows - 1) * self.ldb + b_cols,
                        "C": (self.M - 1) * self.ldc + self.N}
        if lda or ldb or ldc:
            st = gemm_epi_plan_set_ld(self.handle, lda, ldb, ldc)
            if st != OK:
                gemm_epi_destroy(self.handle)
                self.handle = None
                raise GemmEpiError("gemm_epi_plan_set_ld", st)
        if kernel != "auto":
            st = gemm_epi_plan_select(self.handle, kernel, config)
            if st != OK:
                gemm_epi_destroy(self.handle)
                self.handle = None
                raise GemmEpiError("gemm_epi_plan_select", st)
        self.kernel, self.config, self.name = gemm_epi_plan_describe(self.handle)
        self._run = load_library().gemm_epi_run

    def _check(self, t, name, dtype, numel):
        if t is None:
            return None
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name}: expected a contiguous CUDA tensor")
        if _dtype_name(t) != dtype:
            raise ValueError(f"{name}: dtype {t.dtype} does not match {dtype}")
        n = t.numel()
        if n < numel or (n != numel and name not in ("A", "B", "C", "residual")):
            raise ValueError(f"{name}: {n} elements, expected {numel}")
        return t.data_ptr()

    @property
    def workspace_size(self) -> int:
        """Bytes of workspace that let ``run`` split K (0: never splits)."""
        return gemm_epi_workspace_size(self.handle)

    def run(self, A, B, bias, C, stream=None, workspace=None, scale=None, residual=None, out_scale=None):
        """``workspace``: an optional zero-filled uint8 CUDA tensor of at least
        ``workspace_size`` bytes (left zero-filled by every completed run).
        ``scale``: optional fp32 per-column factors (N); ``residual``:
        optional M x N tensor of the output format, added after the
        activation (must not overlap C); ``out_scale``: optional one-element
        fp32 CUDA tensor multiplying the final value (the quantisation
        scale of an fp8 output)."""
        import torch

        a = self._check(A, "A", self.in_dtype, self._extent["A"])
        b = self._check(B, "B", self.in_dtype, self._extent["B"])
        bi = self._check(bias, "bias", self.in_dtype, self.N)
        c = self._check(C, "C", self.out_dtype, self._extent["C"])
        s = stream.cuda_stream if stream is not None else _current_stream_handle(torch)
        if scale is not None or residual is not None or out_scale is not None:
            sc = self._check(scale, "scale", "f32", self.N)
            r = self._check(residual, "residual", self.out_dtype, self._extent["C"])
            q = self._check(out_scale, "out_scale", "f32", 1)
            ws, nbytes = None, 0
            if workspace is not None:
                if not workspace.is_cuda or not workspace.is_contiguous():
                    raise ValueError("workspace: expected a contiguous CUDA tensor")
                ws, nbytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
            st = gemm_epi_run_ex(self.handle, a, b, bi, sc, r, c, ws, nbytes, s, out_scale_ptr=q)
            if st != OK:
                raise GemmEpiError("gemm_epi_run_ex", st)
            return
        if workspace is None:
            st = self._run(self.handle, a, b, bi, c, s)
            fn = "gemm_epi_run"
        else:
            if not workspace.is_cuda or not workspace.is_contiguous():
                raise ValueError("workspace: expected a contiguous CUDA tensor")
            nbytes = workspace.numel() * workspace.element_size()
            st = gemm_epi_run_ws(self.handle, a, b, bi, c, workspace.data_ptr(), nbytes, s)
            fn = "gemm_epi_run_ws"
        if st != OK:
            raise GemmEpiError(fn, st)

    def tune(self, A, B, bias, C, iters=10, stream=None, cold=False) -> float:
        """Measure every configuration that can run this problem on these
        buffers and keep the fastest (also recorded in the tuning table).
        ``cold``: evict the caches before every timed launch.  Returns the
        winner's mean microseconds per launch; synchronises the stream."""
        import torch

        a = self._check(A, "A", self.in_dtype, self._extent["A"])
        b = self._check(B, "B", self.in_dtype, self._extent["B"])
        bi = self._check(bias, "bias", self.in_dtype, self.N)
        c = self._check(C, "C", self.out_dtype, self._extent["C"])
        s = stream.cuda_stream if stream is not None else _current_stream_handle(torch)
        st, us = gemm_epi_tune(self.handle, a, b, bi, c, iters, s, TUNE_COLD if cold else 0)
        if st != OK:
            raise GemmEpiError("gemm_epi_tune", st)
        self.kernel, self.config, self.name = gemm_epi_plan_describe(self.handle)
        return us

    def close(self):
        if self.handle is not None:
            gemm_epi_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
