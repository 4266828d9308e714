"""Benchmark: GEMM+epilogue TFLOP/s (% of dense MFMA peak) and skinny-M GB/s
(% of HBM peak) on one MI355X.

One step = one launch of the library on one batch of synthetic input:
  * main line: C = GELU_tanh(A.B + bias), bf16 in/out, fp32 accumulate,
    M = N = K = 8192, A row-major, B column-major (value = TFLOP/s, 2MNK
    per step);
  * "skinny": C = A.B + bias, bf16, M = 32, N = K = 8192, B column-major
    (GB/s of compulsory A + B + bias + C bytes per step);
  * "epilogue_variants" (the further epilogues on the main shape) and
    "attention" (attention forward, B, H, S, D = 4, 8, 1024, 64, fp16, full
    and causal): reported beside the headline.
Inputs are resident in HBM before timing starts; operand sets are rotated
across launches so that the 256 MB last-level cache cannot serve B from a
previous launch.  Timing uses HIP events on the stream the kernels are
launched on.  The CPU oracle is timed on a bounded sample of the main
workload as a reported baseline (rank 0, N = 1 only).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only main|skinny]
                       [--no-cpu-baseline] [--no-variants] [--calib-copy]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MAIN = "gemm_bias_gelu_bf16_8192x8192x8192_rm_cm"
SKINNY = "skinny_gemm_bias_bf16_32x8192x8192_rm_cm"

# MI355X published peaks
PEAK_BF16_TFLOPS = 2500.0  # dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0

CSRC = os.path.join(ROOT, "epilogue_gemm_amd", "csrc")
# sources that define each kernel family's device code and launch shape
_FAMILY_SOURCES = {
    "tile": ["common.hpp", "kernels.hpp", "gemm_tile.hpp", "gemm_tile16.hpp", "tile_dispatch.hpp",
             "gemm_tile_bf16_bf16.hip", "gemm_tile_bf16_f32.hip", "gemm_tile_bf16_fp8.hip", "gemm_tile_f16_f16.hip",
             "gemm_tile_f16_f32.hip", "gemm_tile_f16_fp8.hip", "gemm_epi.cpp"],
    "skinny": ["common.hpp", "kernels.hpp", "gemm_skinny.hip", "gemm_epi.cpp"],
}


def _code_only(text: str) -> str:
    """C++ source with comments removed and whitespace collapsed."""
    import re

    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_sha(family: str) -> str:
    """sha256 over the code (comments and layout aside) of one kernel
    family's sources: detects a kernel changed since its HBM counters were
    taken."""
    import hashlib

    h = hashlib.sha256()
    for f in _FAMILY_SOURCES[family]:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(f.encode() + b"\0" + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(family: str, kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary of this kernel and workload (profiles/*.txt, copy-calibrated), or
    None when there is none or the kernel's sources changed since."""
    path = os.path.join(ROOT, "profiles", f"{kernel}__{workload}.txt")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        for line in fh:
            if line.startswith("machine-readable:"):
                kv = dict(t.split("=", 1) for t in line.split()[1:])
                if kv.get("src_sha256") == kernel_source_sha(family):
                    return int(float(kv["traffic_bytes"]))
    return None


def _device_sets(w, n_sets, torch, parity, inputs):
    """n_sets independent device copies of the workload's operands."""
    bits = inputs.workload_inputs(w)
    A0 = parity.to_device(bits["A"], w.in_dtype)
    B0 = parity.to_device(bits["B"], w.in_dtype)
    bias0 = parity.to_device(bits["bias"], w.in_dtype) if bits["bias"] is not None else None
    sets = []
    for i in range(n_sets):
        A = A0 if i == 0 else A0.clone()
        B = B0 if i == 0 else B0.clone()
        bias = None if bias0 is None else (bias0 if i == 0 else bias0.clone())
        C = parity.empty_out(w.M * w.N, w.out_dtype)
        sets.append((A, B, bias, C))
    torch.cuda.synchronize()
    return bits, sets


def _time_launches(plan, sets, steps, warmup, torch, extras=None):
    """ms per launch over `steps` launches rotating through `sets`; `extras`
    (optional) is a list, per set, of (column scale, residual) tensors."""
    stream = torch.cuda.current_stream()

    def launch(i):
        A, B, bias, C = sets[i % len(sets)]
        if extras is None:
            plan.run(A, B, bias, C, stream)
        else:
            sc, res = extras[i % len(sets)]
            plan.run(A, B, bias, C, stream, scale=sc, residual=res)

    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        launch(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps  # ms per launch


def _cpu_baseline(w, bits):
    """Oracle rate on a bounded sample of rows of the workload."""
    import numpy as np

    import oracle

    def run_rows(r):
        rows = np.repeat(np.arange(r), w.N)
        cols = np.tile(np.arange(w.N), r)
        t0 = time.perf_counter()
        oracle.gemm_epi_points(bits["A"], bits["B"], bits["bias"], w.M, w.N, w.K, w.in_dtype, w.out_dtype,
                               w.layout_a, w.layout_b, w.epilogue, rows, cols)
        return time.perf_counter() - t0

    t1 = run_rows(1)
    # a one-row run overstates the per-row time (fixed costs), so aim high
    rows = int(max(1, min(w.M, round(18.0 / max(t1, 1e-3)))))
    t = run_rows(rows)
    flops = 2.0 * rows * w.N * w.K
    return {
        "value": flops / t / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.max_threads(),
        "kind": "oracle",
        "sample": f"{rows} full output rows of {w.name} ({rows}x{w.N} outputs, K={w.K}), fp64, {t:.1f} s",
        "seconds": t,
    }


def _run_variants(w, sets, args, variants, binding, inputs, parity, torch):
    """The further epilogues on the main shape and operands (reported beside
    the headline, not in it): bias+SiLU; bias+GELU with a column scale and a
    residual (one residual per operand set, none overlapping C); bias+GELU to
    FP8 E4M3 with an output scale."""
    ex = inputs.extras_inputs(w.M, w.N, w.out_dtype, seed=w.seed)
    scale = torch.from_numpy(ex["scale"]).cuda()
    res0 = parity.to_device_out(ex["residual"], w.out_dtype)
    extras = [(scale, res0 if i == 0 else res0.clone()) for i in range(len(sets))]
    vsteps = min(args.steps, 50)
    warm = max(args.warmup // 2, 5)
    for epi, with_extras in (("bias_silu", False), ("bias_gelu", True)):
        p = binding.Plan(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.layout_a, w.layout_b, epi)
        vms = _time_launches(p, sets, vsteps, warm, torch, extras if with_extras else None)
        variants.append({"epilogue": epi, "out_dtype": w.out_dtype, "col_scale": with_extras,
                         "residual": with_extras, "out_scale": False, "kernel": p.name,
                         "ms_per_step": round(vms, 4), "TFLOP/s": round(w.flops / (vms * 1e-3) / 1e12, 1),
                         "steps": vsteps})
        p.close()
    del extras, res0
    sets8 = [(A, B, bias, parity.empty_out(w.M * w.N, "fp8")) for A, B, bias, _ in sets]
    q = torch.tensor([ex["out_scale"]], dtype=torch.float32, device="cuda")
    p = binding.Plan(w.M, w.N, w.K, w.in_dtype, "fp8", w.layout_a, w.layout_b, "bias_gelu")

    class _WithOutScale:  # runs the plan with the output scale
        def run(self, A, B, bias, C, stream):
            p.run(A, B, bias, C, stream, out_scale=q)

    vms = _time_launches(_WithOutScale(), sets8, vsteps, warm, torch)
    variants.append({"epilogue": "bias_gelu", "out_dtype": "fp8", "col_scale": False, "residual": False,
                     "out_scale": True, "kernel": p.name, "ms_per_step": round(vms, 4),
                     "TFLOP/s": round(w.flops / (vms * 1e-3) / 1e12, 1), "steps": vsteps})
    p.close()


def _bench_attention(steps, warmup, torch, binding, inputs, parity):
    """The attention forward workloads (B, H, S, D = 4, 8, 1024, 64, fp16, full
    and causal): TFLOP/s of 4 B H S^2 D (half when causal) per launch."""
    recs = []
    for w in inputs.ATTENTION_WORKLOADS.values():
        d = inputs.attention_inputs(w.B, w.S, w.H, w.D, w.dtype, w.seed)
        q, k, v = (parity.to_device(d[n], w.dtype).view(w.B, w.S, w.H, w.D) for n in ("Q", "K", "V"))
        o = torch.empty_like(q)
        stream = torch.cuda.current_stream()
        for _ in range(warmup):
            binding.attention_fwd(q, k, v, o, causal=w.causal, stream=stream)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(steps):
            binding.attention_fwd(q, k, v, o, causal=w.causal, stream=stream)
        end.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / steps
        tf = w.flops / (ms * 1e-3) / 1e12
        recs.append({"workload": w.name, "B": w.B, "S": w.S, "H": w.H, "D": w.D, "causal": w.causal,
                     "ms_per_step": round(ms, 5), "TFLOP/s": round(tf, 1), "steps": steps,
                     "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS,
                                  "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None}})
        del q, k, v, o
    return recs


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only", choices=["main", "skinny", "both", "attention"], default="both")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the further-epilogue variants (so that a profile sees the headline kernel only)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after timing, run a plain 1 GiB device copy (elementwise kernel) three times, so that "
                         "HBM byte counters can be scaled against a kernel of known traffic")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU only: the hot path is a single-GPU kernel "
              "(--gpus must be 1)", file=sys.stderr)
        return 2

    import torch

    from epilogue_gemm_amd import binding, inputs
    from tests import parity

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    binding.load_library()
    torch.cuda.set_device(0)

    out = {}
    if args.only in ("main", "both"):
        w = inputs.WORKLOADS[MAIN]
        bits, sets = _device_sets(w, 3, torch, parity, inputs)
        plan = binding.Plan(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.layout_a, w.layout_b, w.epilogue)
        ms = _time_launches(plan, sets, args.steps, args.warmup, torch)
        tflops = w.flops / (ms * 1e-3) / 1e12
        out["main"] = dict(w=w, bits=bits, ms=ms, value=tflops, kernel=plan.name)
        plan.close()
        # the further epilogues on the same shape and operands (_run_variants)
        variants = []
        if args.no_variants:
            del sets
            torch.cuda.empty_cache()
            out["main"]["variants"] = variants
        else:
            _run_variants(w, sets, args, variants, binding, inputs, parity, torch)
            out["main"]["variants"] = variants
            del sets
            torch.cuda.empty_cache()
    if args.only in ("skinny", "both"):
        w = inputs.WORKLOADS[SKINNY]
        # 5 sets x 128 MiB of B: more than the 256 MB last-level cache
        bits_s, sets = _device_sets(w, 5, torch, parity, inputs)
        plan = binding.Plan(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.layout_a, w.layout_b, w.epilogue)
        steps = max(args.steps, 200)
        ms = _time_launches(plan, sets, steps, max(args.warmup, 20), torch)
        gbs = w.compulsory_bytes() / (ms * 1e-3) / 1e9
        out["skinny"] = dict(w=w, ms=ms, value=gbs, kernel=plan.name, steps=steps)
        plan.close()
        del sets
        torch.cuda.empty_cache()

    attention = None
    if args.only in ("both", "attention") and not args.no_variants:
        attention = _bench_attention(max(args.steps, 50), max(args.warmup, 10), torch, binding, inputs, parity)

    if args.calib_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)  # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst

    rec = {}
    if "main" in out:
        m = out["main"]
        w = m["w"]
        rec = {
            "metric": "GEMM+epilogue TFLOP/s (% MFMA peak); skinny-M GB/s (% HBM peak), 1 GPU",
            "value": round(m["value"], 2),
            "unit": "TFLOP/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(m["ms"], 4),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "epilogue": w.epilogue,
                       "layout_a": w.layout_a, "layout_b": w.layout_b, "kernel": m["kernel"],
                       "operand_sets_rotated": 3},
            "roofline": {"bound": "mfma", "achieved": round(m["value"], 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(m["value"] / PEAK_BF16_TFLOPS, 4),
                         "traffic": measured_traffic("tile", m["kernel"], w.name)},
            "epilogue_variants": m.get("variants", []),
        }
    if "skinny" in out:
        s = out["skinny"]
        w = s["w"]
        sk = {
            "metric": "skinny-M GB/s (% HBM peak)",
            "value": round(s["value"], 1),
            "unit": "GB/s",
            "ms_per_step": round(s["ms"], 5),
            "steps": s["steps"],
            "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "epilogue": w.epilogue,
                       "kernel": s["kernel"], "operand_sets_rotated": 5,
                       "compulsory_bytes": w.compulsory_bytes()},
            "roofline": {"bound": "hbm", "achieved": round(s["value"], 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(s["value"] / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic("skinny", s["kernel"], w.name)},
        }
        if rec:
            rec["skinny"] = sk
        else:
            rec = {**sk, "n_gpus": 1, "warmup": args.warmup, "higher_is_better": True, "scaling": "weak",
                   "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}
    if attention is not None:
        if rec:
            rec["attention"] = attention
        else:
            rec = {"metric": "attention forward TFLOP/s", "attention": attention, "n_gpus": 1}
    if "main" in out and not args.no_cpu_baseline:
        rec["cpu_baseline"] = _cpu_baseline(out["main"]["w"], out["main"]["bits"])
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
