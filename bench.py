"""Benchmark: GEMM+epilogue TFLOP/s (% of dense MFMA peak) and skinny-M GB/s
(% of HBM peak) on one MI355X.

One step = one launch of the library on one batch of synthetic input.  The
headline (`value`) is C = GELU_tanh(A.B + bias), bf16 in/out, fp32
accumulate, M = N = K = 8192, A row-major, B column-major, in TFLOP/s of
2MNK per step.  Beside it, under "workloads", every workload the library is
measured on, each through the automatic plan with its own roofline:
  * 128 x 64 x 256 fp16 -> fp32, A row-major, B column-major (one tile);
  * 1024^3 and 4096^3 fp16 ReLU, A and B row-major;
  * 8192^3 bf16 bias+GELU (the headline);
  * the decode shape C = A.B + bias, bf16, M = 32, N = K = 8192, B
    column-major (GB/s of compulsory A + B + bias + C bytes per step; also
    under "skinny").
"probes" holds the on-box ceilings (a streaming HBM read and back-to-back
bf16 MFMAs) that each roofline also reports a fraction of;
"epilogue_variants" the further epilogues on the headline shape and
"attention" the attention forward (B, H, S, D = 4, 8, 1024, 64, fp16, full
and causal).

Warm-up: the W warm-up launches, then untimed launches until 150 ms have run
on the GPU, so that the clock has settled under the power limit (it dips for
some tens of milliseconds after a burst starts).  The timed region is
exactly K launches.  Inputs are resident in HBM before timing starts; operand sets are rotated
across launches so that their total exceeds the 256 MB last-level cache
(3 sets for 8192^3, 5 for the decode shape, enough for 512 MiB for the
others).  Timing uses HIP events on the stream the library launches on: the
mean over one timed region of `steps` launches (`ms_per_step`, `value`), and
a second pass with an event pair around each launch for the median and
p10/p90 (`per_launch`).  The CPU oracle is timed on a bounded sample of the
main workload as a reported baseline (N = 1 only).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
                       [--only all|main|skinny|workloads|attention|probes]
                       [--no-cpu-baseline] [--no-variants] [--no-graph] [--calib-copy]
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
    "tile": ["common.hpp", "kernels.hpp", "gemm_tile.hpp", "gemm_tile16.hpp", "gemm_ring.hpp", "tile_dispatch.hpp",
             "gemm_tile_bf16_bf16.hip", "gemm_tile_bf16_f32.hip", "gemm_tile_bf16_fp8.hip", "gemm_tile_f16_f16.hip",
             "gemm_tile_f16_f32.hip", "gemm_tile_f16_fp8.hip", "gemm_tile16_rowb_f16.hip",
             "gemm_tile16_rowb_bf16.hip", "gemm_ring_bf16_bf16.hip", "gemm_ring_bf16_f32.hip",
             "gemm_ring_bf16_fp8.hip", "gemm_ring_f16_f16.hip", "gemm_ring_f16_f32.hip", "gemm_ring_f16_fp8.hip",
             "gemm_epi.cpp"],
    "skinny": ["common.hpp", "kernels.hpp", "gemm_skinny.hpp", "gemm_skinny.hip", "gemm_skinny_f16_f16.hip",
               "gemm_skinny_f16_f32.hip", "gemm_skinny_f16_fp8.hip", "gemm_skinny_bf16_bf16.hip",
               "gemm_skinny_bf16_f32.hip", "gemm_skinny_bf16_fp8.hip", "gemm_epi.cpp"],
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


def _n_sets(w, floor, cap=64):
    """Operand sets to rotate so that their total exceeds 2 x the 256 MB
    last-level cache (at least `floor`, at most `cap`)."""
    per_set = w.compulsory_bytes()
    return int(max(floor, min(cap, -(-(512 << 20) // per_set))))


def _percentiles(xs):
    import numpy as np

    a = np.asarray(xs, np.float64)
    return {"median_ms": round(float(np.median(a)), 6), "p10_ms": round(float(np.percentile(a, 10)), 6),
            "p90_ms": round(float(np.percentile(a, 90)), 6), "n": int(a.size)}


# Untimed launches continue after the W warm-up steps until at least this
# long has run on the GPU: under the power limit the clock dips after the
# first launches of a burst and takes some tens of milliseconds to settle
# (8192^3: 787, then 990 us at the fourth launch, back near 775 us after
# about 40), so a short warm-up would time the transient.
SETTLE_MS = 150.0


def _settle(launch, n_sets, start_index, torch):
    """Untimed launches until SETTLE_MS have elapsed on the GPU (in batches
    of 8, timed with events); returns the milliseconds spent."""
    stream = torch.cuda.current_stream()
    spent, i = 0.0, start_index
    while spent < SETTLE_MS:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(8):
            launch(i % n_sets)
            i += 1
        b.record(stream)
        torch.cuda.synchronize()
        spent += a.elapsed_time(b)
    return spent


def _time(launch, n_sets, steps, warmup, torch):
    """Times `launch(i)` (i rotating over n_sets operand sets) on torch's
    current stream, where the library enqueues.  Returns (mean ms per launch
    over one timed region of `steps` launches, per-launch statistics of a
    second pass timing each launch with its own event pair)."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        launch(i % n_sets)
    _settle(launch, n_sets, warmup, torch)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        launch(i % n_sets)
    end.record(stream)
    torch.cuda.synchronize()
    mean_ms = start.elapsed_time(end) / steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        launch(i % n_sets)
        b.record(stream)
    torch.cuda.synchronize()
    return mean_ms, _percentiles([a.elapsed_time(b) for a, b in ev])


def _time_graph(launch, n_sets, per_graph, replays, torch):
    """Per-launch time of `launch` with the host out of the way: `per_graph`
    launches (rotating over the operand sets) captured in one HIP graph and
    replayed `replays` times, each replay timed by an event pair on the
    replay stream.  Returns (mean ms per launch over all replays, statistics
    over replays of the mean ms per launch within a replay)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(max(n_sets, 3)):  # warm-up outside the capture
            launch(i % n_sets)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(per_graph):
            launch(i % n_sets)
    stream = torch.cuda.current_stream()
    g.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(replays)]
    for a, b in ev:
        a.record(stream)
        g.replay()
        b.record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) / per_graph for a, b in ev]
    del g
    return sum(per) / len(per), _percentiles(per)


def _plan_launcher(plan, sets, extras=None):
    def launch(i):
        A, B, bias, C = sets[i]
        if extras is None:
            plan.run(A, B, bias, C)
        else:
            sc, res = extras[i]
            plan.run(A, B, bias, C, scale=sc, residual=res)
    return launch


def _roofline(bound, achieved, peak, unit, traffic, probe_peak=None):
    r = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4), "traffic": traffic}
    if probe_peak:
        r["probe_peak"] = round(probe_peak, 1)
        r["frac_of_probe"] = round(achieved / probe_peak, 4)
    return r


def _bench_workload(w, steps, warmup, n_sets, torch, binding, inputs, parity, family, graph=True):
    """One workload through the automatic plan: mean and per-launch times, the
    roofline of its kernel (TFLOP/s of 2MNK, or GB/s of compulsory bytes for
    the HBM-bound decode shape)."""
    bits, sets = _device_sets(w, n_sets, torch, parity, inputs)
    plan = binding.Plan(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.layout_a, w.layout_b, w.epilogue)
    launch = _plan_launcher(plan, sets)
    mean_ms, per = _time(launch, n_sets, steps, warmup, torch)
    rec = {"workload": w.name, "kernel": plan.name, "ms_per_step": round(mean_ms, 6), "per_launch": per,
           "steps": steps, "operand_sets_rotated": n_sets,
           "TFLOP/s": round(w.flops / (mean_ms * 1e-3) / 1e12, 2),
           "GB/s": round(w.compulsory_bytes() / (mean_ms * 1e-3) / 1e9, 1),
           "compulsory_bytes": w.compulsory_bytes(), "flops": w.flops}
    if graph and mean_ms < 0.05:
        # launches this short are paced by the host's launch rate when
        # enqueued one by one from Python: time them replayed from a graph
        # as well, and check that a replay writes what an eager run writes
        ref = sets[0][3].clone()
        gmean, gper = _time_graph(launch, n_sets, max(n_sets, 100), 20, torch)
        same = bool(torch.equal(sets[0][3].view(torch.uint8), ref.view(torch.uint8)))
        rec["graph"] = {"ms_per_launch": round(gmean, 6), "per_replay": gper,
                        "TFLOP/s": round(w.flops / (gmean * 1e-3) / 1e12, 2),
                        "GB/s": round(w.compulsory_bytes() / (gmean * 1e-3) / 1e9, 1),
                        "launches_per_graph": max(n_sets, 100), "replay_equals_eager": same}
    plan.close()
    del sets
    torch.cuda.empty_cache()
    return rec, bits


def _probes(torch, binding):
    """On-box ceilings: streaming read of 5 rotated 128 MiB buffers (640 MiB,
    past the 256 MB last-level cache) and back-to-back bf16 MFMAs."""
    out = {}
    stream = torch.cuda.current_stream().cuda_stream
    nb = 128 << 20
    bufs = [torch.full((nb // 4,), i + 1, dtype=torch.int32, device="cuda") for i in range(5)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")

    def read(i):
        st = binding.gemm_epi_probe_hbm_read(bufs[i].data_ptr(), nb, sink.data_ptr(), stream)
        if st != 0:
            raise RuntimeError(f"gemm_epi_probe_hbm_read: status {st}")

    mean_ms, per = _time(read, len(bufs), 200, 20, torch)
    best = nb / (per["p10_ms"] * 1e-3) / 1e9
    out["hbm_read"] = {"GB/s": round(nb / (mean_ms * 1e-3) / 1e9, 1), "GB/s_p10_launch": round(best, 1),
                       "bytes_per_launch": nb, "buffers_rotated": len(bufs), "ms_per_launch": round(mean_ms, 6),
                       "per_launch": per}
    del bufs
    wg, iters = 1024, 8000
    res = torch.empty(wg * 256, dtype=torch.float32, device="cuda")

    def mfma(_):
        st = binding.gemm_epi_probe_mfma(iters, wg, res.data_ptr(), stream)
        if st != 0:
            raise RuntimeError(f"gemm_epi_probe_mfma: status {st}")

    mean_ms, per = _time(mfma, 1, 20, 5, torch)
    flops = binding.gemm_epi_probe_mfma_flops(iters, wg)
    out["mfma_bf16"] = {"TFLOP/s": round(flops / (mean_ms * 1e-3) / 1e12, 1), "flops_per_launch": flops,
                        "instruction": "v_mfma_f32_16x16x32_bf16", "ms_per_launch": round(mean_ms, 6),
                        "per_launch": per}
    del res
    torch.cuda.empty_cache()
    return out


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


def _run_variants(w, sets, args, binding, inputs, parity, torch):
    """The further epilogues on the main shape and operands (reported beside
    the headline, not in it): bias+SiLU; bias+GELU with a column scale and a
    residual (one residual per operand set, none overlapping C); bias+GELU to
    FP8 E4M3 with an output scale."""
    variants = []
    ex = inputs.extras_inputs(w.M, w.N, w.out_dtype, seed=w.seed)
    scale = torch.from_numpy(ex["scale"]).cuda()
    res0 = parity.to_device_out(ex["residual"], w.out_dtype)
    extras = [(scale, res0 if i == 0 else res0.clone()) for i in range(len(sets))]
    vsteps = min(args.steps, 50)
    warm = max(args.warmup // 2, 5)

    def rec(epi, out_dtype, with_extras, out_scale, kernel, ms, per):
        return {"epilogue": epi, "out_dtype": out_dtype, "col_scale": with_extras, "residual": with_extras,
                "out_scale": out_scale, "kernel": kernel, "ms_per_step": round(ms, 4), "per_launch": per,
                "TFLOP/s": round(w.flops / (ms * 1e-3) / 1e12, 1), "steps": vsteps}

    for epi, with_extras in (("bias_silu", False), ("bias_gelu", True)):
        p = binding.Plan(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.layout_a, w.layout_b, epi)
        ms, per = _time(_plan_launcher(p, sets, extras if with_extras else None), len(sets), vsteps, warm, torch)
        variants.append(rec(epi, w.out_dtype, with_extras, False, p.name, ms, per))
        p.close()
    del extras, res0
    sets8 = [(A, B, bias, parity.empty_out(w.M * w.N, "fp8")) for A, B, bias, _ in sets]
    q = torch.tensor([ex["out_scale"]], dtype=torch.float32, device="cuda")
    p = binding.Plan(w.M, w.N, w.K, w.in_dtype, "fp8", w.layout_a, w.layout_b, "bias_gelu")

    def launch8(i):
        A, B, bias, C = sets8[i]
        p.run(A, B, bias, C, out_scale=q)

    ms, per = _time(launch8, len(sets8), vsteps, warm, torch)
    variants.append(rec("bias_gelu", "fp8", False, True, p.name, ms, per))
    p.close()
    return variants


def _bench_attention(steps, warmup, torch, binding, inputs, parity, graph=True):
    """The attention forward workloads (B, H, S, D = 4, 8, 1024, 64, fp16, full
    and causal): TFLOP/s of 4 B H S^2 D (half when causal) per launch."""
    recs = []
    for w in inputs.ATTENTION_WORKLOADS.values():
        d = inputs.attention_inputs(w.B, w.S, w.H, w.D, w.dtype, w.seed)
        q, k, v = (parity.to_device(d[n], w.dtype).view(w.B, w.S, w.H, w.D) for n in ("Q", "K", "V"))
        o = torch.empty_like(q)

        def launch(_):
            binding.attention_fwd(q, k, v, o, causal=w.causal)

        ms, per = _time(launch, 1, steps, warmup, torch)
        tf = w.flops / (ms * 1e-3) / 1e12
        rec = {"workload": w.name, "B": w.B, "S": w.S, "H": w.H, "D": w.D, "causal": w.causal,
               "ms_per_step": round(ms, 5), "per_launch": per, "TFLOP/s": round(tf, 1), "steps": steps,
               "roofline": _roofline("mfma", tf, PEAK_BF16_TFLOPS, "TFLOP/s", None)}
        if graph:
            # about as long as the host needs to enqueue one launch from
            # Python: replayed from a graph as well (same output as eager)
            ref = o.clone()
            gmean, gper = _time_graph(launch, 1, 100, 20, torch)
            rec["graph"] = {"ms_per_launch": round(gmean, 6), "per_replay": gper,
                            "TFLOP/s": round(w.flops / (gmean * 1e-3) / 1e12, 1), "launches_per_graph": 100,
                            "replay_equals_eager": bool(torch.equal(o.view(torch.uint8), ref.view(torch.uint8)))}
        recs.append(rec)
        del q, k, v, o
    return recs


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only", choices=["all", "main", "skinny", "workloads", "attention", "probes"], default="all",
                    help="main: the 8192^3 headline only; skinny: the decode shape only; workloads: the three "
                         "other GEMM workloads; attention; probes: the on-box ceilings")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the further-epilogue variants and attention (so that a profile of --only main "
                         "sees the headline kernel only)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time short workloads eagerly only (no graph replays; for counter collection)")
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
    sel = args.only

    def say(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    probes = None
    if sel in ("all", "probes"):
        say("probes")
        probes = _probes(torch, binding)
    hbm_probe = probes["hbm_read"]["GB/s"] if probes else None
    mfma_probe = probes["mfma_bf16"]["TFLOP/s"] if probes else None

    workloads = {}
    main_bits, variants, attention = None, None, None
    if sel in ("all", "main"):
        w = inputs.WORKLOADS[MAIN]
        say(w.name)
        rec, main_bits = _bench_workload(w, args.steps, args.warmup, 3, torch, binding, inputs, parity, "tile",
                                         not args.no_graph)
        workloads[w.name] = rec
        if sel == "all" and not args.no_variants:
            say("epilogue variants")
            _, sets = _device_sets(w, 3, torch, parity, inputs)
            variants = _run_variants(w, sets, args, binding, inputs, parity, torch)
            del sets
            torch.cuda.empty_cache()
    if sel in ("all", "skinny"):
        w = inputs.WORKLOADS[SKINNY]
        say(w.name)
        # 5 sets x 128 MiB of B: more than the 256 MB last-level cache
        rec, _ = _bench_workload(w, max(args.steps, 200), max(args.warmup, 20), 5, torch, binding, inputs, parity,
                                 "skinny", not args.no_graph)
        workloads[w.name] = rec
    if sel in ("all", "workloads"):
        for name in inputs.WORKLOADS:
            if name in (MAIN, SKINNY):
                continue
            w = inputs.WORKLOADS[name]
            say(w.name)
            # operand sets past twice the last-level cache (the 128 x 64 x 256
            # case: 64 sets, still cache-resident; one tile, launch-bound)
            rec, _ = _bench_workload(w, max(args.steps, 100), max(args.warmup, 20), _n_sets(w, 3), torch, binding,
                                     inputs, parity, "tile", not args.no_graph)
            workloads[w.name] = rec
    if sel in ("all", "attention") and not args.no_variants:
        say("attention")
        attention = _bench_attention(max(args.steps, 50), max(args.warmup, 10), torch, binding, inputs, parity,
                                     not args.no_graph)

    if args.calib_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)  # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst

    # roofline of each workload's kernel
    for name, r in workloads.items():
        w = inputs.WORKLOADS[name]
        fam = "skinny" if name == SKINNY else "tile"
        traffic = measured_traffic(fam, r["kernel"], name)
        if name == SKINNY:
            r["roofline"] = _roofline("hbm", r["GB/s"], PEAK_HBM_GBS, "GB/s", traffic, hbm_probe)
        else:
            r["roofline"] = _roofline("mfma", r["TFLOP/s"], PEAK_BF16_TFLOPS, "TFLOP/s", traffic, mfma_probe)
        if name == "gemm_f16_f32out_128x64x256_rm_cm":
            r["limited_by"] = "launch latency: one 128 x 64 output block, 4.2 MFLOP"

    rec = {}
    if MAIN in workloads:
        m = workloads[MAIN]
        w = inputs.WORKLOADS[MAIN]
        rec = {
            "metric": "GEMM+epilogue TFLOP/s (% MFMA peak); skinny-M GB/s (% HBM peak), 1 GPU",
            "value": m["TFLOP/s"],
            "unit": "TFLOP/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "warmup_settle_ms": SETTLE_MS,
            "ms_per_step": round(m["ms_per_step"], 5),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "epilogue": w.epilogue,
                       "layout_a": w.layout_a, "layout_b": w.layout_b, "kernel": m["kernel"],
                       "operand_sets_rotated": m["operand_sets_rotated"]},
            "roofline": m["roofline"],
            "per_launch": m["per_launch"],
        }
    elif workloads:
        first = next(iter(workloads.values()))
        rec = {"metric": "GEMM+epilogue TFLOP/s (% MFMA peak); skinny-M GB/s (% HBM peak), 1 GPU",
               "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
               "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
               "config": {"workload": first["workload"]}}
    else:
        rec = {"metric": "on-box probes" if probes else "attention forward TFLOP/s", "n_gpus": 1}
    if workloads:
        rec["workloads"] = workloads
    if SKINNY in workloads:
        rec["skinny"] = workloads[SKINNY]
    if variants is not None:
        rec["epilogue_variants"] = variants
    if attention is not None:
        rec["attention"] = attention
    if probes is not None:
        rec["probes"] = probes
    if main_bits is not None and not args.no_cpu_baseline:
        say("cpu baseline (oracle)")
        rec["cpu_baseline"] = _cpu_baseline(inputs.WORKLOADS[MAIN], main_bits)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
