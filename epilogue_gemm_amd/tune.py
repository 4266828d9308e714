"""Search the fastest kernel configuration for problems on this GPU and save
the tuning table (gemm_epi_tune, gemm_epi_tuning_save).

    python -m epilogue_gemm_amd.tune [--out FILE] [--iters N] [--warm] [--shape M,N,K,in,out,la,lb,epi ...]

Without --shape it tunes the five reference workloads.  Launches are timed
with cold caches (a 512 MiB read before each) unless --warm is given.  Each problem runs on
seeded synthetic operands (epilogue_gemm_amd.inputs); the table file can then
be loaded by any process with gemm_epi_tuning_load before planning.
"""
from __future__ import annotations

import argparse
import json
import sys


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default="gemm_epi_tuning.txt")
    ap.add_argument("--iters", type=int, default=10)
    ap.add_argument("--warm", action="store_true", help="time back-to-back launches (operands may stay cached)")
    ap.add_argument("--shape", action="append", default=[],
                    help="M,N,K,in_dtype,out_dtype,layout_a,layout_b,epilogue (repeatable)")
    args = ap.parse_args(argv)

    import torch

    from epilogue_gemm_amd import binding as gb
    from epilogue_gemm_amd import inputs

    if not torch.cuda.is_available():
        print("tuning needs a GPU", file=sys.stderr)
        return 2
    gb.load_library()
    problems = []
    for s in args.shape:
        f = s.split(",")
        problems.append((int(f[0]), int(f[1]), int(f[2]), *f[3:8]))
    if not problems:
        problems = [(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.layout_a, w.layout_b, w.epilogue)
                    for w in inputs.WORKLOAD_LIST]
    dt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32, "fp8": torch.float8_e4m3fn}
    for (M, N, K, ind, outd, la, lb, epi) in problems:
        bits = inputs.make_inputs(M, N, K, ind, la, lb, epi.startswith("bias"), float(K) ** 0.5, 0.1, seed=0)

        def dev(b):
            return None if b is None else torch.from_numpy(b.view("int16").copy()).view(dt[ind]).cuda()

        A, B, bias = dev(bits["A"]), dev(bits["B"]), dev(bits["bias"])
        C = torch.empty(M * N, dtype=dt[outd], device="cuda")
        plan = gb.Plan(M, N, K, ind, outd, la, lb, epi)
        static = plan.name
        us = plan.tune(A, B, bias, C, iters=args.iters, cold=not args.warm)
        print(json.dumps({"problem": [M, N, K, ind, outd, la, lb, epi], "static": static, "tuned": plan.name,
                          "us": round(us, 2), "TFLOP/s": round(2.0 * M * N * K / us / 1e6, 1)}), flush=True)
        plan.close()
        del A, B, bias, C
        torch.cuda.empty_cache()
    st = gb.gemm_epi_tuning_save(args.out)
    if st != 0:
        print(f"could not write {args.out}", file=sys.stderr)
        return 1
    print(f"saved {gb.gemm_epi_tuning_size()} entries to {args.out}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
