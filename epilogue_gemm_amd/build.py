"""Build the HIP library libgemm_epi.so for gfx950, in-tree.

Every .hip/.cpp file under csrc/ is compiled by hipcc for gfx950 only, in
parallel, then linked into epilogue_gemm_amd/libgemm_epi.so.  build()
recompiles everything by default (it is the "does it build" check);
build(incremental=True) (``python -m epilogue_gemm_amd.build --incremental``)
recompiles only the sources whose object is older than the source or any
header it includes (from the compiler's dependency files).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgemm_epi.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Per-unit flags.  The row-major-B 16x16x32 tile kernel uses the generic
# machine scheduler: under the default AMDGPU scheduler its accumulators are
# copied between AGPRs and VGPRs around every MFMA (about 400 extra moves
# per two k-steps); the generic one keeps them in place.  Its other kernels
# are built as usual.
UNIT_FLAGS = {
    "gemm_tile16_rowb_f16.hip": ["-mllvm", "-misched=ilpmin"],
    "gemm_tile16_rowb_bf16.hip": ["-mllvm", "-misched=ilpmin"],
}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _obj(src: str) -> str:
    return os.path.join(BUILD, os.path.basename(src) + ".o")


def _up_to_date(src: str) -> bool:
    """The object exists and is newer than the source and every file its
    dependency file lists."""
    obj, dep = _obj(src), _obj(src) + ".d"
    if not (os.path.exists(obj) and os.path.exists(dep)):
        return False
    t = os.path.getmtime(obj)
    with open(dep) as fh:
        text = fh.read().replace("\\\n", " ")
    files = text.split(":", 1)[1].split() if ":" in text else []
    for f in [src, *files]:
        if not os.path.exists(f) or os.path.getmtime(f) > t:
            return False
    return True


def _compile(src: str) -> str:
    obj = _obj(src)
    extra = UNIT_FLAGS.get(os.path.basename(src), [])
    cmd = [HIPCC, "-x", "hip", *FLAGS, *extra, "-MMD", "-MF", obj + ".d", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(jobs: int | None = None, verbose: bool = False, incremental: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    todo = [s for s in srcs if not (incremental and _up_to_date(s))]
    jobs = jobs or min(max(len(todo), 1), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        list(ex.map(_compile, todo))
    if verbose and incremental:
        print(f"compiled {len(todo)} of {len(srcs)} sources: {[os.path.basename(s) for s in todo]}")
    objs = [_obj(s) for s in srcs]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build(verbose=True, incremental="--incremental" in sys.argv[1:])
    sys.exit(0)
