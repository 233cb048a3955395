"""Build the gfx950 shared libraries with hipcc: ``libmoe.so`` (the layer,
from ``csrc/``) and ``libmoe_bench.so`` (attainable-rate probes for the
roofline, from ``csrc_bench/``).

Run as ``python -m mixture_experts_moe_amd.build`` or through
``__graft_entry__.build()``.  It always recompiles.
"""

from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmoe.so")
BENCH_LIB = os.path.join(PKG, "libmoe_bench.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    # Packed fp32 VALU ops (v_pk_add/mul/fma_f32) stay off: float code is
    # compiled to scalar-per-lane fp32 instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def sources(folder: str = "csrc"):
    return sorted(glob.glob(os.path.join(PKG, folder, "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature name; drop that note
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False, extra_flags=(), out: str = LIB, folder: str = "csrc") -> str:
    """Compile every <folder>/*.hip into one shared library at `out` (one
    hipcc process per source, in parallel, then one link).  `extra_flags`
    (e.g. -D tuning macros) are appended to every compile line."""
    srcs = sources(folder)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, folder)]
    compile_flags = [f for f in FLAGS if f != "-shared"]
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with tempfile.TemporaryDirectory(prefix="moe_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in srcs]
        cmds = [[HIPCC, *compile_flags, *extra_flags, *inc, "-c", src, "-o", obj]
                for src, obj in zip(srcs, objs)]
        with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = out + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


def build_bench(verbose: bool = False) -> str:
    """The attainable-rate probe library (include/moe_bench.h)."""
    return build(verbose=verbose, out=BENCH_LIB, folder="csrc_bench")


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_bench(verbose=True))
