"""Build libiq.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(_HERE)
SOURCES = [os.path.join(_HERE, "csrc", "iq_kernels.hip"), os.path.join(_HERE, "csrc", "iq_api.cpp")]
OUT = os.path.join(_HERE, "libiq.so")
BENCH_SOURCES = [os.path.join(_HERE, "csrc", "bench_copy.hip")]
BENCH_OUT = os.path.join(_HERE, "libiq_bench.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no FMA contraction: x - s*q and the statistics must round as written
    "-ffp-contract=off",
    # no packed FP32 (v_pk_fma_f32 / v_pk_mul_f32 / v_pk_add_f32) in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def _hipcc(sources, out, verbose):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-o", out + ".tmp", *sources]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(out + ".tmp", out)
    return out


def build(verbose: bool = False) -> str:
    """Compile libiq.so (the library) and libiq_bench.so (the benchmark's
    reference copy kernel)."""
    _hipcc(BENCH_SOURCES, BENCH_OUT, verbose)
    return _hipcc(SOURCES, OUT, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
