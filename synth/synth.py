"""Seeded synthetic inputs (ctypes front end of synth.c).

Holds the workload table: shapes, dtypes, value distributions and outlier
structure of the five quantization workloads, the activations that the
MXFP4 weights of c3 are multiplied with, and the 2 GiB streaming pass.
Nothing here performs any quantization arithmetic; GPU tests, the bench and
the CPU oracle all read the same bytes produced here.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

F32, BF16 = 0, 1
AXIS_NONE, AXIS_ROWS, AXIS_COLS = 0, 1, 2


def build() -> str:
    """Compile libsynth.so with gcc (always recompiles)."""
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
           "-o", _LIB + ".tmp", _SRC, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.synth_fill.restype = ctypes.c_int
        lib.synth_fill.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                                   ctypes.c_int, ctypes.c_double, ctypes.c_double, ctypes.c_uint64,
                                   ctypes.c_int]
        lib.synth_outlier_mask.restype = ctypes.c_int
        lib.synth_outlier_mask.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p]
        lib.synth_normal.restype = ctypes.c_double
        lib.synth_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_u64.restype = ctypes.c_uint64
        lib.synth_u64.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        _lib = lib
    return _lib


@dataclass(frozen=True)
class Workload:
    name: str
    rows: int
    cols: int
    dtype: int          # F32 or BF16
    sigma: float
    outlier_axis: int
    outlier_frac: float
    outlier_factor: float
    seed: int
    formats: tuple      # ((format, granularity), ...) exercised on this workload

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == F32 else 2


# The five workloads and the streaming pass (shapes and distributions as the
# quantization study describes them: activations N(0,1) with outlier channels,
# weights N(0, 0.02^2) with outlier output rows).
WORKLOADS = {
    "c1": Workload("c1", 1024, 4096, F32, 1.0, AXIS_COLS, 0.01, 20.0, 1,
                   (("int8", "tensor"), ("e4m3", "tensor"))),
    "c2": Workload("c2", 8192, 8192, BF16, 1.0, AXIS_COLS, 0.005, 200.0, 2,
                   (("e4m3", "row"), ("e5m2", "row"))),
    "c3": Workload("c3", 14336, 4096, BF16, 0.02, AXIS_ROWS, 0.01, 20.0, 3,
                   (("mxfp4", "block"),)),
    "c4": Workload("c4", 16384, 8192, BF16, 1.0, AXIS_COLS, 0.005, 200.0, 4,
                   (("nvfp4", "block"),)),
    "c5": Workload("c5", 28672, 8192, BF16, 0.02, AXIS_ROWS, 0.01, 30.0, 5,
                   (("int4", "block"),)),
    # activations for the c3 weights (K = 4096): the MXFP4 x MXFP4 product
    "a3": Workload("a3", 8192, 4096, BF16, 1.0, AXIS_COLS, 0.005, 200.0, 7, (("mxfp4", "block"),)),
    "stream": Workload("stream", 65536, 16384, BF16, 1.0, AXIS_COLS, 0.005, 200.0, 6,
                       (("int8", "tensor"), ("e4m3", "tensor"), ("e4m3", "row"), ("e5m2", "row"),
                        ("mxfp4", "block"), ("nvfp4", "block"), ("int4", "block"))),
}


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def fill(rows: int, cols: int, dtype: int, sigma: float = 1.0, outlier_axis: int = AXIS_NONE,
         outlier_frac: float = 0.0, outlier_factor: float = 1.0, seed: int = 0,
         ld: int | None = None, threads: int | None = None, out: np.ndarray | None = None,
         row0: int = 0, nrows: int | None = None) -> np.ndarray:
    """Return rows [row0, row0+nrows) of a rows x cols synthetic tensor as a
    [nrows, ld] array (float32, or uint16 BF16 bits).

    Columns [cols, ld) hold a 1e30 sentinel (BF16: its rounding).
    """
    ld = cols if ld is None else ld
    nrows = rows - row0 if nrows is None else nrows
    if ld < cols:
        raise ValueError("ld must be >= cols")
    if row0 < 0 or nrows < 0 or row0 + nrows > rows:
        raise ValueError("row range outside the tensor")
    npdt = np.float32 if dtype == F32 else np.uint16
    if out is None:
        out = np.empty((nrows, ld), dtype=npdt)
    elif out.dtype != npdt or out.shape != (nrows, ld) or not out.flags.c_contiguous:
        raise ValueError("out has the wrong dtype, shape or layout")
    if nrows == 0 or cols == 0:
        return out
    k = _load().synth_fill(out.ctypes.data, dtype, rows, row0, nrows, cols, ld, sigma, outlier_axis,
                           outlier_frac, outlier_factor, seed, threads or default_threads())
    if k < 0:
        raise MemoryError("synth_fill failed")
    return out


def make(name: str, row0: int = 0, nrows: int | None = None, ld: int | None = None,
         threads: int | None = None, out: np.ndarray | None = None) -> np.ndarray:
    """Rows [row0, row0+nrows) of workload `name` (all rows by default)."""
    w = WORKLOADS[name]
    return fill(w.rows, w.cols, w.dtype, w.sigma, w.outlier_axis, w.outlier_frac, w.outlier_factor,
                w.seed, ld, threads, out, row0, nrows)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """FP32 -> BF16 bit patterns by round to nearest even (input synthesis only)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def outlier_mask(seed: int, dim: int, frac: float) -> np.ndarray:
    m = np.zeros(dim, dtype=np.uint8)
    _load().synth_outlier_mask(seed, dim, frac, m.ctypes.data)
    return m


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen BF16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
