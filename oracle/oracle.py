"""ctypes front end of the CPU oracle (iq_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the bench's
cpu_baseline leg.  The GPU library never imports or calls it.

Arrays are numpy: inputs as float32 or uint16 (BF16 bits); codes uint8;
scales float32 (per-tensor / per-row), uint8 (E8M0 / E4M3 block codes) or
uint16 (FP16 group scales).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "iq_oracle.c")
_LIB = os.path.join(_HERE, "libiq_oracle.so")

FORMATS = {"int8": 0, "e4m3": 1, "e5m2": 2, "mxfp4": 3, "nvfp4": 4, "int4": 5, "int4zp": 6}
GRANS = {"tensor": 0, "row": 1, "block": 2}
F32, BF16 = 0, 1
K_E4M3, K_E5M2, K_E2M1, K_F16 = 0, 1, 2, 3
FLAG_MX_ROUND_NEAREST, FLAG_MX_ROUND_UP, FLAG_NV_SCALE_RNE = 1, 2, 4
QMAX = {"int8": 127.0, "e4m3": 448.0, "e5m2": 57344.0, "mxfp4": 6.0, "nvfp4": 6.0, "int4": 7.0}
FOUR_BIT = ("mxfp4", "nvfp4", "int4", "int4zp")


def build() -> str:
    """Compile libiq_oracle.so with gcc (always recompiles)."""
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
           "-fno-fast-math", "-frounding-math", "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class Desc(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int), ("gran", ctypes.c_int), ("in_dtype", ctypes.c_int),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("ld", ctypes.c_int64),
                ("flags", ctypes.c_uint32)]


class Stats(ctypes.Structure):
    _fields_ = [("n", ctypes.c_uint64), ("n_zero_flush", ctypes.c_uint64),
                ("n_saturated", ctypes.c_uint64), ("n_nonfinite", ctypes.c_uint64),
                ("sum_x2", ctypes.c_double), ("sum_err2", ctypes.c_double),
                ("sum_abs_err", ctypes.c_double), ("max_abs_err", ctypes.c_float),
                ("reserved", ctypes.c_uint32)]

    def as_dict(self) -> dict:
        return {k: getattr(self, k) for k, _ in self._fields_ if k != "reserved"}


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P, I64, F, U32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_uint32
        sig = {
            "iqo_bf16_to_f32": (F, [ctypes.c_uint16]),
            "iqo_f32_to_bf16": (ctypes.c_uint16, [F]),
            "iqo_fp_encode": (U32, [ctypes.c_int, F]),
            "iqo_fp_decode": (F, [ctypes.c_int, U32]),
            "iqo_int_encode": (ctypes.c_int, [F, ctypes.c_int]),
            "iqo_e8m0_code": (ctypes.c_uint8, [F, U32]),
            "iqo_e8m0_value": (F, [ctypes.c_uint8]),
            "iqo_e4m3_ceil": (ctypes.c_uint8, [F]),
            "iqo_fp_encode_n": (None, [ctypes.c_int, P, P, I64]),
            "iqo_fp_decode_n": (None, [ctypes.c_int, P, P, I64]),
            "iqo_int_encode_n": (None, [P, P, I64, ctypes.c_int]),
            "iqo_block_size": (I64, [ctypes.c_int, ctypes.c_int]),
            "iqo_check": (ctypes.c_int, [ctypes.POINTER(Desc)]),
            "iqo_amax": (F, [ctypes.POINTER(Desc), P]),
            "iqo_quantize_rows": (ctypes.c_int, [ctypes.POINTER(Desc), P, I64, I64, F, P, P, P, P,
                                                 ctypes.POINTER(Stats)]),
            "iqo_quantize": (ctypes.c_int, [ctypes.POINTER(Desc), P, P, P, P, P, ctypes.POINTER(Stats)]),
            "iqo_static_amax": (F, [F]),
            "iqo_quantize_zp_rows": (ctypes.c_int, [ctypes.POINTER(Desc), P, I64, I64, P, P, P, P,
                                                    ctypes.POINTER(Stats)]),
            "iqo_dequantize_zp": (ctypes.c_int, [ctypes.POINTER(Desc), P, P, P, P, ctypes.c_int]),
            "iqo_zp_gemm": (ctypes.c_int, [ctypes.POINTER(Desc), P, P, P, P, ctypes.c_int, I64, P, P]),
            "iqo_mx_gemm": (ctypes.c_int, [ctypes.POINTER(Desc), P, P, P, P, I64, P, P]),
            "iqo_mxw_gemm": (ctypes.c_int, [ctypes.POINTER(Desc), P, P, P, ctypes.c_int, I64, P, P]),
            "iqo_quantize_static": (ctypes.c_int, [ctypes.POINTER(Desc), P, F, P, P, P, P,
                                                   ctypes.POINTER(Stats)]),
            "iqo_dequantize": (ctypes.c_int, [ctypes.POINTER(Desc), P, P, P, P, ctypes.c_int]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


# ---- scalar codecs ---------------------------------------------------------
def fp_encode(kind: int, v: float) -> int:
    return int(_load().iqo_fp_encode(kind, float(v)))


def fp_decode(kind: int, code: int) -> float:
    return float(_load().iqo_fp_decode(kind, int(code)))


def fp_encode_array(kind: int, v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint32)
    _load().iqo_fp_encode_n(kind, v.ctypes.data, out.ctypes.data, v.size)
    return out


def fp_decode_array(kind: int, codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint32)
    out = np.empty(c.shape, dtype=np.float32)
    _load().iqo_fp_decode_n(kind, c.ctypes.data, out.ctypes.data, c.size)
    return out


def int_encode_array(v, qmax: int) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.int32)
    _load().iqo_int_encode_n(v.ctypes.data, out.ctypes.data, v.size, int(qmax))
    return out


def int_encode(v: float, qmax: int) -> int:
    return int(_load().iqo_int_encode(float(v), int(qmax)))


def e8m0_code(A: float, flags: int = 0) -> int:
    return int(_load().iqo_e8m0_code(float(A), int(flags)))


def e8m0_value(code: int) -> float:
    return float(_load().iqo_e8m0_value(int(code)))


def e4m3_ceil(t: float) -> int:
    return int(_load().iqo_e4m3_ceil(float(t)))


def bf16_to_f32(b: int) -> float:
    return float(_load().iqo_bf16_to_f32(int(b)))


def f32_to_bf16(f: float) -> int:
    return int(_load().iqo_f32_to_bf16(float(f)))


def block_size(fmt: str, gran: str) -> int:
    return int(_load().iqo_block_size(FORMATS[fmt], GRANS[gran]))


# ---- layouts ---------------------------------------------------------------
def codes_shape(fmt: str, rows: int, cols: int) -> tuple:
    return (rows, cols // 2) if fmt in FOUR_BIT else (rows, cols)


def scales_spec(fmt: str, gran: str, rows: int, cols: int) -> tuple:
    """(shape, numpy dtype) of the scales array."""
    if fmt in ("int8", "e4m3", "e5m2"):
        return ((1,) if gran == "tensor" else (rows,)), np.float32
    if fmt == "mxfp4":
        return (rows, cols // 32), np.uint8
    if fmt == "nvfp4":
        return (rows, cols // 16), np.uint8
    if fmt == "int4zp":
        return (rows, cols // 128), np.float32
    return (rows, cols // 128), np.uint16


def shifts_shape(rows: int, cols: int) -> tuple:
    """Asymmetric INT4 shifts: two 4-bit values per byte, group 2t in bits 3:0."""
    return (rows, cols // 256)


def _desc(fmt, gran, x, cols=None, flags=0):
    rows, ld = x.shape
    cols = ld if cols is None else cols
    in_dtype = F32 if x.dtype == np.float32 else BF16
    if x.dtype not in (np.float32, np.uint16) or not x.flags.c_contiguous:
        raise TypeError("x must be a C-contiguous float32 or uint16 (BF16) array")
    d = Desc(FORMATS[fmt], GRANS[gran], in_dtype, rows, cols, ld, flags)
    if _load().iqo_check(ctypes.byref(d)):
        raise ValueError(f"illegal descriptor {fmt}/{gran} rows={rows} cols={cols} ld={ld}")
    return d


def _p(a):
    return None if a is None else a.ctypes.data


def amax(x: np.ndarray, cols: int | None = None, fmt: str = "e4m3", gran: str = "tensor") -> float:
    d = _desc(fmt, gran, x, cols)
    return float(_load().iqo_amax(ctypes.byref(d), _p(x)))


def quantize(x: np.ndarray, fmt: str, gran: str, cols: int | None = None, flags: int = 0,
             want_xhat: bool = True, threads: int = 1, static_amax: float | None = None) -> dict:
    """Quantize a whole [rows, ld] array; returns codes, scales, global_scale, xhat, stats.

    threads > 1 splits rows across threads (the oracle itself is serial per
    row range; ctypes releases the GIL).  Codes, scales and x^ do not depend
    on the split; the double-precision sums may differ in the last bits.
    static_amax: per-tensor formats and NVFP4 only; the absmax is the given
    value (iqo_static_amax's rule) instead of the measured one.
    """
    d = _desc(fmt, gran, x, cols, flags)
    rows, c = d.rows, d.cols
    codes = np.zeros(codes_shape(fmt, rows, c), dtype=np.uint8)
    sshape, sdt = scales_spec(fmt, gran, rows, c)
    scales = np.zeros(sshape, dtype=sdt)
    g = np.zeros(1, dtype=np.float32)
    xhat = np.zeros((rows, c), dtype=np.float32) if want_xhat else None
    L = _load()
    tensor_amax = 0.0
    if static_amax is not None:
        if not (gran == "tensor" or fmt == "nvfp4"):
            raise ValueError("static_amax needs a per-tensor format or NVFP4")
        tensor_amax = L.iqo_static_amax(float(static_amax))
    elif gran == "tensor" or fmt == "nvfp4":
        tensor_amax = L.iqo_amax(ctypes.byref(d), _p(x))
    parts = _split(rows, threads)
    stats = [Stats() for _ in parts]
    shifts = np.zeros(shifts_shape(rows, c), dtype=np.uint8) if fmt == "int4zp" else None

    def run(i):
        r0, r1 = parts[i]
        if shifts is not None:
            rc = L.iqo_quantize_zp_rows(ctypes.byref(d), _p(x), r0, r1, _p(codes), _p(scales), _p(shifts),
                                        _p(xhat), ctypes.byref(stats[i]))
        else:
            rc = L.iqo_quantize_rows(ctypes.byref(d), _p(x), r0, r1, tensor_amax, _p(codes), _p(scales),
                                     _p(g), _p(xhat), ctypes.byref(stats[i]))
        if rc:
            raise RuntimeError("iqo_quantize_rows failed")

    if len(parts) == 1:
        run(0)
    else:
        with ThreadPoolExecutor(len(parts)) as ex:
            list(ex.map(run, range(len(parts))))
    st = merge_stats([s.as_dict() for s in stats])
    out = {"codes": codes, "scales": scales, "global_scale": g, "xhat": xhat, "stats": st,
           "tensor_amax": tensor_amax}
    if shifts is not None:
        out["shifts"] = shifts
    return out


def quantize_rows(x: np.ndarray, fmt: str, gran: str, row0: int, nrows: int, tensor_amax: float,
                  cols: int | None = None, flags: int = 0) -> dict:
    """Quantize only rows [row0, row0+nrows) of x, given the tensor absmax
    (used by per-tensor formats and NVFP4).  x holds just those rows."""
    d = _desc(fmt, gran, x, cols, flags)
    rows, c = d.rows, d.cols
    codes = np.zeros(codes_shape(fmt, rows, c), dtype=np.uint8)
    sshape, sdt = scales_spec(fmt, gran, rows, c)
    scales = np.zeros(sshape, dtype=sdt)
    g = np.zeros(1, dtype=np.float32)
    xhat = np.zeros((rows, c), dtype=np.float32)
    st = Stats()
    out = {"codes": codes, "scales": scales, "global_scale": g, "xhat": xhat}
    if fmt == "int4zp":
        out["shifts"] = np.zeros(shifts_shape(rows, c), dtype=np.uint8)
        rc = _load().iqo_quantize_zp_rows(ctypes.byref(d), _p(x), 0, rows, _p(codes), _p(scales),
                                          _p(out["shifts"]), _p(xhat), ctypes.byref(st))
    else:
        rc = _load().iqo_quantize_rows(ctypes.byref(d), _p(x), 0, rows, float(tensor_amax), _p(codes),
                                       _p(scales), _p(g), _p(xhat), ctypes.byref(st))
    if rc:
        raise RuntimeError("iqo_quantize_rows failed")
    out["stats"] = st.as_dict()
    return out


def dequantize(codes: np.ndarray, scales: np.ndarray, fmt: str, gran: str, rows: int, cols: int,
               global_scale: np.ndarray | None = None, out_dtype: int = F32,
               shifts: np.ndarray | None = None) -> np.ndarray:
    d = Desc(FORMATS[fmt], GRANS[gran], F32, rows, cols, cols, 0)
    if _load().iqo_check(ctypes.byref(d)):
        raise ValueError("illegal descriptor")
    out = np.zeros((rows, cols), dtype=np.float32 if out_dtype == F32 else np.uint16)
    if fmt == "int4zp":
        rc = _load().iqo_dequantize_zp(ctypes.byref(d), _p(np.ascontiguousarray(codes)),
                                       _p(np.ascontiguousarray(scales, dtype=np.float32)),
                                       _p(np.ascontiguousarray(shifts, dtype=np.uint8)), _p(out), out_dtype)
        if rc:
            raise RuntimeError("iqo_dequantize_zp failed")
        return out
    g = None if global_scale is None else np.ascontiguousarray(global_scale, dtype=np.float32)
    rc = _load().iqo_dequantize(ctypes.byref(d), _p(np.ascontiguousarray(codes)),
                                _p(np.ascontiguousarray(scales)), _p(g), _p(out), out_dtype)
    if rc:
        raise RuntimeError("iqo_dequantize failed")
    return out


def merge_stats(parts: list) -> dict:
    out = {"n": 0, "n_zero_flush": 0, "n_saturated": 0, "n_nonfinite": 0, "sum_x2": 0.0,
           "sum_err2": 0.0, "sum_abs_err": 0.0, "max_abs_err": 0.0}
    for p in parts:
        for k in ("n", "n_zero_flush", "n_saturated", "n_nonfinite", "sum_x2", "sum_err2", "sum_abs_err"):
            out[k] += p[k]
        out["max_abs_err"] = max(out["max_abs_err"], p["max_abs_err"])
    return out


def _split(rows: int, threads: int) -> list:
    threads = max(1, min(threads, rows)) if rows else 1
    return [(rows * t // threads, rows * (t + 1) // threads) for t in range(threads)]


def zp_gemm(codes: np.ndarray, scales: np.ndarray, shifts: np.ndarray, x: np.ndarray) -> tuple:
    """Puzzle 12's z[j, k] = sum_l sc * (w - sh) * y[l, k] for asymmetric INT4
    weights (N0 x K) and token-major activations x [n1, K] (float32 or BF16
    bits); returns (z, zabs) as float64 [N0, n1]."""
    n0 = codes.shape[0]
    K = codes.shape[1] * 2
    n1 = x.shape[0]
    if x.shape[1] != K:
        raise ValueError("activations must be [n1, K]")
    d = Desc(FORMATS["int4zp"], GRANS["block"], F32, n0, K, K, 0)
    z = np.zeros((n0, n1), dtype=np.float64)
    zabs = np.zeros((n0, n1), dtype=np.float64)
    xd = F32 if x.dtype == np.float32 else BF16
    rc = _load().iqo_zp_gemm(ctypes.byref(d), _p(np.ascontiguousarray(codes)),
                             _p(np.ascontiguousarray(scales, dtype=np.float32)),
                             _p(np.ascontiguousarray(shifts)), _p(np.ascontiguousarray(x)), xd, n1, _p(z), _p(zabs))
    if rc:
        raise RuntimeError("iqo_zp_gemm failed")
    return z, zabs


def mx_gemm(codes_w: np.ndarray, scales_w: np.ndarray, codes_a: np.ndarray, scales_a: np.ndarray) -> tuple:
    """FP4 GEMM over two MXFP4 operands: z[j, t] = sum_k xw[j, k] * xa[t, k]
    of the dequantized weights (codes [N0, K/2], E8M0 scales [N0, K/32]) and
    activations (codes [n1, K/2], scales [n1, K/32]); returns (z, zabs) as
    float64 [N0, n1]."""
    n0, K = codes_w.shape[0], codes_w.shape[1] * 2
    n1 = codes_a.shape[0]
    if codes_a.shape[1] * 2 != K or scales_w.shape != (n0, K // 32) or scales_a.shape != (n1, K // 32):
        raise ValueError("operand shapes do not match")
    d = Desc(FORMATS["mxfp4"], GRANS["block"], F32, n0, K, K, 0)
    z = np.zeros((n0, n1), dtype=np.float64)
    zabs = np.zeros((n0, n1), dtype=np.float64)
    rc = _load().iqo_mx_gemm(ctypes.byref(d), _p(np.ascontiguousarray(codes_w)), _p(np.ascontiguousarray(scales_w)),
                             _p(np.ascontiguousarray(codes_a)), _p(np.ascontiguousarray(scales_a)), n1, _p(z), _p(zabs))
    if rc:
        raise RuntimeError("iqo_mx_gemm failed")
    return z, zabs


def mxw_gemm(codes_w: np.ndarray, scales_w: np.ndarray, x: np.ndarray) -> tuple:
    """MXFP4 weights (codes [N0, K/2], E8M0 scales [N0, K/32]) against
    token-major activations x [n1, K] (float32 or BF16 bits):
    z[j, t] = sum_k xw[j, k] * x[t, k]; returns (z, zabs) as float64 [N0, n1]."""
    n0, K = codes_w.shape[0], codes_w.shape[1] * 2
    n1 = x.shape[0]
    if x.shape[1] != K or scales_w.shape != (n0, K // 32):
        raise ValueError("operand shapes do not match")
    d = Desc(FORMATS["mxfp4"], GRANS["block"], F32, n0, K, K, 0)
    z = np.zeros((n0, n1), dtype=np.float64)
    zabs = np.zeros((n0, n1), dtype=np.float64)
    xd = F32 if x.dtype == np.float32 else BF16
    rc = _load().iqo_mxw_gemm(ctypes.byref(d), _p(np.ascontiguousarray(codes_w)), _p(np.ascontiguousarray(scales_w)),
                              _p(np.ascontiguousarray(x)), xd, n1, _p(z), _p(zabs))
    if rc:
        raise RuntimeError("iqo_mxw_gemm failed")
    return z, zabs
