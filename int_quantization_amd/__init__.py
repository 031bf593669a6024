"""Python binding of libiq (block-scaled quantization on MI355X).

A thin ctypes layer over the C ABI declared in include/iq.h: the functions
below carry the C names and only marshal arguments.  torch provides device
memory (torch.empty) and the current HIP stream; every step of quantization
runs in the HIP kernels of libiq.so.  There is no CPU fallback: importing
works anywhere, but any call raises if the library is missing.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libiq.so")

# iq_format / iq_gran / iq_dtype / iq_status values of include/iq.h
FORMATS = {"int8": 0, "e4m3": 1, "e5m2": 2, "mxfp4": 3, "nvfp4": 4, "int4": 5, "int4zp": 6}
GRANS = {"tensor": 0, "row": 1, "block": 2}
IQ_F32, IQ_BF16 = 0, 1
IQ_OK, IQ_EINVAL, IQ_EALIGN, IQ_EUNSUPPORTED, IQ_EHIP = 0, 1, 2, 3, 4
# iq_desc.flags: scale-rule variants (MXFP4 exponent rounding, NVFP4 block-scale rounding)
IQ_FLAG_MX_ROUND_NEAREST, IQ_FLAG_MX_ROUND_UP, IQ_FLAG_NV_SCALE_RNE = 0x1, 0x2, 0x4
FOUR_BIT = ("mxfp4", "nvfp4", "int4", "int4zp")


class IQDesc(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("gran", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
                ("reserved0", ctypes.c_int32), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("ld_in", ctypes.c_int64), ("flags", ctypes.c_uint32), ("reserved1", ctypes.c_uint32)]


class IQStats(ctypes.Structure):
    _fields_ = [("n", ctypes.c_uint64), ("n_zero_flush", ctypes.c_uint64),
                ("n_saturated", ctypes.c_uint64), ("n_nonfinite", ctypes.c_uint64),
                ("sum_x2", ctypes.c_double), ("sum_err2", ctypes.c_double),
                ("sum_abs_err", ctypes.c_double), ("max_abs_err", ctypes.c_float),
                ("reserved", ctypes.c_uint32)]

    def as_dict(self) -> dict:
        return {k: getattr(self, k) for k, _ in self._fields_ if k != "reserved"}


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libiq.so (raises OSError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise OSError(f"libiq.so not found at {path}: build it with __graft_entry__.build()")
    L = ctypes.CDLL(path)
    P, S = ctypes.c_void_p, ctypes.c_size_t
    D = ctypes.POINTER(IQDesc)
    L.iq_codes_bytes.restype, L.iq_codes_bytes.argtypes = S, [D]
    L.iq_scales_bytes.restype, L.iq_scales_bytes.argtypes = S, [D]
    L.iq_workspace_bytes.restype, L.iq_workspace_bytes.argtypes = S, [D]
    L.iq_quantize.restype = ctypes.c_int
    L.iq_quantize.argtypes = [D, P, P, P, P, P, P, ctypes.c_int32, P, P]
    L.iq_quantize_noalloc.restype = ctypes.c_int
    L.iq_quantize_noalloc.argtypes = [D, P, P, P, P, P, P, ctypes.c_int32, P]
    L.iq_quantize_static.restype = ctypes.c_int
    L.iq_quantize_static.argtypes = [D, P, P, P, P, P, P, P, ctypes.c_int32, P, P]
    L.iq_quantize_zp.restype = ctypes.c_int
    L.iq_quantize_zp.argtypes = [D, P, P, P, P, P, P, ctypes.c_int32, P, P]
    L.iq_dequantize_zp.restype = ctypes.c_int
    L.iq_dequantize_zp.argtypes = [D, P, P, P, P, ctypes.c_int32, P]
    L.iq_shifts_bytes.restype, L.iq_shifts_bytes.argtypes = S, [D]
    L.iq_zp_gemm.restype = ctypes.c_int
    L.iq_zp_gemm.argtypes = [D, P, P, P, P, ctypes.c_int32, ctypes.c_int64, P, P]
    L.iq_mx_gemm.restype = ctypes.c_int
    L.iq_mx_gemm.argtypes = [D, P, P, P, P, ctypes.c_int64, P, P]
    L.iq_mxw_gemm.restype = ctypes.c_int
    L.iq_mxw_gemm.argtypes = [D, P, P, P, ctypes.c_int32, ctypes.c_int64, P, P]
    L.iq_dequantize.restype = ctypes.c_int
    L.iq_dequantize.argtypes = [D, P, P, P, P, ctypes.c_int32, P]
    L.iq_amax.restype = ctypes.c_int
    L.iq_amax.argtypes = [D, P, P, P, P]
    L.iq_status_str.restype, L.iq_status_str.argtypes = ctypes.c_char_p, [ctypes.c_int]
    L.iq_abi_version.restype, L.iq_abi_version.argtypes = ctypes.c_int, []
    _lib = L
    return L


class IQError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {iq_status_str(status)} ({status})")
        self.status = status


def _check(status: int, what: str) -> None:
    if status != IQ_OK:
        raise IQError(status, what)


# ---- C entry points (same names, marshalling only) -------------------------
def iq_abi_version() -> int:
    return load_library().iq_abi_version()


def iq_status_str(status: int) -> str:
    return load_library().iq_status_str(status).decode()


def iq_codes_bytes(d: IQDesc) -> int:
    return load_library().iq_codes_bytes(ctypes.byref(d))


def iq_scales_bytes(d: IQDesc) -> int:
    return load_library().iq_scales_bytes(ctypes.byref(d))


def iq_workspace_bytes(d: IQDesc) -> int:
    return load_library().iq_workspace_bytes(ctypes.byref(d))


def iq_quantize(d: IQDesc, x: int, codes: int, scales: int, global_scale: int | None, stats: int | None,
                xhat: int | None, xhat_dtype: int, workspace: int, stream: int | None) -> int:
    """Raw call with integer device addresses; returns the iq_status."""
    return load_library().iq_quantize(ctypes.byref(d), x, codes, scales, global_scale, stats, xhat,
                                      xhat_dtype, workspace, stream)


def iq_quantize_noalloc(d: IQDesc, x: int, codes: int, scales: int, global_scale: int | None, stats: int | None,
                        xhat: int | None, xhat_dtype: int, stream: int | None) -> int:
    """Raw call with integer device addresses; the library's own workspace."""
    return load_library().iq_quantize_noalloc(ctypes.byref(d), x, codes, scales, global_scale, stats, xhat,
                                              xhat_dtype, stream)


def iq_quantize_static(d: IQDesc, x: int, amax_in: int, codes: int, scales: int, global_scale: int | None,
                       stats: int | None, xhat: int | None, xhat_dtype: int, workspace: int,
                       stream: int | None) -> int:
    """Raw call with integer device addresses (amax_in: device float32 [1])."""
    return load_library().iq_quantize_static(ctypes.byref(d), x, amax_in, codes, scales, global_scale, stats,
                                             xhat, xhat_dtype, workspace, stream)


def iq_quantize_zp(d: IQDesc, x: int, codes: int, scales: int, shifts: int, stats: int | None,
                   xhat: int | None, xhat_dtype: int, workspace: int, stream: int | None) -> int:
    return load_library().iq_quantize_zp(ctypes.byref(d), x, codes, scales, shifts, stats, xhat, xhat_dtype,
                                         workspace, stream)


def iq_dequantize_zp(d: IQDesc, codes: int, scales: int, shifts: int, xhat: int, xhat_dtype: int,
                     stream: int | None) -> int:
    return load_library().iq_dequantize_zp(ctypes.byref(d), codes, scales, shifts, xhat, xhat_dtype, stream)


def iq_shifts_bytes(d: IQDesc) -> int:
    return load_library().iq_shifts_bytes(ctypes.byref(d))


def iq_zp_gemm(d: IQDesc, codes: int, scales: int, shifts: int, x: int, x_dtype: int, n1: int, z: int,
               stream: int | None) -> int:
    return load_library().iq_zp_gemm(ctypes.byref(d), codes, scales, shifts, x, x_dtype, n1, z, stream)


def iq_mx_gemm(d: IQDesc, codes_w: int, scales_w: int, codes_a: int, scales_a: int, n1: int, z: int,
               stream: int | None) -> int:
    return load_library().iq_mx_gemm(ctypes.byref(d), codes_w, scales_w, codes_a, scales_a, n1, z, stream)


def iq_mxw_gemm(d: IQDesc, codes: int, scales: int, x: int, x_dtype: int, n1: int, z: int,
                stream: int | None) -> int:
    return load_library().iq_mxw_gemm(ctypes.byref(d), codes, scales, x, x_dtype, n1, z, stream)


def iq_dequantize(d: IQDesc, codes: int, scales: int, global_scale: int | None, xhat: int,
                  xhat_dtype: int, stream: int | None) -> int:
    return load_library().iq_dequantize(ctypes.byref(d), codes, scales, global_scale, xhat, xhat_dtype,
                                        stream)


def iq_amax(d: IQDesc, x: int, amax_out: int, workspace: int, stream: int | None) -> int:
    return load_library().iq_amax(ctypes.byref(d), x, amax_out, workspace, stream)


# ---- torch-facing helpers (allocation with torch.empty + the calls above) ---
def _torch():
    import torch
    return torch


def make_desc(fmt: str, gran: str, rows: int, cols: int, in_dtype: int = IQ_BF16, ld: int | None = None,
              flags: int = 0) -> IQDesc:
    return IQDesc(FORMATS[fmt], GRANS[gran], in_dtype, 0, rows, cols, cols if ld is None else ld, flags, 0)


def desc_for(x, fmt: str, gran: str, cols: int | None = None, flags: int = 0) -> IQDesc:
    """Descriptor of a 2-D CUDA/HIP tensor (float32 or bfloat16, unit column stride)."""
    torch = _torch()
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    if x.dtype == torch.float32:
        dt = IQ_F32
    elif x.dtype == torch.bfloat16:
        dt = IQ_BF16
    else:
        raise TypeError("x must be float32 or bfloat16")
    rows = x.shape[0]
    c = x.shape[1] if cols is None else cols
    ld = x.stride(0) if rows > 1 else c   # a single row is read at ld-independent offsets
    return IQDesc(FORMATS[fmt], GRANS[gran], dt, 0, rows, c, ld, flags, 0)


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def empty_outputs(d: IQDesc, device, fmt: str, gran: str):
    """codes, scales, global_scale tensors for a descriptor (torch.empty)."""
    torch = _torch()
    rows, cols = d.rows, d.cols
    codes = torch.empty((rows, cols // 2 if fmt in FOUR_BIT else cols), dtype=torch.uint8, device=device)
    if fmt in ("int8", "e4m3", "e5m2"):
        scales = torch.empty((1,) if gran == "tensor" else (rows,), dtype=torch.float32, device=device)
    elif fmt == "mxfp4":
        scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=device)
    elif fmt == "nvfp4":
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=device)
    elif fmt == "int4zp":
        scales = torch.empty((rows, cols // 128), dtype=torch.float32, device=device)
    else:
        scales = torch.empty((rows, cols // 128), dtype=torch.int16, device=device)
    gscale = torch.empty((1,), dtype=torch.float32, device=device) if fmt == "nvfp4" else None
    return codes, scales, gscale


def workspace_for(d: IQDesc, device):
    """A zero-filled workspace (the library's tickets start at zero and every
    call leaves them there); 256-byte aligned."""
    torch = _torch()
    n = iq_workspace_bytes(d)
    return torch.zeros((n + 255) // 256 * 64, dtype=torch.float32, device=device)


def _check_buffer(t, nbytes: int, what: str, device, dtype=None):
    """A caller-supplied device buffer must be contiguous, on the input's
    device, of the expected dtype and hold at least nbytes."""
    if t is None:
        raise ValueError(f"{what} is missing")
    if t.device != device:
        raise ValueError(f"{what} is on {t.device}, the input on {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{what} holds {t.numel() * t.element_size()} bytes, needs {nbytes}")


def _check_out(out: "Quantized", d: IQDesc, fmt: str, gran: str, device):
    """A Quantized passed as `out` must match the descriptor of this call."""
    torch = _torch()
    if out.fmt != fmt or out.gran != gran or out.rows != d.rows or out.cols != d.cols:
        raise ValueError("out was made for another format, granularity or shape")
    _check_buffer(out.codes, iq_codes_bytes(d), "out.codes", device, torch.uint8)
    _check_buffer(out.scales, iq_scales_bytes(d), "out.scales", device)
    if fmt == "nvfp4":
        _check_buffer(out.global_scale, 4, "out.global_scale", device, torch.float32)
    if fmt == "int4zp":
        _check_buffer(out.shifts, iq_shifts_bytes(d), "out.shifts", device, torch.uint8)
    if out.stats_buf is not None:
        _check_buffer(out.stats_buf, ctypes.sizeof(IQStats), "out.stats_buf", device)
    if out.xhat is not None:
        if out.xhat.dtype not in (torch.float32, torch.bfloat16):
            raise TypeError("out.xhat must be float32 or bfloat16")
        _check_buffer(out.xhat, d.rows * d.cols * out.xhat.element_size(), "out.xhat", device)


@dataclass
class Quantized:
    codes: object
    scales: object
    global_scale: object
    xhat: object
    stats_buf: object
    fmt: str
    gran: str
    rows: int
    cols: int
    shifts: object = None   # asymmetric INT4: uint8 [rows, cols / 256]

    def stats(self) -> dict:
        """Copy the statistics to the host (synchronizes with the device)."""
        if self.stats_buf is None:
            return None
        raw = bytes(self.stats_buf.cpu().numpy().tobytes())
        return IQStats.from_buffer_copy(raw).as_dict()


def quantize(x, fmt: str, gran: str, *, stats: bool = True, xhat_dtype=None, cols: int | None = None,
             flags: int = 0, workspace=None, out=None, stream=None, static_amax=None) -> Quantized:
    """Quantize a device tensor; outputs are allocated with torch.empty unless
    `out` (a Quantized from a previous call of the same shape) is given.
    static_amax (a device float32 tensor of one element) selects static
    scaling: iq_quantize_static with that absmax instead of the measured one."""
    torch = _torch()
    d = desc_for(x, fmt, gran, cols, flags)
    if out is None:
        codes, scales, gscale = empty_outputs(d, x.device, fmt, gran)
        sbuf = torch.empty((64,), dtype=torch.uint8, device=x.device) if stats else None
        xh = None
        if xhat_dtype is not None:
            xh = torch.empty((d.rows, d.cols), dtype=xhat_dtype, device=x.device)
        shifts = (torch.empty((d.rows, d.cols // 256), dtype=torch.uint8, device=x.device)
                  if fmt == "int4zp" else None)
        out = Quantized(codes, scales, gscale, xh, sbuf, fmt, gran, d.rows, d.cols, shifts)
    else:
        _check_out(out, d, fmt, gran, x.device)
    if workspace is None:
        ws = workspace_for(d, x.device)
    else:
        _check_buffer(workspace, iq_workspace_bytes(d), "workspace", x.device)
        ws = workspace
    xdt = IQ_F32
    if out.xhat is not None:
        xdt = IQ_F32 if out.xhat.dtype == torch.float32 else IQ_BF16
    if fmt == "int4zp":
        if static_amax is not None:
            raise ValueError("static_amax needs a per-tensor format or NVFP4")
        st = iq_quantize_zp(d, x.data_ptr(), _ptr(out.codes), _ptr(out.scales), _ptr(out.shifts),
                            _ptr(out.stats_buf), _ptr(out.xhat), xdt, ws.data_ptr(), _stream(stream))
        _check(st, "iq_quantize_zp")
    elif static_amax is None:
        st = iq_quantize(d, x.data_ptr(), _ptr(out.codes), _ptr(out.scales), _ptr(out.global_scale),
                         _ptr(out.stats_buf), _ptr(out.xhat), xdt, ws.data_ptr(), _stream(stream))
        _check(st, "iq_quantize")
    else:
        if static_amax.dtype != torch.float32 or static_amax.numel() != 1 or static_amax.device != x.device:
            raise ValueError("static_amax must be one float32 on the input's device")
        st = iq_quantize_static(d, x.data_ptr(), static_amax.data_ptr(), _ptr(out.codes), _ptr(out.scales),
                                _ptr(out.global_scale), _ptr(out.stats_buf), _ptr(out.xhat), xdt,
                                ws.data_ptr(), _stream(stream))
        _check(st, "iq_quantize_static")
    return out


def dequantize(q: Quantized, out_dtype=None, out=None, stream=None):
    torch = _torch()
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    d = make_desc(q.fmt, q.gran, q.rows, q.cols)
    if out is None:
        out = torch.empty((q.rows, q.cols), dtype=out_dtype, device=q.codes.device)
    elif out.dtype not in (torch.float32, torch.bfloat16) or tuple(out.shape) != (q.rows, q.cols):
        raise ValueError("out must be a float32 or bfloat16 [rows, cols] tensor")
    else:
        _check_buffer(out, q.rows * q.cols * out.element_size(), "out", q.codes.device)
    _check_buffer(q.codes, iq_codes_bytes(d), "codes", q.codes.device, torch.uint8)
    _check_buffer(q.scales, iq_scales_bytes(d), "scales", q.codes.device)
    if q.fmt == "nvfp4":
        _check_buffer(q.global_scale, 4, "global_scale", q.codes.device, torch.float32)
    if q.fmt == "int4zp":
        _check_buffer(q.shifts, iq_shifts_bytes(d), "shifts", q.codes.device, torch.uint8)
    dt = IQ_F32 if out.dtype == torch.float32 else IQ_BF16
    if q.fmt == "int4zp":
        st = iq_dequantize_zp(d, q.codes.data_ptr(), q.scales.data_ptr(), _ptr(q.shifts), out.data_ptr(), dt,
                              _stream(stream))
        _check(st, "iq_dequantize_zp")
        return out
    st = iq_dequantize(d, q.codes.data_ptr(), q.scales.data_ptr(), _ptr(q.global_scale), out.data_ptr(), dt,
                       _stream(stream))
    _check(st, "iq_dequantize")
    return out


def amax(x, workspace=None, stream=None):
    torch = _torch()
    d = desc_for(x, "e4m3", "tensor")
    out = torch.empty((1,), dtype=torch.float32, device=x.device)
    if workspace is None:
        ws = workspace_for(d, x.device)
    else:
        _check_buffer(workspace, iq_workspace_bytes(d), "workspace", x.device)
        ws = workspace
    _check(iq_amax(d, x.data_ptr(), out.data_ptr(), ws.data_ptr(), _stream(stream)), "iq_amax")
    return out


def _gemm_out(out, n0: int, n1: int, device):
    """z float32 [n0, n1]: a new tensor, or the caller's after checks."""
    torch = _torch()
    if out is None:
        return torch.empty((n0, n1), dtype=torch.float32, device=device)
    if tuple(out.shape) != (n0, n1):
        raise ValueError(f"out must be [{n0}, {n1}], got {tuple(out.shape)}")
    _check_buffer(out, n0 * n1 * 4, "out", device, torch.float32)
    return out


def zp_gemm(q: "Quantized", x, out=None, stream=None):
    """Puzzle 12's z[j, k] = sum_l sc (w - sh) y[l, k] for asymmetric INT4
    weights q (from quantize(..., "int4zp", "block")) and token-major BF16
    activations x [n1, K]; returns z float32 [N0, n1]."""
    torch = _torch()
    if q.fmt != "int4zp":
        raise ValueError("zp_gemm needs asymmetric INT4 weights")
    if x.dim() != 2 or x.shape[1] != q.cols or x.dtype != torch.bfloat16 or not x.is_contiguous():
        raise ValueError("x must be a contiguous BF16 [n1, K] tensor")
    n1 = x.shape[0]
    out = _gemm_out(out, q.rows, n1, x.device)
    d = make_desc("int4zp", "block", q.rows, q.cols)
    _check_buffer(q.codes, iq_codes_bytes(d), "codes", x.device, torch.uint8)
    _check_buffer(q.scales, iq_scales_bytes(d), "scales", x.device, torch.float32)
    _check_buffer(q.shifts, iq_shifts_bytes(d), "shifts", x.device, torch.uint8)
    st = iq_zp_gemm(d, q.codes.data_ptr(), q.scales.data_ptr(), q.shifts.data_ptr(), x.data_ptr(), IQ_BF16, n1,
                    out.data_ptr(), _stream(stream))
    _check(st, "iq_zp_gemm")
    return out


def mx_gemm(qw: "Quantized", qa: "Quantized", out=None, stream=None):
    """FP4 GEMM z[j, t] = sum_k xw[j, k] xa[t, k] of two MXFP4 operands (from
    quantize(..., "mxfp4", "block")), weights qw [N0, K] and activations
    qa [n1, K]; returns z float32 [N0, n1]."""
    torch = _torch()
    if qw.fmt != "mxfp4" or qa.fmt != "mxfp4":
        raise ValueError("mx_gemm needs two MXFP4 operands")
    if qa.cols != qw.cols:
        raise ValueError("operands disagree on K")
    n1 = qa.rows
    out = _gemm_out(out, qw.rows, n1, qw.codes.device)
    d = make_desc("mxfp4", "block", qw.rows, qw.cols)
    da = make_desc("mxfp4", "block", qa.rows, qa.cols)
    dev = qw.codes.device
    _check_buffer(qw.codes, iq_codes_bytes(d), "weight codes", dev, torch.uint8)
    _check_buffer(qw.scales, iq_scales_bytes(d), "weight scales", dev, torch.uint8)
    _check_buffer(qa.codes, iq_codes_bytes(da), "activation codes", dev, torch.uint8)
    _check_buffer(qa.scales, iq_scales_bytes(da), "activation scales", dev, torch.uint8)
    st = iq_mx_gemm(d, qw.codes.data_ptr(), qw.scales.data_ptr(), qa.codes.data_ptr(), qa.scales.data_ptr(), n1,
                    out.data_ptr(), _stream(stream))
    _check(st, "iq_mx_gemm")
    return out


def mxw_gemm(qw: "Quantized", x, out=None, stream=None):
    """MXFP4 weights qw [N0, K] (from quantize(..., "mxfp4", "block")) against
    token-major BF16 activations x [n1, K]: z[j, t] = sum_k xw[j, k] x[t, k];
    returns z float32 [N0, n1]."""
    torch = _torch()
    if qw.fmt != "mxfp4":
        raise ValueError("mxw_gemm needs MXFP4 weights")
    if x.dim() != 2 or x.shape[1] != qw.cols or x.dtype != torch.bfloat16 or not x.is_contiguous():
        raise ValueError("x must be a contiguous BF16 [n1, K] tensor")
    n1 = x.shape[0]
    out = _gemm_out(out, qw.rows, n1, x.device)
    d = make_desc("mxfp4", "block", qw.rows, qw.cols)
    _check_buffer(qw.codes, iq_codes_bytes(d), "weight codes", x.device, torch.uint8)
    _check_buffer(qw.scales, iq_scales_bytes(d), "weight scales", x.device, torch.uint8)
    st = iq_mxw_gemm(d, qw.codes.data_ptr(), qw.scales.data_ptr(), x.data_ptr(), IQ_BF16, n1, out.data_ptr(),
                     _stream(stream))
    _check(st, "iq_mxw_gemm")
    return out
