"""Shared helpers of the GPU parity tests (comparison with the CPU oracle)."""
import numpy as np


def to_device(x_np, device="cuda:0"):
    """numpy float32 / uint16 (BF16 bits) -> torch tensor on the GPU."""
    import torch
    if x_np.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x_np).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x_np)).to(device)


def as_bits(a):
    a = np.ascontiguousarray(a)
    if a.dtype in (np.float32, np.int32, np.uint32):
        return a.view(np.uint32)
    if a.dtype in (np.uint16, np.int16, np.float16):
        return a.view(np.uint16)
    return a.view(np.uint8)


def assert_bits_equal(got, want, what, nan_equal=True):
    """Bitwise equality; with nan_equal, any NaN matches any NaN (payloads are
    not specified by the method)."""
    g, w = as_bits(got), as_bits(want)
    assert g.shape == w.shape, f"{what}: shape {g.shape} vs {w.shape}"
    bad = g != w
    if nan_equal and np.asarray(got).dtype == np.float32:
        bad &= ~(np.isnan(np.asarray(got)) & np.isnan(np.asarray(want)))
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} differ; first at {idx.tolist()}: "
                             f"got {[hex(int(g[tuple(i)])) for i in idx]} want {[hex(int(w[tuple(i)])) for i in idx]}")


def assert_stats_match(got: dict, want: dict, what: str, rel=1e-6):
    for k in ("n", "n_zero_flush", "n_saturated", "n_nonfinite"):
        assert got[k] == want[k], f"{what}: {k} {got[k]} vs {want[k]}"
    assert np.float32(got["max_abs_err"]) == np.float32(want["max_abs_err"]), \
        f"{what}: max_abs_err {got['max_abs_err']} vs {want['max_abs_err']}"
    for k in ("sum_x2", "sum_err2", "sum_abs_err"):
        g, w = got[k], want[k]
        if g == w or (np.isnan(g) and np.isnan(w)):      # identical, including +-inf
            continue
        assert abs(g - w) <= rel * abs(w) + 1e-300, f"{what}: {k} {g} vs {w} (rel {abs(g - w) / max(abs(w), 1e-300):.3g})"


def widen(x_np):
    return (x_np.astype(np.uint32) << 16).view(np.float32) if x_np.dtype == np.uint16 else x_np
