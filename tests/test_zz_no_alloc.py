"""iq_quantize_noalloc, the entry point that allocates nothing (its workspace
is the library's own device array), against iq_quantize with a workspace
of the caller's, through the C ABI: the same codes, scales, global scale,
x^ and statistics, bit for bit, on two calls in a row, the second on a
smaller input, for each format family."""
import numpy as np
import pytest

from helpers import to_device

pytestmark = pytest.mark.gpu

CASES = [("e4m3", "row"), ("int8", "tensor"), ("nvfp4", "block"), ("mxfp4", "block"), ("int4", "block"),
         ("e5m2", "tensor")]


@pytest.fixture(scope="module")
def iq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int_quantization_amd as m
    m.load_library()
    return m


def bytes_of(t):
    import torch
    return t.contiguous().view(torch.uint8).cpu().numpy()


def noalloc_call(iq, x, fmt, gran, want_stats, want_xhat):
    """iq_quantize_noalloc into freshly poisoned outputs."""
    import torch
    d = iq.desc_for(x, fmt, gran)
    codes, scales, gs = iq.empty_outputs(d, x.device, fmt, gran)
    codes.fill_(0xA5)
    scales.view(torch.uint8).fill_(0xA5)
    if gs is not None:
        gs.fill_(-1.0)
    stats = torch.full((64,), 0xA5, dtype=torch.uint8, device=x.device) if want_stats else None
    xh = torch.full((d.rows, d.cols), float("nan"), dtype=torch.float32, device=x.device) if want_xhat else None
    st = iq.iq_quantize_noalloc(d, x.data_ptr(), codes.data_ptr(), scales.data_ptr(),
                                None if gs is None else gs.data_ptr(), None if stats is None else stats.data_ptr(),
                                None if xh is None else xh.data_ptr(), iq.IQ_F32,
                                torch.cuda.current_stream().cuda_stream)
    assert st == iq.IQ_OK, iq.iq_status_str(st)
    return codes, scales, gs, stats, xh


@pytest.mark.parametrize("fmt,gran", CASES)
def test_noalloc_equals_workspace_call(iq, fmt, gran):
    import torch

    from synth import synth
    for rows in (4096, 37):                       # the second call on a smaller input
        x = to_device(synth.make("c4", nrows=rows))   # BF16 [rows, 8192], outlier channels
        for want_stats, want_xhat in ((True, True), (True, False), (False, False)):
            ref = iq.quantize(x, fmt, gran, stats=want_stats, xhat_dtype=torch.float32 if want_xhat else None)
            got = noalloc_call(iq, x, fmt, gran, want_stats, want_xhat)
            torch.cuda.synchronize()
            what = f"{fmt}/{gran} rows={rows} stats={want_stats} xhat={want_xhat}"
            assert np.array_equal(bytes_of(got[0]), bytes_of(ref.codes)), f"{what}: codes"
            assert np.array_equal(bytes_of(got[1]), bytes_of(ref.scales)), f"{what}: scales"
            if ref.global_scale is not None:
                assert np.array_equal(bytes_of(got[2]), bytes_of(ref.global_scale)), f"{what}: global scale"
            if want_stats:
                assert got[3][:64].cpu().tolist() == ref.stats_buf[:64].cpu().tolist(), f"{what}: statistics"
                assert ref.stats()["n"] == rows * 8192
            if want_xhat:
                assert np.array_equal(bytes_of(got[4]), bytes_of(ref.xhat)), f"{what}: x^"


def test_noalloc_rejects_bad_arguments_before_any_launch(iq):
    import torch
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda:0")
    d = iq.desc_for(x, "int4zp", "block")
    assert iq.iq_quantize_noalloc(d, x.data_ptr(), 0, 0, None, None, None, iq.IQ_F32, None) == iq.IQ_EINVAL
    d = iq.desc_for(x, "e4m3", "row")
    codes = torch.empty((4, 64), dtype=torch.uint8, device="cuda:0")
    assert iq.iq_quantize_noalloc(d, x.data_ptr(), codes.data_ptr(), 0, None, None, None, iq.IQ_F32,
                                  None) == iq.IQ_EINVAL              # no scales
