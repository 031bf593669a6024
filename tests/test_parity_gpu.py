"""GPU parity: libiq (HIP, gfx950) against the CPU oracle, element by element.

Codes, scales, the NVFP4 global scale and x^ must match bit for bit (any NaN
matches any NaN); counts and the maximum error exactly; the summed
statistics within 1e-6 relative.  Inputs come from the seeded generator in
synth/ (shared by both sides); nothing here feeds GPU output to the oracle.
"""
import os

import numpy as np
import pytest

from helpers import assert_bits_equal, assert_stats_match, to_device, widen

pytestmark = pytest.mark.gpu

THREADS = max(1, min(16, os.cpu_count() or 1))

ALL = [("int8", "tensor"), ("e4m3", "tensor"), ("e5m2", "tensor"), ("int8", "row"), ("e4m3", "row"),
       ("e5m2", "row"), ("mxfp4", "block"), ("nvfp4", "block"), ("int4", "block"), ("int4zp", "block")]


def fits(O, fmt, gran, cols):
    """Whether a row length is legal for the format (asymmetric INT4 needs
    whole shift bytes: cols a multiple of 256)."""
    bs = O.block_size(fmt, gran)
    return not (bs and cols % bs) and not (fmt == "int4zp" and cols % 256)


@pytest.fixture(scope="module")
def iq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int_quantization_amd as m
    m.load_library()
    return m


@pytest.fixture(scope="module")
def O():
    from oracle import oracle
    return oracle


@pytest.fixture(scope="module")
def S():
    from synth import synth
    return synth


def run_gpu(iq, x_np, fmt, gran, cols=None, xhat="f32", flags=0, stats=True, x_dev=None):
    """One iq_quantize call; stats=False passes no statistics buffer (the
    statistics-free kernels), x_dev an input already on the device."""
    import torch
    x = to_device(x_np) if x_dev is None else x_dev
    if cols is not None:
        x = x[:, :cols]
    xdt = {"f32": torch.float32, "bf16": torch.bfloat16, None: None}[xhat]
    q = iq.quantize(x, fmt, gran, xhat_dtype=xdt, flags=flags, stats=stats)
    torch.cuda.synchronize()
    out = {"codes": q.codes.cpu().numpy(), "scales": q.scales.cpu().numpy(), "stats": q.stats(), "q": q}
    if q.global_scale is not None:
        out["global_scale"] = q.global_scale.cpu().numpy()
    if q.shifts is not None:
        out["shifts"] = q.shifts.cpu().numpy()
    if q.xhat is not None:
        out["xhat"] = (q.xhat.cpu().numpy() if q.xhat.dtype == torch.float32
                       else q.xhat.cpu().view(torch.int16).numpy().view(np.uint16))
    return out


def compare(g, r, fmt, what, O=None, S=None, xhat="f32"):
    assert_bits_equal(g["codes"], r["codes"], f"{what} codes")
    gs = g["scales"]
    if gs.dtype == np.int16:
        gs = gs.view(np.uint16)
    assert_bits_equal(gs, r["scales"], f"{what} scales")
    if fmt == "nvfp4":
        assert_bits_equal(g["global_scale"], r["global_scale"], f"{what} global scale")
    if fmt == "int4zp":
        assert_bits_equal(g["shifts"], r["shifts"], f"{what} shifts")
    if "xhat" in g and r.get("xhat") is not None:
        want = r["xhat"]
        if xhat == "bf16":
            want = S.f32_to_bf16_bits(want)
        assert_bits_equal(g["xhat"], want, f"{what} xhat")
    if g["stats"] is not None:
        assert_stats_match(g["stats"], r["stats"], what)


def oracle_ref(O, x_np, fmt, gran, cols=None, want_xhat=True, flags=0):
    return O.quantize(x_np, fmt, gran, cols=cols, flags=flags, want_xhat=want_xhat, threads=THREADS)


# ---- shapes spanning several tiles, ragged tails, padded rows -----------------
SHAPES = [
    (37, 8192, None),      # per-row: 4 chunks per thread
    (5, 2072, None),       # per-row: 259 chunks, ragged over 256 threads
    (3, 40000, None),      # per-row: long rows, two-pass kernel
    (2100, 16, None),      # more rows than workgroups, 2 chunks per row
    (33, 1024, 1056),      # padded rows (ld > cols), power-of-two chunks per row
    (13, 384, 400),        # padded rows, non-power-of-two chunks per row
    (1, 8192, None),
    (6, 2048, None),       # per-row: one wave, 4 chunks per lane
    (9, 16384, None),      # per-row: 8 chunks per lane (the stream's row length)
    (4, 12288, 12296),     # per-row: 8 chunks per lane, partial, padded rows
]


def make_input(S, dtype, rows, cols, ld, seed):
    w = S.fill(rows, cols, dtype, sigma=1.0, outlier_axis=S.AXIS_COLS, outlier_frac=0.02,
               outlier_factor=50.0, seed=seed, ld=ld or cols)
    return w


@pytest.mark.parametrize("stats", [True, False], ids=["stats", "nostats"])
@pytest.mark.parametrize("dtype", [1, 0], ids=["bf16", "f32"])
@pytest.mark.parametrize("fmt,gran", ALL)
def test_parity_shapes(iq, O, S, fmt, gran, dtype, stats):
    """Every row-kernel width (1, 2, 4 chunks per lane on one wave; 2, 4, 8 on
    four; the two-pass kernel), full and partial flat tiles, padded rows,
    with and without the statistics, with and without x^."""
    for i, (rows, cols, ld) in enumerate(SHAPES):
        if not fits(O, fmt, gran, cols):
            continue
        x = make_input(S, dtype, rows, cols, ld, seed=100 + i)
        r = oracle_ref(O, x, fmt, gran, cols=cols if ld else None)
        for xhat in ("f32", None):
            g = run_gpu(iq, x, fmt, gran, cols=cols if ld else None, xhat=xhat, stats=stats)
            compare(g, r, fmt, f"{fmt}/{gran}/{'bf16' if dtype else 'f32'} {rows}x{cols} ld={ld} stats={stats} "
                               f"xhat={xhat}", O)


def sweep_shapes(O, fmt, gran, seed, n=20):
    """n legal (rows, cols, ld, stats, xhat) drawn from a seeded generator:
    row lengths log-uniform from one chunk (or block) to 65536 columns, up to
    about 2 M elements, padded rows (ld > cols) about a third of the time,
    statistics and x^ on or off; per-tensor adds contiguous shapes whose
    element count is a multiple of 16384 (the per-tensor kernel over rows of
    16384), without x^, which that kernel requires."""
    rng = np.random.default_rng(seed)
    step = 256 if fmt == "int4zp" else max(8, O.block_size(fmt, gran) or 8)
    out = []
    for _ in range(n):
        cols = max(step, int(np.exp(rng.uniform(np.log(step), np.log(65536)))) // step * step)
        rows = int(rng.integers(1, max(2, min(400, 2_000_000 // cols)) + 1))
        ld = cols + 8 * int(rng.integers(1, 9)) if rng.random() < 0.35 else None
        out.append((rows, cols, ld, bool(rng.random() < 0.7), [None, "f32", "bf16"][int(rng.integers(0, 3))]))
    if gran == "tensor":
        for rows, cols in ((2, 8192), (3, 16384), (1, 65536), (int(rng.integers(2, 40)) * 4, 4096)):
            out.append((rows, cols, None, bool(rng.random() < 0.7), None))
    return out


@pytest.mark.parametrize("dtype", [1, 0], ids=["bf16", "f32"])
@pytest.mark.parametrize("fmt,gran", ALL)
def test_parity_random_shapes(iq, O, S, fmt, gran, dtype):
    """A seeded sweep across the kernel selection: every drawn shape, with
    its statistics and x^ choice, against the oracle bit for bit; the
    standalone dequantize of every third contiguous shape as well."""
    seed = 7000 + 10 * ALL.index((fmt, gran)) + dtype
    for i, (rows, cols, ld, stats, xhat) in enumerate(sweep_shapes(O, fmt, gran, seed)):
        x = make_input(S, dtype, rows, cols, ld, seed=seed * 100 + i)
        what = f"{fmt}/{gran}/{'bf16' if dtype else 'f32'} {rows}x{cols} ld={ld} (seed {seed}, case {i})"
        r = oracle_ref(O, x, fmt, gran, cols=cols if ld else None, want_xhat=xhat is not None)
        g = run_gpu(iq, x, fmt, gran, cols=cols if ld else None, xhat=xhat, stats=stats)
        compare(g, r, fmt, f"{what} stats={stats} xhat={xhat}", O, S, xhat=xhat or "f32")
        if ld is None and i % 3 == 0:
            check_dequantize(iq, O, S, x, fmt, gran, what)


def gemm_shapes(seed, k_step, n=12, max_macs=60e6):
    """n seeded (n0, K, n1): n0 up to 384 weight rows, K a multiple of k_step
    up to 4096, n1 log-uniform from 1 to 1200 tokens (the few-token, tiled,
    k-split and ragged-tile paths); n0 is drawn below max_macs / (K n1), to
    bound the oracle's time."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        K = k_step * int(rng.integers(1, 4096 // k_step + 1))
        n1 = int(np.exp(rng.uniform(0.0, np.log(1200.0))))
        top = min(384, int(max_macs // (K * n1)))
        if top >= 1:
            out.append((int(rng.integers(1, top + 1)), K, n1))
    return out


@pytest.mark.parametrize("kind", ["zp", "mx", "mxw"])
def test_gemm_random_shapes(iq, O, S, kind):
    """The three consumers over seeded shapes, each against the oracle's
    exact sum within the FP32 bound."""
    seed = {"zp": 8100, "mx": 8200, "mxw": 8300}[kind]
    shapes = gemm_shapes(seed, 256 if kind == "zp" else 128, max_macs=20e6 if kind == "mx" else 60e6)
    for i, (n0, K, n1) in enumerate(shapes):
        what = f"{kind} {n0}x{K}x{n1} (seed {seed}, case {i})"
        if kind == "zp":
            zp_gemm_case(iq, O, S, n0, K, n1, seed=seed + i)
            continue
        if kind == "mxw":
            z, zr, zabs = mxw_case(iq, O, S, n0, K, n1, seed=seed + i)
        else:
            rw = mx_operand(O, S, n0, K, seed=seed + i, sigma=0.02, outlier_axis=S.AXIS_ROWS)
            ra = mx_operand(O, S, n1, K, seed=seed + 50 + i, sigma=1.0, outlier_axis=S.AXIS_COLS)
            z = iq.mx_gemm(mx_gpu(iq, rw, n0, K), mx_gpu(iq, ra, n1, K)).cpu().numpy().astype(np.float64)
            zr, zabs = O.mx_gemm(rw["codes"], rw["scales"], ra["codes"], ra["scales"])
        bound = (K + 2) * 2.0 ** -24 * zabs + 1e-30
        err = np.abs(z - zr)
        assert np.all(err <= bound), f"{what}: max err/bound {np.max(err / bound):.3g}"


@pytest.mark.parametrize("fmt,gran", ALL)
def test_parity_bf16_xhat(iq, O, S, fmt, gran):
    x = make_input(S, 1, 64, 4096, None, seed=7)
    g = run_gpu(iq, x, fmt, gran, xhat="bf16")
    r = oracle_ref(O, x, fmt, gran)
    compare(g, r, fmt, f"{fmt}/{gran} bf16 xhat", O, S, xhat="bf16")


# ---- special values and degenerate units --------------------------------------
def bf16_special_matrix(S, rows=16, cols=512, seed=3):
    x = S.fill(rows, cols, 1, sigma=1.0, seed=seed)
    rng = np.random.default_rng(seed)
    x[0] = 0                                                       # all zero
    x[1] = 0x8000                                                  # all -0
    x[2] = rng.integers(1, 0x80, cols) | (rng.integers(0, 2, cols) << 15)   # BF16 subnormals
    x[3] = S.f32_to_bf16_bits((rng.standard_normal(cols) * 1e-30).astype(np.float32))  # tiny scale
    x[4] = S.f32_to_bf16_bits((rng.standard_normal(cols) * 1e30).astype(np.float32))   # huge values
    x[5, ::37] = 0x7FC0                                            # NaN
    x[6, ::41] = 0x7F80                                            # +Inf
    x[6, 5::41] = 0xFF80                                           # -Inf
    x[7, ::3] = 0x7F7F                                             # max finite
    x[8, :] = 0x7FC0                                               # all NaN
    x[9, 17] = 0xFFC1                                              # negative NaN with payload
    x[10, :] = S.f32_to_bf16_bits((rng.standard_normal(cols) * 1e-38).astype(np.float32))
    x[11, 3::7] = 0x8000
    x[11, 4::7] = 0x0000
    x[12, :] = S.f32_to_bf16_bits((rng.standard_normal(cols) * 2.0 ** -125).astype(np.float32))
    x[13, 100:] = 0                                                # mostly zero
    return x


def f32_special_matrix(S, rows=16, cols=512, seed=4):
    x = S.fill(rows, cols, 0, sigma=1.0, seed=seed)
    rng = np.random.default_rng(seed)
    x[0] = 0.0
    x[1] = -0.0
    x[2] = (rng.integers(1, 1 << 20, cols).astype(np.uint32) | (rng.integers(0, 2, cols).astype(np.uint32) << 31)).view(np.float32)
    x[3] = (rng.standard_normal(cols) * 1e-30).astype(np.float32)
    x[4] = (rng.standard_normal(cols) * 1e36).astype(np.float32)
    x[5, ::37] = np.nan
    x[6, ::41] = np.inf
    x[6, 5::41] = -np.inf
    x[7, ::3] = np.float32(3.4028235e38)
    x[8, :] = np.nan
    x[10, :] = (rng.standard_normal(cols) * 1e-41).astype(np.float32)
    x[12, :] = (rng.standard_normal(cols) * 2.0 ** -126).astype(np.float32)
    x[13, 100:] = 0.0
    return x


@pytest.mark.parametrize("dtype", [1, 0], ids=["bf16", "f32"])
@pytest.mark.parametrize("fmt,gran", ALL)
def test_parity_special_values(iq, O, S, fmt, gran, dtype):
    x = bf16_special_matrix(S) if dtype else f32_special_matrix(S)
    if gran == "tensor" or fmt == "nvfp4":
        # per-tensor scales: check with and without the non-finite rows
        cases = [x, np.ascontiguousarray(np.delete(x, [5, 6, 8, 9], axis=0))]
    else:
        cases = [x]
    for k, xc in enumerate(cases):
        g = run_gpu(iq, xc, fmt, gran)
        r = oracle_ref(O, xc, fmt, gran)
        compare(g, r, fmt, f"{fmt}/{gran} special case {k}", O)


@pytest.mark.parametrize("fmt,gran", ALL)
def test_parity_ties(iq, O, S, fmt, gran):
    """Inputs on the midpoints between grid values, where round-to-nearest-even decides."""
    rows, cols = 4, 1024
    x = np.zeros((rows, cols), np.float32)
    rng = np.random.default_rng(5)
    if fmt in ("int8",):
        top, mids = 127.0, np.arange(-127, 127) + 0.5
    elif fmt in ("e4m3", "e5m2"):
        kind = O.K_E4M3 if fmt == "e4m3" else O.K_E5M2
        vals = np.unique(O.fp_decode_array(kind, np.arange(0x7C if fmt == "e5m2" else 0x7F)))
        mids = (vals[:-1] + vals[1:]) / 2
        mids = np.concatenate([mids, -mids])
        top = vals.max()
    elif fmt == "int4":
        top, mids = 7.0, np.arange(-7, 7) + 0.5
    else:
        vals = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
        mids = (vals[:-1] + vals[1:]) / 2
        mids = np.concatenate([mids, -mids])
        top = 6.0
    for r in range(rows):
        x[r] = rng.choice(mids, cols).astype(np.float32)
        if fmt == "int4":
            x[r, ::128] = top                    # every group's maximum gives s = 1
        elif fmt == "mxfp4":
            x[r, ::32] = 4.0                     # floor(log2 4) - 2 = 0: s = 1
        elif fmt == "nvfp4":
            x[r, ::16] = 6.0                     # block max 6
        else:
            x[r, 0] = top                        # alpha = top: s = 1
    if fmt == "nvfp4":
        x[0, 0] = 2688.0                         # s_global = 1, so t = 1 and s_nv = 1 elsewhere
    for dtype in (0, 1):
        xi = x if dtype == 0 else S.f32_to_bf16_bits(x)
        g = run_gpu(iq, xi, fmt, gran)
        rr = oracle_ref(O, xi, fmt, gran)
        compare(g, rr, fmt, f"{fmt}/{gran} ties dtype {dtype}", O)


@pytest.mark.parametrize("fmt,gran", ALL)
def test_empty(iq, O, fmt, gran):
    import torch
    cols = 256
    x = torch.zeros((0, cols), dtype=torch.bfloat16, device="cuda:0")
    q = iq.quantize(x, fmt, gran, xhat_dtype=torch.float32)
    torch.cuda.synchronize()
    st = q.stats()
    assert st["n"] == 0 and st["sum_err2"] == 0.0 and st["n_saturated"] == 0
    if gran == "tensor":
        assert q.scales.cpu().item() == 0.0
    if fmt == "nvfp4":
        assert q.global_scale.cpu().item() == 0.0
    d = iq.dequantize(q)
    assert d.shape == (0, cols)


def test_determinism(iq, S):
    import torch
    x = to_device(S.make("c4", nrows=512))
    outs = []
    for _ in range(2):
        q = iq.quantize(x, "nvfp4", "block", xhat_dtype=torch.float32)
        torch.cuda.synchronize()
        outs.append((q.codes.cpu(), q.scales.cpu(), q.xhat.cpu(), q.stats()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(outs[0][2].view(torch.int32), outs[1][2].view(torch.int32))
    assert outs[0][3] == outs[1][3]


# ---- dequantize (separate call) -------------------------------------------------
def dev_raw(a):
    """Upload an array's raw bytes (codes, scales, shifts) as a device tensor
    of the same element size."""
    import torch
    a = np.ascontiguousarray(a)
    view = {1: np.uint8, 2: np.int16, 4: np.float32}[a.dtype.itemsize]
    return torch.from_numpy(a.view(view)).to("cuda:0")


def oracle_quantized(iq, r, fmt, gran, rows, cols):
    """The oracle's codes and scales as the binding's Quantized (device copies)."""
    gs = dev_raw(r["global_scale"]) if fmt == "nvfp4" else None
    sh = dev_raw(r["shifts"]) if fmt == "int4zp" else None
    return iq.Quantized(dev_raw(r["codes"]), dev_raw(r["scales"]), gs, None, None, fmt, gran, rows, cols, sh)


def check_dequantize(iq, O, S, x, fmt, gran, what, flags=0):
    """GPU dequantize of the oracle's codes and scales: FP32 equals the
    oracle's x^ (the fused x^ of the quantizer), BF16 its RNE."""
    import torch
    rows, cols = x.shape
    r = O.quantize(x, fmt, gran, flags=flags, want_xhat=True, threads=THREADS)
    q = oracle_quantized(iq, r, fmt, gran, rows, cols)
    for dt in (torch.float32, torch.bfloat16):
        d = iq.dequantize(q, dt)
        torch.cuda.synchronize()
        got = d.cpu().numpy() if dt == torch.float32 else d.cpu().view(torch.int16).numpy().view(np.uint16)
        want = r["xhat"] if dt == torch.float32 else S.f32_to_bf16_bits(r["xhat"])
        assert_bits_equal(got, want, f"{what} dequantize {dt}")
        del d
    del q


@pytest.mark.parametrize("fmt,gran", ALL)
def test_dequantize_parity(iq, O, S, fmt, gran):
    """Power-of-two (2048 columns) and non-power-of-two (768 columns: 96
    chunks per row) row lengths."""
    for i, cols in enumerate((2048, 768)):
        x = make_input(S, 1, 48, cols, None, seed=11 + i)
        check_dequantize(iq, O, S, x, fmt, gran, f"{fmt}/{gran} 48x{cols}")


@pytest.mark.parametrize("cfg,fmt,gran", [("c1", "int8", "tensor"), ("c1", "e4m3", "tensor"), ("c2", "e4m3", "row"),
                                          ("c2", "e5m2", "row"), ("c3", "mxfp4", "block"), ("c4", "nvfp4", "block"),
                                          ("c5", "int4", "block"), ("c5", "int4zp", "block")])
def test_dequantize_full_size(iq, O, S, cfg, fmt, gran):
    check_dequantize(iq, O, S, S.make(cfg), fmt, gran, f"{cfg} {fmt}/{gran} full size")


def test_amax(iq, O, S):
    for dtype in (1, 0):
        x = bf16_special_matrix(S) if dtype else f32_special_matrix(S)
        a = iq.amax(to_device(x)).cpu().item()
        assert np.float32(a) == np.float32(O.amax(x))


# ---- division strategy: every BF16 input against many scales ---------------------
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2", "int8"])
def test_bf16_division_sweep(iq, O, S, fmt):
    """Rows [alpha, every BF16 value with |x| <= alpha]: the per-row scale is
    alpha / FMAX, and every BF16 input passes the divide + cast path."""
    allv = np.arange(0x10000, dtype=np.uint32)
    fin = allv[((allv & 0x7FFF) < 0x7F80)].astype(np.uint16)
    alphas = np.arange(0x0080, 0x7F80, 61, dtype=np.uint16)       # ~500 alphas over the normal range
    mag = widen(fin)
    cols = 66 * 1024
    x = np.zeros((len(alphas), cols), np.uint16)
    for i, a in enumerate(alphas):
        av = widen(np.array([a], np.uint16))[0]
        keep = fin[np.abs(mag) <= av]
        row = np.concatenate([[a], keep])
        x[i, :len(row)] = row
    g = run_gpu(iq, x, fmt, "row", xhat=None)
    r = O.quantize(x, fmt, "row", want_xhat=False, threads=THREADS)
    assert_bits_equal(g["codes"], r["codes"], f"{fmt} sweep codes")
    assert_bits_equal(g["scales"], r["scales"], f"{fmt} sweep scales")
    assert_stats_match(g["stats"], r["stats"], f"{fmt} sweep")


def division_rows_8192(step=8):
    """Rows of exactly 8192 BF16 columns for every `step`-th normal BF16
    absmax alpha: each row starts with alpha and holds BF16 values of
    magnitude <= alpha (both signs, zeros included); the values of one alpha
    fill as many rows as they need, the last one padded with +0."""
    alphas = np.arange(0x0080, 0x7F80, step, dtype=np.uint32)
    per = 8191
    counts = [(2 * (int(a) + 1) + per - 1) // per for a in alphas]
    x = np.zeros((sum(counts), 8192), np.uint16)
    r = 0
    for a, nrows in zip(alphas, counts):
        mags = np.arange(int(a) + 1, dtype=np.uint32)
        vals = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
        body = np.zeros(nrows * per, np.uint16)
        body[:vals.size] = vals
        x[r:r + nrows, 0] = a
        x[r:r + nrows, 1:] = body.reshape(nrows, per)
        r += nrows
    return x


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2", "int8"])
def test_bf16_division_sweep_8192(iq, O, S, fmt):
    """Every 8th normal BF16 absmax with every BF16 input at or below it,
    in rows of 8192 columns: the per-row kernel the bench times (4 chunks
    per lane, full rows, no x^) and its scale derivation, with and without
    statistics, and the x^-writing kernel."""
    x = division_rows_8192()
    xd = to_device(x)
    r = O.quantize(x, fmt, "row", want_xhat=True, threads=THREADS)
    for xhat, stats in ((None, True), (None, False), ("f32", True)):
        g = run_gpu(iq, None, fmt, "row", xhat=xhat, stats=stats, x_dev=xd)
        compare(g, r, fmt, f"{fmt} 8192-column sweep stats={stats} xhat={xhat}")
        del g
    del xd


@pytest.mark.parametrize("fmt,flags", [("int4", 0), ("nvfp4", 0), ("mxfp4", 0), ("nvfp4", 4), ("mxfp4", 1),
                                       ("mxfp4", 2), ("int4zp", 0)],
                         ids=["int4", "nvfp4", "mxfp4", "nvfp4-rne", "mxfp4-nearest", "mxfp4-up", "int4zp"])
def test_bf16_block_sweep(iq, O, S, fmt, flags):
    """Blocks whose maximum walks the BF16 range while the other elements take
    every BF16 magnitude at or below it."""
    B = {"int4": 128, "int4zp": 128, "nvfp4": 16, "mxfp4": 32}[fmt]
    rng = np.random.default_rng(17)
    rows, cols = 256, 8192
    nb = cols // B
    tops = rng.integers(0x0080, 0x7F80, (rows, nb)).astype(np.uint32)
    te = np.repeat(tops, B, axis=1)
    mags = (rng.random((rows, cols)) * (te + 1)).astype(np.uint32)          # any BF16 magnitude <= top
    signs = rng.integers(0, 2, (rows, cols)).astype(np.uint32) << 15
    x = (np.minimum(mags, te) | signs).astype(np.uint16)
    pos = rng.integers(0, B, (rows, nb)) + np.arange(nb) * B                 # one element per block = top
    np.put_along_axis(x, pos, tops.astype(np.uint16), axis=1)
    if fmt == "nvfp4":
        x[0, 0] = 0x7F7F
    g = run_gpu(iq, x, fmt, "block", flags=flags)
    rr = oracle_ref(O, x, fmt, "block", flags=flags)
    compare(g, rr, fmt, f"{fmt} block sweep flags={flags}", O)


# ---- the five workloads at full size (the configuration the bench times) ----------
FULL = [("c1", "int8", "tensor", 0), ("c1", "e4m3", "tensor", 0), ("c2", "e4m3", "row", 0),
        ("c2", "e5m2", "row", 0), ("c3", "mxfp4", "block", 0), ("c4", "nvfp4", "block", 0),
        ("c5", "int4", "block", 0), ("c3", "mxfp4", "block", 1), ("c3", "mxfp4", "block", 2),
        ("c4", "nvfp4", "block", 4), ("c5", "int4zp", "block", 0)]


@pytest.mark.parametrize("cfg,fmt,gran,flags", FULL)
def test_full_size_workloads(iq, O, S, cfg, fmt, gran, flags):
    """The kernels the bench times (no x^) with statistics on and off, and
    the x^-writing kernels, element by element against the oracle."""
    x = S.make(cfg)
    xd = to_device(x)
    r = O.quantize(x, fmt, gran, flags=flags, want_xhat=True, threads=THREADS)
    for xhat, stats in ((None, True), (None, False), ("f32", True)):
        g = run_gpu(iq, None, fmt, gran, xhat=xhat, flags=flags, stats=stats, x_dev=xd)
        compare(g, r, fmt, f"{cfg} {fmt}/{gran} flags={flags} full size stats={stats} xhat={xhat}", O)
        del g
    del xd


FLAT = [f for f in ALL if f[1] != "row"]


def saturating_alpha(fmt):
    """A BF16 absmax alpha whose per-tensor scale s = RN(alpha / Q) puts
    RN(alpha / s) above Q, so the elements equal to alpha saturate."""
    Q = {"int8": 127.0, "e4m3": 448.0, "e5m2": 57344.0}[fmt]
    for bits in range(0x4000, 0x4800):                  # BF16 values in [2, 2^17)
        a = np.float32(np.array([bits << 16], np.uint32).view(np.float32)[0])
        s = np.float32(a / np.float32(Q))
        if np.float32(a / s) > np.float32(Q):
            return a
    raise AssertionError("no saturating absmax found")


@pytest.mark.parametrize("fmt", ["int8", "e4m3", "e5m2"])
def test_tensor_rows_special_and_saturating(iq, O, S, fmt):
    """Per-tensor INT8 / FP8 of BF16 tensors of 16384 elements, which the
    library quantizes as rows of 16384 under the tensor's scale: the special
    values (NaN and +-Inf send the whole tensor to the general path), the
    rows without the non-finite and huge ones (zeros, subnormals and tiny
    values on the fast path), and a tensor whose absmax saturates under its
    own scale (two elements at +-alpha), each against the oracle."""
    x = bf16_special_matrix(S, rows=32, cols=512)
    assert x.size % 16384 == 0
    # without the non-finite and the huge rows: the fast path, with exact zeros, -0, subnormals and tiny values
    finite = np.concatenate([np.delete(x, [4, 5, 6, 7, 8, 9], axis=0), S.fill(6, 512, 1, sigma=1.0, seed=9)], axis=0)
    alpha = saturating_alpha(fmt)
    sat = S.fill(2, 16384, 1, sigma=float(alpha) / 8, seed=10)
    abits = int(np.array([alpha], np.float32).view(np.uint32)[0] >> 16)
    mag = sat & 0x7FFF
    sat[mag > abits] = (sat[mag > abits] & 0x8000) | abits   # clip to |x| <= alpha
    sat[0, 7] = abits
    sat[1, 9000] = abits | 0x8000
    for k, xc in enumerate((x, finite, sat)):
        g = run_gpu(iq, np.ascontiguousarray(xc), fmt, "tensor", xhat=None)
        r = oracle_ref(O, np.ascontiguousarray(xc), fmt, "tensor")
        compare(g, r, fmt, f"{fmt}/tensor rows case {k}", O)
        if k == 2:
            assert r["stats"]["n_saturated"] >= 2


@pytest.mark.parametrize("fmt,gran", FLAT)
def test_many_tiles_ragged(iq, O, S, fmt, gran):
    """The flat kernels with many tiles per workgroup and a ragged last
    tile (BF16 2500 x 8448: 2578 full tiles of 1024 chunks and one of 128),
    so the persistent loop runs its in-flight buffers down to a partial
    tile: with and without statistics, and with x^."""
    x = make_input(S, 1, 2500, 8448, None, seed=77)
    assert (2500 * 8448 // 8) % 1024 == 128
    xd = to_device(x)
    r = oracle_ref(O, x, fmt, gran)
    for xhat, stats in ((None, True), (None, False), ("f32", False)):
        g = run_gpu(iq, None, fmt, gran, xhat=xhat, stats=stats, x_dev=xd)
        compare(g, r, fmt, f"{fmt}/{gran} 2500x8448 stats={stats} xhat={xhat}", O)
        del g
    del xd


@pytest.fixture(scope="module")
def stream_input(S):
    """The 2 GiB streaming workload, on the host and the device."""
    x = S.make("stream")
    yield x, to_device(x)


@pytest.mark.parametrize("fmt,gran", [("int8", "tensor"), ("e4m3", "tensor"), ("e4m3", "row"), ("e5m2", "row"),
                                      ("mxfp4", "block"), ("nvfp4", "block"), ("int4", "block")])
def test_stream_every_row(iq, O, S, stream_input, fmt, gran):
    """The 2 GiB streaming workload in every format: every code and scale and
    the statistics against the oracle over the whole tensor; the call
    without statistics gives the same codes and scales."""
    x, xd = stream_input
    r = O.quantize(x, fmt, gran, want_xhat=False, threads=THREADS)
    for stats in (True, False):
        g = run_gpu(iq, None, fmt, gran, xhat=None, stats=stats, x_dev=xd)
        compare(g, r, fmt, f"stream {fmt}/{gran} stats={stats}")
        del g
    del r


# ---- graph capture: replays match eager calls -------------------------------------
@pytest.mark.parametrize("fmt,gran", [("e4m3", "row"), ("e4m3", "tensor"), ("nvfp4", "block"), ("int4", "block"),
                                      ("int4zp", "block")])
def test_graph_replay_matches_eager(iq, S, fmt, gran):
    """The library enqueues only kernels (no memset nodes), so a captured call
    replays to the same bytes every time, also with eager work in between."""
    import torch
    x = to_device(S.make("c4", nrows=256))
    ws = iq.workspace_for(iq.desc_for(x, fmt, gran), x.device)
    ref = iq.quantize(x, fmt, gran, xhat_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    want = (ref.codes.cpu(), ref.scales.cpu(), ref.xhat.cpu(), ref.stats())
    out = iq.quantize(x, fmt, gran, xhat_dtype=torch.float32, workspace=ws)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        iq.quantize(x, fmt, gran, workspace=ws, out=out)
    for rep in range(4):
        out.codes.zero_(); out.scales.zero_(); out.xhat.zero_(); out.stats_buf.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (out.codes.cpu(), out.scales.cpu(), out.xhat.cpu(), out.stats())
        assert torch.equal(got[0], want[0]) and torch.equal(got[1], want[1]), rep
        assert torch.equal(got[2].view(torch.int32), want[2].view(torch.int32)), rep
        assert got[3] == want[3], rep
        iq.quantize(x, "mxfp4", "block", workspace=ws)     # eager work on the same workspace between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("n1", [1, 24, 64, 100, 256])
def test_gemm_repeat_bit_identical(iq, O, S, n1):
    """Every consumer path returns the same bits on every call, on a
    1024-row grid over five calls with other work between them: the INT4
    k split (atomic adds: the 64-token tile adding directly at 64 tokens,
    the 128-token tile row by row at 100, the 256-token tile directly at
    256), the W4A16 and FP4 64-row tiles and the few-token kernels."""
    import torch
    n0, K = 1024, 1024
    rzp = O.quantize((S.bf16_to_f32(S.make("c5", nrows=n0))[:, :K]).copy(), "int4zp", "block")
    qzp = iq.Quantized(to_device(rzp["codes"]), to_device(rzp["scales"]), None, None, None, "int4zp", "block",
                       n0, K, to_device(rzp["shifts"]))
    qw = mx_gpu(iq, mx_operand(O, S, n0, K, seed=51, sigma=0.02, outlier_axis=S.AXIS_ROWS), n0, K)
    qa = mx_gpu(iq, mx_operand(O, S, n1, K, seed=52, sigma=1.0, outlier_axis=S.AXIS_COLS), n1, K)
    x = to_device(S.make("c2", nrows=n1)[:, :K].copy())
    calls = (lambda: iq.zp_gemm(qzp, x), lambda: iq.mxw_gemm(qw, x), lambda: iq.mx_gemm(qw, qa))
    first = [c().cpu().view(torch.int32) for c in calls]
    for rep in range(4):
        iq.quantize(x, "e4m3", "row", stats=True)         # other work on the stream between the calls
        for c, want in zip(calls, first):
            assert torch.equal(c().cpu().view(torch.int32), want), rep


@pytest.mark.parametrize("off", [1, 2, 3])
def test_gemm_split_output_offsets(iq, O, S, off):
    """An INT4 call whose k is split zeroes z first, with 16-byte stores from
    the first 16-byte boundary and single floats around them, then adds row
    by row; the W4A16 call (64-row tiles) writes z directly.  Either way an
    output 4, 8 or 12 bytes past a boundary gets the bits of an aligned
    output, and the floats just before and after it keep their values."""
    import torch
    n0, K, n1 = 96, 512, 300                       # small grid: INT4 splits k (128-token tiles)
    rzp = O.quantize((S.bf16_to_f32(S.make("c5", nrows=n0))[:, :K]).copy(), "int4zp", "block")
    qzp = iq.Quantized(to_device(rzp["codes"]), to_device(rzp["scales"]), None, None, None, "int4zp", "block",
                       n0, K, to_device(rzp["shifts"]))
    qw = mx_gpu(iq, mx_operand(O, S, n0, K, seed=41, sigma=0.02, outlier_axis=S.AXIS_ROWS), n0, K)
    x = to_device(S.make("c2", nrows=n1)[:, :K].copy())
    sentinel = 0x7FC0BEEF
    for name, call in (("zp", lambda out=None: iq.zp_gemm(qzp, x, out=out)),
                       ("mxw", lambda out=None: iq.mxw_gemm(qw, x, out=out))):
        want = call().cpu()
        buf = torch.full((n0 * n1 + 8,), sentinel, dtype=torch.int32, device="cuda:0")
        out = buf[off:off + n0 * n1].view(torch.float32).view(n0, n1)
        call(out)
        torch.cuda.synchronize()
        b = buf.cpu()
        assert torch.equal(b[off:off + n0 * n1], want.view(torch.int32).reshape(-1)), name
        assert bool((b[:off] == sentinel).all()) and bool((b[off + n0 * n1:] == sentinel).all()), name


@pytest.mark.parametrize("n1", [16, 300])
def test_gemm_graph_replay_matches_eager(iq, O, S, n1):
    """The GEMMs (their few-token and their tiled kernels) add in a fixed
    order, so a captured call replays to the eager call's exact bits, also
    with eager work in between."""
    import torch
    K = 512
    rzp = O.quantize((S.bf16_to_f32(S.make("c5", nrows=96))[:, :K]).copy(), "int4zp", "block")
    qzp = iq.Quantized(to_device(rzp["codes"]), to_device(rzp["scales"]), None, None, None, "int4zp", "block",
                       96, K, to_device(rzp["shifts"]))
    x = to_device(S.make("c2", nrows=n1)[:, :K].copy())
    rw = mx_operand(O, S, 96, K, seed=31, sigma=0.02, outlier_axis=S.AXIS_ROWS)
    ra = mx_operand(O, S, n1, K, seed=32, sigma=1.0, outlier_axis=S.AXIS_COLS)
    qw, qa = mx_gpu(iq, rw, 96, K), mx_gpu(iq, ra, n1, K)
    want_zp, want_mx, want_w = iq.zp_gemm(qzp, x), iq.mx_gemm(qw, qa), iq.mxw_gemm(qw, x)
    torch.cuda.synchronize()
    want_zp, want_mx, want_w = want_zp.cpu(), want_mx.cpu(), want_w.cpu()
    out_zp = torch.empty((96, n1), dtype=torch.float32, device="cuda:0")
    out_mx = torch.empty((96, n1), dtype=torch.float32, device="cuda:0")
    out_w = torch.empty((96, n1), dtype=torch.float32, device="cuda:0")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        iq.zp_gemm(qzp, x, out=out_zp)
        iq.mx_gemm(qw, qa, out=out_mx)
        iq.mxw_gemm(qw, x, out=out_w)
    for rep in range(4):
        out_zp.zero_(); out_mx.zero_(); out_w.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_zp.cpu().view(torch.int32), want_zp.view(torch.int32)), rep
        assert torch.equal(out_mx.cpu().view(torch.int32), want_mx.view(torch.int32)), rep
        assert torch.equal(out_w.cpu().view(torch.int32), want_w.view(torch.int32)), rep
        iq.mx_gemm(qw, qa)                                   # eager work between replays
        torch.cuda.synchronize()


# ---- one workspace across many calls ------------------------------------------------
def test_workspace_reuse_across_calls(iq, O, S):
    """One workspace serves a sequence of calls with different grids, formats,
    the absmax pre-pass and calls without statistics in between; every call's
    outputs and statistics still match the oracle."""
    import torch
    plan = [("c2", 96, "e4m3", "row"), ("c4", 128, "nvfp4", "block"), ("c1", 64, "int8", "tensor"),
            ("c3", 64, "mxfp4", "block"), ("c5", 32, "int4", "block"), ("c2", 3, "e5m2", "row"),
            ("c1", 1, "e4m3", "tensor"), ("c2", 96, "e4m3", "row")]
    ws = None
    for name, nrows, fmt, gran in plan:
        x_np = S.make(name, nrows=nrows)
        x = to_device(x_np)
        if ws is None:
            ws = iq.workspace_for(iq.desc_for(x, fmt, gran), x.device)
        iq.quantize(x, fmt, gran, stats=False, workspace=ws)          # a call without statistics in between
        a = iq.amax(x, workspace=ws)
        q = iq.quantize(x, fmt, gran, xhat_dtype=torch.float32, workspace=ws)
        torch.cuda.synchronize()
        ref = oracle_ref(O, x_np, fmt, gran)
        what = f"{name}[{nrows}] {fmt}/{gran} on a shared workspace"
        assert np.float32(a.cpu().item()) == np.float32(O.amax(x_np)), what
        g = {"codes": q.codes.cpu().numpy(), "scales": q.scales.cpu().numpy(), "stats": q.stats(),
             "xhat": q.xhat.cpu().numpy()}
        if q.global_scale is not None:
            g["global_scale"] = q.global_scale.cpu().numpy()
        compare(g, ref, fmt, what)


# ---- tiny magnitudes: global and block scales near the bottom of the range ------------
@pytest.mark.parametrize("fmt,gran", ALL)
@pytest.mark.parametrize("shift", [60, 100, 118, 126, 130])
def test_tiny_magnitudes(iq, O, S, fmt, gran, shift):
    """The activation workload scaled by 2^-shift (BF16, subnormals included):
    quotients and scales that leave the normal range take the correctly
    rounded divisions; every output still matches the oracle."""
    x32 = S.bf16_to_f32(S.make("c2", nrows=48)) * np.float32(2.0 ** -shift)
    x = S.f32_to_bf16_bits(x32.astype(np.float32))
    g = run_gpu(iq, x, fmt, gran)
    r = oracle_ref(O, x, fmt, gran)
    compare(g, r, fmt, f"{fmt}/{gran} x 2^-{shift}", O)


# ---- INT4: group maxima whose A / 7 is an exact FP16 tie ---------------------------------
@pytest.mark.parametrize("dtype", [0, 1], ids=["f32", "bf16"])
def test_int4_fp16_scale_ties(iq, O, S, dtype):
    """Every group's maximum is 7 * m with m halfway between two FP16 values,
    so A / 7 = m exactly and the FP16 scale is decided by ties-to-even after
    the FP32 quotient (a fused fma-to-FP16 would round once and differ)."""
    rng = np.random.default_rng(23)
    rows, cols = 64, 1024
    ng = cols // 128
    k = rng.integers(0, 1024, (rows, ng))
    e = rng.integers(-10, 12, (rows, ng))
    m = (1.0 + (2 * k + 1) / 2048.0) * np.exp2(e)              # FP16 midpoints (12 significant bits)
    A = (7.0 * m).astype(np.float32)                          # exact: 15 significant bits
    if dtype:                                                 # BF16 keeps 8 bits: use maxima it can hold
        A = S.bf16_to_f32(S.f32_to_bf16_bits(A))
    x = (rng.standard_normal((rows, cols)) * 0.3).astype(np.float32) * np.repeat(A, 128, axis=1) / 4
    x = np.clip(x, -np.repeat(A, 128, axis=1), np.repeat(A, 128, axis=1)).astype(np.float32)
    pos = rng.integers(0, 128, (rows, ng)) + np.arange(ng) * 128
    np.put_along_axis(x, pos, A * np.where(rng.random((rows, ng)) < 0.5, -1, 1).astype(np.float32), axis=1)
    if dtype:
        x = S.f32_to_bf16_bits(x)
    g = run_gpu(iq, x, "int4", "block")
    r = oracle_ref(O, x, "int4", "block")
    compare(g, r, "int4", f"int4 FP16 scale ties ({'bf16' if dtype else 'f32'})", O)


# ---- scale-rule variants (iq_desc.flags) ------------------------------------------
RULES = [("mxfp4", 1), ("mxfp4", 2), ("nvfp4", 4)]
RULE_IDS = ["mx-nearest", "mx-up", "nv-rne"]


@pytest.mark.parametrize("fmt,flags", RULES, ids=RULE_IDS)
@pytest.mark.parametrize("dtype", [1, 0], ids=["bf16", "f32"])
def test_rule_variant_parity(iq, O, S, fmt, flags, dtype):
    """Each rule variant over the multi-tile shapes, the special-value matrix
    and the activation workload scaled toward the bottom of the range."""
    bs = O.block_size(fmt, "block")
    for i, (rows, cols, ld) in enumerate(SHAPES):
        if cols % bs:
            continue
        x = make_input(S, dtype, rows, cols, ld, seed=300 + i)
        c = cols if ld else None
        g = run_gpu(iq, x, fmt, "block", cols=c, flags=flags)
        r = oracle_ref(O, x, fmt, "block", cols=c, flags=flags)
        compare(g, r, fmt, f"{fmt} flags={flags} {rows}x{cols} ld={ld}", O)
    x = bf16_special_matrix(S) if dtype else f32_special_matrix(S)
    cases = [x, np.ascontiguousarray(np.delete(x, [5, 6, 8, 9], axis=0))]
    for k, xc in enumerate(cases):
        g = run_gpu(iq, xc, fmt, "block", flags=flags)
        r = oracle_ref(O, xc, fmt, "block", flags=flags)
        compare(g, r, fmt, f"{fmt} flags={flags} special case {k}", O)
    for shift in (100, 126, 130):
        x32 = S.bf16_to_f32(S.make("c2", nrows=16)) * np.float32(2.0 ** -shift)
        x = S.f32_to_bf16_bits(x32.astype(np.float32)) if dtype else x32.astype(np.float32)
        g = run_gpu(iq, x, fmt, "block", flags=flags)
        r = oracle_ref(O, x, fmt, "block", flags=flags)
        compare(g, r, fmt, f"{fmt} flags={flags} x 2^-{shift}", O)


@pytest.mark.parametrize("flags", [0, 1, 2], ids=["floor", "nearest", "up"])
def test_mx_exponent_rule_boundaries(iq, O, S, flags):
    """FP32 block maxima whose significand sits on, or next to, the point
    where each exponent rule changes its answer (3*sqrt(2)/4 for the nearest
    rule, 3/2 for the round-up rule, the binade ends for the default), with
    exponents over the whole FP32 range, subnormals included."""
    rng = np.random.default_rng(41)
    rows, cols = 64, 2048
    nb = cols // 32
    mants = np.array([0x0, 0x1, 0x07C3B5, 0x07C3B6, 0x07C3B7, 0x07C3B8, 0x3FFFFF, 0x400000, 0x400001,
                      0x7FFFFE, 0x7FFFFF], np.uint32)
    m = rng.choice(mants, (rows, nb))
    e = rng.integers(0, 255, (rows, nb)).astype(np.uint32)       # 0: subnormal maxima
    e[:, :8] = np.arange(0, 8, dtype=np.uint32)                  # the bottom of the range on every row
    e[:, 8:12] = np.arange(251, 255, dtype=np.uint32)            # and the top
    m[e == 0] |= 1                                               # keep subnormal maxima nonzero
    tops = ((e << 23) | m).astype(np.uint32).view(np.float32)
    te = np.repeat(tops, 32, axis=1)
    x = (te * rng.random((rows, cols)).astype(np.float32)).astype(np.float32)
    x *= np.where(rng.random((rows, cols)) < 0.5, -1, 1).astype(np.float32)
    pos = rng.integers(0, 32, (rows, nb)) + np.arange(nb) * 32
    np.put_along_axis(x, pos, tops * np.where(rng.random((rows, nb)) < 0.5, -1, 1).astype(np.float32), axis=1)
    g = run_gpu(iq, x, "mxfp4", "block", flags=flags)
    r = oracle_ref(O, x, "mxfp4", "block", flags=flags)
    compare(g, r, "mxfp4", f"mxfp4 exponent-rule boundaries flags={flags}", O)


@pytest.mark.parametrize("flags", [0, 4], ids=["ceil", "rne"])
def test_nv_block_scale_rounding(iq, O, S, flags):
    """NVFP4 with s_global = 1 (tensor absmax 2688): each block's maximum is
    6 t with t an E4M3 value, a midpoint between two neighbours (below the
    smallest subnormal too), or a few FP32 steps off one, so the rounding
    rule alone decides the block scale code, including code 0 for A > 0."""
    rng = np.random.default_rng(43)
    vals = np.asarray(O.fp_decode_array(O.K_E4M3, np.arange(0x7F)), np.float64)      # 0 .. 448
    mids = (vals[:-1] + vals[1:]) / 2
    targets = []
    for t in np.concatenate([vals[1:], mids]):
        a = np.float32(6.0 * t)                                                       # exact
        for k in (-2, -1, 0, 1, 2):
            b = a
            for _ in range(abs(k)):
                b = np.nextafter(b, np.float32(np.inf) if k > 0 else np.float32(0))
            if 0 < b <= 2688.0:
                targets.append(b)
    targets = np.array(targets, np.float32)
    rows, cols = 64, 1024
    nb = cols // 16
    tops = rng.choice(targets, (rows, nb)).astype(np.float32)
    tops[0, 0] = np.float32(2688.0)
    te = np.repeat(tops, 16, axis=1)
    x = (te * rng.random((rows, cols)).astype(np.float32)).astype(np.float32)
    x *= np.where(rng.random((rows, cols)) < 0.5, -1, 1).astype(np.float32)
    pos = rng.integers(0, 16, (rows, nb)) + np.arange(nb) * 16
    np.put_along_axis(x, pos, tops, axis=1)
    g = run_gpu(iq, x, "nvfp4", "block", flags=flags)
    r = oracle_ref(O, x, "nvfp4", "block", flags=flags)
    assert r["global_scale"][0] == np.float32(1.0)
    compare(g, r, "nvfp4", f"nvfp4 block-scale rounding flags={flags}", O)


# ---- static (calibrated) scaling: iq_quantize_static -------------------------------
STATIC = [("int8", "tensor"), ("e4m3", "tensor"), ("e5m2", "tensor"), ("nvfp4", "block")]


def run_gpu_static(iq, x_np, fmt, gran, alpha, cols=None, xhat="f32"):
    import torch
    x = to_device(x_np)
    if cols is not None:
        x = x[:, :cols]
    a = torch.tensor([alpha], dtype=torch.float32, device=x.device)
    xdt = {"f32": torch.float32, "bf16": torch.bfloat16, None: None}[xhat]
    q = iq.quantize(x, fmt, gran, xhat_dtype=xdt, static_amax=a)
    torch.cuda.synchronize()
    out = {"codes": q.codes.cpu().numpy(), "scales": q.scales.cpu().numpy(), "stats": q.stats(), "q": q}
    if q.global_scale is not None:
        out["global_scale"] = q.global_scale.cpu().numpy()
    if q.xhat is not None:
        out["xhat"] = q.xhat.cpu().numpy()
    return out


def static_alphas(G):
    """Calibrated absmaxes around the data's own G: equal, below (clipping),
    above, tiny, huge, and the invalid values taken as 0."""
    return [G, 0.5 * G, 0.01 * G, 4.0 * G, 1e-30, 1e30, 0.0, -0.0, -1.0, float("nan"), float("inf")]


@pytest.mark.parametrize("dtype", [1, 0], ids=["bf16", "f32"])
@pytest.mark.parametrize("fmt,gran", STATIC)
def test_static_parity(iq, O, S, fmt, gran, dtype):
    """Every calibrated absmax on multi-tile and ragged shapes, and on the
    special-value matrix (non-finite inputs, zeros, subnormals)."""
    for i, (rows, cols, ld) in enumerate(SHAPES):
        if cols % 16:
            continue
        x = make_input(S, dtype, rows, cols, ld, seed=500 + i)
        c = cols if ld else None
        G = float(O.quantize(x, fmt, gran, cols=c, want_xhat=False)["tensor_amax"])
        for alpha in static_alphas(G):
            g = run_gpu_static(iq, x, fmt, gran, alpha, cols=c)
            r = O.quantize(x, fmt, gran, cols=c, static_amax=alpha, threads=THREADS)
            compare(g, r, fmt, f"static {fmt}/{gran} {rows}x{cols} ld={ld} alpha={alpha!r}", O)
    x = bf16_special_matrix(S) if dtype else f32_special_matrix(S)
    for alpha in (1.0, 1e-30, 3e38, float("nan")):
        g = run_gpu_static(iq, x, fmt, gran, alpha)
        r = O.quantize(x, fmt, gran, static_amax=alpha, threads=THREADS)
        compare(g, r, fmt, f"static {fmt}/{gran} special alpha={alpha!r}", O)


@pytest.mark.parametrize("cfg,fmt,gran", [("c1", "int8", "tensor"), ("c1", "e4m3", "tensor"),
                                          ("c4", "nvfp4", "block")])
def test_static_full_size(iq, O, S, cfg, fmt, gran):
    """The per-tensor workloads at full size with a calibrated absmax below
    the data's (outlier columns clip)."""
    x = S.make(cfg)
    G = float(np.max(np.abs(S.bf16_to_f32(x) if x.dtype == np.uint16 else x)))
    alpha = 0.3 * G
    g = run_gpu_static(iq, x, fmt, gran, alpha, xhat=None)
    r = O.quantize(x, fmt, gran, static_amax=alpha, want_xhat=False, threads=THREADS)
    compare(g, r, fmt, f"static {cfg} {fmt}/{gran} full size", O)
    assert r["stats"]["n_saturated"] > 0


@pytest.mark.parametrize("fmt,gran", STATIC)
def test_static_after_amax_equals_dynamic(iq, S, fmt, gran):
    """iq_amax then iq_quantize_static on the same stream reproduces
    iq_quantize bit for bit (codes, scales, x^ and statistics)."""
    import torch
    x = to_device(make_input(S, 1, 96, 4096, None, seed=61))
    a = iq.amax(x)
    qs = iq.quantize(x, fmt, gran, xhat_dtype=torch.float32, static_amax=a)
    qd = iq.quantize(x, fmt, gran, xhat_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(qs.codes, qd.codes) and torch.equal(qs.scales.view(torch.uint8), qd.scales.view(torch.uint8))
    assert torch.equal(qs.xhat.view(torch.int32), qd.xhat.view(torch.int32))
    if fmt == "nvfp4":
        assert torch.equal(qs.global_scale, qd.global_scale)
    assert qs.stats() == qd.stats()


@pytest.mark.parametrize("fmt,gran", STATIC)
def test_static_empty(iq, O, fmt, gran):
    """An empty input still gets the scale derived from the supplied absmax."""
    import torch
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda:0")
    a = torch.tensor([254.0], dtype=torch.float32, device="cuda:0")
    q = iq.quantize(x, fmt, gran, static_amax=a)
    torch.cuda.synchronize()
    r = O.quantize(np.zeros((0, 256), np.uint16), fmt, gran, static_amax=254.0)
    st = q.stats()
    assert st["n"] == 0 and st["sum_x2"] == 0.0
    if gran == "tensor":
        assert np.float32(q.scales.cpu().item()) == r["scales"][0]
    else:
        assert np.float32(q.global_scale.cpu().item()) == r["global_scale"][0]


@pytest.mark.parametrize("fmt,gran", [("e4m3", "tensor"), ("nvfp4", "block")])
def test_static_graph_replay(iq, S, fmt, gran):
    """A captured iq_quantize_static (the calibrated mode a serving loop
    captures) reads its absmax buffer at replay time: refilled before each
    replay, it reproduces the eager bytes, with eager work in between."""
    import torch
    x = to_device(S.make("c4", nrows=256))
    ws = iq.workspace_for(iq.desc_for(x, fmt, gran), x.device)
    a = iq.amax(x)
    ref = iq.quantize(x, fmt, gran, xhat_dtype=torch.float32, workspace=ws, static_amax=a)
    torch.cuda.synchronize()
    want = (ref.codes.cpu(), ref.scales.cpu(), ref.xhat.cpu(), ref.stats())
    a2 = torch.empty_like(a)
    out = iq.quantize(x, fmt, gran, xhat_dtype=torch.float32, workspace=ws, static_amax=a)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        iq.quantize(x, fmt, gran, workspace=ws, out=out, static_amax=a2)
    for rep in range(3):
        out.codes.zero_(); out.scales.zero_(); out.xhat.zero_(); out.stats_buf.zero_()
        a2.copy_(a)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (out.codes.cpu(), out.scales.cpu(), out.xhat.cpu(), out.stats())
        assert torch.equal(got[0], want[0]) and torch.equal(got[1], want[1]), rep
        assert torch.equal(got[2].view(torch.int32), want[2].view(torch.int32)), rep
        assert got[3] == want[3], rep
        a2.fill_(-1.0)                                       # invalid absmax: taken as 0 if replayed now
        iq.quantize(x, "mxfp4", "block", workspace=ws)
        torch.cuda.synchronize()



# ---- asymmetric INT4: groups at the edges of the encoder ----------------------------
@pytest.mark.parametrize("dtype", [0, 1], ids=["f32", "bf16"])
def test_int4zp_edge_groups(iq, O, S, dtype):
    """Groups that are all positive, all negative, constant, all zero, a
    single nonzero, spanning the whole float range (the scale clamps), with
    code ties (sc a power of two, x on half steps) and a shift tie
    (-lo / sc = 7.5), beside weight-like groups."""
    rng = np.random.default_rng(29)
    rows, cols = 32, 2048
    x = S.bf16_to_f32(S.make("c5", nrows=rows))[:, :cols].astype(np.float32).copy()
    x[0, 0:128] = np.abs(x[0, 0:128])
    x[0, 128:256] = -np.abs(x[0, 128:256])
    x[0, 256:384] = np.float32(0.75)
    x[0, 384:512] = 0.0
    x[0, 512:640] = 0.0
    x[0, 600] = np.float32(-3.5)
    x[1, 0:128] = np.float32(3e38) * np.where(rng.random(128) < 0.5, -1, 1).astype(np.float32)
    x[1, 0], x[1, 1] = np.float32(3.3e38), np.float32(-3.3e38)
    half = (np.arange(128) % 15).astype(np.float32) + np.float32(0.5)
    x[2, 0:128] = half * np.float32(2.0 ** -5)              # lo = 0, hi = 14.5 * 2^-5
    x[2, 127] = np.float32(15 * 2.0 ** -5)                  # hi = 15 * 2^-5: sc = 2^-5, ties at k + 0.5
    x[3, 0:128] = np.linspace(-7.5, 7.5, 128, dtype=np.float32)   # sc = 1, -lo / sc = 7.5
    x[3, 128:256] = np.round(np.linspace(-7.5, 7.5, 128) * 2) / 2
    x[4, 0:256] = rng.standard_normal(256).astype(np.float32) * np.float32(2.0 ** -130)   # subnormal range
    if dtype:
        x = S.f32_to_bf16_bits(x)
    g = run_gpu(iq, x, "int4zp", "block")
    r = oracle_ref(O, x, "int4zp", "block")
    compare(g, r, "int4zp", f"int4zp edge groups ({'bf16' if dtype else 'f32'})", O)


# ---- Puzzle 12's consumer: dequantize-then-dot on the matrix cores ------------------
def zp_gemm_case(iq, O, S, n0, K, n1, seed, x_scale=1.0):
    """Weights quantized by the oracle (asymmetric INT4), BF16 activations;
    the GPU result against the oracle's exact sum, within the FP32 bound."""
    import torch
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n0, K)) * 0.02).astype(np.float32)
    w[:, :: 97] *= 30.0                                           # outlier columns
    r = O.quantize(w, "int4zp", "block")
    x = S.f32_to_bf16_bits((rng.standard_normal((n1, K)) * x_scale).astype(np.float32))
    q = iq.Quantized(to_device(r["codes"]), to_device(r["scales"]), None, None, None, "int4zp", "block", n0, K,
                     to_device(r["shifts"]))
    z = iq.zp_gemm(q, to_device(x)).cpu().numpy()
    zr, zabs = O.zp_gemm(r["codes"], r["scales"], r["shifts"], x)
    bound = (K + 2) * 2.0 ** -24 * zabs + 1e-30
    err = np.abs(z.astype(np.float64) - zr)
    assert np.all(err <= bound), f"{n0}x{K}x{n1}: max err/bound {np.max(err / bound):.3g}"
    return err, bound, zr


# n1 <= 32: the few-token kernel (1 or 2 token tiles of 16, stripes of 32
# weight rows up to 8 tokens and of 64 above); up to 64 tokens 64-token
# tiles; above: 128- or
# 256-token tiles, whose k is split in two halves added atomically when the
# tile grid is small (every tiled case here; K = 256 gives each half one group).
@pytest.mark.parametrize("n0,K,n1", [(128, 256, 128), (200, 512, 75), (32, 1024, 300), (1, 256, 1),
                                     (257, 768, 129), (384, 2048, 256), (100, 512, 1), (64, 768, 16),
                                     (300, 1024, 33), (48, 256, 64), (17, 2048, 50), (40, 512, 1100),
                                     (70, 256, 40), (96, 768, 100), (33, 512, 24),
                                     (40, 16896, 1), (40, 16896, 7), (24, 16896, 40), (100, 512, 9),
                                     (130, 16896, 12), (70, 768, 31), (1, 256, 12), (1, 256, 24), (5, 512, 40),
                                     (3, 512, 300)])
def test_zp_gemm_parity(iq, O, S, n0, K, n1):
    err, bound, zr = zp_gemm_case(iq, O, S, n0, K, n1, seed=n0 + K + n1)
    assert np.abs(zr).max() > 0
    assert np.max(err / bound) < 0.05          # the bound is loose; a real fault is not small


def test_zp_gemm_zero_and_empty(iq, O, S):
    import torch
    zp_gemm_case(iq, O, S, 64, 512, 40, seed=3, x_scale=0.0)
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((16, 256)) * 0.02).astype(np.float32)
    r = O.quantize(w, "int4zp", "block")
    q = iq.Quantized(to_device(r["codes"]), to_device(r["scales"]), None, None, None, "int4zp", "block", 16, 256,
                     to_device(r["shifts"]))
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda:0")
    assert iq.zp_gemm(q, x).shape == (16, 0)


def zp_gemm_run(iq, O, S, n0, K, x, seed, w_scale=0.02):
    """Random asymmetric INT4 weights (by the oracle) against the BF16 bits x;
    returns the GPU result and the oracle's exact sum and sum of |terms|."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n0, K)) * w_scale).astype(np.float32)
    r = O.quantize(w, "int4zp", "block")
    q = iq.Quantized(to_device(r["codes"]), to_device(r["scales"]), None, None, None, "int4zp", "block", n0, K,
                     to_device(r["shifts"]))
    z = iq.zp_gemm(q, to_device(x)).cpu().numpy().astype(np.float64)
    zr, zabs = O.zp_gemm(r["codes"], r["scales"], r["shifts"], x)
    return z, zr, zabs


@pytest.mark.parametrize("n1", [5, 130, 300])
def test_zp_gemm_nonfinite_activations(iq, O, S, n1):
    """NaN and +-Inf activations: the non-finite pattern (NaN, and Inf with its
    sign; Inf times a zero weight is NaN) equals the oracle's FP64 sums, and
    every finite output is within the FP32 bound."""
    n0, K = 70, 512
    rng = np.random.default_rng(n1)
    x = S.f32_to_bf16_bits(rng.standard_normal((n1, K)).astype(np.float32))
    x[0, 7] = 0x7F80                       # +Inf
    x[1 % n1, 300] = 0xFF80                # -Inf
    x[2 % n1, 100] = 0x7FC0                # NaN
    x[3 % n1, 5] = 0x7F80
    x[3 % n1, 6] = 0xFF80                  # +Inf and -Inf in one group
    z, zr, zabs = zp_gemm_run(iq, O, S, n0, K, x, seed=11)
    assert np.array_equal(np.isnan(z), np.isnan(zr))
    assert np.array_equal(np.isposinf(z), np.isposinf(zr))
    assert np.array_equal(np.isneginf(z), np.isneginf(zr))
    fin = np.isfinite(zr)
    assert (~fin).any() and fin.any()
    err = np.abs(z[fin] - zr[fin])
    assert np.all(err <= (K + 2) * 2.0 ** -24 * zabs[fin] + 1e-30)


def test_zp_gemm_subnormal_activations(iq, O, S):
    """A token whose activations are all BF16 subnormals (2^-133 .. 2^-127
    in magnitude) beside ordinary tokens: its outputs too are within the
    bound of the exact sums, i.e. the matrix cores keep subnormal inputs.
    Weights near 1e4 keep those outputs normal FP32 numbers, and every
    product and partial sum is a multiple of 2^-133, exact in FP32."""
    n0, K, n1 = 40, 256, 20
    rng = np.random.default_rng(5)
    x = S.f32_to_bf16_bits(rng.standard_normal((n1, K)).astype(np.float32))
    mant = rng.integers(1, 128, size=K).astype(np.uint16)
    sign = (rng.integers(0, 2, size=K) << 15).astype(np.uint16)
    x[4] = sign | mant                     # exponent field 0: subnormal
    z, zr, zabs = zp_gemm_run(iq, O, S, n0, K, x, seed=12, w_scale=1e4)
    assert np.abs(zr[:, 4]).max() > 1e-36
    assert np.abs(zr[:, 4]).max() > 0
    err = np.abs(z - zr)
    bound = (K + 2) * 2.0 ** -24 * zabs + 1e-300
    assert np.all(err <= bound), f"max err/bound {np.max(err / bound):.3g} (token 4: {np.max(err[:, 4] / bound[:, 4]):.3g})"


@pytest.fixture(scope="module")
def c5_int4zp(O, S):
    """The c5 weight matrix (28672 x 8192) as asymmetric INT4, by the oracle."""
    return O.quantize(S.make("c5"), "int4zp", "block", want_xhat=False, threads=THREADS)


@pytest.mark.parametrize("n1", [1, 16, 50, 64, 100, 256, 384, 2048])
def test_zp_gemm_full_size_sampled(iq, O, S, c5_int4zp, n1):
    """The c5 weights against n1 tokens of BF16 activations; rows sampled
    for the oracle.  At 28672 rows the kernels are: the few-token kernel
    (1, 16); the 64-token tile with k split in halves, adding row by row at
    50 tokens and directly at 64; the 128-token tile with the k split,
    adding row by row (100, not a multiple of 16); the 128- and 256-token
    tiles whole (256, 384, 2048)."""
    import torch
    r = c5_int4zp
    n0, K = 28672, 8192
    x = S.make("c2", nrows=n1)                                  # BF16 activations [n1, 8192]
    q = iq.Quantized(to_device(r["codes"]), to_device(r["scales"]), None, None, None, "int4zp", "block", n0, K,
                     to_device(r["shifts"]))
    z = iq.zp_gemm(q, to_device(x))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, n0, 997), [n0 - 1, 1, 128, 8191]]))
    zs = z[torch.from_numpy(rows).cuda()].cpu().numpy()
    zr, zabs = O.zp_gemm(np.ascontiguousarray(r["codes"][rows]), np.ascontiguousarray(r["scales"][rows]),
                         np.ascontiguousarray(r["shifts"][rows]), x)
    bound = (K + 2) * 2.0 ** -24 * zabs + 1e-30
    err = np.abs(zs.astype(np.float64) - zr)
    assert np.all(err <= bound), f"max err/bound {np.max(err / bound):.3g}"
    assert np.max(err / bound) < 0.05


# ---- FP4 GEMM over two MXFP4 operands on the block-scaled matrix cores -------------
def mx_operand(O, S, rows, K, seed, sigma, outlier_axis):
    x = S.fill(rows, K, S.F32, sigma=sigma, outlier_axis=outlier_axis, outlier_frac=0.02, outlier_factor=30.0,
               seed=seed, ld=K)
    r = O.quantize(x, "mxfp4", "block", want_xhat=False)
    return r


def mx_gpu(iq, r, rows, K):
    return iq.Quantized(to_device(r["codes"]), to_device(r["scales"]), None, None, None, "mxfp4", "block", rows, K)


# n1 <= 64: the few-token kernel (1, 2 or 4 token tiles of 16); above, the
# 128 x 128 tiles, 64 x 128 where the grid is small (each such case here; 1100
# tokens take 128 x 256 tiles).  Odd step counts (K / 128) exercise the last half pair;
# K = 8320 (65 steps) takes two LDS chunks of scale words, the second one step.
@pytest.mark.parametrize("n0,K,n1", [(128, 128, 128), (200, 256, 75), (1, 128, 1), (257, 384, 129),
                                     (384, 1024, 256), (64, 512, 1100), (33, 4096, 40), (50, 640, 24),
                                     (70, 2048, 64), (24, 8320, 3), (24, 8320, 50), (100, 384, 65), (5, 512, 128),
                                     (130, 4096, 100)])
def test_mx_gemm_parity(iq, O, S, n0, K, n1):
    """Weights and activations quantized to MXFP4 by the oracle; the GPU
    product against the oracle's exact sum, within the FP32 bound."""
    rw = mx_operand(O, S, n0, K, seed=n0 + K, sigma=0.02, outlier_axis=S.AXIS_ROWS)
    ra = mx_operand(O, S, n1, K, seed=n1 + 3 * K, sigma=1.0, outlier_axis=S.AXIS_COLS)
    z = iq.mx_gemm(mx_gpu(iq, rw, n0, K), mx_gpu(iq, ra, n1, K)).cpu().numpy().astype(np.float64)
    zr, zabs = O.mx_gemm(rw["codes"], rw["scales"], ra["codes"], ra["scales"])
    bound = (K + 2) * 2.0 ** -24 * zabs + 1e-30
    err = np.abs(z - zr)
    assert np.all(err <= bound), f"{n0}x{K}x{n1}: max err/bound {np.max(err / bound):.3g}"
    assert np.abs(zr).max() > 0
    assert np.max(err / bound) < 0.05


def test_mx_gemm_zero_and_empty(iq, O, S):
    import torch
    n0, K = 64, 256
    rw = mx_operand(O, S, n0, K, seed=9, sigma=0.02, outlier_axis=S.AXIS_ROWS)
    ra = O.quantize(np.zeros((40, K), dtype=np.float32), "mxfp4", "block", want_xhat=False)
    z = iq.mx_gemm(mx_gpu(iq, rw, n0, K), mx_gpu(iq, ra, 40, K)).cpu().numpy()
    assert np.all(z == 0)
    empty = iq.Quantized(torch.zeros((0, K // 2), dtype=torch.uint8, device="cuda:0"),
                         torch.zeros((0, K // 32), dtype=torch.uint8, device="cuda:0"), None, None, None,
                         "mxfp4", "block", 0, K)
    assert iq.mx_gemm(mx_gpu(iq, rw, n0, K), empty).shape == (n0, 0)


@pytest.mark.parametrize("n1", [24, 300])
def test_mx_gemm_nan_scale(iq, O, S, n1):
    """E8M0 byte 255 is NaN: a weight row or a token with such a block scale
    gives NaN outputs (NaN times zero included), as in the oracle; every
    other output stays within the FP32 bound."""
    n0, K = 40, 512
    rw = mx_operand(O, S, n0, K, seed=21, sigma=0.02, outlier_axis=S.AXIS_ROWS)
    ra = mx_operand(O, S, n1, K, seed=22, sigma=1.0, outlier_axis=S.AXIS_COLS)
    rw["scales"][3, 2] = 255
    ra["scales"][5, 0] = 255
    z = iq.mx_gemm(mx_gpu(iq, rw, n0, K), mx_gpu(iq, ra, n1, K)).cpu().numpy().astype(np.float64)
    zr, zabs = O.mx_gemm(rw["codes"], rw["scales"], ra["codes"], ra["scales"])
    assert np.isnan(zr[3]).all() and np.isnan(zr[:, 5]).all()
    assert np.array_equal(np.isnan(z), np.isnan(zr))
    fin = np.isfinite(zr)
    assert np.all(np.abs(z[fin] - zr[fin]) <= (K + 2) * 2.0 ** -24 * zabs[fin] + 1e-30)


@pytest.fixture(scope="module")
def c3_mxfp4(O, S):
    """The c3 weight matrix (14336 x 4096) as MXFP4, by the oracle."""
    return O.quantize(S.make("c3"), "mxfp4", "block", want_xhat=False, threads=THREADS)


@pytest.mark.parametrize("n1", [16, 128, 2048])
def test_mx_gemm_full_size_sampled(iq, O, S, c3_mxfp4, n1):
    """The c3 weights against n1 tokens of the a3 activations (both MXFP4
    from the oracle); rows sampled for the oracle."""
    import torch
    rw = c3_mxfp4
    n0, K = 14336, 4096
    ra = O.quantize(S.make("a3", nrows=n1), "mxfp4", "block", want_xhat=False, threads=THREADS)
    z = iq.mx_gemm(mx_gpu(iq, rw, n0, K), mx_gpu(iq, ra, n1, K))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, n0, 997), [n0 - 1, 1, 128, 8191]]))
    zs = z[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    zr, zabs = O.mx_gemm(np.ascontiguousarray(rw["codes"][rows]), np.ascontiguousarray(rw["scales"][rows]),
                         ra["codes"], ra["scales"])
    bound = (K + 2) * 2.0 ** -24 * zabs + 1e-30
    err = np.abs(zs - zr)
    assert np.all(err <= bound), f"max err/bound {np.max(err / bound):.3g}"
    assert np.max(err / bound) < 0.05


@pytest.mark.parametrize("kind", ["mx", "mxw"])
def test_gemm_large_grid_random_shapes(iq, O, S, kind):
    """Seeded ragged shapes large enough for the 256 x 256 kernels (LDS DMA
    for the FP4 GEMM, the wide W4A16 tile): 4100 to 6000 weight rows and
    2100 to 4096 tokens (at least 153 tiles of 256 x 256 and 297 of
    128 x 256), K a multiple of 128 up to 768 (odd step counts included);
    24 sampled weight rows per case, among them the last one, against the
    oracle."""
    import torch
    rng = np.random.default_rng(8400 if kind == "mx" else 8500)
    for case in range(4):
        n0 = int(rng.integers(4100, 6000))
        n1 = int(rng.integers(2100, 4097))
        K = 128 * int(rng.integers(1, 7))
        rw = mx_operand(O, S, n0, K, seed=8600 + case, sigma=0.02, outlier_axis=S.AXIS_ROWS)
        if kind == "mx":
            ra = mx_operand(O, S, n1, K, seed=8700 + case, sigma=1.0, outlier_axis=S.AXIS_COLS)
            z = iq.mx_gemm(mx_gpu(iq, rw, n0, K), mx_gpu(iq, ra, n1, K))
        else:
            x = S.f32_to_bf16_bits(np.random.default_rng(8800 + case).standard_normal((n1, K)).astype(np.float32))
            z = iq.mxw_gemm(mx_gpu(iq, rw, n0, K), to_device(x))
        torch.cuda.synchronize()
        rows = np.unique(np.concatenate([rng.choice(n0, 22, replace=False), [0, n0 - 1]]))
        zs = z[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
        wc, ws = np.ascontiguousarray(rw["codes"][rows]), np.ascontiguousarray(rw["scales"][rows])
        zr, zabs = O.mx_gemm(wc, ws, ra["codes"], ra["scales"]) if kind == "mx" else O.mxw_gemm(wc, ws, x)
        bound = (K + 2) * 2.0 ** -24 * zabs + 1e-30
        err = np.abs(zs - zr)
        assert np.all(err <= bound), f"{kind} {n0}x{K}x{n1} (case {case}): max err/bound {np.max(err / bound):.3g}"


def test_mx_gemm_dma_tiles_sampled(iq, O, S):
    """From 1024 tokens, grids of at least 128 tiles of 256 x 256 copy their
    operands by LDS DMA in pairs of k steps: a ragged 2100 x 384 x 3600
    product (9 x 15 tiles; three steps, so the last pair has one), the last
    token with a NaN block scale, on sampled rows against the oracle; a
    second call returns the same bits."""
    import torch
    n0, K, n1 = 2100, 384, 3600
    rw = mx_operand(O, S, n0, K, seed=91, sigma=0.02, outlier_axis=S.AXIS_ROWS)
    ra = mx_operand(O, S, n1, K, seed=92, sigma=1.0, outlier_axis=S.AXIS_COLS)
    ra["scales"][n1 - 1, 1] = 255
    qw, qa = mx_gpu(iq, rw, n0, K), mx_gpu(iq, ra, n1, K)
    z = iq.mx_gemm(qw, qa)
    torch.cuda.synchronize()
    assert torch.equal(iq.mx_gemm(qw, qa).view(torch.int32), z.view(torch.int32))
    rows = np.unique(np.concatenate([np.arange(0, n0, 53), [1, 255, 256, 2047, 2048, n0 - 2, n0 - 1]]))
    zs = z[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    zr, zabs = O.mx_gemm(np.ascontiguousarray(rw["codes"][rows]), np.ascontiguousarray(rw["scales"][rows]),
                         ra["codes"], ra["scales"])
    assert np.isnan(zr[:, -1]).all() and np.array_equal(np.isnan(zs), np.isnan(zr))
    fin = np.isfinite(zr)
    bound = (K + 2) * 2.0 ** -24 * zabs[fin] + 1e-30
    err = np.abs(zs[fin] - zr[fin])
    assert np.all(err <= bound), f"max err/bound {np.max(err / bound):.3g}"
    assert np.max(err / bound) < 0.05


# ---- MXFP4 weights against BF16 activations (W4A16) ---------------------------------
def mxw_case(iq, O, S, n0, K, n1, seed, nan_row=None):
    rw = mx_operand(O, S, n0, K, seed=seed, sigma=0.02, outlier_axis=S.AXIS_ROWS)
    if nan_row is not None:
        rw["scales"][nan_row, 1] = 255
    rng = np.random.default_rng(seed + 1)
    x = S.f32_to_bf16_bits(rng.standard_normal((n1, K)).astype(np.float32))
    z = iq.mxw_gemm(mx_gpu(iq, rw, n0, K), to_device(x)).cpu().numpy().astype(np.float64)
    zr, zabs = O.mxw_gemm(rw["codes"], rw["scales"], x)
    return z, zr, zabs


# n1 <= 64: the few-token kernel (1, 2 or 4 token tiles); 65 .. 255: 128-token
# tiles; from 256: 256-token tiles (256 x 256 where the 128 x 256 tiles exceed
# one round of resident workgroups, which no case here does; see the sampled
# tests).  Odd step counts (K / 128) included.  The
# tiled cases' grids are small, so k is split in halves (one step each for
# K = 256, 1 and 2 steps for K = 384), except for K = 128 (one step).
@pytest.mark.parametrize("n0,K,n1", [(128, 256, 128), (200, 512, 75), (257, 384, 129), (40, 512, 300),
                                     (64, 1024, 1100), (1, 128, 1), (33, 640, 24), (70, 2048, 64), (50, 384, 16),
                                     (80, 128, 90), (24, 8320, 1), (24, 8320, 20), (24, 8320, 70),
                                     (70, 1024, 12), (130, 384, 8), (1, 384, 12), (2, 256, 24), (5, 640, 70),
                                     (3, 512, 300)])
def test_mxw_gemm_parity(iq, O, S, n0, K, n1):
    z, zr, zabs = mxw_case(iq, O, S, n0, K, n1, seed=n0 + 7 * K + n1)
    bound = (K + 2) * 2.0 ** -24 * zabs + 1e-30
    err = np.abs(z - zr)
    assert np.all(err <= bound), f"{n0}x{K}x{n1}: max err/bound {np.max(err / bound):.3g}"
    assert np.abs(zr).max() > 0 and np.max(err / bound) < 0.05


def test_mxw_gemm_wide_tiles_sampled(iq, O, S):
    """More 128 x 256 tiles than one round of resident workgroups (33 x 9
    here) take 256 x 256 tiles: a ragged 4100 x 384 x 2100 product, the last
    weight row with a NaN block scale, on sampled rows (both ends of the
    ragged last row tile among them) against the oracle; a second call and
    two replays of a captured call return the same bits."""
    import torch
    n0, K, n1 = 4100, 384, 2100
    rw = mx_operand(O, S, n0, K, seed=77, sigma=0.02, outlier_axis=S.AXIS_ROWS)
    rw["scales"][n0 - 1, 2] = 255
    rng = np.random.default_rng(78)
    x = S.f32_to_bf16_bits(rng.standard_normal((n1, K)).astype(np.float32))
    qw, xd = mx_gpu(iq, rw, n0, K), to_device(x)
    z = iq.mxw_gemm(qw, xd)
    torch.cuda.synchronize()
    assert torch.equal(iq.mxw_gemm(qw, xd).view(torch.int32), z.view(torch.int32))
    out = torch.empty_like(z)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        iq.mxw_gemm(qw, xd, out=out)
    for rep in range(2):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), z.view(torch.int32)), rep
    rows = np.unique(np.concatenate([np.arange(0, n0, 97), [1, 255, 256, 3839, 3840, 4095, 4096, n0 - 2, n0 - 1]]))
    zs = z[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    zr, zabs = O.mxw_gemm(np.ascontiguousarray(rw["codes"][rows]), np.ascontiguousarray(rw["scales"][rows]), x)
    assert np.isnan(zr[-1]).all() and np.array_equal(np.isnan(zs), np.isnan(zr))
    fin = np.isfinite(zr)
    bound = (K + 2) * 2.0 ** -24 * zabs[fin] + 1e-30
    err = np.abs(zs[fin] - zr[fin])
    assert np.all(err <= bound), f"max err/bound {np.max(err / bound):.3g}"
    assert np.max(err / bound) < 0.05


@pytest.mark.parametrize("n1", [24, 300])
def test_mxw_gemm_nan_scale_and_empty(iq, O, S, n1):
    """E8M0 255 on one weight block: that row's outputs are NaN, as in the
    oracle; other outputs within the bound; no tokens writes nothing."""
    import torch
    n0, K = 40, 512
    z, zr, zabs = mxw_case(iq, O, S, n0, K, n1, seed=5, nan_row=3)
    assert np.isnan(zr[3]).all() and np.array_equal(np.isnan(z), np.isnan(zr))
    fin = np.isfinite(zr)
    assert np.all(np.abs(z[fin] - zr[fin]) <= (K + 2) * 2.0 ** -24 * zabs[fin] + 1e-30)
    rw = mx_operand(O, S, n0, K, seed=6, sigma=0.02, outlier_axis=S.AXIS_ROWS)
    x0 = torch.zeros((0, K), dtype=torch.bfloat16, device="cuda:0")
    assert iq.mxw_gemm(mx_gpu(iq, rw, n0, K), x0).shape == (n0, 0)


@pytest.mark.parametrize("n1", [1, 16, 128, 255, 2048])
def test_mxw_gemm_full_size_sampled(iq, O, S, c3_mxfp4, n1):
    """The c3 weights (MXFP4 from the oracle) against n1 BF16 tokens of a3
    (few-token kernel; 128-token tiles with k split in halves; 256-token
    tiles whole); rows sampled for the oracle."""
    import torch
    rw = c3_mxfp4
    n0, K = 14336, 4096
    x = S.make("a3", nrows=n1)
    z = iq.mxw_gemm(mx_gpu(iq, rw, n0, K), to_device(x))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, n0, 997), [n0 - 1, 1, 128, 8191]]))
    zs = z[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    zr, zabs = O.mxw_gemm(np.ascontiguousarray(rw["codes"][rows]), np.ascontiguousarray(rw["scales"][rows]), x)
    bound = (K + 2) * 2.0 ** -24 * zabs + 1e-30
    err = np.abs(zs - zr)
    assert np.all(err <= bound), f"max err/bound {np.max(err / bound):.3g}"
    assert np.max(err / bound) < 0.05
