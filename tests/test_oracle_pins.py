"""Pins of the CPU oracle against what the pages and mathematics fix.

Every test here checks the oracle (oracle/iq_oracle.c) against something other
than its own formulas: values printed on the pages (tests/golden/), closed-form
error bounds, library routines (torch float8 casts, numpy float16 / rint,
struct), and brute-force nearest-code search over tiny code tables.

Pages: Lorn blog, post "浅谈低精度浮点数" (sections "IEEE 754 标准浮点数",
"FP8", "FP4 / MXFP4 / NVFP4"), and post "Triton" (Puzzle 12, extract()).
"""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import golden_map, read_golden

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def bits_f32(u: int) -> float:
    return struct.unpack("<f", struct.pack("<I", u))[0]


# ---- independent code tables ------------------------------------------------
def torch_fp8_table(dtype) -> np.ndarray:
    """Decode of all 256 FP8 codes by torch's float8 dtypes (library routine)."""
    return torch.arange(256, dtype=torch.uint8).view(dtype).float().numpy()


def e2m1_table() -> np.ndarray:
    """The 16 E2M1 values from the page's printed value set (sign in bit 3)."""
    pos = np.array([float(v) for v in read_golden("e2m1_values.txt")[0]], dtype=np.float32)
    return np.concatenate([pos, -pos]).astype(np.float32)


def brute_nearest(v: np.ndarray, table: np.ndarray, sign_bit: int, nan_code: int) -> np.ndarray:
    """Nearest finite code by exhaustive scan, ties to the even code, sign kept,
    saturating beyond the largest finite magnitude.  Independent of the oracle."""
    v = np.asarray(v, dtype=np.float64)
    mags = table[:sign_bit].astype(np.float64)
    finite = np.nonzero(np.isfinite(mags))[0]
    vals = mags[finite]
    a = np.abs(v)
    out = np.zeros(v.shape, dtype=np.int64)
    for i in range(v.size):
        ai = a.flat[i]
        if np.isnan(ai):
            out.flat[i] = nan_code
            continue
        if ai >= vals.max():
            c = finite[np.argmax(vals)]
        else:
            d = np.abs(vals - ai)
            best = np.nonzero(d == d.min())[0]
            cands = finite[best]
            c = cands[0] if len(cands) == 1 else [k for k in cands if k % 2 == 0][0]
        out.flat[i] = c | (sign_bit if np.signbit(v.flat[i]) else 0)
    return out


# ---- P1: the 25.125 worked example ------------------------------------------
def test_p1_worked_example_fields(O):
    g = golden_map("fp32_worked_example.txt")
    val = float(g["value"][0])
    word = int(g["word"][0], 16)
    assert f32_bits(val) == word
    assert (word >> 31) == int(g["sign"][0])
    assert ((word >> 23) & 0xFF) == int(g["exponent_field"][0])
    assert format(word & 0x7FFFFF, "023b") == g["fraction_bits"][0]
    # BF16 is the top half of the word: widening and narrowing are exact here.
    assert O.bf16_to_f32(word >> 16) == val
    assert O.f32_to_bf16(val) == word >> 16
    # The MX exponent is floor(log2 A): 25.125 lies in [2^4, 2^5).
    assert O.e8m0_code(val) == int(g["exponent_unbiased"][0]) - 2 + 127


def test_p2_fp32_limits(O):
    g = golden_map("fp32_limits.txt")
    vmax, wmax = float(g["max_finite"][0]), int(g["max_finite"][1], 16)
    vmin, wmin = float(g["min_normal"][0]), int(g["min_normal"][1], 16)
    assert bits_f32(wmax) == pytest.approx(vmax, rel=1e-7)
    assert bits_f32(wmin) == pytest.approx(vmin, rel=1e-7)
    emax, emin = int(g["exponent_max"][0]), int(g["exponent_min"][0])
    assert O.e8m0_code(bits_f32(wmax)) == emax - 2 + 127
    assert O.e8m0_code(bits_f32(wmin)) == max(0, emin - 2 + 127)
    assert O.e8m0_code(2.0 ** -124) == 1
    assert O.bf16_to_f32(wmax >> 16) == bits_f32(wmax & 0xFFFF0000)


# ---- P3, P4, P5: printed value sets and constants ----------------------------
def test_p3_e2m1_value_set(O):
    tab = e2m1_table()
    got = O.fp_decode_array(O.K_E2M1, np.arange(16))
    assert np.array_equal(got, tab)
    assert np.array_equal(np.signbit(got), np.arange(16) >= 8)


def test_p4_constants(O):
    g = golden_map("format_constants.txt")
    e4m3 = O.fp_decode_array(O.K_E4M3, np.arange(256))
    assert O.fp_decode(O.K_E4M3, 0x7E) == float(g["e4m3_max"][0])
    assert np.nanmax(e4m3) == float(g["e4m3_max"][0])
    assert O.fp_decode(O.K_E2M1, 0x7) == float(g["e2m1_max"][0])
    assert float(g["e2m1_max"][0]) * float(g["e4m3_max"][0]) == float(g["nvfp4_global_divisor"][0])
    # the NVFP4 global scale is the tensor absmax over 6*448
    for G in (2688.0, 448.0, 1000.0):
        x = np.full((1, 16), 0.5, dtype=np.float32)
        x[0, 3] = -G
        r = O.quantize(x, "nvfp4", "block")
        assert r["global_scale"][0] == np.float32(G) / np.float32(2688.0)
    assert O.block_size("mxfp4", "block") == int(g["mxfp4_block"][0])
    assert O.block_size("nvfp4", "block") == int(g["nvfp4_block"][0])


def test_p5_samples_per_binade(O):
    g = golden_map("format_constants.txt")
    for kind, key in ((O.K_E5M2, "e5m2_values_in_2_4"), (O.K_E4M3, "e4m3_values_in_2_4")):
        v = O.fp_decode_array(kind, np.arange(128))
        assert len({float(t) for t in v if 2.0 <= t < 4.0}) == int(g[key][0])


# ---- P12: exhaustive code tables and brute force -------------------------------
FP8 = [("e4m3", 0, torch.float8_e4m3fn, 448.0, 3), ("e5m2", 1, torch.float8_e5m2, 57344.0, 2)]


@pytest.mark.parametrize("name,kind,tdt,fmax,mbits", FP8)
def test_p12_fp8_decode_matches_torch(O, name, kind, tdt, fmax, mbits):
    ref = torch_fp8_table(tdt)
    got = O.fp_decode_array(kind, np.arange(256))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


@pytest.mark.parametrize("name,kind,tdt,fmax,mbits", FP8)
def test_p12_fp8_roundtrip_midpoints_saturation(O, name, kind, tdt, fmax, mbits):
    ref = torch_fp8_table(tdt)
    codes = np.arange(256)
    finite = np.isfinite(ref)
    # decode -> encode is the identity on every finite code (also -0 -> 0x80)
    enc = O.fp_encode_array(kind, ref[finite])
    assert np.array_equal(enc, codes[finite])
    # midpoints between adjacent positive values go to the even code;
    # one FP32 ulp either side goes to the nearer code
    pos = sorted((float(ref[c]), c) for c in range(128) if np.isfinite(ref[c]))
    for (a, ca), (b, cb) in zip(pos, pos[1:]):
        m = np.float32((a + b) / 2)
        assert float(m) == (a + b) / 2
        even = ca if ca % 2 == 0 else cb
        assert O.fp_encode(kind, m) == even
        assert O.fp_encode(kind, -m) == even | 0x80
        assert O.fp_encode(kind, np.nextafter(m, np.float32(np.inf))) == cb
        assert O.fp_encode(kind, np.nextafter(m, np.float32(0))) == ca
    # saturation beyond the largest finite value
    maxc = int(codes[finite & (ref == fmax)][0])
    for v in (fmax * 1.01, fmax * 1.0625, fmax * 1.2, 1e30, float("inf")):
        assert O.fp_encode(kind, v) == maxc
        assert O.fp_encode(kind, -v) == maxc | 0x80


@pytest.mark.parametrize("name,kind,tdt,fmax,mbits", FP8)
def test_p12_fp8_bruteforce_random(O, name, kind, tdt, fmax, mbits):
    rng = np.random.default_rng(12)
    ref = torch_fp8_table(tdt)
    # random magnitudes over the whole format range plus subnormals and beyond max
    e = rng.uniform(-20 if kind == 0 else -19, math.log2(fmax) + 2, 20000)
    v = (np.exp2(e) * rng.choice([-1, 1], e.size)).astype(np.float32)
    got = O.fp_encode_array(kind, v)
    want = brute_nearest(v, ref, 0x80, 0x7F)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("name,kind,tdt,fmax,mbits", FP8)
def test_p12_fp8_matches_torch_cast_in_range(O, name, kind, tdt, fmax, mbits):
    """Third opinion: torch's float8 casts round to nearest even inside the
    finite range (they do not saturate, so only |v| <= max is compared)."""
    rng = np.random.default_rng(7)
    v = (rng.standard_normal(1_000_000) * rng.choice([1e-4, 1e-2, 1, 30, fmax / 4], 1_000_000)).astype(np.float32)
    v = v[np.abs(v) <= fmax]
    t = torch.from_numpy(v).to(tdt).view(torch.uint8).numpy()
    assert np.array_equal(O.fp_encode_array(kind, v), t.astype(np.uint32))


def test_p12_e2m1_exhaustive(O):
    tab = e2m1_table()
    assert np.array_equal(O.fp_encode_array(O.K_E2M1, tab), np.arange(16))
    pos = sorted((float(tab[c]), c) for c in range(8))
    for (a, ca), (b, cb) in zip(pos, pos[1:]):
        m = np.float32((a + b) / 2)
        even = ca if ca % 2 == 0 else cb
        assert O.fp_encode(O.K_E2M1, m) == even
        assert O.fp_encode(O.K_E2M1, np.nextafter(m, np.float32(np.inf))) == cb
        assert O.fp_encode(O.K_E2M1, np.nextafter(m, np.float32(0))) == ca
    for v in (6.5, 7.0, 100.0, float("inf")):
        assert O.fp_encode(O.K_E2M1, v) == 0x7
        assert O.fp_encode(O.K_E2M1, -v) == 0xF
    rng = np.random.default_rng(3)
    v = (rng.uniform(-8, 8, 20000)).astype(np.float32)
    assert np.array_equal(O.fp_encode_array(O.K_E2M1, v), brute_nearest(v, tab, 0x8, 0))


def test_p12_e8m0_values(O):
    for c in range(255):
        assert O.e8m0_value(c) == math.ldexp(1.0, c - 127)
    assert math.isnan(O.e8m0_value(255))


def test_p12_f16_scale_matches_numpy(O):
    """The INT4 group scale is FP16 by round to nearest even (numpy's cast),
    saturated at 65504 instead of overflowing."""
    rng = np.random.default_rng(5)
    v = np.exp2(rng.uniform(-27, 17, 200000)).astype(np.float32)
    got = O.fp_encode_array(O.K_F16, v)
    want = v.astype(np.float16).view(np.uint16).astype(np.uint32)
    big = v > 65504
    want[big] = 0x7BFF
    assert np.array_equal(got, want)
    h = np.arange(0x7C00, dtype=np.uint16)
    assert np.array_equal(O.fp_decode_array(O.K_F16, h), h.view(np.float16).astype(np.float32))


# ---- P13: textbook reductions -------------------------------------------------
def test_p13_int_path_is_rint_and_clip(O):
    rng = np.random.default_rng(9)
    v = np.concatenate([rng.uniform(-200, 200, 100000), np.arange(-140, 140) + 0.5,
                        np.arange(-140, 140, dtype=np.float64)]).astype(np.float32)
    for qmax in (127, 7):
        want = np.clip(np.rint(v.astype(np.float64)), -qmax, qmax).astype(np.int32)
        assert np.array_equal(O.int_encode_array(v, qmax), want)
    assert O.int_encode(float("nan"), 127) == 0


def test_p13_mx_scale_is_exponent_field(O):
    rng = np.random.default_rng(11)
    bits = rng.integers(1, 0x7F800000, 200000, dtype=np.uint32)
    A = bits.view(np.float32)
    for a, b in zip(A[:50000], bits[:50000]):
        field = int(b) >> 23
        e = field - 127 if field else (int(b) & 0x7FFFFF).bit_length() - 1 - 149
        assert O.e8m0_code(float(a)) == min(254, max(0, e - 2 + 127))
    assert O.e8m0_code(0.0) == 0


def test_p13_e5m2_is_rounded_fp16(O):
    """E5M2 has FP16's exponent layout, so encoding an FP16 value equals
    rounding its bit pattern to the top byte, ties to even."""
    h = np.arange(0x0400, 0x7C00, dtype=np.uint32)          # positive normal FP16
    vals = h.astype(np.uint16).view(np.float16).astype(np.float32)
    keep = vals <= 57344
    h, vals = h[keep], vals[keep]
    low = h & 0xFF
    up = h >> 8
    want = up + ((low > 0x80) | ((low == 0x80) & (up & 1) == 1))
    assert np.array_equal(O.fp_encode_array(O.K_E5M2, vals), want)
    assert np.array_equal(O.fp_encode_array(O.K_E5M2, -vals), want | 0x80)


# ---- P6, P7, P8: error bounds of the FP8 section -------------------------------
def test_p6_int8_bound(O, S):
    x = S.make("c1")
    r = O.quantize(x, "int8", "tensor")
    alpha = float(np.max(np.abs(x)))
    s = float(r["scales"][0])
    assert s == float(np.float32(alpha) / np.float32(127.0))
    x64 = x.astype(np.float64)
    err = np.abs(x64 - r["xhat"].astype(np.float64))
    g = golden_map("error_bounds.txt")
    assert err.max() <= s / 2 * (1 + 2 ** -20)
    assert err.max() <= alpha * float(g["int8_abs_err_over_alpha"][0]) * (1 + 2 ** -20)
    q = r["codes"].view(np.int8).astype(np.float64)
    assert np.abs(x64 / s - q).max() <= 0.5 + 1e-6


@pytest.mark.parametrize("fmt,fmax,mbits,key", [("e4m3", 448.0, 3, "e4m3_rel_err"),
                                                 ("e5m2", 57344.0, 2, "e5m2_rel_err")])
def test_p7_fp8_relative_bound(O, fmt, fmax, mbits, key):
    """Every BF16 value in the format's normal range, quantized with s = 1
    (alpha = FMAX), has relative error below 2^-(M+1)."""
    bound = float(golden_map("error_bounds.txt")[key][0])
    assert bound == 2.0 ** -(mbits + 1)
    bits = np.arange(0x0000, 0x7F80, dtype=np.uint16)
    v = (bits.astype(np.uint32) << 16).view(np.float32)
    min_normal = 2.0 ** -6 if fmt == "e4m3" else 2.0 ** -14
    v = v[(v >= min_normal) & (v <= fmax)]
    x = np.concatenate([v, -v, [fmax]]).astype(np.float32)[None, :]
    cols = x.shape[1] - x.shape[1] % 16
    x = np.ascontiguousarray(x[:, :cols])
    x[0, 0] = fmax
    r = O.quantize(x, fmt, "tensor")
    assert r["scales"][0] == 1.0
    # |v| == FMAX is on the grid: represented exactly, so not counted as saturated
    assert r["stats"]["n_saturated"] == 0
    rel = np.abs(x - r["xhat"]).astype(np.float64) / np.abs(x).astype(np.float64)
    assert rel.max() < bound
    assert rel.max() > 0.9 * bound / (1 + bound)


def test_p8_int8_fp8_crossover(O, S):
    """Binned by |x|/alpha, the worst relative error of per-tensor INT8 falls
    below per-tensor E4M3's near |x| ~ 0.063 alpha and not far from it."""
    x = S.make("c1")
    alpha = float(np.max(np.abs(x)))
    xi = O.quantize(x, "int8", "tensor")["xhat"]
    xf = O.quantize(x, "e4m3", "tensor")["xhat"]
    ax = np.abs(x.astype(np.float64))
    nz = ax > 0
    rel_i = np.abs(x - xi)[nz] / ax[nz]
    rel_f = np.abs(x - xf)[nz] / ax[nz]
    ratio = ax[nz] / alpha
    edges = np.exp2(np.arange(-7.0, 0.01, 0.125))
    worse = []
    for lo, hi in zip(edges, edges[1:]):
        m = (ratio >= lo) & (ratio < hi)
        if m.sum() < 200:
            continue
        worse.append((np.sqrt(lo * hi), rel_i[m].max() > rel_f[m].max()))
    above = [c for c, w in worse if not w]
    below = [c for c, w in worse if w]
    cross = min(above)
    assert max(below) < cross
    page = float(golden_map("error_bounds.txt")["int8_e4m3_crossover"][0])
    assert 0.75 * page < cross < 1.35 * page
    assert all(w for c, w in worse if c < 0.5 * page)
    assert not any(w for c, w in worse if c > 2 * page)


# ---- P9: MXFP4 ------------------------------------------------------------------
def test_p9_mx_alignment_example(O):
    """The page's example A/6 = 1.99 vs 2.01: round-up gives scales 2 and 4.
    The default floor(log2 A) - 2 rule gives 2 for both."""
    rows = read_golden("mx_alignment_example.txt")
    for r in rows:
        A = np.float32(float(r[1]) * 6)
        assert O.e8m0_value(O.e8m0_code(float(A), O.FLAG_MX_ROUND_UP)) == float(r[3])
        assert O.e8m0_value(O.e8m0_code(float(A))) == 2.0
    # default rule with block maximum 12.06: s = 2, v = 6.03 saturates to 6
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 12.06
    x[0, 1] = -1.0
    r = O.quantize(x, "mxfp4", "block")
    assert r["scales"][0, 0] == 128
    assert r["xhat"][0, 0] == 12.0
    assert r["stats"]["n_saturated"] == 1
    assert r["codes"][0, 0] == 0x7 | (0x9 << 4)  # +6 low nibble, -1/2 = -0.5 (0x9) high nibble


def test_p9_mx_bounds(O, S):
    x = S.make("c3", nrows=256)
    for flags in (0, O.FLAG_MX_ROUND_UP):
        r = O.quantize(x, "mxfp4", "block", flags=flags)
        xb = x_f32(S, x).reshape(-1, 32).astype(np.float64)
        xh = r["xhat"].reshape(-1, 32).astype(np.float64)
        s = np.exp2(r["scales"].reshape(-1).astype(np.float64) - 127)[:, None]
        A = np.abs(xb).max(axis=1, keepdims=True)
        v = xb / s
        err = np.abs(xb - xh)
        if flags == 0:
            assert ((A / s >= 4) & (A / s < 8)).all()
            inr = np.abs(v) <= 6
            assert (err[inr] <= s.repeat(32, 1)[inr]).all()
            top = np.abs(v) > 6
            assert (np.abs(xh[top]) == 6 * s.repeat(32, 1)[top]).all()
            assert (err[top] < 2 * s.repeat(32, 1)[top]).all()
        else:
            g = golden_map("error_bounds.txt")
            rho = s / (A / 6)
            assert ((rho >= 1) & (rho < 2)).all()
            assert (err <= s).all()
            assert (err.max(axis=1, keepdims=True) < A * float(g["mx_err_worst"][0])).all()
            zt = np.where(xh == 0, np.abs(xb), 0).max(axis=1, keepdims=True)
            assert (zt <= A * float(g["mx_zero_hi"][0])).all()
            assert (zt <= 0.25 * s).all()
        assert (np.where(np.abs(v) <= 0.25, xh, 0) == 0).all()


def x_f32(S, x):
    return S.bf16_to_f32(x) if x.dtype == np.uint16 else x


def mx_rule_exact(A: float, rule: str) -> int:
    """E8M0 code of a block maximum A > 0 by exact rational arithmetic.
    floor: the largest k with 2^k <= A, minus 2; nearest: the k closest to
    log2(A/6), decided by (A/6)^2 >= 2^(2k+1); up: the least k with
    6 * 2^k >= A.  Biased by 127 and clamped to [0, 254]."""
    from fractions import Fraction
    a = Fraction(A)
    k = math.frexp(A)[1] - 1                       # 2^k <= A < 2^(k+1), exact for floats
    assert Fraction(2) ** k <= a < Fraction(2) ** (k + 1)
    if rule == "floor":
        e = k - 2
    else:
        a6 = a / 6
        j = k - 3                                  # 2^j <= A/6 < 2^(j+1) for one of j, j+1
        while Fraction(2) ** (j + 1) <= a6:
            j += 1
        assert Fraction(2) ** j <= a6 < Fraction(2) ** (j + 1)
        if rule == "nearest":
            e = j + 1 if a6 * a6 >= Fraction(2) ** (2 * j + 1) else j
        else:
            e = j if a6 == Fraction(2) ** j else j + 1
    return min(max(e + 127, 0), 254)


def test_p9_mx_rule_variants_exact(O):
    """The three MXFP4 exponent rules of the page against exact rational
    arithmetic, for maxima over the whole FP32 range (subnormals included),
    with significands at random and next to 3*sqrt(2)/4 and 3/2, where the
    nearest and round-up rules change their answer."""
    rng = np.random.default_rng(9)
    mants = list(rng.integers(0, 1 << 23, 12)) + [0, 1, 0x07C3B5, 0x07C3B6, 0x07C3B7, 0x07C3B8,
                                                   0x3FFFFF, 0x400000, 0x400001, 0x7FFFFF]
    flags = {"floor": 0, "nearest": O.FLAG_MX_ROUND_NEAREST, "up": O.FLAG_MX_ROUND_UP}
    for e in range(0, 255):
        for m in mants:
            u = (e << 23) | int(m)
            if u == 0:
                continue
            A = bits_f32(u)
            for rule, f in flags.items():
                assert O.e8m0_code(A, f) == mx_rule_exact(A, rule), (hex(u), rule)
    # saturation ranges: nearest keeps A/s below 6*sqrt(2), round-up at most 6
    x = np.zeros((1, 64), np.float32)
    x[0, 0] = 8.4                                  # A/6 = 1.4 < sqrt(2): s = 1, v = 8.4 saturates
    x[0, 32] = 6.0                                 # exact power-of-two boundary for round-up
    r = O.quantize(x, "mxfp4", "block", flags=O.FLAG_MX_ROUND_NEAREST)
    assert r["scales"][0, 0] == 127 and r["xhat"][0, 0] == 6.0 and r["stats"]["n_saturated"] == 1
    r = O.quantize(x, "mxfp4", "block", flags=O.FLAG_MX_ROUND_UP)
    assert r["scales"][0, 0] == 128 and r["scales"][0, 1] == 127
    assert r["xhat"][0, 32] == 6.0 and r["stats"]["n_saturated"] == 0


# ---- P10: NVFP4 -----------------------------------------------------------------
def test_p10_nv_bounds(O, S):
    x = S.make("c4", nrows=128)
    G = float(np.max(np.abs(x_f32(S, x))))
    r = O.quantize(x, "nvfp4", "block")
    g = golden_map("error_bounds.txt")
    sb = r["scales"].reshape(-1)
    assert sb.max() <= 0x7E
    s_g = float(r["global_scale"][0])
    assert s_g == float(np.float32(G) / np.float32(2688))
    dec = O.fp_decode_array(O.K_E4M3, sb).astype(np.float64)
    s_nv = (np.float32(s_g) * dec.astype(np.float32)).astype(np.float64)[:, None]
    xb = x_f32(S, x).reshape(-1, 16).astype(np.float64)
    xh = r["xhat"].reshape(-1, 16).astype(np.float64)
    A = np.abs(xb).max(axis=1, keepdims=True)
    t = (A / 6) / s_g
    normal = (t >= 2.0 ** -6) & (t <= 448)
    rho = (s_nv / (A / 6))[normal]
    assert rho.min() >= 1 - 1e-6
    assert rho.max() <= float(g["nv_rho_max"][0]) + 1e-6
    err = np.abs(xb - xh)
    nb = normal[:, 0]
    assert (err[nb].max(axis=1) <= A[nb, 0] * float(g["nv_err"][0]) * (1 + 1e-6)).all()
    zt = np.where(xh == 0, np.abs(xb), 0).max(axis=1)
    assert (zt[nb] <= A[nb, 0] * float(g["nv_zero"][0])).all()


def test_p10_e4m3_ceil_is_smallest_not_below(O):
    """Rounding the block scale up: the smallest E4M3 value >= t, with the
    E4M3 table taken from torch's decode."""
    tab = torch_fp8_table(torch.float8_e4m3fn)
    for c in range(0x7F):
        v = np.float32(tab[c])
        assert O.e4m3_ceil(v) == c
        if c < 0x7E:
            assert O.e4m3_ceil(np.nextafter(v, np.float32(np.inf))) == c + 1
    assert O.e4m3_ceil(1e6) == 0x7E


def test_p10_nv_aligned_block_is_exact(O):
    """rho = 1 (the aligned case): G = 2688 gives s_global = 1, and a block
    whose maximum is 6 gets t = 1 exactly, so E2M1 values come back exact."""
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 2688.0
    vals = np.array([6, -3, 1.5, 0.5, -4, 2, 1, -6, 0, 3, 4, -0.5, 1.5, 2, -1, 6], np.float32)
    x[0, 16:] = vals
    r = O.quantize(x, "nvfp4", "block")
    assert r["global_scale"][0] == 1.0
    assert r["scales"][0, 1] == 0x38                     # E4M3 1.0
    assert np.array_equal(r["xhat"][0, 16:], vals)


def test_p10_nv_rne_block_scale_exact(O):
    """Block scale by RNE (flag): with s_global = 1 each block's code is the
    E4M3 value nearest to t = A/6 (torch's decode table, exhaustive search,
    ties to the even code), for maxima on E4M3 values, on midpoints between
    neighbours (below the smallest subnormal too) and a few FP32 steps off;
    blocks that round to code 0 quantize to +0, and elements beyond
    6 * s_block saturate."""
    tab = torch_fp8_table(torch.float8_e4m3fn)[:0x7F].astype(np.float64)      # codes 0 .. 0x7E
    order = np.argsort(tab, kind="stable")
    vals = tab[order]
    mids = (vals[:-1] + vals[1:]) / 2
    targets = []
    for t in np.concatenate([vals[1:], mids]):
        a = np.float32(6.0 * t)
        for k in (-2, -1, 0, 1, 2):
            b = a
            for _ in range(abs(k)):
                b = np.nextafter(b, np.float32(np.inf) if k > 0 else np.float32(0))
            if 0 < b <= 2688.0:
                targets.append(b)
    targets = np.array(targets, np.float32)
    nb = len(targets) + 1
    x = np.zeros((1, 16 * nb), np.float32)
    x[0, 0] = 2688.0                                       # s_global = 1
    x[0, 16::16] = targets
    x[0, 17::16] = -targets                                # a second element equal in magnitude
    x[0, 18::16] = targets * np.float32(0.3)
    r = O.quantize(x, "nvfp4", "block", flags=O.FLAG_NV_SCALE_RNE)
    assert r["global_scale"][0] == 1.0
    for i, A in enumerate(targets):
        t = float(np.float32(A) / np.float32(6.0))
        d = np.abs(tab - t)
        best = np.flatnonzero(d == d.min())
        want = int(best[0]) if len(best) == 1 else int([c for c in best if c % 2 == 0][0])
        got = int(r["scales"][0, i + 1])
        assert got == want, (float(A), t, got, want)
        s_nv = tab[got]
        xh = r["xhat"][0, 16 * (i + 1): 16 * (i + 2)].astype(np.float64)
        assert (np.abs(xh) <= 6 * s_nv).all()
        if got == 0:
            assert (xh == 0).all() and not np.signbit(xh).any()
    # rounding up never lands below t; RNE does for about half the targets
    up = O.quantize(x, "nvfp4", "block")
    assert (tab[up["scales"][0, 1:]] >= (targets.astype(np.float64) / 6) * (1 - 2 ** -23)).all()
    assert (r["scales"][0, 1:] != up["scales"][0, 1:]).any()


# ---- static (calibrated) scaling: the absmax is given, not measured ---------------
def test_static_scale_matches_measured_and_textbook(O, S):
    """With alpha equal to the measured absmax, static scaling is the
    dynamic path; with any alpha, INT8 codes are rint(x / s) clipped to
    [-127, 127] (numpy), s = alpha / 127 in FP32, and the saturation count
    is the number of |x / s| > 127."""
    x = S.make("c1", nrows=64)
    x32 = x_f32(S, x)
    G = float(np.max(np.abs(x32)))
    for fmt, gran in (("int8", "tensor"), ("e4m3", "tensor"), ("e5m2", "tensor"), ("nvfp4", "block")):
        a = O.quantize(x, fmt, gran)
        b = O.quantize(x, fmt, gran, static_amax=G)
        for k in ("codes", "scales", "global_scale", "xhat"):
            assert np.array_equal(a[k], b[k]), (fmt, k)
        assert a["stats"] == b["stats"]
    for alpha in (0.25 * G, G, 3.0 * G, 1e-3):
        s = np.float32(np.float32(alpha) / np.float32(127.0))
        r = O.quantize(x, "int8", "tensor", static_amax=alpha)
        assert r["scales"][0] == s
        v = x32 / s
        q = np.clip(np.rint(v), -127, 127).astype(np.int8)
        assert np.array_equal(r["codes"].view(np.int8), q)
        assert np.array_equal(r["xhat"], (s * q.astype(np.float32)).astype(np.float32))
        assert r["stats"]["n_saturated"] == int(np.count_nonzero(np.abs(v) > 127))


def test_static_scale_fp8_saturates_to_torch_clamp(O, S):
    """E4M3 / E5M2 with alpha below the data: codes equal torch's float8 cast
    of clamp(x / s, -FMAX, FMAX) (torch's cast rounds to nearest even and
    does not saturate, hence the clamp)."""
    x = S.make("c1", nrows=32)
    x32 = x_f32(S, x)
    G = float(np.max(np.abs(x32)))
    for fmt, tdt, fmax in (("e4m3", torch.float8_e4m3fn, 448.0), ("e5m2", torch.float8_e5m2, 57344.0)):
        alpha = 0.1 * G
        r = O.quantize(x, fmt, "tensor", static_amax=alpha)
        s = np.float32(np.float32(alpha) / np.float32(fmax))
        v = np.clip(x32 / s, -fmax, fmax).astype(np.float32)
        want = torch.from_numpy(v).to(tdt).view(torch.uint8).numpy()
        assert np.array_equal(r["codes"], want), fmt
        assert r["stats"]["n_saturated"] == int(np.count_nonzero(np.abs(x32 / s) > fmax))


def test_static_scale_invalid_alpha_is_zero(O, S):
    """NaN, negative and infinite alphas are taken as 0 (every code +0,
    scale 0, x^ = 0); -0 as +0."""
    x = S.make("c1", nrows=8)
    assert O._load().iqo_static_amax(float("nan")) == 0.0
    assert O._load().iqo_static_amax(-1.0) == 0.0
    assert O._load().iqo_static_amax(float("inf")) == 0.0
    assert not math.copysign(1.0, O._load().iqo_static_amax(-0.0)) < 0
    assert O._load().iqo_static_amax(2.5) == 2.5
    for alpha in (float("nan"), -3.0, float("inf"), -0.0):
        for fmt, gran in (("int8", "tensor"), ("e4m3", "tensor"), ("nvfp4", "block")):
            r = O.quantize(x, fmt, gran, static_amax=alpha)
            assert not r["codes"].any() and not r["scales"].any()
            assert not r["xhat"].any() and not np.signbit(r["xhat"]).any()
            if fmt == "nvfp4":
                assert r["global_scale"][0] == 0.0 and not np.signbit(r["global_scale"][0])


# ---- P11: INT4 and the nibble order of Puzzle 12 ---------------------------------
def test_p11_int4_bound_and_nibbles(O, S):
    x = S.make("c5", nrows=64)
    r = O.quantize(x, "int4", "block")
    xb = x_f32(S, x).astype(np.float64)
    sf = r["scales"].view(np.float16).astype(np.float64)                 # [rows, groups]
    sfe = np.repeat(sf, 128, axis=1)
    A = np.abs(xb).reshape(x.shape[0], -1, 128).max(axis=2)
    assert np.allclose(sf, A / 7, rtol=2 ** -10)
    q = r["xhat"].astype(np.float64) / sfe
    assert np.array_equal(q, np.rint(q))
    v = xb / sfe
    assert (np.abs(v - q) <= 0.5 + 1e-6).all()
    assert (np.abs(xb[q == 0]) <= sfe[q == 0] / 2 * (1 + 1e-6)).all()
    g = golden_map("error_bounds.txt")
    Ae = np.repeat(A, 128, axis=1)
    assert (np.abs(xb - r["xhat"]) <= Ae * float(g["int4_err"][0]) * (1 + 1e-3)).all()
    # Puzzle 12's extract(): element i of a packed 32-bit word is (w >> 4i) & 0xF
    words = r["codes"].view("<u4")
    for i in range(8):
        nib = (words >> (4 * i)) & 0xF
        assert np.array_equal(nib, (q[:, i::8].astype(np.int64) & 0xF))


# ---- P11: the INT4 FP16 group scale on FP16 rounding boundaries -------------------
def rne_grid(v: Fraction, mbits: int, emin: int) -> Fraction:
    """The binary floating-point value nearest to the rational v >= 0 with
    mbits fraction bits and smallest normal exponent emin (a fixed spacing
    2^(emin - mbits) below it), ties to the even significand; unbounded above."""
    if v == 0:
        return Fraction(0)
    e = v.numerator.bit_length() - v.denominator.bit_length()
    while Fraction(2) ** e > v:
        e -= 1
    while Fraction(2) ** (e + 1) <= v:
        e += 1
    ulp = Fraction(2) ** (max(e, emin) - mbits)
    n = v / ulp
    k = n.numerator // n.denominator
    rem = n - k
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and k % 2 == 1):
        k += 1
    return k * ulp


def fp16_bits_of(v: Fraction) -> int:
    """IEEE binary16 bit pattern of a non-negative value on the binary16 grid."""
    if v < Fraction(2) ** -14:
        return int(v / Fraction(2) ** -24)
    e = v.numerator.bit_length() - v.denominator.bit_length()
    while Fraction(2) ** e > v:
        e -= 1
    while Fraction(2) ** (e + 1) <= v:
        e += 1
    return ((e + 15) << 10) | int((v / Fraction(2) ** e - 1) * 1024)


def int4_scale_expected(A: float) -> int:
    """s = A/7 as the method states it: one binary32 quotient (exact rational,
    rounded to nearest even), then binary16 by round to nearest even,
    saturating at the largest finite binary16 value 65504."""
    s32 = rne_grid(Fraction(A) / 7, 23, -126)
    s16 = rne_grid(s32, 10, -14)
    return 0x7BFF if s16 > 65504 else fp16_bits_of(s16)


def test_p11_int4_fp16_scale_ties_exact():
    """Self-check of the exact-rational helpers on printed binary16 facts."""
    assert fp16_bits_of(Fraction(1)) == 0x3C00 and fp16_bits_of(Fraction(65504)) == 0x7BFF
    assert fp16_bits_of(Fraction(2) ** -24) == 0x0001 and fp16_bits_of(Fraction(2) ** -14) == 0x0400
    assert rne_grid(Fraction(2049, 2048), 10, -14) == 1                          # tie, even below
    assert rne_grid(Fraction(2051, 2048), 10, -14) == Fraction(1026, 1024)        # tie, even above
    assert rne_grid(Fraction(1, 3), 23, -126) == Fraction(bits_f32(0x3EAAAAAB))


def test_p11_int4_fp16_scale_rounding(O):
    """Groups whose maximum A puts A/7 on a binary16 midpoint m (A = 7m, exact
    in binary32) and on the binary32 values next to 7m: the stored FP16 scale
    is fp16(fl32(A/7)) with ties to even and saturation at 65504."""
    ulp16 = lambda h: Fraction(2) ** -24 if h < 0x0400 else Fraction(2) ** (((h >> 10) - 15) - 10)
    val16 = lambda h: Fraction(fp16_value(h))
    mids = [val16(h) + ulp16(h) / 2 for h in (0x3C00, 0x3C01, 0x0400, 0x03FF, 0x5000, 0x1234, 0x2F01, 0x7BFE,
                                              0x7BFF, 0x0000, 0x0001, 0x0002)]
    As, want = [], []
    for m in mids:
        a0 = float(7 * m)
        assert Fraction(a0) == 7 * m                     # 7m is exact in binary32 (m has <= 12 bits)
        for a in (np.nextafter(np.float32(a0), np.float32(0)), np.float32(a0), np.nextafter(np.float32(a0),
                                                                                              np.float32(np.inf))):
            As.append(float(a))
            want.append(int4_scale_expected(float(a)))
    x = np.zeros((len(As), 128), dtype=np.float32)
    for i, a in enumerate(As):
        x[i] = np.linspace(0.0, a, 128, dtype=np.float32)
        x[i, 37] = np.float32(a)
        x[i] = np.minimum(x[i], np.float32(a))
    r = O.quantize(x, "int4", "block")
    got = r["scales"].view(np.uint16)[:, 0].astype(int)
    assert got.tolist() == want, [(hex(g), hex(w)) for g, w in zip(got, want) if g != w]
    # the cases really sit on the boundaries: every tie (A = 7m) goes to the
    # even code, some down and some up, and 65520 saturates where a plain
    # binary16 cast would give Inf
    ties = want[1::3]
    assert all(t % 2 == 0 for i, t in enumerate(ties) if i != 8)   # 8: the saturating tie
    assert any(Fraction(fp16_value(t)) < m for t, m in zip(ties, mids) if t != 0x7BFF)
    assert any(Fraction(fp16_value(t)) > m for t, m in zip(ties, mids))
    assert want[3 * 8 + 1] == 0x7BFF and rne_grid(mids[8], 10, -14) > 65504
    # planted mistakes this pin catches: a product with RN(1/7), ties away
    # from zero, and an unsaturated binary16 cast
    a32 = np.array(As, dtype=np.float32)
    mult = (a32 * np.float32(1.0 / 7.0)).astype(np.float16).view(np.uint16).astype(int)
    assert (mult != np.array(want)).any()
    assert np.isinf((a32 / np.float32(7.0)).astype(np.float16)).any()
    away = [fp16_bits_of(min(rne_grid(Fraction(a) / 7, 23, -126) + Fraction(1, 2 ** 60), Fraction(65504)))
            for a in As]
    away = [0x7BFF if a > 0x7BFF else a for a in away]
    assert away != want


def fp16_value(h: int) -> float:
    return float(np.array([h], dtype=np.uint16).view(np.float16)[0])


# ---- P15: asymmetric INT4 of Puzzle 12 (decoder printed, encoder read) ------------
def puzzle12_extract(words: np.ndarray) -> np.ndarray:
    """The page's extract(): value i of a 32-bit word is (word >> 4i) & 0xF."""
    over = np.arange(8, dtype=np.uint32) * 4
    return ((words[..., None] >> over) & np.uint32(0xF)).reshape(*words.shape[:-1], -1)


def zp_input(S, rows=48, cols=1024, seed=71):
    """Weight-like rows (c5 recipe), one group all positive, one all
    negative, one all zero, one symmetric, one constant."""
    x = S.bf16_to_f32(S.make("c5", nrows=rows))[:, :cols].copy()
    x[0, 0:128] = np.abs(x[0, 0:128])
    x[0, 128:256] = -np.abs(x[0, 128:256])
    x[0, 256:384] = 0.0
    x[1, 0:128] = np.linspace(-1, 1, 128, dtype=np.float32)
    x[1, 128:256] = np.float32(0.37)
    return np.ascontiguousarray(x.astype(np.float32))


def test_p15_zp_decoder_is_puzzle12(O, S):
    """Codes and shifts read as 32-bit words through the page's extract(),
    decoded by its sc * (w - sh), give the oracle's x^ bit for bit."""
    x = zp_input(S)
    r = O.quantize(x, "int4zp", "block")
    rows, cols = x.shape
    assert (cols // 128) % 8 == 0                        # whole 32-bit words of shifts per row
    w = puzzle12_extract(r["codes"].view("<u4")).astype(np.int32)                 # [rows, cols]
    sh = puzzle12_extract(r["shifts"].view("<u4")).astype(np.int32)               # [rows, cols / 128]
    assert sh.shape == (rows, cols // 128)
    sc = r["scales"].astype(np.float32)
    want = (np.repeat(sc, 128, axis=1) * (w - np.repeat(sh, 128, axis=1)).astype(np.float32)).astype(np.float32)
    assert np.array_equal(r["xhat"], want)
    d = O.dequantize(r["codes"], r["scales"], "int4zp", "block", rows, cols, shifts=r["shifts"])
    assert np.array_equal(d, r["xhat"])


def test_p15_zp_nearest_grid_point(O, S):
    """Exhaustive search: each code is the grid point k in [-sh, 15 - sh]
    nearest to v = x / sc (binary32 quotient), ties to even k; the scale
    spans the range [min(0, x), max(0, x)] in 15 steps, and the shift puts
    0 within half a step of -lo / sc."""
    x = zp_input(S)
    r = O.quantize(x, "int4zp", "block")
    rows, cols = x.shape
    ng = cols // 128
    w = puzzle12_extract(r["codes"].view("<u4")).astype(np.int64)
    sh = puzzle12_extract(r["shifts"].view("<u4")).astype(np.int64)
    ks = np.arange(-15, 16)
    for i in range(rows):
        for g in range(ng):
            xb = x[i, g * 128:(g + 1) * 128]
            sc, s = np.float32(r["scales"][i, g]), int(sh[i, g])
            lo, hi = min(0.0, float(xb.min())), max(0.0, float(xb.max()))
            if hi == lo:
                assert sc == 0 and s == 0 and not w[i, g * 128:(g + 1) * 128].any()
                continue
            assert abs(15 * float(sc) - (hi - lo)) <= (hi - lo) * 2.0 ** -23
            assert abs(s - (-lo / float(sc))) <= 0.5 + 1e-6
            v = (xb / sc).astype(np.float32).astype(np.float64)
            grid = ks[(ks >= -s) & (ks <= 15 - s)]
            dist = np.abs(v[:, None] - grid[None, :])
            best = dist == dist.min(axis=1, keepdims=True)
            pick = np.array([grid[b][0] if b.sum() == 1 else grid[b][grid[b] % 2 == 0][0] for b in best])
            assert np.array_equal(w[i, g * 128:(g + 1) * 128] - s, pick), (i, g)


def test_p15_zp_bounds_and_textbook_cases(O, S):
    """|x - x^| <= sc/2 inside the grid and <= sc at its ends; an all-positive
    group is unsigned 4-bit quantization (sh = 0, w = clip(rint(x / sc), 0, 15),
    numpy); an all-negative group has sh = 15; an all-zero group has sc = 0;
    the statistics' counts match brute force."""
    x = zp_input(S)
    r = O.quantize(x, "int4zp", "block")
    rows, cols = x.shape
    sh = puzzle12_extract(r["shifts"].view("<u4")).astype(np.int64)
    sc = np.repeat(r["scales"].astype(np.float64), 128, axis=1)
    shr = np.repeat(sh, 128, axis=1)
    v = (x / np.repeat(r["scales"], 128, axis=1)).astype(np.float32).astype(np.float64)
    err = np.abs(x.astype(np.float64) - r["xhat"].astype(np.float64))
    inside = (v <= 15 - shr) & (v >= -shr)
    assert (err[inside] <= sc[inside] * 0.5 * (1 + 2.0 ** -20)).all()
    assert (err <= sc * (1 + 2.0 ** -20)).all()
    assert sh[0, 0] == 0 and sh[0, 1] == 15 and r["scales"][0, 2] == 0.0 and sh[0, 2] == 0
    s0 = np.float32(r["scales"][0, 0])
    want = np.clip(np.rint(x[0, :128] / s0), 0, 15).astype(np.int64)
    assert np.array_equal(puzzle12_extract(r["codes"][0:1, :64].copy().view("<u4"))[0], want)
    st = r["stats"]
    assert st["n_saturated"] == int(np.count_nonzero(~inside & (sc > 0)))
    assert st["n_zero_flush"] == int(np.count_nonzero((x != 0) & (r["xhat"] == 0)))
    assert st["n"] == x.size


def test_p15_zp_special_values(O):
    """NaN maps to w = sh (x^ = 0), +-Inf to the grid ends; a group whose
    range overflows binary32 takes the largest float as its scale."""
    x = np.zeros((2, 256), np.float32)
    x[0, :128] = np.linspace(-2, 2, 128, dtype=np.float32)
    x[0, 5], x[0, 6], x[0, 7] = np.nan, np.inf, -np.inf
    x[1, 0], x[1, 1] = np.float32(3e38), np.float32(-3e38)
    x[1, 128] = np.nan
    r = O.quantize(x, "int4zp", "block")
    w = puzzle12_extract(r["codes"].view("<u4"))
    sh = np.stack([r["shifts"] & 0xF, r["shifts"] >> 4], axis=-1).reshape(2, -1)   # one byte per row
    assert w[0, 5] == sh[0, 0] and r["xhat"][0, 5] == 0.0
    assert w[0, 6] == 15 and w[0, 7] == 0
    assert r["stats"]["n_nonfinite"] == 4
    assert r["scales"][1, 0] == np.float32(3.4028235e38)
    assert np.isfinite(r["xhat"][1]).all()
    assert r["scales"][1, 1] == 0.0 and w[1, 128] == 0


# ---- P16: Puzzle 12's dequantize-then-dot -------------------------------------------
def zp_weights(O, S, n0=48, K=1024, seed=77):
    w = (S.bf16_to_f32(S.make("c5", nrows=n0))[:, :K]).astype(np.float32).copy()
    r = O.quantize(np.ascontiguousarray(w), "int4zp", "block")
    return w, r


def test_p16_zp_gemm_is_puzzle12(O, S):
    """The oracle's loop against the page's own procedure: extract() the
    32-bit words, reshape into groups, broadcast scale and offset, then a
    dot with the activations (numpy, float64)."""
    w, r = zp_weights(O, S)
    n0, K = w.shape
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((24, K)) * 0.7).astype(np.float32)
    z, zabs = O.zp_gemm(r["codes"], r["scales"], r["shifts"], x)
    wq = puzzle12_extract(r["codes"].view("<u4")).astype(np.float64)                  # [n0, K]
    sh = puzzle12_extract(r["shifts"].view("<u4")).astype(np.float64)                 # [n0, K/128]
    G = K // 128
    wd = r["scales"].astype(np.float64)[:, :, None] * (wq.reshape(n0, G, 128) - sh[:, :, None])
    want = wd.reshape(n0, K) @ x.T.astype(np.float64)
    assert np.all(np.abs(z - want) <= 1e-12 * zabs + 1e-300)
    assert np.all(zabs >= np.abs(z))


def test_p16_zp_gemm_identity_and_bound(O, S):
    """Identity activations return the format's x^ exactly (sc * (w - sh)
    rounded once to FP32); any activations give z within the quantization
    bound of the unquantized product, |z - W y| <= sum_l sc_l |y_l|."""
    w, r = zp_weights(O, S, n0=16, K=256)
    n0, K = w.shape
    eye = np.eye(K, dtype=np.float32)
    z, _ = O.zp_gemm(r["codes"], r["scales"], r["shifts"], eye)
    assert np.array_equal(z.astype(np.float32), r["xhat"])
    rng = np.random.default_rng(6)
    x = rng.standard_normal((8, K)).astype(np.float32)
    z, _ = O.zp_gemm(r["codes"], r["scales"], r["shifts"], x)
    exact = w.astype(np.float64) @ x.T.astype(np.float64)
    sc = np.repeat(r["scales"].astype(np.float64), 128, axis=1)
    bound = sc @ np.abs(x.T.astype(np.float64))
    assert np.all(np.abs(z - exact) <= bound * (1 + 1e-9))
    # BF16 activations read as the same values
    xb = S.f32_to_bf16_bits(x)
    zb, _ = O.zp_gemm(r["codes"], r["scales"], r["shifts"], xb)
    z2, _ = O.zp_gemm(r["codes"], r["scales"], r["shifts"], S.bf16_to_f32(xb).astype(np.float32))
    assert np.array_equal(zb, z2)


# ---- P17: FP4 GEMM over two MXFP4 operands -------------------------------------------
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])       # the page's E2M1 value set


def mx_decode_numpy(codes, scales):
    """Dequantize MXFP4 with numpy alone: element 2t in the low nibble,
    E2M1 magnitude by the value table, bit 3 the sign, 2^(E - 127) per 32."""
    lo, hi = codes & 0xF, codes >> 4
    q = np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1).astype(np.int64)
    v = E2M1_VALUES[q & 7] * np.where(q & 8, -1.0, 1.0)
    return v * np.repeat(np.exp2(scales.astype(np.float64) - 127.0), 32, axis=1)


def test_p17_mx_gemm_is_the_product_of_dequantized_operands(O, S):
    """Weights (c3) and activations (a3) quantized to MXFP4 by the oracle:
    the GEMM equals the float64 product of the operands decoded by numpy
    from the page's value table, exactly (every partial sum is a dyadic
    number well inside binary64), and equals the product of the oracle's
    own x^."""
    K = 512
    w = np.ascontiguousarray(S.bf16_to_f32(S.make("c3", nrows=40))[:, :K])
    a = np.ascontiguousarray(S.bf16_to_f32(S.make("a3", nrows=24))[:, :K])
    rw, ra = O.quantize(w, "mxfp4", "block"), O.quantize(a, "mxfp4", "block")
    z, zabs = O.mx_gemm(rw["codes"], rw["scales"], ra["codes"], ra["scales"])
    want = mx_decode_numpy(rw["codes"], rw["scales"]) @ mx_decode_numpy(ra["codes"], ra["scales"]).T
    assert np.array_equal(z, want)
    assert np.array_equal(z, rw["xhat"].astype(np.float64) @ ra["xhat"].astype(np.float64).T)
    assert np.all(zabs >= np.abs(z)) and np.abs(z).max() > 0


def test_p17_mx_gemm_closed_forms(O):
    """All-ones operands give K; a scale of 2^3 on the weights and -1 codes
    on the activations give -8 K; a single nonzero pair gives its product."""
    n0, n1, K = 3, 5, 256
    ones_c = np.full((n0, K // 2), 0x22, dtype=np.uint8)             # E2M1 code 2 = 1.0 in both nibbles
    unit = np.full((n0, K // 32), 127, dtype=np.uint8)
    a_c = np.full((n1, K // 2), 0x22, dtype=np.uint8)
    a_s = np.full((n1, K // 32), 127, dtype=np.uint8)
    z, _ = O.mx_gemm(ones_c, unit, a_c, a_s)
    assert np.all(z == K)
    z, zabs = O.mx_gemm(ones_c, unit + 3, np.full((n1, K // 2), 0xAA, dtype=np.uint8), a_s)   # code 0xA = -1.0
    assert np.all(z == -8.0 * K) and np.all(zabs == 8.0 * K)
    wc = np.zeros((n0, K // 2), dtype=np.uint8)
    ac = np.zeros((n1, K // 2), dtype=np.uint8)
    wc[1, 100] = 0x70                    # element 201 of row 1: 6.0
    ac[4, 100] = 0xD0                    # element 201 of token 4: -3.0
    ws = unit.copy()
    ws[1, 201 // 32] = 125               # 2^-2
    z, _ = O.mx_gemm(wc, ws, ac, a_s)
    want = np.zeros((n0, n1))
    want[1, 4] = 6.0 * 0.25 * -3.0
    assert np.array_equal(z, want)


def test_p17_mxw_gemm_is_the_product_with_dequantized_weights(O, S):
    """MXFP4 weights (c3) against BF16 and FP32 activations: the float64
    product of the numpy-decoded weights with the activations (within the
    float64 rounding of numpy's own sum order), identity activations return
    the weights' x^ exactly, and BF16 bits read as their FP32 values."""
    K = 512
    w = np.ascontiguousarray(S.bf16_to_f32(S.make("c3", nrows=24))[:, :K])
    rw = O.quantize(w, "mxfp4", "block")
    xb = np.ascontiguousarray(S.make("a3", nrows=20)[:, :K])
    z, zabs = O.mxw_gemm(rw["codes"], rw["scales"], xb)
    want = mx_decode_numpy(rw["codes"], rw["scales"]) @ S.bf16_to_f32(xb).astype(np.float64).T
    assert np.all(np.abs(z - want) <= 1e-13 * zabs + 1e-300) and np.abs(z).max() > 0
    z2, _ = O.mxw_gemm(rw["codes"], rw["scales"], S.bf16_to_f32(xb).astype(np.float32))
    assert np.array_equal(z, z2)
    eye, _ = O.mxw_gemm(rw["codes"], rw["scales"], np.eye(K, dtype=np.float32))
    assert np.array_equal(eye.astype(np.float32), rw["xhat"])


# ---- P14: statistics by brute force ------------------------------------------------
@pytest.mark.parametrize("fmt,gran,cfg", [("e4m3", "row", "c2"), ("e5m2", "row", "c2"),
                                          ("int8", "tensor", "c1"), ("mxfp4", "block", "c3"),
                                          ("nvfp4", "block", "c4"), ("int4", "block", "c5")])
def test_p14_stats_bruteforce(O, S, fmt, gran, cfg):
    x = S.make(cfg, nrows=64)
    x.reshape(-1)[::97] = 0          # exact zeros must not count as flushed
    x.reshape(-1)[5::193] = 0x8000 if x.dtype == np.uint16 else np.float32(-0.0)
    r = O.quantize(x, fmt, gran)
    xf = x_f32(S, x)
    x64 = xf.astype(np.float64)
    xh = r["xhat"]
    d = (xf - xh).astype(np.float64)
    st = r["stats"]
    assert st["n"] == x.size
    assert st["n_nonfinite"] == 0
    assert st["sum_x2"] == pytest.approx(np.sum(x64 * x64), rel=1e-12)
    assert st["sum_err2"] == pytest.approx(np.sum(d * d), rel=1e-12)
    assert st["sum_abs_err"] == pytest.approx(np.sum(np.abs(d)), rel=1e-12)
    assert st["max_abs_err"] == np.float32(np.abs(d).max())
    assert st["n_zero_flush"] == int(np.sum((xf != 0) & (xh == 0)))
    assert st["n_zero_flush"] < int(np.sum(xh == 0))
    # d = x - x^ is exact: recomputing in double gives the same values
    assert np.array_equal(d, x64 - xh.astype(np.float64))


def test_dequantize_reproduces_xhat(O, S):
    for fmt, gran, cfg in [("e4m3", "row", "c2"), ("e5m2", "row", "c2"), ("int8", "tensor", "c1"),
                           ("e4m3", "tensor", "c1"), ("mxfp4", "block", "c3"), ("nvfp4", "block", "c4"),
                           ("int4", "block", "c5")]:
        x = S.make(cfg, nrows=32)
        r = O.quantize(x, fmt, gran)
        rows, cols = x.shape
        d = O.dequantize(r["codes"], r["scales"], fmt, gran, rows, cols, r["global_scale"])
        assert np.array_equal(d.view(np.uint32), r["xhat"].view(np.uint32)), fmt
        b = O.dequantize(r["codes"], r["scales"], fmt, gran, rows, cols, r["global_scale"], O.BF16)
        assert np.array_equal(b, S.f32_to_bf16_bits(r["xhat"])), fmt


# ---- readings where the pages are silent (parity unpinned; documented rules) ------
def test_readings_special_values(O):
    x = np.array([[0.0, -0.0, -1e-30, np.nan, np.inf, -np.inf, 1.0, -2.0] * 4], dtype=np.float32)
    r = O.quantize(x, "e4m3", "row")
    c = r["codes"][0]
    assert r["scales"][0] == np.float32(2.0) / np.float32(448.0)   # absmax over finite values
    assert c[0] == 0x00 and c[1] == 0x80 and c[2] == 0x80            # sign kept on zero
    assert c[3] == 0x7F                                               # NaN -> NaN code
    assert c[4] == 0x7E and c[5] == 0xFE                              # +-Inf saturate
    st = r["stats"]
    assert st["n_nonfinite"] == 12 and st["n"] == 32
    assert st["n_saturated"] == 8                                     # the infinities
    assert np.isfinite(st["sum_err2"])
    z = O.quantize(np.zeros((2, 32), np.float32), "int8", "row")
    assert (z["codes"] == 0).all() and (z["scales"] == 0).all() and (z["xhat"] == 0).all()
    m = O.quantize(x, "mxfp4", "block")
    nib = [(m["codes"][0, i // 2] >> (4 * (i % 2))) & 0xF for i in range(8)]
    assert nib[3] == 0 and nib[4] == 0x7 and nib[5] == 0xF and nib[1] == 0x8


def test_empty_and_invalid(O):
    r = O.quantize(np.zeros((0, 32), np.float32), "e4m3", "row")
    assert r["stats"]["n"] == 0
    with pytest.raises(ValueError):
        O.quantize(np.zeros((2, 48), np.float32), "mxfp4", "block")   # 48 % 32 != 0
    with pytest.raises(ValueError):
        O.quantize(np.zeros((2, 32), np.float32), "mxfp4", "row")
