"""CPU proof that the GPU fast paths compute the method's quotient x / s.

The post "浅谈低精度浮点数" (section "FP8") defines v = x / s, one correctly
rounded binary32 division.  The kernels replace the division by a
correction step from a rounded reciprocal (a constant one for the scale
derivations alpha / Q and A / 6, A / 7; a per-unit one for x / s), and the
INT4 kernel takes the reciprocals of its FP16 scales from a table.
division_check.c restates that arithmetic in C and compares it bit for bit
with the division over every input the kernels apply it to (or, for the
NVFP4 scales and FP32 inputs, over seeded samples).  Any mismatch fails.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path_factory.mktemp("divcheck") / "division_check")
    cmd = ["gcc", "-O3", "-march=native", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-o", exe,
           os.path.join(HERE, "division_check.c"), "-lm"]
    subprocess.run(cmd, check=True)
    return exe


def run(checker, what):
    threads = str(max(1, min(8, os.cpu_count() or 1)))
    out = subprocess.run([checker, what], check=True, capture_output=True, text=True,
                         env={**os.environ, "OMP_NUM_THREADS": threads}).stdout
    rows = [ln.split() for ln in out.strip().splitlines()]
    return {r[0]: (int(r[1]), int(r[2])) for r in rows}


def test_constant_divisors_exhaustive(checker):
    """alpha / 127, / 448, / 57344, A / 6, A / 7 and the asymmetric INT4
    span / 15 for every finite binary32 value >= 0."""
    res = run(checker, "divconst")
    assert set(res) == {"divconst_6", "divconst_7", "divconst_15", "divconst_127", "divconst_448",
                        "divconst_57344"}
    for name, (n, bad) in res.items():
        assert n == 0x7F800000, name          # every non-negative finite binary32 pattern
        assert bad == 0, f"{name}: {bad} quotients differ from the division"


def test_row_scales_every_bf16_pair(checker):
    """Per-row INT8 / E4M3 / E5M2 on BF16 input: every absmax alpha of the
    fast range and every BF16 x with |x| <= alpha."""
    res = run(checker, "row_bf16")
    for q in ("127", "448", "57344"):
        n, bad = res[f"row_bf16_{q}"]
        assert n > 4e8 and bad == 0, (q, n, bad)


def test_int4_fp16_scales(checker):
    """Every normal FP16 group scale: the table reciprocal is RN(1/sf), and
    every BF16 x with |x| <= 7.5 sf divides exactly."""
    res = run(checker, "int4_fp16")
    assert res["int4_fp16_table"] == (30720, 0)
    n, bad = res["int4_fp16"]
    assert n > 1e9 and bad == 0


def test_nvfp4_block_scales(checker):
    res = run(checker, "nvfp4")
    n, bad = res["nvfp4"]
    assert n > 2e8 and bad == 0
    n, bad = res["nvfp4_block_scale"]
    assert n > 1e5 and bad == 0


def test_random_fp32_pairs(checker):
    res = run(checker, "random_f32")
    assert len(res) == 5
    for name, (n, bad) in res.items():
        assert n == 10 ** 8 and bad == 0, name


def test_int4zp_groups(checker):
    """Asymmetric INT4 (Triton post, Puzzle 12): the group scale span / 15
    by the constant-divisor correction, the shift RNE(nlo / sc) from the
    corrected quotient, and the corrected quotient of every BF16 x of the
    group's range, over seeded group ranges."""
    res = run(checker, "int4zp")
    groups, bad = res["int4zp_scale"]
    assert groups > 20000 and bad == 0
    assert res["int4zp_shift"] == (groups, 0)
    n, bad = res["int4zp"]
    assert n > 5e8 and bad == 0


def test_int4_scale_double_rounding(checker):
    """The INT4 scale is fp16(fl32(A / 7)) (post "浅谈低精度浮点数", section
    "FP4 / MXFP4 / NVFP4": s = A / 7 kept in FP16).  Rounding the quotient
    to binary32 first never changes the binary16 result: every finite
    binary32 A up to the binary16 range gives the same code as one rounding
    of the exact quotient."""
    n, bad = run(checker, "a7_double_rounding")["a7_double_rounding"]
    assert n > 1e9 and bad == 0
