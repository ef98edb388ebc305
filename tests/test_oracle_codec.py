"""Pins of the oracle's FP8 codec (C1) against what the pages and the
mathematics fix: the printed format constants, the worked E2M2 grid, the
1.75 / 0.875 mantissa checks, brute force over all codes, torch's own FP8
dtypes (an independent implementation) and the round-to-nearest-even rule."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import golden_rows

FMTS = ["e4m3", "e5m2"]
TORCH_DT = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


def test_page_constants(orc):
    rows = golden_rows("fp8_formats.txt")
    assert {r[0] for r in rows} == set(FMTS)
    for fmt, s, e, m, vmax, lmin, sp1 in rows:
        assert orc.fmt_max(fmt) == float(vmax)
        assert orc.fmt_min_subnormal(fmt) == 2.0 ** int(lmin)
        one = orc.encode(fmt, 1.0)
        assert orc.decode(fmt, one) == 1.0
        assert orc.decode(fmt, one + 1) - 1.0 == float(sp1)
        # the bit split is what the grid size says: 2^(1+e+m) codes in all
        assert 1 + int(e) + int(m) == 8 and int(s) == 1
        n_mant = 2 ** int(m)
        # subnormal step = min subnormal; first normal = 2^(1-bias) = n_mant * min_sub
        assert orc.decode(fmt, n_mant) == n_mant * orc.fmt_min_subnormal(fmt)


def test_coat_e4m3_range(orc):
    # the COAT explainer's E4M3 range 448 / 2^-9 ~ 2e5
    r = orc.fmt_max("e4m3") / orc.fmt_min_subnormal("e4m3")
    assert r == 448 * 2 ** 9 and 1.5e5 < r < 2.5e5


def test_mantissa_checks(orc):
    for fmt, code, sig, exp in golden_rows("fp8_mantissa_checks.txt"):
        assert orc.decode(fmt, int(code, 16)) == float(sig) * 2.0 ** int(exp)


def test_e2m2_worked_grid(orc):
    (row,) = golden_rows("e2m2_grid.txt")
    want = [float(Fraction(v)) for v in row]
    got = [orc.decode("e2m2", c) for c in range(16)]
    assert got == want
    # negative half mirrors it
    assert [orc.decode("e2m2", 16 + c) for c in range(16)] == [-w for w in want]


@pytest.mark.parametrize("fmt", FMTS)
def test_decode_all_codes_vs_torch(orc, fmt):
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.decode_all(fmt, codes)
    ref = torch.from_numpy(codes).view(TORCH_DT[fmt]).to(torch.float64).numpy()
    nan_ours, nan_ref = np.isnan(ours), np.isnan(ref)
    assert (nan_ours == nan_ref).all()
    assert (ours[~nan_ours] == ref[~nan_ref]).all()
    # inf only in E5M2
    assert np.isinf(ours).sum() == (2 if fmt == "e5m2" else 0)


@pytest.mark.parametrize("fmt", FMTS)
def test_grid_is_monotone_and_roundtrips(orc, fmt):
    top = orc.fmt_max_code(fmt)
    assert top == (0x7E if fmt == "e4m3" else 0x7B)
    vals = [orc.decode(fmt, c) for c in range(top + 1)]
    assert all(b > a for a, b in zip(vals, vals[1:]))
    for c in range(256):
        d = orc.decode(fmt, c)
        if not np.isfinite(d):
            continue
        want = 0 if d == 0 else c
        assert orc.encode(fmt, d) == want


@pytest.mark.parametrize("fmt", FMTS)
def test_midpoints_round_to_even(orc, fmt):
    top = orc.fmt_max_code(fmt)
    for c in range(top):
        lo, hi = orc.decode(fmt, c), orc.decode(fmt, c + 1)
        mid = (lo + hi) / 2  # exact in binary64
        even = c if c % 2 == 0 else c + 1
        assert orc.encode(fmt, mid) == (0 if even == 0 else even)
        assert orc.encode(fmt, -mid) == (0 if even == 0 else 0x80 | even)
        above = np.nextafter(mid, np.inf)
        below = np.nextafter(mid, -np.inf)
        assert orc.encode(fmt, above) == c + 1
        assert orc.encode(fmt, below) == c


@pytest.mark.parametrize("fmt", FMTS)
def test_saturation(orc, fmt):
    top = orc.fmt_max_code(fmt)
    vmax = orc.fmt_max(fmt)
    for x in [vmax, vmax * 1.03, vmax * 1.2, vmax * 2, 1e30, np.inf]:
        assert orc.encode(fmt, x) == top
        assert orc.encode(fmt, -x) == 0x80 | top


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_vs_torch_cast_in_range(orc, fmt):
    """torch's FP8 casts round to nearest even but do not saturate, so they
    check the oracle on |x| <= MAX only (inputs are FP32 values)."""
    rng = np.random.default_rng(7)
    vmax = orc.fmt_max(fmt)
    lo = np.log2(orc.fmt_min_subnormal(fmt)) - 3
    mag = np.exp2(rng.uniform(lo, np.log2(vmax), 20000))
    x = (mag * rng.choice([-1.0, 1.0], mag.size)).astype(np.float32)
    x = x[np.abs(x) <= vmax]
    ours = orc.encode_all(fmt, x.astype(np.float64))
    ref = torch.from_numpy(x).to(TORCH_DT[fmt]).view(torch.uint8).numpy().copy()
    ref[(ref & 0x7F) == 0] = 0  # the oracle writes no negative zero
    assert (ours == ref).all()
