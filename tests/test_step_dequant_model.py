"""The optimizer step's dequantization, instruction by instruction, in exact
FP32 arithmetic on the CPU (tests/fp32_model.py).

The kernel decodes a stored moment as amax * 2^(L(c)/k), L(c) = log2(|dec c|
/ MAX) read from a per-code table as a hi + lo FP32 pair and 1/k carried as
hi + lo, so that only the final exp2 rounds noticeably:

    ih = rcp(k);  il = fma(-k, ih, 1) * ih
    ph = L.hi * ih;  pl = fma(L.hi, ih, -ph);  pl = fma(L.hi, il, pl);  pl = fma(L.lo, ih, pl)
    x  = exp2(ph) * fma(amax * ln2, pl, amax)             (fast form)
    x  = ldexp(exp2(ph - n) * fma(ma * ln2, pl, ma), ea + n),  n = max(rint(ph), -1024),
         amax = ma 2^ea                                    (wide form)

A zero code has no logarithm; its table entry is a large negative number Z
so that exp2(ph) is exactly 0.  The method maps zero to zero (the COAT
explainer, section "expansion function": the expansion keeps sign(x), with
sign(0) = 0), so the product must be exactly 0 -- which needs the second
factor finite.  It is not when Z is so large that the correction term
Z * il, times amax ln2, overflows: with Z = -2^100 a zero code in a group
with amax around 1e17 and k of a few decodes to 0 * inf = NaN.  The step now
uses Z = -2^40, which still sends exp2 to 0 for every k the step can store,
and takes the fast form only for amax <= 2^100, where the correction term is
bounded far below FP32's range.  These tests show the old failure and check
the bound of the new scheme over the whole (k, amax) range, with the native
reciprocal's one-ulp error.
"""
import math

import numpy as np
import pytest

import fp32_model as F
import oracle as orc

LN2F = float(np.float32(math.log(2.0)))
MAX = {"e4m3": 448.0, "e5m2": 57344.0}
# log2(MAX / smallest subnormal), rounded to FP32 as the host passes it
LOG2_RANGE = {"e4m3": float(np.float32(math.log2(448.0) + 9.0)), "e5m2": float(np.float32(math.log2(57344.0) + 16.0))}
Z_OLD, Z_NEW = -(2.0 ** 100), -(2.0 ** 40)
FAST_AMAX_MAX = 2.0 ** 100   # the fast form is taken only for amax at most this
LG_FLOOR = float(np.float32(8.5e-8))  # the step's floor on log2(amax / amin) when forming k


def table_entry(fmt, code, zero_entry):
    """(hi, lo) of log2(|dec c| / MAX), binary64 rounded hi then lo, as the host builds it."""
    mag = code & 0x7F
    if mag == 0 or mag > orc.fmt_max_code(fmt):
        return zero_entry, 0.0
    L = math.log2(orc.decode(fmt, mag)) - math.log2(MAX[fmt])
    hi = float(np.float32(L))
    return hi, float(np.float32(L - hi))


def corrections(entry, k, ih):
    il = F.mul(F.fma(-k, ih, 1.0), ih)
    ph = F.mul(entry[0], ih)
    pl = F.fma(entry[0], ih, -ph)
    pl = F.fma(entry[0], il, pl)
    pl = F.fma(entry[1], ih, pl)
    return ph, pl


def dequant_fast(entry, amax, k, ih):
    ph, pl = corrections(entry, k, ih)
    return F.mul(F.exp2(ph), F.fma(F.mul(amax, LN2F), pl, amax))


def dequant_wide(entry, amax, k, ih):
    ph, pl = corrections(entry, k, ih)
    if amax == 0.0:
        ma, ea = 0.0, 0
    else:
        ma, ea = F.frexp(amax)
    n = max(F.rint(ph), -1024.0)
    return F.ldexp(F.mul(F.exp2(F.add(ph, -n)), F.fma(F.mul(ma, LN2F), pl, ma)), ea + int(n))


def fast_form_allowed(fmt, k, amax):
    return F.mul(k, 120.0) >= LOG2_RANGE[fmt] and amax <= FAST_AMAX_MAX


def k_extremes(fmt):
    """The smallest and largest k the step stores: log2 R_fmt over the widest
    FP32 group range (max float over min denormal) and over the floor of the
    narrowest one."""
    k_min = F.rn(np.float64(LOG2_RANGE[fmt]) / math.log2(float(np.finfo(np.float32).max) / 2.0 ** -149))
    k_max = F.mul(LOG2_RANGE[fmt], F.rcp(LG_FLOOR)) * (1 + 2.0 ** -22)
    return k_min, k_max


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_old_zero_entry_gives_nan_for_large_narrow_groups(fmt):
    """The cause of the failure: Z = -2^100, amax 1e17 .. 1e20, k of a few --
    some zero codes decode to NaN (0 * inf) in the fast form."""
    e = table_entry(fmt, 0, Z_OLD)
    nan_ks = []
    for amax in (float(np.float32(1e17)), float(np.float32(1e20))):
        for k in np.float32(np.linspace(1.5, 12.5, 221)):
            k = float(k)
            if not (F.mul(k, 120.0) >= LOG2_RANGE[fmt]):
                continue
            x = dequant_fast(e, amax, k, F.rcp(k))
            if math.isnan(x):
                nan_ks.append((amax, k))
            else:
                assert x == 0.0
    assert nan_ks, "expected the old table entry to overflow"


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_zero_code_decodes_to_zero_over_the_whole_state_range(fmt):
    """Z = -2^40: every zero code decodes to exactly 0 in both forms, for k
    over [k_min, k_max] (with the reciprocal one ulp either way) and amax
    from the smallest denormal to the largest float; the fast form is only
    checked where the step takes it."""
    rng = np.random.default_rng(5)
    k_min, k_max = k_extremes(fmt)
    ks = sorted(set(float(np.float32(v)) for v in
                    list(np.geomspace(k_min, k_max, 100)) + list(10 ** rng.uniform(math.log10(k_min),
                                                                                    math.log10(k_max), 40))
                    + [k_min, k_max, 1.0, 2.05, 3.3, 5.37, 7.0, 12.5]))
    amaxes = sorted(set([2.0 ** -149, 2.0 ** -126, 2.0 ** -120, 1.0, 1e17, 1e20, 1e30, FAST_AMAX_MAX,
                         float(np.nextafter(np.float32(FAST_AMAX_MAX), np.float32(np.inf))), 1e35,
                         float(np.finfo(np.float32).max)]
                        + [float(np.float32(v)) for v in 10 ** rng.uniform(-44, 38, 12)]))
    for code in (0x00, 0x80):
        e = table_entry(fmt, code, Z_NEW)
        for k in ks:
            for ih in F.ulp_neighbours(F.rcp(k)):
                for amax in amaxes:
                    assert dequant_wide(e, amax, k, ih) == 0.0, (code, k, ih, amax)
                    if fast_form_allowed(fmt, k, amax):
                        assert dequant_fast(e, amax, k, ih) == 0.0, (code, k, ih, amax)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_zero_entry_bound(fmt):
    """The two facts the choice of Z rests on, at their worst cases:
    exp2(Z / k_max) is 0, and |Z * il| * amax ln2 stays finite for the
    largest 1/k of the fast form at amax = 2^100."""
    k_min, k_max = k_extremes(fmt)
    assert F.exp2(F.mul(Z_NEW, F.ulp_neighbours(F.rcp(k_max))[2])) == 0.0
    k_fast = float(np.float32(LOG2_RANGE[fmt] / 120.0))
    while F.mul(k_fast, 120.0) < LOG2_RANGE[fmt]:
        k_fast = float(np.nextafter(np.float32(k_fast), np.float32(np.inf)))
    worst = 0.0
    for k in np.float32(np.linspace(k_fast, 2 * k_fast, 400)):
        for ih in F.ulp_neighbours(F.rcp(float(k))):
            _, pl = corrections((Z_NEW, 0.0), float(k), ih)
            worst = max(worst, abs(pl))
    assert worst < 2.0 ** 24
    assert math.isfinite(F.fma(F.mul(FAST_AMAX_MAX, LN2F), worst, FAST_AMAX_MAX))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_nonzero_codes_unchanged_and_accurate(fmt):
    """Nonzero codes do not read Z: both forms agree with the binary64 value
    amax (|dec c| / MAX)^(1/k) to a few ulps (the model's exp2 is correctly
    rounded; the hardware's is within an ulp)."""
    rng = np.random.default_rng(9)
    codes = [c for c in range(1, orc.fmt_max_code(fmt) + 1)]
    for _ in range(300):
        c = int(rng.choice(codes))
        k = float(np.float32(10 ** rng.uniform(math.log10(LOG2_RANGE[fmt] / 120.0) + 0.01, 3)))
        amax = float(np.float32(10 ** rng.uniform(-30, 30)))
        want = amax * (orc.decode(fmt, c) / MAX[fmt]) ** (1.0 / k)
        e = table_entry(fmt, c, Z_NEW)
        for form in (dequant_fast, dequant_wide):
            got = form(e, amax, k, F.rcp(k))
            assert abs(got - want) <= 4 * float(np.spacing(np.float32(want))), (form.__name__, c, k, amax)
