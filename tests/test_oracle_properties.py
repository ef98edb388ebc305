"""Property tests of the oracle's expansion quantizer over generated groups
(hypothesis): the invariants that hold by construction -- the group max on
the top code, the smallest nonzero magnitude on code 1, signs kept, zeros
kept, no nonzero value on a zero code -- the dequant(quant) bound, and
exact invariance under a power-of-two scale of the whole group."""
import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

FMTS = ["e4m3", "e5m2"]


def groups(G):
    """A 1xG FP32 group: per-element log10 magnitude within a random window,
    random signs, some exact zeros; at least one nonzero."""
    return st.tuples(
        st.floats(min_value=-30.0, max_value=30.0),                       # window centre
        st.floats(min_value=0.0, max_value=12.0),                         # window width, decades
        st.lists(st.floats(min_value=0.0, max_value=1.0), min_size=G, max_size=G),
        st.lists(st.booleans(), min_size=G, max_size=G),                  # signs
        st.lists(st.integers(min_value=0, max_value=19), min_size=G, max_size=G),  # 0 -> zero (5%)
    ).map(lambda t: _build(*t)).filter(lambda x: (x != 0).any())


def _build(centre, width, u, neg, z):
    mag = 10.0 ** (centre - width * np.asarray(u))
    x = np.where(np.asarray(neg), -mag, mag)
    x[np.asarray(z) == 0] = 0.0
    return x.astype(np.float32)


def half_spacing(fmt, y):
    mbits = 3 if fmt == "e4m3" else 2
    emin = -6 if fmt == "e4m3" else -14
    e = np.maximum(np.floor(np.log2(np.maximum(y, 1e-300))), emin)
    return 0.5 * np.exp2(e - mbits)


@pytest.mark.parametrize("fmt", FMTS)
@settings(max_examples=150, deadline=None)
@given(x=groups(32))
def test_invariants(orc, fmt, x):
    codes, amax, k = orc.expand_quantize(fmt, x)
    a = np.abs(x.astype(np.float64))
    nz = a > 0
    mag = codes & 0x7F
    assert amax == a.max()
    assert (mag[a == a.max()] == orc.fmt_max_code(fmt)).all()
    if a[nz].min() < a.max():
        assert (mag[a == a[nz].min()] == 1).all()
    else:
        assert k == 1.0
    assert ((codes & 0x80)[x < 0] == 0x80).all() and ((codes & 0x80)[x > 0] == 0).all()
    assert (codes[~nz] == 0).all() and (mag[nz] > 0).all()


@pytest.mark.parametrize("fmt", FMTS)
@settings(max_examples=150, deadline=None)
@given(x=groups(32))
def test_roundtrip_bound(orc, fmt, x):
    codes, amax, k = orc.expand_quantize(fmt, x)
    back = orc.expand_dequantize(fmt, codes, amax, k)
    a = np.abs(x.astype(np.float64))
    nz = a > 0
    y = orc.fmt_max(fmt) * (a[nz] / amax) ** np.float64(k)
    h = half_spacing(fmt, y) * (1 + 1e-6)
    lo = (np.maximum(y - h, 0) / y) ** (1 / np.float64(k))
    hi = ((y + h) / y) ** (1 / np.float64(k))
    ratio = np.abs(back[nz]) / a[nz]
    assert (ratio >= lo * (1 - 1e-12)).all() and (ratio <= hi * (1 + 1e-12)).all()
    assert (back[~nz] == 0).all()


@pytest.mark.parametrize("fmt", FMTS)
@settings(max_examples=100, deadline=None)
@given(x=groups(32), p=st.integers(min_value=-20, max_value=20))
def test_power_of_two_scale_invariance(orc, fmt, x, p):
    """Scaling a group by 2^p scales amax by 2^p and changes neither k nor any
    code (every ratio |x|/amax is unchanged), while no value leaves the
    normal FP32 range."""
    a = np.abs(x[x != 0]).astype(np.float64)
    if a.min() * 2.0 ** p < 2.0 ** -120 or a.max() * 2.0 ** p > 2.0 ** 120 or \
            a.min() < 2.0 ** -120 or a.max() > 2.0 ** 120:
        return
    c1, a1, k1 = orc.expand_quantize(fmt, x)
    c2, a2, k2 = orc.expand_quantize(fmt, (x.astype(np.float64) * 2.0 ** p).astype(np.float32))
    assert (c1 == c2).all() and k1 == k2 and a2 == np.float32(a1 * 2.0 ** p)
