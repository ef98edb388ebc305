"""Pins of the oracle's dynamic-range expansion (C2 quantize, C3 dequantize).

What fixes them, with no implementation to compare against:
* k = 1 is plain absmax scaling -- the "naive" baseline the COAT explainer
  compares against -- so forcing k = 1 must reproduce the oracle's 1xG group
  quantization (a separate division-based code path) code for code;
* by construction the expanded group spans exactly the format's range: the
  group max lands on the largest code and the smallest nonzero magnitude on
  the smallest subnormal code; signs survive (sign(0) = 0);
* dequantize(quantize(x)) is within the format's half-spacing, mapped back
  through the inverse power 1/k;
* degenerate groups (all zero, all equal, a single nonzero) follow the
  readings stated in coat_oracle.c.
"""
import numpy as np
import pytest

FMTS = ["e4m3", "e5m2"]


def bf16_round(x):
    """Round float32 values to the nearest BF16 value (RNE), as uint16 bits."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_to_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def random_groups(rng, n_groups, G, decades, signed=True, zero_frac=0.0):
    """Groups with log-uniform magnitudes over `decades` decades around a
    per-group random scale."""
    scale = 10.0 ** rng.uniform(-12, 2, (n_groups, 1))
    mag = scale * 10.0 ** rng.uniform(-decades, 0, (n_groups, G))
    sign = rng.choice([-1.0, 1.0], (n_groups, G)) if signed else 1.0
    x = (mag * sign).astype(np.float32)
    if zero_frac:
        x[rng.random((n_groups, G)) < zero_frac] = 0.0
    return x


def test_k1_is_plain_absmax_scaling(orc):
    rng = np.random.default_rng(11)
    G = 128
    x = bf16_round(rng.standard_normal((64, G)) * 10.0 ** rng.uniform(-3, 3, (64, 1)))
    x[3, :] = 0  # an all-zero group too
    codes_g, scales, partial = orc.quant_group(x, G)
    for gi in range(x.shape[0]):
        codes_e, amax, k = orc.expand_quantize("e4m3", bf16_to_f32(x[gi]), k_force=1.0)
        assert (codes_e == codes_g[gi * G:(gi + 1) * G]).all(), gi
        assert amax == partial[gi]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("G", [32, 128, 512])
@pytest.mark.parametrize("decades", [0.5, 3, 6, 12])
def test_expanded_group_fills_range(orc, fmt, G, decades):
    rng = np.random.default_rng(FMTS.index(fmt) * 100000 + G * 100 + int(decades * 10))
    top = orc.fmt_max_code(fmt)
    x = random_groups(rng, 24, G, decades, zero_frac=0.05)
    for row in x:
        codes, amax, k = orc.expand_quantize(fmt, row)
        a = np.abs(row.astype(np.float64))
        nz = a > 0
        assert amax == a.max()
        mag = codes & 0x7F
        # group max -> largest code; smallest nonzero -> smallest subnormal code
        assert (mag[a == a.max()] == top).all()
        assert (mag[a == a[nz].min()] == 1).all()
        # signs preserved, zeros map to code 0, nonzero never to a zero code
        assert ((codes & 0x80)[row < 0] == 0x80).all()
        assert ((codes & 0x80)[row > 0] == 0).all()
        assert (codes[~nz] == 0).all()
        assert (mag[nz] > 0).all()
        # k stretches the group's range onto the format's range
        r_fmt = orc.fmt_max(fmt) / orc.fmt_min_subnormal(fmt)
        r_grp = a.max() / a[nz].min()
        assert abs(np.log(r_grp) * k - np.log(r_fmt)) < 1e-6 * np.log(r_fmt)
        # a narrow group is stretched (k > 1); one wider than the format is squeezed
        assert (k > 1) == (r_grp < r_fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_nonnegative_groups_have_no_sign_bits(orc, fmt):
    rng = np.random.default_rng(5)
    x = random_groups(rng, 16, 128, 2, signed=False)
    for row in x:
        codes, _, _ = orc.expand_quantize(fmt, row)
        assert (codes & 0x80 == 0).all()


def half_spacing(fmt, y):
    """Half the distance between neighbouring grid values at magnitude y."""
    mbits = 3 if fmt == "e4m3" else 2
    emin = -6 if fmt == "e4m3" else -14  # exponent of the smallest normal
    e = np.maximum(np.floor(np.log2(np.maximum(y, 1e-300))), emin)
    return 0.5 * np.exp2(e - mbits)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("decades", [1, 4, 8])
def test_roundtrip_error_bound(orc, fmt, decades):
    rng = np.random.default_rng(17 + decades)
    vmax = orc.fmt_max(fmt)
    x = random_groups(rng, 16, 128, decades, zero_frac=0.02)
    for row in x:
        codes, amax, k = orc.expand_quantize(fmt, row)
        back = orc.expand_dequantize(fmt, codes, amax, k)
        a = np.abs(row.astype(np.float64))
        nz = a > 0
        assert (back[~nz] == 0).all()
        assert (np.sign(back[nz]) == np.sign(row[nz])).all()
        y = vmax * (a[nz] / amax) ** np.float64(k)   # expanded magnitude
        h = half_spacing(fmt, y) * (1 + 1e-6)        # + FP32 rounding of y
        lo = (np.maximum(y - h, 0) / y) ** (1 / np.float64(k))
        hi = ((y + h) / y) ** (1 / np.float64(k))
        ratio = np.abs(back[nz]) / a[nz]
        assert (ratio >= lo * (1 - 1e-12)).all() and (ratio <= hi * (1 + 1e-12)).all()


def test_dequantize_of_special_codes(orc):
    # code 0 / 0x80 and an all-zero group decode to zero
    assert orc.expand_dequantize("e4m3", [0x00, 0x80], 3.0, 2.0).tolist() == [0.0, 0.0]
    assert orc.expand_dequantize("e4m3", [0x7E, 0x01], 0.0, 1.0).tolist() == [0.0, 0.0]
    # the largest code gives back amax for any k; its negative gives -amax
    for k in [0.3, 1.0, 7.5]:
        assert orc.expand_dequantize("e5m2", [0x7B, 0xFB], 2.5, k).tolist() == [2.5, -2.5]


@pytest.mark.parametrize("fmt", FMTS)
def test_degenerate_groups(orc, fmt):
    top = orc.fmt_max_code(fmt)
    z = np.zeros(128, np.float32)
    codes, amax, k = orc.expand_quantize(fmt, z)
    assert (codes == 0).all() and amax == 0 and k == 1
    eq = np.full(128, -0.75, np.float32)
    eq[::3] = 0.75
    codes, amax, k = orc.expand_quantize(fmt, eq)
    assert k == 1 and amax == np.float32(0.75)
    assert ((codes & 0x7F) == top).all()
    one = np.zeros(128, np.float32)
    one[17] = -3e-7
    codes, amax, k = orc.expand_quantize(fmt, one)
    assert k == 1 and codes[17] == 0x80 | top and (np.delete(codes, 17) == 0).all()


def test_wide_group_gets_k_below_one(orc):
    # ten decades exceed both formats' ranges, so the group is compressed (k < 1)
    x = np.array([1e-8, 1e-5, -3e-3, 1e2] * 32, dtype=np.float32)
    for fmt in FMTS:
        codes, amax, k = orc.expand_quantize(fmt, x)
        assert 0 < k < 1
        assert (codes[x == np.float32(1e-8)] & 0x7F == 1).all()


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_with_given_scale_and_k(orc, fmt):
    """The quantizer's last step on its own (orc_expand_encode): with a group's
    own stored (amax, k) it gives the group's codes; the stored max maps to
    the largest code, amax (min_sub / MAX)^(1/k) to the smallest subnormal
    code, zero to zero, and the sign is carried; with k = 1 it is the plain
    absmax cast of a value that need not be FP32."""
    rng = np.random.default_rng(23)
    G = 128
    x = random_groups(rng, 40, G, 5, zero_frac=0.05)
    codes, amax, k = orc.expand_quantize_groups(fmt, x.ravel(), G)
    again = orc.expand_encode_groups(fmt, x.ravel().astype(np.float64), G, amax, k)
    assert (again == codes).all()
    top, mx, ms = orc.fmt_max_code(fmt), orc.fmt_max(fmt), orc.fmt_min_subnormal(fmt)
    a = np.float32(3.0e-5)
    for kk in (0.3, 1.0, 2.5, 9.0):
        kf = np.float32(kk)
        lo = float(a) * (ms / mx) ** (1.0 / float(kf))
        got = orc.expand_encode_groups(fmt, np.array([float(a), -float(a), lo, -lo, 0.0, 0.0] + [0.0] * (G - 6)), G,
                                       np.array([a], np.float32), np.array([kf], np.float32))
        assert list(got[:5]) == [top, 0x80 | top, 1, 0x81, 0]
    # k = 1: RNE_sat(MAX x / amax) of binary64 x, e.g. a midpoint between two codes
    c = 0x30 if fmt == "e4m3" else 0x30
    mid = 0.5 * (orc.decode(fmt, c) + orc.decode(fmt, c + 1))
    want = orc.encode(fmt, float(np.float32(mid)))
    got = orc.expand_encode_groups(fmt, np.array([mid * float(a) / mx] + [0.0] * (G - 1)), G,
                                   np.array([a], np.float32), np.array([1.0], np.float32))
    assert got[0] == want
