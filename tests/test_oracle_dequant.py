"""Pins of the oracle's BF16 rounding, the BF16 working copy of the step, and
the activation dequantization for the backward pass -- against torch's own
BF16 and FP8 conversions (independent implementations) and against the
error bound of a quantize/dequantize round trip."""
import numpy as np
import pytest
import torch

from activation_compression_amd import inputs


def torch_bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_rne_matches_torch(orc):
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 20000).astype(np.float32),
        # exact BF16 midpoints (ties) and their neighbours
        ((rng.integers(0, 1 << 15, 4000).astype(np.uint32) << 16) | 0x8000).view(np.float32),
        ((rng.integers(0, 1 << 15, 4000).astype(np.uint32) << 16) | 0x8001).view(np.float32),
        ((rng.integers(0, 1 << 15, 4000).astype(np.uint32) << 16) | 0x7FFF).view(np.float32),
        # FP32 subnormals and the top of the range
        (rng.integers(1, 1 << 23, 2000).astype(np.uint32)).view(np.float32),
        np.array([3.3895313e38, 3.39e38, 3.4028235e38, -3.4028235e38, 0.0, -0.0], np.float32),
    ])
    x = x[np.isfinite(x)]
    assert (orc.bf16_rne(x) == torch_bf16_bits(x)).all()


def test_dequant_matches_torch_casts(orc):
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 256, 64 * 256).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x12  # no NaN codes
    scales = (np.abs(rng.standard_normal(64 * 2)) * 10.0 ** rng.uniform(-4, 4, 128)).astype(np.float32)
    got = orc.dequant_group(codes, 64, 256, 128, scales)
    val = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().reshape(64, 2, 128)
    want = (val * torch.from_numpy(scales).reshape(64, 2, 1)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (got == want.reshape(-1)).all()
    got_t = orc.dequant_per_tensor(codes, scales[0])
    want_t = (torch.from_numpy(codes).view(torch.float8_e4m3fn).float() * float(scales[0])).to(torch.bfloat16)
    assert (got_t == want_t.view(torch.int16).numpy().view(np.uint16)).all()


def test_power_of_two_scale_is_exact(orc):
    # an E4M3 value times 2^j is exactly representable in BF16
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]
    for j in (-20, 0, 7):
        got = orc.dequant_per_tensor(codes, 2.0 ** j)
        exact = np.array([orc.decode("e4m3", c) * 2.0 ** j for c in codes], np.float32)
        assert (got == torch_bf16_bits(exact)).all()
        assert ((got.astype(np.uint32) << 16).view(np.float32) == exact).all()


@pytest.mark.parametrize("G", [32, 128])
def test_group_roundtrip_error_bound(orc, G):
    """quantize then dequantize: within half an E4M3 spacing (scaled) plus half
    a BF16 spacing of the result."""
    spec = inputs.ActivationSpec("t", 32, 1024, seed=3)
    x = inputs.gen_activation(spec).numpy().view(np.uint16)
    codes, scales, partial = orc.quant_group(x, G)
    back = orc.dequant_group(codes, 32, 1024, G, scales)
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64).reshape(-1)
    bf = (back.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    sc = np.repeat(scales.astype(np.float64), G)
    y = np.abs(xf) / sc  # the value on the E4M3 grid scale, <= 448
    e = np.maximum(np.floor(np.log2(np.maximum(y, 1e-300))), -6)
    half_fp8 = 0.5 * np.exp2(e - 3) * sc
    half_bf16 = 0.5 * np.spacing(np.abs(bf).astype(np.float32)).astype(np.float64) * 2 ** 16
    assert (np.abs(bf - xf) <= half_fp8 * (1 + 1e-6) + half_bf16).all()


def test_step_bf16_copy(orc):
    from test_oracle_adamw import B1, B2, EPS, LR, WD, bf16_bits, fresh
    rng = np.random.default_rng(4)
    G, n = 128, 128 * 32
    th = rng.normal(0, 0.02, n).astype(np.float32)
    g = bf16_bits(rng.normal(0, 1e-3, n))
    st_a, st_b = fresh(n, G), fresh(n, G)
    th_a, th_b = th.copy(), th.copy()
    copy = np.zeros(n, np.uint16)
    hp = orc.hparams(LR, B1, B2, EPS, WD, 1)
    orc.adamw_step(th_a, g, st_a["m_codes"], st_a["m_amax"], st_a["m_k"], st_a["v_codes"], st_a["v_amax"],
                   st_a["v_k"], G=G, v_fmt="e4m3", hp=hp)
    orc.adamw_step_bf16(th_b, g, st_b["m_codes"], st_b["m_amax"], st_b["m_k"], st_b["v_codes"], st_b["v_amax"],
                        st_b["v_k"], copy, G=G, v_fmt="e4m3", hp=hp, threads=3)
    assert (th_a == th_b).all() and all((st_a[k] == st_b[k]).all() for k in st_a)
    assert (copy == torch_bf16_bits(th_b)).all()
