"""Pins of the oracle's RMSNorm producer with fused Group Scaling stage 1:
y against torch.nn.functional.rms_norm in float64 (rounded through FP32 to
BF16), the closed form of a constant row, invariance under power-of-two
scaling of a row, and the partials against torch.amax of |y|."""
import numpy as np
import pytest
import torch

from activation_compression_amd import inputs


def bits_to_f64(b):
    return torch.from_numpy((np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)).double()


def to_bf16_bits(t64):
    return t64.float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).reshape(-1)


@pytest.mark.parametrize("G, weighted", [(32, False), (128, True)])
def test_rmsnorm_matches_torch(orc, G, weighted):
    rows, cols = 24, 1024
    x = inputs.gen_activation(inputs.ActivationSpec("x", rows, cols, seed=31)).numpy().view(np.uint16)
    w = None
    if weighted:
        w = inputs.gen_activation(inputs.ActivationSpec("w", 1, cols, seed=32)).numpy().view(np.uint16)
    eps = 1e-5
    y, partial, rstd = orc.rmsnorm_absmax(x, w, G, eps)
    xt = bits_to_f64(x)
    wt = None if w is None else bits_to_f64(w).reshape(-1)
    yt = torch.nn.functional.rms_norm(xt, (cols,), wt, eps=float(np.float32(eps)))
    want = to_bf16_bits(yt)
    assert (y == want).all()
    rs = torch.rsqrt(xt.pow(2).mean(dim=-1) + float(np.float32(eps))).float().numpy()
    assert np.array_equal(rstd, rs)
    yb = bits_to_f64(want).reshape(rows, cols // G, G)
    assert (partial == torch.amax(yb.abs(), dim=-1).reshape(-1).float().numpy()).all()


def test_rmsnorm_constant_row(orc):
    """x = +-c everywhere: mean x^2 = c^2, so y = x / sqrt(c^2 + eps) = +-1 for
    eps far below c^2 (the mean divides by cols, not by anything else)."""
    cols = 512
    x = np.empty((3, cols), np.uint16)
    x[0] = 0x4040               # 3.0
    x[1, ::2], x[1, 1::2] = 0x3E80, 0xBE80   # +-0.25
    x[2] = 0x4700               # 32768
    y, partial, rstd = orc.rmsnorm_absmax(x, None, 128, 1e-12)
    y = y.reshape(3, cols)
    assert (y[0] == 0x3F80).all() and (y[2] == 0x3F80).all()
    assert (y[1, ::2] == 0x3F80).all() and (y[1, 1::2] == 0xBF80).all()
    assert (partial == 1.0).all()
    assert rstd[0] == np.float32(1 / 3.0) and rstd[1] == 4.0 and rstd[2] == np.float32(2.0 ** -15)


def test_rmsnorm_zero_row_and_eps(orc):
    """A zero row gives y = 0 and rstd = 1/sqrt(eps); eps matters exactly as
    its closed form says for a row of ones: y = 1/sqrt(1 + eps)."""
    x = np.zeros((2, 256), np.uint16)
    x[1] = 0x3F80
    eps = 0.25
    y, partial, rstd = orc.rmsnorm_absmax(x, None, 256, eps)
    assert (y[:256] == 0).all() and partial[0] == 0 and rstd[0] == 2.0
    assert (y[256:] == to_bf16_bits(torch.tensor([1 / np.sqrt(1.25)], dtype=torch.float64))[0]).all()
    assert rstd[1] == np.float32(1 / np.sqrt(1.25))


def test_rmsnorm_power_of_two_scale_invariance(orc):
    """With eps negligible, y(4x) = y(x) bit for bit (every step scales exactly)."""
    x = inputs.gen_activation(inputs.ActivationSpec("x", 8, 2048, seed=33)).numpy().view(np.uint16)
    x4 = (((x.astype(np.uint32) << 16).view(np.float32) * 4).view(np.uint32) >> 16).astype(np.uint16)
    y1, p1, r1 = orc.rmsnorm_absmax(x, None, 128, 1e-30)
    y4, p4, r4 = orc.rmsnorm_absmax(x4, None, 128, 1e-30)
    assert (y1 == y4).all() and (p1 == p4).all() and (r4 * 4 == r1).all()
