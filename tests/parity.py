"""Helpers shared by the GPU parity tests: run one step on each side from the
same inputs and compare to the stated tolerances.

Tolerances (the product's contract with the oracle):
* theta (FP32 master weights): |gpu - ref| <= 1e-6 |ref| + 1e-6 lr.  The
  absolute floor covers parameters that land near zero, where a relative
  bound is undefined; 1e-6 lr is a millionth of a typical update.
* FP8 codes, two criteria:
  (A) identical (0x00 == 0x80) to the oracle's on >= 99.99% of each moment
      tensor (at least one mismatch is allowed, so tensors under 10 000
      elements may hold a single one);
  (B) every code within one grid step of the oracle's encoding of the
      oracle's own new moment with the GPU's stored k for that group -- or,
      for a first moment that is itself a near-total cancellation
      b1 m + (1-b1) g, within 1 + ceil(8 k 2^-21 cond / ln 2) steps, where
      cond = (b1 amax_prev + (1-b1)|g|) / |m_new| bounds the condition number
      of that sum (|m_old| <= amax_prev).  2^-21 is a few ulps of FP32
      relative error on the terms; 8 k / ln 2 turns a relative error of the
      moment into FP8 grid steps (8 steps per binade, stretched by k).  The
      second moment is a sum of non-negative terms (cond = 1): one step.
  The GPU evaluates the power with FP32 exp2/log2 while the oracle uses
  binary64 pow, so an element within an ulp or so of a rounding midpoint may
  land on the neighbouring code.  (B) uses the GPU's k so that it also judges
  groups whose smallest moment is such a cancellation: there the FP32 value
  of that moment, and with it k, is ill-conditioned for any FP32 evaluation,
  and a whole group's codes may shift against the oracle's while still being
  the right encoding for the k stored beside them (k is judged separately).
* amax: within the FP32 rounding bound of the moment update, 2^-21 (2 amax_prev
  + amax) (a few ulps: the dequantized old moment carries the exp2 rounding).
* k: within 1e-5 relative, plus the first-order effect on k of the FP32
  rounding bound of the group's smallest moment (dk/k = (d amin/amin) /
  ln(amax/amin)).  The smallest moment of a group is often a near-cancellation
  b1 m + (1-b1) g, whose FP32 value carries an absolute error of a few ulps of
  the terms, i.e. of max(amax_prev, amax); that error is bounded here by
  2^-21 (2 amax_prev + amax).  Groups whose range is below 1.01 or whose
  smallest moment is within that bound of zero are judged by their codes only.
* Activation path: partial maxima, amax, scales and codes bit-exact.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle as orc
from activation_compression_amd import coat, inputs

LR, B1, B2, EPS, WD = (float(np.float32(v)) for v in
                       (inputs.LR, inputs.BETA1, inputs.BETA2, inputs.EPS, inputs.WEIGHT_DECAY))
THREADS = 8
CODE_MATCH_MIN = 0.9999
STATS = []  # (what, elements, mismatching codes) of every code comparison, for the report
BF16_STATS = []  # (what, elements, elements not bit-identical) of every BF16 output compared in value space


def flush(msg: str):
    print(msg, flush=True)


def gpu_hp(step):
    return coat.adamw_hparams(LR, B1, B2, EPS, WD, step)


def orc_hp(step):
    return orc.hparams(LR, B1, B2, EPS, WD, step)


def np_state(n, G):
    return {k: v.numpy() for k, v in inputs.fresh_state(n, G).items()}


def dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    a = t.cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def gpu_step(theta, g_bits, st, G, v_fmt, t):
    """One coat_adamw_step on copies of the given host arrays; returns host copies."""
    th = dev(theta)
    s = {k: dev(v) for k, v in st.items()}
    coat.coat_adamw_step(th, dev(g_bits), s["m_codes"], s["m_amax"], s["m_k"], s["v_codes"],
                         s["v_amax"], s["v_k"], group_size=G, v_format=v_fmt, hp=gpu_hp(t))
    torch.cuda.synchronize()
    return host(th), {k: host(v) for k, v in s.items()}


class StepResult(tuple):
    """(theta, state) of one oracle step; .moments holds the oracle's new FP32
    moments (m, v) before requantization, .G the group size, .v_fmt v's format."""
    moments = None
    G = None
    v_fmt = None
    grad_bits = None


def oracle_step(theta, g_bits, st, G, v_fmt, t, threads=THREADS):
    th = theta.copy()
    s = {k: v.copy() for k, v in st.items()}
    m_new = np.empty(th.size, np.float32)
    v_new = np.empty(th.size, np.float32)
    orc.adamw_step(th, g_bits, s["m_codes"], s["m_amax"], s["m_k"], s["v_codes"], s["v_amax"], s["v_k"],
                   G=G, v_fmt=v_fmt, hp=orc_hp(t), threads=threads, moments_out=(m_new, v_new))
    r = StepResult((th, s))
    r.moments, r.G, r.v_fmt = (m_new, v_new), G, v_fmt
    r.grad_bits = g_bits
    return r


def _signed(c):
    c = c.astype(np.int32)
    return np.where(c & 0x80, -1, 1) * (c & 0x7F)


def differing(gpu: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Indices where two code arrays differ, with 0x00 == 0x80 (byte ops only,
    so that billion-element arenas stay cheap)."""
    g, r = gpu.reshape(-1), ref.reshape(-1)
    ne = g != r
    ne &= ((g & 0x7F) != 0) | ((r & 0x7F) != 0)
    return np.flatnonzero(ne)


def code_diff(gpu: np.ndarray, ref: np.ndarray):
    """(fraction identical, max grid-step distance) with 0x00 == 0x80."""
    idx = differing(gpu, ref)
    n = gpu.size
    if idx.size == 0:
        return 1.0, 0
    g, r = gpu.reshape(-1)[idx], ref.reshape(-1)[idx]
    return 1.0 - idx.size / n, int(np.abs(_signed(g) - _signed(r)).max())


def assert_codes(gpu, ref, what, min_frac=CODE_MATCH_MIN, max_steps=1, record=True, check=True):
    """Identical codes (0x00 == 0x80) on at least min_frac of the elements and
    no code more than max_steps grid steps away; check=False only records the
    counts for the report."""
    frac, steps = code_diff(gpu, ref)
    n = gpu.size
    bad = int(round((1.0 - frac) * n))
    if record:
        STATS.append((what, n, bad, steps))
    if not check:
        return frac
    allowed = max(1, int((1.0 - min_frac) * n))
    assert bad <= allowed, f"{what}: {bad} of {n} codes differ ({frac:.6%} identical)"
    if max_steps is not None:
        assert steps <= max_steps, f"{what}: a code differs by {steps} grid steps"
    return frac


def assert_codes_given_k(gpu_codes, moments, gpu_k, fmt, G, what, cond=None, threads=THREADS,
                         min_frac=CODE_MATCH_MIN):
    # cond: None, or a function of element indices giving the condition bound there
    """The GPU's codes against the oracle's encoding of the oracle's own
    moments with the GPU's stored k: (A) at least min_frac identical, (B) every
    code within its step bound -- one step, or for a first moment that is a
    near-cancellation (cond: per-element condition number bound of the moment
    update, None for 1) 1 + ceil(8 k 2^-21 cond / ln 2) steps."""
    want, _, _ = orc.expand_quantize_groups(fmt, moments, G, k_given=gpu_k, threads=threads)
    frac = assert_codes(gpu_codes, want, what + " (GPU k)", min_frac=min_frac, max_steps=None, record=False)
    idx = differing(gpu_codes, want)
    dist = np.abs(_signed(gpu_codes.reshape(-1)[idx]) - _signed(want.reshape(-1)[idx]))
    if cond is None:
        allowed = np.ones_like(dist)
    else:
        k_el = gpu_k.astype(np.float64)[idx // G]
        allowed = 1 + np.ceil(8.0 * k_el * 2.0 ** -21 * cond(idx) / math.log(2.0))
    bad = dist > allowed
    assert not bad.any(), (f"{what} (GPU k): {int(bad.sum())} codes beyond their step bound; "
                           f"worst {int(dist[bad].max())} steps where {int(np.max(np.where(bad, allowed, 0)))} allowed")
    return frac


def assert_theta(gpu, ref, what):
    ref64 = ref.astype(np.float64)
    err = np.abs(gpu.astype(np.float64) - ref64)
    tol = 1e-6 * np.abs(ref64) + 1e-6 * LR
    bad = err > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} params out of tolerance; worst "
                           f"err {err[bad].max():.3e} at |ref| {np.abs(ref64[bad][np.argmax(err[bad])]):.3e}")


def assert_amax(gpu, ref, amax_prev, what):
    ref = ref.astype(np.float64)
    tol = np.maximum(2.0 ** -21 * (2 * np.abs(amax_prev.astype(np.float64)) + ref),
                     np.spacing(np.abs(ref).astype(np.float32)))
    d = np.abs(gpu.astype(np.float64) - ref)
    bad = d > tol
    assert not bad.any(), f"{what}: amax off in {int(bad.sum())} groups (worst {(d / np.maximum(ref, 1e-45)).max():.3e} rel)"


def k_conditioning(ref_k, amax_ref, amax_prev, v_fmt_name):
    """Per group: (well, tol, ln_ratio).  k = ln R_fmt / ln(amax/amin) is
    well-conditioned where the group range is at least 1.01 and the smallest
    moment exceeds the FP32 rounding bound delta of the moment update; tol is
    the relative bound on k there."""
    r_fmt = orc.fmt_max(v_fmt_name) / orc.fmt_min_subnormal(v_fmt_name)
    ref = ref_k.astype(np.float64)
    amax = amax_ref.astype(np.float64)
    ln_ratio = math.log(r_fmt) / ref                 # ln(amax / amin) from the stored k
    amin = amax * np.exp(-ln_ratio)
    delta = 2.0 ** -21 * (2 * np.abs(amax_prev.astype(np.float64)) + amax)
    well = (ln_ratio >= math.log(1.01)) & (delta < 0.5 * amin) & (amax > 0)
    tol = 1e-5 + 2.0 * (delta / np.where(amin > 0, amin, 1.0)) / ln_ratio
    return well, tol


def assert_k(gpu, ref, amax_ref, amax_prev, v_fmt_name, what):
    well, tol = k_conditioning(ref, amax_ref, amax_prev, v_fmt_name)
    ref = ref.astype(np.float64)
    rel = np.abs(gpu.astype(np.float64) - ref) / ref
    bad = well & (rel > tol)
    assert not bad.any(), f"{what}: k off by {rel[bad].max():.3e} relative in {int(bad.sum())} groups"


def assert_step_parity(gpu, ref, v_fmt, what, prev=None):
    """prev: the state both sides started from (None: a fresh state)."""
    th_g, st_g = gpu
    th_r, st_r = ref
    zeros = np.zeros_like(st_r["m_amax"])
    prev_m = zeros if prev is None else prev["m_amax"]
    prev_v = zeros if prev is None else prev["v_amax"]
    assert_theta(th_g, th_r, what + " theta")
    moments = getattr(ref, "moments", None)
    # Without the oracle's unquantized moments: identical codes on >= 99.99%,
    # every mismatch one grid step.  With them, the codes are judged against
    # the oracle's encoding of its own moments with the k the GPU stored beside
    # them -- (A) >= 99.99% identical, (B) within the step bound -- because k is
    # itself ill-conditioned wherever a group's smallest moment is a partial
    # cancellation (any FP32 evaluation of the update moves it), and a whole
    # group's codes then legitimately shift with it.  k is judged against the
    # oracle's on its own, to its conditioning bound (assert_k); the mismatch
    # count against the oracle's own codes is recorded for the report.
    if moments is None:
        fm = assert_codes(st_g["m_codes"], st_r["m_codes"], what + " m codes")
        fv = assert_codes(st_g["v_codes"], st_r["v_codes"], what + " v codes")
    else:
        assert_codes(st_g["m_codes"], st_r["m_codes"], what + " m codes", check=False)
        assert_codes(st_g["v_codes"], st_r["v_codes"], what + " v codes", check=False)
        G = ref.G

        def cond(idx):  # (b1 amax_prev + (1 - b1)|g|) / |m_new| at the given elements
            g_abs = np.abs((ref.grad_bits[idx].astype(np.uint32) << 16).view(np.float32).astype(np.float64))
            m_new = np.abs(moments[0][idx].astype(np.float64))
            terms = B1 * np.abs(prev_m[idx // G].astype(np.float64)) + (1.0 - B1) * g_abs
            with np.errstate(divide="ignore", invalid="ignore"):
                return np.where(m_new > 0, terms / m_new, np.inf)

        fm = assert_codes_given_k(st_g["m_codes"], moments[0], st_g["m_k"], "e4m3", ref.G, what + " m codes",
                                  cond=cond)
        fv = assert_codes_given_k(st_g["v_codes"], moments[1], st_g["v_k"], ref.v_fmt, ref.G, what + " v codes")
    assert_amax(st_g["m_amax"], st_r["m_amax"], prev_m, what + " m amax")
    assert_amax(st_g["v_amax"], st_r["v_amax"], prev_v, what + " v amax")
    assert_k(st_g["m_k"], st_r["m_k"], st_r["m_amax"], prev_m, "e4m3", what + " m k")
    assert_k(st_g["v_k"], st_r["v_k"], st_r["v_amax"], prev_v, v_fmt, what + " v k")
    return fm, fv
