"""CPU oracle for COAT-style FP8 optimizer-state and activation compression.

TEST INFRASTRUCTURE ONLY.  The slow, obviously-correct binary64 reference the
GPU path is checked against.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the product package never does.

This module is a thin ctypes wrapper over ``liboracle.so`` (plain C, built by
``oracle/build.py``).  Every function takes and returns numpy arrays and works
on the host only.  Arithmetic lives in ``coat_oracle.c``; see its comments for
the passages of the pages each step follows.
"""
from __future__ import annotations

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# COAT_ORACLE_LIB names another build of coat_oracle.c (the pin tests' own
# check that planted mistakes fail them loads mutated builds this way).
LIB_PATH = os.environ.get("COAT_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")

E4M3, E5M2, E2M2 = 0, 1, 2
FORMATS = {"e4m3": E4M3, "e5m2": E5M2, "e2m2": E2M2}

_lib = None


class HParams(ctypes.Structure):
    _fields_ = [
        ("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
        ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float), ("step", ctypes.c_int64),
    ]


def fmt_id(fmt) -> int:
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def lib():
    """Load (building first if needed) the oracle library."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _build
        _build.build()
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i64, f32, f64, u32, i32 = ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_uint32, ctypes.c_int
    L.orc_fp8_decode.argtypes, L.orc_fp8_decode.restype = [i32, u32], f64
    L.orc_fp8_encode.argtypes, L.orc_fp8_encode.restype = [i32, f64], u32
    L.orc_fp8_max.argtypes, L.orc_fp8_max.restype = [i32], f64
    L.orc_fp8_min_subnormal.argtypes, L.orc_fp8_min_subnormal.restype = [i32], f64
    L.orc_fp8_max_code.argtypes, L.orc_fp8_max_code.restype = [i32], u32
    L.orc_expand_quantize.argtypes = [i32, P, i64, f64, P, P, P]
    L.orc_expand_quantize.restype = None
    L.orc_expand_dequantize.argtypes, L.orc_expand_dequantize.restype = [i32, u32, f32, f32], f64
    L.orc_expand_encode.argtypes, L.orc_expand_encode.restype = [i32, f64, f32, f32], u32
    L.orc_expand_encode_each.argtypes = [i32, P, P, P, i64, P]
    L.orc_expand_encode_each.restype = None
    L.orc_expand_encode_groups.argtypes = [i32, P, i64, i64, i64, P, P, P]
    L.orc_expand_encode_groups.restype = None
    L.orc_expand_quantize_groups.argtypes = [i32, P, i64, i64, i64, P, P, P, P]
    L.orc_expand_quantize_groups.restype = None
    L.orc_expand_dequantize_groups.argtypes = [i32, P, i64, i64, i64, P, P, P]
    L.orc_expand_dequantize_groups.restype = None
    L.orc_bf16_rne.argtypes, L.orc_bf16_rne.restype = [f32], ctypes.c_uint16
    L.orc_adamw_step_bf16.argtypes = [P, P, P, P, P, P, P, P, i64, i64, i64, i32, ctypes.POINTER(HParams), P]
    L.orc_adamw_step_bf16.restype = None
    L.orc_dequant_per_tensor.argtypes = [P, i64, f32, P]
    L.orc_dequant_per_tensor.restype = None
    L.orc_dequant_group.argtypes = [P, i64, i64, i64, P, P]
    L.orc_dequant_group.restype = None
    L.orc_silu.argtypes, L.orc_silu.restype = [f64], f64
    L.orc_swiglu_absmax.argtypes = [P, P, i64, i64, i64, P, P]
    L.orc_swiglu_absmax.restype = None
    L.orc_rmsnorm_absmax.argtypes = [P, P, i64, i64, i64, ctypes.c_float, P, P, P]
    L.orc_rmsnorm_absmax.restype = None
    L.orc_adamw_step.argtypes = [P, P, P, P, P, P, P, P, i64, i64, i64, i32, ctypes.POINTER(HParams), P, P]
    L.orc_adamw_step.restype = None
    L.orc_adamw_step_f64.argtypes = [P, P, P, P, i64, ctypes.POINTER(HParams)]
    L.orc_adamw_step_f64.restype = None
    L.orc_group_absmax.argtypes = [P, i64, i64, i64, P, P]
    L.orc_group_absmax.restype = None
    L.orc_absmax_reduce.argtypes, L.orc_absmax_reduce.restype = [P, i64], f32
    L.orc_quant_per_tensor.argtypes = [P, i64, f32, P, P]
    L.orc_quant_per_tensor.restype = None
    L.orc_quant_group.argtypes = [P, i64, i64, i64, P, P, P]
    L.orc_quant_group.restype = None
    _lib = L
    return L


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def hparams(lr, beta1, beta2, eps, weight_decay, step) -> HParams:
    return HParams(lr, beta1, beta2, eps, weight_decay, int(step))


# ---------------------------------------------------------------- C1 codec
def decode(fmt, code: int) -> float:
    return lib().orc_fp8_decode(fmt_id(fmt), int(code))


def encode(fmt, x: float) -> int:
    return int(lib().orc_fp8_encode(fmt_id(fmt), float(x)))


def decode_all(fmt, codes) -> np.ndarray:
    f = fmt_id(fmt)
    return np.array([lib().orc_fp8_decode(f, int(c)) for c in np.asarray(codes).ravel()])


def encode_all(fmt, xs) -> np.ndarray:
    f = fmt_id(fmt)
    return np.array([lib().orc_fp8_encode(f, float(x)) for x in np.asarray(xs, dtype=np.float64).ravel()],
                    dtype=np.uint8 if f != E2M2 else np.uint8)


def fmt_max(fmt) -> float:
    return lib().orc_fp8_max(fmt_id(fmt))


def fmt_min_subnormal(fmt) -> float:
    return lib().orc_fp8_min_subnormal(fmt_id(fmt))


def fmt_max_code(fmt) -> int:
    return int(lib().orc_fp8_max_code(fmt_id(fmt)))


# ------------------------------------------------------------- C2/C3 expansion
def expand_quantize(fmt, x, k_force: float = 0.0):
    """Quantize one group; returns (codes uint8[G], amax float32, k float32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.zeros(x.size, dtype=np.uint8)
    amax = np.zeros(1, dtype=np.float32)
    k = np.zeros(1, dtype=np.float32)
    lib().orc_expand_quantize(fmt_id(fmt), _ptr(x), x.size, float(k_force), _ptr(codes), _ptr(amax), _ptr(k))
    return codes, np.float32(amax[0]), np.float32(k[0])


def expand_quantize_groups(fmt, x, G: int, k_given=None, threads: int = 1):
    """Quantize every G-element group of x; k_given (float32 per group) fixes
    each group's k instead of recomputing it.  Returns (codes, amax, k)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    ng = x.size // G
    codes = np.zeros(x.size, dtype=np.uint8)
    amax = np.zeros(ng, dtype=np.float32)
    k = np.zeros(ng, dtype=np.float32)
    kg = None if k_given is None else np.ascontiguousarray(k_given, dtype=np.float32)
    L = lib()
    f = fmt_id(fmt)
    ptrs = (_ptr(x), _ptr(kg) if kg is not None else None, _ptr(codes), _ptr(amax), _ptr(k))

    def run(lo, hi):
        L.orc_expand_quantize_groups(f, ptrs[0], lo, hi, G, ptrs[1], ptrs[2], ptrs[3], ptrs[4])

    _run_blocks(run, _row_blocks(ng, threads), threads)
    return codes, amax, k


def expand_encode_groups(fmt, x, G: int, amax, k, threads: int = 1) -> np.ndarray:
    """The code of every value of x (binary64) in its group stored with the
    given (amax, k) (float32 per group): the quantizer's last step alone."""
    xx = np.ascontiguousarray(x, dtype=np.float64)
    a = np.ascontiguousarray(amax, dtype=np.float32)
    kk = np.ascontiguousarray(k, dtype=np.float32)
    codes = np.zeros(xx.size, dtype=np.uint8)
    L = lib()
    f = fmt_id(fmt)

    def run(lo, hi):
        L.orc_expand_encode_groups(f, _ptr(xx), lo, hi, G, _ptr(a), _ptr(kk), _ptr(codes))

    _run_blocks(run, _row_blocks(xx.size // G, threads), threads)
    return codes


def expand_encode_each(fmt, x, amax, k) -> np.ndarray:
    """The code of every x[i] (binary64) in a group stored with (amax[i], k[i])."""
    xx = np.ascontiguousarray(x, dtype=np.float64)
    a = np.ascontiguousarray(amax, dtype=np.float32)
    kk = np.ascontiguousarray(k, dtype=np.float32)
    assert a.size == xx.size and kk.size == xx.size
    codes = np.zeros(xx.size, dtype=np.uint8)
    lib().orc_expand_encode_each(fmt_id(fmt), _ptr(xx), _ptr(a), _ptr(kk), xx.size, _ptr(codes))
    return codes


def expand_dequantize_groups(fmt, codes, G: int, amax, k, threads: int = 1) -> np.ndarray:
    """Inverse expansion of every code (binary64 values)."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    a = np.ascontiguousarray(amax, dtype=np.float32)
    kk = np.ascontiguousarray(k, dtype=np.float32)
    out = np.zeros(c.size, dtype=np.float64)
    L = lib()
    f = fmt_id(fmt)

    def run(lo, hi):
        L.orc_expand_dequantize_groups(f, _ptr(c), lo, hi, G, _ptr(a), _ptr(kk), _ptr(out))

    _run_blocks(run, _row_blocks(c.size // G, threads), threads)
    return out


def bf16_rne(x) -> np.ndarray:
    """BF16 bit patterns (uint16) of FP32 values, round to nearest even."""
    L = lib()
    return np.array([L.orc_bf16_rne(float(v)) for v in np.asarray(x, dtype=np.float32).ravel()], dtype=np.uint16)


def expand_dequantize(fmt, codes, amax, k) -> np.ndarray:
    f = fmt_id(fmt)
    L = lib()
    return np.array([L.orc_expand_dequantize(f, int(c), float(amax), float(k))
                     for c in np.asarray(codes).ravel()])


# ------------------------------------------------------------------ C4 AdamW
def adamw_step(param, grad_bf16, m_codes, m_amax, m_k, v_codes, v_amax, v_k, *,
               G: int, v_fmt, hp: HParams, groups=None, threads: int = 1, moments_out=None) -> None:
    """One FP8-state AdamW step, in place on numpy arrays.

    ``groups`` = (g0, g1) restricts the step to a group range; ``threads``
    splits that range over host threads (the C code runs without the GIL).
    ``moments_out`` = (m_new, v_new) float32 arrays like ``param`` receive the
    new moments before requantization.
    """
    arrs = [param, grad_bf16, m_codes, m_amax, m_k, v_codes, v_amax, v_k]
    for a in arrs:
        assert a.flags["C_CONTIGUOUS"]
    assert param.dtype == np.float32 and grad_bf16.dtype == np.uint16
    assert m_codes.dtype == np.uint8 and v_codes.dtype == np.uint8
    n_groups = param.size // G
    g0, g1 = groups if groups is not None else (0, n_groups)
    ptrs = [_ptr(a) for a in arrs]
    if moments_out is not None:
        for a in moments_out:
            assert a.dtype == np.float32 and a.size == param.size and a.flags["C_CONTIGUOUS"]
        outs = [_ptr(a) for a in moments_out]
    else:
        outs = [None, None]
    L = lib()
    vf = fmt_id(v_fmt)

    def run(lo, hi):
        L.orc_adamw_step(*ptrs, lo, hi, G, vf, ctypes.byref(hp), *outs)

    if threads <= 1 or g1 - g0 < 2 * threads:
        run(g0, g1)
        return
    bounds = np.linspace(g0, g1, threads + 1).astype(np.int64)
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda i: run(int(bounds[i]), int(bounds[i + 1])), range(threads)))


def adamw_step_bf16(param, grad_bf16, m_codes, m_amax, m_k, v_codes, v_amax, v_k, param_bf16, *,
                    G: int, v_fmt, hp: HParams, threads: int = 1) -> None:
    """adamw_step that also writes the BF16 working copy of the new weights."""
    arrs = [param, grad_bf16, m_codes, m_amax, m_k, v_codes, v_amax, v_k, param_bf16]
    for a in arrs:
        assert a.flags["C_CONTIGUOUS"]
    assert param_bf16.dtype == np.uint16 and param_bf16.size == param.size
    ptrs = [_ptr(a) for a in arrs]
    L = lib()
    vf = fmt_id(v_fmt)
    ng = param.size // G

    def run(lo, hi):
        L.orc_adamw_step_bf16(*ptrs[:8], lo, hi, G, vf, ctypes.byref(hp), ptrs[8])

    _run_blocks(run, _row_blocks(ng, threads), threads)


def adamw_step_f64(param, grad, m, v, hp: HParams) -> None:
    for a in (param, grad, m, v):
        assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"]
    lib().orc_adamw_step_f64(_ptr(param), _ptr(grad), _ptr(m), _ptr(v), param.size, ctypes.byref(hp))


# ------------------------------------------------------------ C5 Group Scaling
def _row_blocks(rows: int, threads: int):
    t = max(1, min(threads, rows))
    b = np.linspace(0, rows, t + 1).astype(np.int64)
    return [(int(b[i]), int(b[i + 1])) for i in range(t) if b[i + 1] > b[i]]


def _run_blocks(fn, blocks, threads):
    if len(blocks) == 1 or threads <= 1:
        for lo, hi in blocks:
            fn(lo, hi)
        return
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda b: fn(*b), blocks))


def group_absmax(x_bf16, G: int, threads: int = 1):
    """Two-stage absmax of a 2-D BF16 (uint16 bits) tensor: (partial, amax).
    ``threads`` splits stage 1 by rows; stage 2 runs once over all partials."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, cols = x.shape
    gpr = cols // G
    partial = np.zeros(rows * gpr, dtype=np.float32)
    L = lib()

    def run(lo, hi):
        tmp = np.zeros(1, dtype=np.float32)
        L.orc_group_absmax(_ptr(x[lo:hi]), hi - lo, cols, G, _ptr(partial[lo * gpr:hi * gpr]), _ptr(tmp))

    _run_blocks(run, _row_blocks(rows, threads), threads)
    return partial, absmax_reduce(partial)


def absmax_reduce(partial) -> np.float32:
    p = np.ascontiguousarray(partial, dtype=np.float32)
    return np.float32(lib().orc_absmax_reduce(_ptr(p), p.size))


def quant_per_tensor(x_bf16, amax, threads: int = 1):
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16).reshape(-1)
    codes = np.zeros(x.size, dtype=np.uint8)
    scale = np.zeros(1, dtype=np.float32)
    L = lib()
    n = x.size
    bounds = [(lo * 16, min(n, hi * 16)) for lo, hi in _row_blocks((n + 15) // 16, threads)]

    def run(lo, hi):
        L.orc_quant_per_tensor(_ptr(x[lo:hi]), hi - lo, float(amax), _ptr(codes[lo:hi]), _ptr(scale))

    _run_blocks(run, bounds, threads)
    return codes, np.float32(scale[0])


def quant_group(x_bf16, G: int, threads: int = 1):
    """1xG E4M3 group quantization: (codes uint8[rows*cols], scales, partial)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, cols = x.shape
    gpr = cols // G
    codes = np.zeros(rows * cols, dtype=np.uint8)
    scales = np.zeros(rows * gpr, dtype=np.float32)
    partial = np.zeros(rows * gpr, dtype=np.float32)
    L = lib()

    def run(lo, hi):
        L.orc_quant_group(_ptr(x[lo:hi]), hi - lo, cols, G, _ptr(codes[lo * cols:hi * cols]),
                          _ptr(scales[lo * gpr:hi * gpr]), _ptr(partial[lo * gpr:hi * gpr]))

    _run_blocks(run, _row_blocks(rows, threads), threads)
    return codes, scales, partial


# ------------------------------------------------ activation dequantization
def dequant_per_tensor(codes, scale, threads: int = 1) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1)
    out = np.zeros(c.size, dtype=np.uint16)
    L = lib()
    bounds = [(lo * 16, min(c.size, hi * 16)) for lo, hi in _row_blocks((c.size + 15) // 16, threads)]

    def run(lo, hi):
        L.orc_dequant_per_tensor(_ptr(c[lo:hi]), hi - lo, float(scale), _ptr(out[lo:hi]))

    _run_blocks(run, bounds, threads)
    return out


def dequant_group(codes, rows: int, cols: int, G: int, scales, threads: int = 1) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8).reshape(rows, cols)
    sc = np.ascontiguousarray(scales, dtype=np.float32)
    gpr = cols // G
    out = np.zeros(rows * cols, dtype=np.uint16)
    L = lib()

    def run(lo, hi):
        L.orc_dequant_group(_ptr(c[lo:hi]), hi - lo, cols, G, _ptr(sc[lo * gpr:hi * gpr]),
                            _ptr(out[lo * cols:hi * cols]))

    _run_blocks(run, _row_blocks(rows, threads), threads)
    return out


# ------------------------------------------- SwiGLU producer with stage 1
def silu(x: float) -> float:
    return lib().orc_silu(float(x))


def swiglu_absmax(gate_bf16, up_bf16, G: int, threads: int = 1):
    """(h BF16 bits [rows*cols], partial absmax of h per 1xG slice)."""
    g = np.ascontiguousarray(gate_bf16, dtype=np.uint16)
    u = np.ascontiguousarray(up_bf16, dtype=np.uint16)
    rows, cols = g.shape
    gpr = cols // G
    h = np.zeros(rows * cols, dtype=np.uint16)
    partial = np.zeros(rows * gpr, dtype=np.float32)
    L = lib()

    def run(lo, hi):
        L.orc_swiglu_absmax(_ptr(g[lo:hi]), _ptr(u[lo:hi]), hi - lo, cols, G, _ptr(h[lo * cols:hi * cols]),
                            _ptr(partial[lo * gpr:hi * gpr]))

    _run_blocks(run, _row_blocks(rows, threads), threads)
    return h, partial


# ------------------------------------------ RMSNorm producer with stage 1
def rmsnorm_absmax(x_bf16, weight_bf16, G: int, eps: float, threads: int = 1):
    """(y BF16 bits [rows*cols], partial absmax of y per 1xG slice, rstd FP32 [rows]);
    weight_bf16 may be None (no gain)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, cols = x.shape
    w = None if weight_bf16 is None else np.ascontiguousarray(weight_bf16, dtype=np.uint16).reshape(-1)
    assert w is None or w.size == cols
    gpr = cols // G
    y = np.zeros(rows * cols, dtype=np.uint16)
    partial = np.zeros(rows * gpr, dtype=np.float32)
    rstd = np.zeros(rows, dtype=np.float32)
    L = lib()

    def run(lo, hi):
        L.orc_rmsnorm_absmax(_ptr(x[lo:hi]), None if w is None else _ptr(w), hi - lo, cols, G, float(eps),
                             _ptr(y[lo * cols:hi * cols]), _ptr(partial[lo * gpr:hi * gpr]), _ptr(rstd[lo:hi]))

    _run_blocks(run, _row_blocks(rows, threads), threads)
    return y, partial, rstd
