"""Python binding of the C ABI in include/coat.h (libcoat.so).

Argument marshalling only: every step of the path runs in the HIP kernels.
Tensors are torch device tensors (torch supplies device memory and streams);
each function checks dtype, device, size and contiguity, passes raw device
pointers and the current HIP stream, and raises on a non-zero status.  There
is no CPU fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcoat.so")

E4M3, E5M2 = 0, 1
_FMT = {"e4m3": E4M3, "e5m2": E5M2, E4M3: E4M3, E5M2: E5M2}

_lib = None
_P = ctypes.c_void_p


class CoatError(RuntimeError):
    pass


class AdamWHParams(ctypes.Structure):
    _fields_ = [
        ("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
        ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float), ("step", ctypes.c_int64),
    ]


class AdamWTensor(ctypes.Structure):
    """coat_adamw_tensor: one tensor's optimizer-state buffers (device pointers)."""
    _fields_ = [("param", _P), ("grad_bf16", _P), ("m_codes", _P), ("m_amax", _P), ("m_k", _P),
                ("v_codes", _P), ("v_amax", _P), ("v_k", _P), ("param_bf16", _P), ("n", ctypes.c_int64)]


def lib():
    """Load libcoat.so (built by activation_compression_amd/build.py)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise CoatError(f"{LIB_PATH} is missing: build it with `python activation_compression_amd/build.py`")
    L = ctypes.CDLL(LIB_PATH)
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    L.coat_adamw_step.argtypes = [P, P, P, P, P, P, P, P, i64, i32, ctypes.c_int,
                                  ctypes.POINTER(AdamWHParams), P]
    L.coat_group_absmax.argtypes = [P, i64, i64, i32, P, P, P]
    L.coat_absmax_reduce.argtypes = [P, i64, P, P]
    L.coat_quant_per_tensor.argtypes = [P, i64, P, P, P, P]
    L.coat_quant_group.argtypes = [P, i64, i64, i32, P, P, P, P]
    L.coat_adamw_step_bf16.argtypes = [P, P, P, P, P, P, P, P, P, i64, i32, ctypes.c_int,
                                       ctypes.POINTER(AdamWHParams), P]
    L.coat_dequant_per_tensor.argtypes = [P, i64, P, P, P]
    L.coat_dequant_group.argtypes = [P, i64, i64, i32, P, P, P]
    L.coat_swiglu_fused.argtypes = [P, P, i64, i64, i32, P, P, P, P, P, P, P]
    L.coat_swiglu_fused.restype = ctypes.c_int
    L.coat_rmsnorm_fused.argtypes = [P, P, i64, i64, ctypes.c_float, i32, P, P, P, P, P, P]
    L.coat_rmsnorm_fused.restype = ctypes.c_int
    for f in (L.coat_adamw_step, L.coat_group_absmax, L.coat_absmax_reduce,
              L.coat_quant_per_tensor, L.coat_quant_group, L.coat_adamw_step_bf16,
              L.coat_dequant_per_tensor, L.coat_dequant_group):
        f.restype = ctypes.c_int
    L.coat_adamw_list_bytes.argtypes = [i32]
    L.coat_adamw_list_bytes.restype = i64
    L.coat_adamw_list_pack.argtypes = [ctypes.POINTER(AdamWTensor), i32, i32, P]
    L.coat_adamw_list_pack.restype = ctypes.c_int
    L.coat_adamw_step_list.argtypes = [P, P, ctypes.c_int, ctypes.POINTER(AdamWHParams), P]
    L.coat_adamw_step_list.restype = ctypes.c_int
    L.coat_adamw_step_list_noalloc.argtypes = [P, ctypes.c_int, ctypes.POINTER(AdamWHParams), P]
    L.coat_adamw_step_list_noalloc.restype = ctypes.c_int
    L.coat_status_string.argtypes = [ctypes.c_int]
    L.coat_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def status_string(s: int) -> str:
    return lib().coat_status_string(int(s)).decode()


def _check(status: int, what: str):
    if status != 0:
        raise CoatError(f"{what}: {status_string(status)} (status {status})")


def _ptr(t: torch.Tensor | None, dtypes, name: str, numel: int | None = None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}, but the launch goes to the current device "
                         f"cuda:{torch.cuda.current_device()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name}: needs at least {numel} elements, has {t.numel()}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


_U16 = (torch.int16, torch.bfloat16, torch.uint16)
_U8 = (torch.uint8,)
_F32 = (torch.float32,)


def adamw_hparams(lr, beta1, beta2, eps, weight_decay, step) -> AdamWHParams:
    return AdamWHParams(lr, beta1, beta2, eps, weight_decay, int(step))


def coat_adamw_step(param, grad_bf16, m_codes, m_amax, m_k, v_codes, v_amax, v_k, *,
                    group_size: int = 128, v_format="e4m3", hp: AdamWHParams, n: int | None = None,
                    stream=None) -> None:
    """One fused FP8-state AdamW step (see coat_adamw_step in include/coat.h)."""
    n = param.numel() if n is None else int(n)
    ng = n // group_size if group_size > 0 else 0
    args = [_ptr(param, _F32, "param", n), _ptr(grad_bf16, _U16, "grad_bf16", n),
            _ptr(m_codes, _U8, "m_codes", n), _ptr(m_amax, _F32, "m_amax", ng), _ptr(m_k, _F32, "m_k", ng),
            _ptr(v_codes, _U8, "v_codes", n), _ptr(v_amax, _F32, "v_amax", ng), _ptr(v_k, _F32, "v_k", ng)]
    _check(lib().coat_adamw_step(*args, n, group_size, _FMT[v_format], ctypes.byref(hp), _stream(stream)),
           "coat_adamw_step")


def coat_adamw_step_bf16(param, grad_bf16, m_codes, m_amax, m_k, v_codes, v_amax, v_k, param_bf16, *,
                         group_size: int = 128, v_format="e4m3", hp: AdamWHParams, n: int | None = None,
                         stream=None) -> None:
    """coat_adamw_step that also writes the BF16 working copy of the new weights."""
    n = param.numel() if n is None else int(n)
    ng = n // group_size if group_size > 0 else 0
    args = [_ptr(param, _F32, "param", n), _ptr(grad_bf16, _U16, "grad_bf16", n),
            _ptr(m_codes, _U8, "m_codes", n), _ptr(m_amax, _F32, "m_amax", ng), _ptr(m_k, _F32, "m_k", ng),
            _ptr(v_codes, _U8, "v_codes", n), _ptr(v_amax, _F32, "v_amax", ng), _ptr(v_k, _F32, "v_k", ng),
            _ptr(param_bf16, _U16, "param_bf16", n)]
    _check(lib().coat_adamw_step_bf16(*args, n, group_size, _FMT[v_format], ctypes.byref(hp), _stream(stream)),
           "coat_adamw_step_bf16")


def coat_group_absmax(x_bf16, partial_amax, amax, *, group_size: int = 128, stream=None) -> None:
    """Two-stage Group Scaling absmax of a 2-D BF16 tensor."""
    rows, cols = x_bf16.shape
    _check(lib().coat_group_absmax(_ptr(x_bf16, _U16, "x_bf16"), rows, cols, group_size,
                                   _ptr(partial_amax, _F32, "partial_amax", rows * (cols // group_size)),
                                   _ptr(amax, _F32, "amax", 1), _stream(stream)), "coat_group_absmax")


def coat_absmax_reduce(partial, amax, *, stream=None) -> None:
    """Stage 2 of Group Scaling alone."""
    _check(lib().coat_absmax_reduce(_ptr(partial, _F32, "partial"), partial.numel(),
                                    _ptr(amax, _F32, "amax", 1), _stream(stream)), "coat_absmax_reduce")


def coat_quant_per_tensor(x_bf16, amax, codes, scale, *, stream=None) -> None:
    """Per-tensor E4M3 cast with the device-resident tensor absmax."""
    n = x_bf16.numel()
    _check(lib().coat_quant_per_tensor(_ptr(x_bf16, _U16, "x_bf16"), n, _ptr(amax, _F32, "amax", 1),
                                       _ptr(codes, _U8, "codes", n), _ptr(scale, _F32, "scale", 1),
                                       _stream(stream)), "coat_quant_per_tensor")


def coat_quant_group(x_bf16, codes, scales, partial_amax=None, *, group_size: int = 128, stream=None) -> None:
    """1xG E4M3 quantization of a 2-D BF16 tensor (optionally also stage 1)."""
    rows, cols = x_bf16.shape
    ng = rows * (cols // group_size)
    _check(lib().coat_quant_group(_ptr(x_bf16, _U16, "x_bf16"), rows, cols, group_size,
                                  _ptr(codes, _U8, "codes", rows * cols), _ptr(scales, _F32, "scales", ng),
                                  _ptr(partial_amax, _F32, "partial_amax", ng), _stream(stream)),
           "coat_quant_group")


def coat_dequant_per_tensor(codes, scale, out_bf16, *, stream=None) -> None:
    """E4M3 codes times the per-tensor scale, to BF16."""
    n = codes.numel()
    _check(lib().coat_dequant_per_tensor(_ptr(codes, _U8, "codes"), n, _ptr(scale, _F32, "scale", 1),
                                         _ptr(out_bf16, _U16, "out_bf16", n), _stream(stream)),
           "coat_dequant_per_tensor")


def coat_dequant_group(codes, scales, out_bf16, *, rows: int, cols: int, group_size: int = 128, stream=None) -> None:
    """1xG E4M3 codes times their slice scales, to BF16."""
    ng = rows * (cols // group_size)
    _check(lib().coat_dequant_group(_ptr(codes, _U8, "codes", rows * cols), rows, cols, group_size,
                                    _ptr(scales, _F32, "scales", ng), _ptr(out_bf16, _U16, "out_bf16", rows * cols),
                                    _stream(stream)), "coat_dequant_group")


def coat_swiglu_fused(gate_bf16, up_bf16, h_bf16, h_partial, saved=None, *, group_size: int = 128,
                      stream=None) -> None:
    """h = silu(gate) * up (BF16) with the per-1xG maxima of h (Group Scaling
    stage 1); saved = (gate_codes, gate_scales, up_codes, up_scales) also
    stores the inputs in 1xG E4M3 for the backward pass."""
    rows, cols = gate_bf16.shape
    n, ng = rows * cols, rows * (cols // group_size)
    if saved is None:
        sv = [None, None, None, None]
    else:
        gc, gs, uc, us = saved
        sv = [_ptr(gc, _U8, "gate_codes", n), _ptr(gs, _F32, "gate_scales", ng),
              _ptr(uc, _U8, "up_codes", n), _ptr(us, _F32, "up_scales", ng)]
    _check(lib().coat_swiglu_fused(_ptr(gate_bf16, _U16, "gate_bf16", n), _ptr(up_bf16, _U16, "up_bf16", n),
                                   rows, cols, group_size, _ptr(h_bf16, _U16, "h_bf16", n),
                                   _ptr(h_partial, _F32, "h_partial", ng), *sv, _stream(stream)),
           "coat_swiglu_fused")


def coat_rmsnorm_fused(x_bf16, weight_bf16, y_bf16, y_partial, rstd=None, saved=None, *, eps: float = 1e-5,
                       group_size: int = 128, stream=None) -> None:
    """y = rmsnorm(x) * w (BF16) with the per-1xG maxima of y (Group Scaling
    stage 1); rstd (FP32 [rows]) and saved = (x_codes, x_scales) optionally
    keep what the backward pass needs, x in 1xG E4M3."""
    rows, cols = x_bf16.shape
    n, ng = rows * cols, rows * (cols // group_size)
    xc, xs = (None, None) if saved is None else saved
    _check(lib().coat_rmsnorm_fused(_ptr(x_bf16, _U16, "x_bf16", n), _ptr(weight_bf16, _U16, "weight_bf16", cols),
                                    rows, cols, float(eps), group_size, _ptr(y_bf16, _U16, "y_bf16", n),
                                    _ptr(y_partial, _F32, "y_partial", ng), _ptr(rstd, _F32, "rstd", rows),
                                    _ptr(xc, _U8, "x_codes", n), _ptr(xs, _F32, "x_scales", ng), _stream(stream)),
           "coat_rmsnorm_fused")


class AdamWTensorList:
    """A packed tensor-list table (host and device copies) for
    coat_adamw_step_list.  `states` is a sequence of dicts with the keys
    param, grad, m_codes, m_amax, m_k, v_codes, v_amax, v_k and optionally
    param_bf16 (device tensors, one allocation each is fine).  Build it once;
    it stays valid while those tensors live, and keeps references to them."""

    def __init__(self, states, *, group_size: int = 128, device_copy: bool = True):
        n_t = len(states)
        arr = (AdamWTensor * max(n_t, 1))()
        for i, s in enumerate(states):
            n = s["param"].numel()
            ng = n // group_size
            arr[i] = AdamWTensor(
                _ptr(s["param"], _F32, "param", n), _ptr(s["grad"], _U16, "grad", n),
                _ptr(s["m_codes"], _U8, "m_codes", n), _ptr(s["m_amax"], _F32, "m_amax", ng),
                _ptr(s["m_k"], _F32, "m_k", ng), _ptr(s["v_codes"], _U8, "v_codes", n),
                _ptr(s["v_amax"], _F32, "v_amax", ng), _ptr(s["v_k"], _F32, "v_k", ng),
                _ptr(s.get("param_bf16"), _U16, "param_bf16", n), n)
        nbytes = lib().coat_adamw_list_bytes(n_t)
        if nbytes <= 0:
            raise CoatError("coat_adamw_list_bytes: empty tensor list")
        import numpy as np

        self.host = np.zeros(nbytes, dtype=np.uint8)
        _check(lib().coat_adamw_list_pack(arr, n_t, group_size, ctypes.c_void_p(self.host.ctypes.data)),
               "coat_adamw_list_pack")
        # device_copy=False: for coat_adamw_step_list_noalloc only, which copies the table itself
        self.device = torch.from_numpy(self.host).to("cuda") if device_copy else None
        self.group_size = group_size
        self._refs = list(states)


def coat_adamw_step_list(tlist: AdamWTensorList, *, v_format="e4m3", hp: AdamWHParams, stream=None) -> None:
    """One fused FP8-state AdamW step over every tensor of the list, one launch."""
    _check(lib().coat_adamw_step_list(ctypes.c_void_p(tlist.host.ctypes.data), _ptr(tlist.device, _U8, "table"),
                                      _FMT[v_format], ctypes.byref(hp), _stream(stream)), "coat_adamw_step_list")


def coat_adamw_step_list_noalloc(tlist: AdamWTensorList, *, v_format="e4m3", hp: AdamWHParams, stream=None) -> None:
    """coat_adamw_step_list with the table in the library's own device array
    (no device memory is allocated by the call).  The host table stays alive
    with `tlist`, which the caller keeps until the stream has run the call."""
    _check(lib().coat_adamw_step_list_noalloc(ctypes.c_void_p(tlist.host.ctypes.data), _FMT[v_format],
                                              ctypes.byref(hp), _stream(stream)), "coat_adamw_step_list_noalloc")
