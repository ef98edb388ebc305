"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/coat.h declares, and rejects invalid arguments
before anything is enqueued (these calls return before any HIP call)."""
import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "coat.h")


@pytest.fixture(scope="module")
def L():
    from activation_compression_amd import coat
    if not os.path.exists(coat.LIB_PATH):
        pytest.skip("libcoat.so not built")
    return coat.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(coat_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_path():
    names = declared_functions()
    for want in ("coat_adamw_step", "coat_adamw_step_bf16", "coat_group_absmax", "coat_absmax_reduce",
                 "coat_quant_per_tensor", "coat_quant_group", "coat_dequant_per_tensor",
                 "coat_dequant_group", "coat_swiglu_fused", "coat_rmsnorm_fused", "coat_status_string"):
        assert want in names


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings(L):
    from activation_compression_amd import coat
    for s in range(8):
        assert coat.status_string(s)
    assert coat.status_string(0) == "ok"
    assert "unknown" in coat.status_string(99)


FAKE = 0x10000  # an aligned, never-dereferenced address


def hp(**kw):
    from activation_compression_amd.coat import AdamWHParams
    d = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1, step=1)
    d.update(kw)
    return AdamWHParams(**d)


def step_call(L, n=1024, G=128, fmt=0, hparams=None, **ptr_over):
    ptrs = dict(param=FAKE, grad=FAKE, mc=FAKE, ma=FAKE, mk=FAKE, vc=FAKE, va=FAKE, vk=FAKE)
    ptrs.update(ptr_over)
    P = ctypes.c_void_p
    return L.coat_adamw_step(*(P(v) for v in ptrs.values()), n, G, fmt,
                             ctypes.byref(hparams or hp()), P(0))


@pytest.mark.parametrize("over, want", [
    (dict(param=0), 1), (dict(vk=0), 1), (dict(grad=FAKE + 2), 2), (dict(mc=FAKE + 8), 2),
    (dict(ma=FAKE + 2), 2),
])
def test_step_rejects_bad_pointers(L, over, want):
    assert step_call(L, **over) == want


@pytest.mark.parametrize("n, G, want", [(1024, 48, 4), (1024, 16, 4), (4096, 2048, 4), (0, 128, 3),
                                        (1000, 128, 3), (-128, 128, 3)])
def test_step_rejects_bad_shapes(L, n, G, want):
    assert step_call(L, n=n, G=G) == want


def test_step_rejects_bad_format_and_hparams(L):
    assert step_call(L, fmt=2) == 5
    assert step_call(L, hparams=hp(beta1=1.0)) == 6
    assert step_call(L, hparams=hp(beta2=-0.1)) == 6
    assert step_call(L, hparams=hp(eps=0.0)) == 6
    assert step_call(L, hparams=hp(step=0)) == 6
    assert step_call(L, hparams=hp(lr=float("nan"))) == 6
    assert L.coat_adamw_step(*([ctypes.c_void_p(FAKE)] * 8), 1024, 128, 0, None, None) == 1


def test_activation_entry_points_validate(L):
    P = ctypes.c_void_p
    f = P(FAKE)
    assert L.coat_group_absmax(P(0), 4, 256, 128, f, f, None) == 1
    assert L.coat_group_absmax(P(FAKE + 4), 4, 256, 128, f, f, None) == 2
    assert L.coat_group_absmax(f, 4, 200, 128, f, f, None) == 3
    assert L.coat_group_absmax(f, 0, 256, 128, f, f, None) == 3
    assert L.coat_group_absmax(f, 4, 256, 100, f, f, None) == 4
    assert L.coat_absmax_reduce(f, 0, f, None) == 3
    assert L.coat_absmax_reduce(P(FAKE + 1), 8, f, None) == 2
    assert L.coat_quant_per_tensor(f, 12, f, f, f, None) == 3
    assert L.coat_quant_per_tensor(f, 16, f, P(FAKE + 8), f, None) == 2
    assert L.coat_quant_per_tensor(f, 16, P(0), f, f, None) == 1
    assert L.coat_quant_group(f, 4, 256, 128, f, f, P(FAKE + 2), None) == 2
    assert L.coat_quant_group(f, 4, 256, 64 * 3, f, f, None, None) == 4
    assert L.coat_quant_group(f, 4, 96, 32, P(0), f, None, None) == 1


def test_new_entry_points_validate(L):
    P = ctypes.c_void_p
    f = P(FAKE)
    ptrs = [f] * 8
    assert L.coat_adamw_step_bf16(*ptrs, P(0), 1024, 128, 0, ctypes.byref(hp()), None) == 1
    assert L.coat_adamw_step_bf16(*ptrs, P(FAKE + 8), 1024, 128, 0, ctypes.byref(hp()), None) == 2
    assert L.coat_adamw_step_bf16(*ptrs, f, 1000, 128, 0, ctypes.byref(hp()), None) == 3
    assert L.coat_dequant_per_tensor(f, 12, f, f, None) == 3
    assert L.coat_dequant_per_tensor(P(FAKE + 4), 16, f, f, None) == 2
    assert L.coat_dequant_per_tensor(f, 16, P(0), f, None) == 1
    assert L.coat_dequant_group(f, 4, 256, 100, f, f, None) == 4
    assert L.coat_dequant_group(f, 4, 200, 128, f, f, None) == 3
    assert L.coat_dequant_group(f, 4, 256, 128, f, P(FAKE + 2), None) == 2


def test_swiglu_validates(L):
    P = ctypes.c_void_p
    f = P(FAKE)
    assert L.coat_swiglu_fused(P(0), f, 4, 256, 128, f, f, None, None, None, None, None) == 1
    assert L.coat_swiglu_fused(f, f, 4, 256, 128, f, f, f, None, None, None, None) == 1  # partial save set
    assert L.coat_swiglu_fused(f, P(FAKE + 2), 4, 256, 128, f, f, None, None, None, None, None) == 2
    assert L.coat_swiglu_fused(f, f, 4, 200, 128, f, f, None, None, None, None, None) == 3
    assert L.coat_swiglu_fused(f, f, 4, 256, 96, f, f, None, None, None, None, None) == 4


def test_rmsnorm_validates(L):
    P, F = ctypes.c_void_p, ctypes.c_float
    f = P(FAKE)
    call = lambda x=f, w=None, rows=4, cols=256, eps=1e-5, G=128, xc=None, xs=None, y=f: L.coat_rmsnorm_fused(
        x, w, rows, cols, F(eps), G, y, f, None, xc, xs, None)
    assert call(x=P(0)) == 1
    assert call(xc=f) == 1  # codes without scales
    assert call(w=P(FAKE + 8)) == 2
    assert call(cols=200) == 3
    assert call(cols=16384, G=1024) == 3  # a row must fit one wave
    assert call(rows=0) == 3
    assert call(G=48) == 4
    assert call(eps=0.0) == 6
    assert call(eps=float("nan")) == 6
