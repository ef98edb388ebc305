"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/coat.h declares, and rejects invalid arguments
before anything is enqueued (these calls return before any HIP call)."""
import ctypes
import os
import re

import numpy as np

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
                 "coat_dequant_group", "coat_swiglu_fused", "coat_rmsnorm_fused", "coat_adamw_list_bytes",
                 "coat_adamw_list_pack", "coat_adamw_step_list", "coat_status_string"):
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
    # eps must be normal: 1 / eps overflows FP32 below about 2.9e-39
    assert step_call(L, hparams=hp(eps=1e-40)) == 6
    # lr / (1 - b1^t) and 1 - lr wd must be finite in FP32
    assert step_call(L, hparams=hp(lr=3e38)) == 6
    assert step_call(L, hparams=hp(weight_decay=3e38, lr=10.0)) == 6
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


def _tensor(base, n, bf16=False):
    from activation_compression_amd.coat import AdamWTensor
    a = base
    return AdamWTensor(a, a + 0x100000, a + 0x200000, a + 0x300000, a + 0x400000, a + 0x500000, a + 0x600000,
                       a + 0x700000, a + 0x800000 if bf16 else None, n)


def _list_lib():
    from activation_compression_amd import coat
    return coat.lib(), coat


def test_list_bytes():
    L, _ = _list_lib()
    assert L.coat_adamw_list_bytes(0) == 0 and L.coat_adamw_list_bytes(-3) == 0
    assert L.coat_adamw_list_bytes(1) == 32 + 16 + 80
    assert L.coat_adamw_list_bytes(3) == 32 + 32 + 240
    assert L.coat_adamw_list_bytes(130) == 32 + 1056 + 130 * 80


def test_list_pack_layout():
    """Header, chunk prefix (ceil(n/1024) per tensor, in order) and entries,
    read back with numpy from the packed bytes."""
    L, coat = _list_lib()
    sizes = [128, 1024, 1152, 384, 2048 * 5 + 128]
    arr = (coat.AdamWTensor * len(sizes))(*[_tensor(0x1000000 * (i + 1), n) for i, n in enumerate(sizes)])
    buf = np.zeros(L.coat_adamw_list_bytes(len(sizes)), np.uint8)
    assert L.coat_adamw_list_pack(arr, len(sizes), 128, ctypes.c_void_p(buf.ctypes.data)) == 0
    hdr = buf[:32].view(np.int32)
    assert hdr[2] == len(sizes) and hdr[3] == 128 and hdr[4] == 0
    chunks = [-(-n // 1024) for n in sizes]
    assert buf[24:32].view(np.int64)[0] == sum(chunks)
    starts = buf[32:32 + 8 * (len(sizes) + 1)].view(np.int64)
    assert list(starts) == list(np.concatenate([[0], np.cumsum(chunks)]))
    ent = buf[32 + 48:].view(np.int64).reshape(len(sizes), 10)
    for i, n in enumerate(sizes):
        base = 0x1000000 * (i + 1)
        assert list(ent[i, :8]) == [base + 0x100000 * j for j in range(8)]
        assert ent[i, 8] == 0 and ent[i, 9] == n


def test_list_pack_validates():
    L, coat = _list_lib()
    buf = np.zeros(4096, np.uint8)
    out = ctypes.c_void_p(buf.ctypes.data)

    def pack(ts, G=128):
        arr = (coat.AdamWTensor * len(ts))(*ts)
        return L.coat_adamw_list_pack(arr, len(ts), G, out)

    good = _tensor(0x1000000, 1024)
    assert pack([good, _tensor(0x2000000, 256)]) == 0
    bad_null = _tensor(0x2000000, 256); bad_null.m_k = None
    assert pack([good, bad_null]) == 1
    assert pack([good, _tensor(0x2000008, 256)]) == 2     # param not 16-byte aligned
    assert pack([good, _tensor(0x2000000, 200)]) == 3     # n % G
    assert pack([good, _tensor(0x2000000, 0)]) == 3
    assert pack([good], G=96) == 4
    assert pack([good, _tensor(0x2000000, 256, bf16=True)]) == 1  # BF16 copy on some entries only
    assert L.coat_adamw_list_pack((coat.AdamWTensor * 1)(good), 0, 128, out) == 3
    assert L.coat_adamw_list_pack(None, 1, 128, out) == 1


def test_step_list_validates_before_launch():
    """Every error below is found on the host; nothing is launched."""
    L, coat = _list_lib()
    arr = (coat.AdamWTensor * 2)(_tensor(0x1000000, 1024), _tensor(0x2000000, 256))
    buf = np.zeros(L.coat_adamw_list_bytes(2), np.uint8)
    assert L.coat_adamw_list_pack(arr, 2, 128, ctypes.c_void_p(buf.ctypes.data)) == 0
    host = ctypes.c_void_p(buf.ctypes.data)
    hp = coat.adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.1, 1)
    devp = ctypes.c_void_p(FAKE)
    assert L.coat_adamw_step_list(None, devp, 0, ctypes.byref(hp), None) == 1
    assert L.coat_adamw_step_list(host, None, 0, ctypes.byref(hp), None) == 1
    assert L.coat_adamw_step_list(host, ctypes.c_void_p(FAKE + 4), 0, ctypes.byref(hp), None) == 2
    assert L.coat_adamw_step_list(host, devp, 7, ctypes.byref(hp), None) == 5
    bad = coat.adamw_hparams(1e-3, 1.0, 0.999, 1e-8, 0.1, 1)
    assert L.coat_adamw_step_list(host, devp, 0, ctypes.byref(bad), None) == 6
    junk = np.zeros_like(buf)
    assert L.coat_adamw_step_list(ctypes.c_void_p(junk.ctypes.data), devp, 0, ctypes.byref(hp), None) == 3


def test_sizes_beyond_the_launch_grid_are_rejected(L):
    """(2^31 - 1) * 4096 elements is the most one launch covers; validation
    rejects more before anything is enqueued."""
    P = ctypes.c_void_p
    f = P(FAKE)
    big = (2 ** 31) * 4096
    assert L.coat_quant_per_tensor(f, big, f, f, f, None) == 3
    assert L.coat_quant_group(f, big // 4096, 4096, 128, f, f, None, None) == 3
    assert L.coat_dequant_per_tensor(f, big, f, f, None) == 3
    from activation_compression_amd import coat
    hp = coat.adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.1, 1)
    lib = coat.lib()
    assert lib.coat_adamw_step(f, f, f, f, f, f, f, f, big, 128, 0, ctypes.byref(hp), None) == 3
    assert L.coat_rmsnorm_fused(f, None, 2 ** 33 + 8, 1024, ctypes.c_float(1e-5), 128, f, f, None, None, None,
                                None) == 3


def test_empty_inputs_are_rejected(L):
    """Zero-size inputs are a shape error everywhere (nothing is enqueued)."""
    P = ctypes.c_void_p
    f = P(FAKE)
    from activation_compression_amd import coat
    lib = coat.lib()
    hp = coat.adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.1, 1)
    assert lib.coat_adamw_step(f, f, f, f, f, f, f, f, 0, 128, 0, ctypes.byref(hp), None) == 3
    assert L.coat_quant_per_tensor(f, 0, f, f, f, None) == 3
    assert L.coat_dequant_per_tensor(f, 0, f, f, None) == 3
    assert L.coat_quant_group(f, 0, 4096, 128, f, f, None, None) == 3
    assert L.coat_quant_group(f, 16, 0, 128, f, f, None, None) == 3
    assert L.coat_dequant_group(f, 16, 0, 128, f, f, None) == 3
    assert L.coat_swiglu_fused(f, f, 0, 256, 128, f, f, None, None, None, None, None) == 3
    assert L.coat_group_absmax(f, 16, 0, 128, f, f, None) == 3


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No fallback: without libcoat.so every entry point raises before doing
    any work (the product path has no CPU implementation to fall back to)."""
    from activation_compression_amd import coat
    monkeypatch.setattr(coat, "_lib", None)
    monkeypatch.setattr(coat, "LIB_PATH", str(tmp_path / "libcoat.so"))
    with pytest.raises(coat.CoatError, match="missing"):
        coat.lib()
    with pytest.raises(coat.CoatError, match="missing"):
        coat.status_string(0)
