"""coat_adamw_step_list_noalloc: the tensor-list step with its packed table
in the library's own device array, so that the call allocates nothing.

* On the host (no GPU): arguments are validated before anything is
  enqueued, and a table larger than COAT_LIST_NOALLOC_MAX_BYTES is refused
  with COAT_ERR_SCRATCH.
* On the GPU: against coat_adamw_step_list (the caller-owned device table)
  on the same inputs, byte for byte -- both launch the same kernel, so every
  output must be identical -- over calls in a row: a list of nine tensors, then
  a smaller list of three smaller tensors (a shorter table over the longer
  one's leftovers), then the first list again with the state of its first
  step.  The tables' host copies are the only table memory the caller holds.
"""
import ctypes

import numpy as np
import pytest
import torch

from conftest import ROOT  # noqa: F401  (puts the repository on sys.path)

FAKE = 0x10000
MAX_BYTES = 65536
ERR_SCRATCH = 8
KEYS = ("m_codes", "m_amax", "m_k", "v_codes", "v_amax", "v_k")


def _tensor(coat, base, n):
    a = base
    return coat.AdamWTensor(a, a + 0x100000, a + 0x200000, a + 0x300000, a + 0x400000, a + 0x500000,
                            a + 0x600000, a + 0x700000, None, n)


def test_noalloc_validates_before_anything_is_enqueued():
    from activation_compression_amd import coat
    L = coat.lib()
    hp = coat.adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.1, 1)
    # the largest list that fits, and one tensor more
    n_fit = max(n for n in range(1, 2000) if L.coat_adamw_list_bytes(n) <= MAX_BYTES)
    assert n_fit == 744
    for n_t, want in ((n_fit + 1, ERR_SCRATCH), (3000, ERR_SCRATCH)):
        arr = (coat.AdamWTensor * n_t)(*[_tensor(coat, 0x10000000 + 0x1000000 * i, 1024) for i in range(n_t)])
        buf = np.zeros(L.coat_adamw_list_bytes(n_t), np.uint8)
        assert L.coat_adamw_list_pack(arr, n_t, 128, ctypes.c_void_p(buf.ctypes.data)) == 0
        assert L.coat_adamw_step_list_noalloc(ctypes.c_void_p(buf.ctypes.data), 0, ctypes.byref(hp), None) == want
    arr = (coat.AdamWTensor * 2)(_tensor(coat, 0x1000000, 1024), _tensor(coat, 0x2000000, 256))
    buf = np.zeros(L.coat_adamw_list_bytes(2), np.uint8)
    assert L.coat_adamw_list_pack(arr, 2, 128, ctypes.c_void_p(buf.ctypes.data)) == 0
    host = ctypes.c_void_p(buf.ctypes.data)
    assert L.coat_adamw_step_list_noalloc(None, 0, ctypes.byref(hp), None) == 1
    assert L.coat_adamw_step_list_noalloc(host, 0, None, None) == 1
    assert L.coat_adamw_step_list_noalloc(host, 7, ctypes.byref(hp), None) == 5
    bad = coat.adamw_hparams(1e-3, 1.0, 0.999, 1e-8, 0.1, 1)
    assert L.coat_adamw_step_list_noalloc(host, 0, ctypes.byref(bad), None) == 6
    junk = np.zeros_like(buf)
    assert L.coat_adamw_step_list_noalloc(ctypes.c_void_p(junk.ctypes.data), 0, ctypes.byref(hp), None) == 3
    assert coat.status_string(ERR_SCRATCH) != coat.status_string(99)


def _buffers(spec, G, seed):
    """Two identical sets of per-tensor device buffers (random theta, a fresh
    state), one allocation per tensor and array."""
    from activation_compression_amd import inputs
    theta = inputs.gen_params(spec)
    sets = []
    for _ in range(2):
        views = []
        for _, off, n, _ in spec.offsets():
            st = inputs.fresh_state(n, G, device="cuda")
            d = {"param": theta[off:off + n].clone().cuda(), "grad": torch.empty(n, dtype=torch.int16, device="cuda")}
            d.update(st)
            views.append(d)
        sets.append(views)
    return sets


def _grads(spec, sets, t):
    from activation_compression_amd import inputs
    g = inputs.gen_grads(spec, t)
    for views in sets:
        for (_, off, n, _), d in zip(spec.offsets(), views):
            d["grad"].copy_(g[off:off + n])


def _same(a, b):
    for x, y in zip(a, b):
        for k in ("param",) + KEYS:
            assert torch.equal(x[k].view(torch.uint8) if x[k].dtype != torch.uint8 else x[k],
                               y[k].view(torch.uint8) if y[k].dtype != torch.uint8 else y[k]), k


@pytest.mark.gpu
@pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
def test_noalloc_matches_the_list_step_over_calls_in_a_row():
    from activation_compression_amd import coat, inputs
    from parity import flush, gpu_hp
    G = 128
    big = inputs.ragged_list(G, "e4m3")                                   # nine tensors
    small = inputs.ArenaSpec("noalloc-small", 7, (("a", (2, G)), ("b", (7, G)), ("c", (1, G))), "e4m3", G,
                             "tensor")                                     # three smaller tensors
    b_ref, b_new = _buffers(big, G, 1)
    s_ref, s_new = _buffers(small, G, 2)
    lists = {}
    for name, spec, ref, new in (("big", big, b_ref, b_new), ("small", small, s_ref, s_new)):
        lists[name] = (spec, ref, new, coat.AdamWTensorList(ref, group_size=G),
                       coat.AdamWTensorList(new, group_size=G, device_copy=False))
        assert lists[name][4].host.size < MAX_BYTES
    for call, (name, t) in enumerate((("big", 1), ("small", 1), ("big", 2))):
        spec, ref, new, tl_ref, tl_new = lists[name]
        flush(f"no-alloc list step: call {call + 1}, {name} list, step {t}")
        _grads(spec, (ref, new), t)
        coat.coat_adamw_step_list(tl_ref, v_format="e4m3", hp=gpu_hp(t))
        coat.coat_adamw_step_list_noalloc(tl_new, v_format="e4m3", hp=gpu_hp(t))
        torch.cuda.synchronize()
        _same(ref, new)
        assert all(bool((d["m_amax"] > 0).any()) for d in new)
