"""The hot path driven from a plain C program through the C ABI alone
(tests/c_abi/gpu_path.c: hipMalloc'd buffers, a hipStreamCreate'd stream, no
Python between the caller and the library).  Its results are judged against
the oracle here: the fused step to the lockstep parity bar, Group Scaling and
both casts bit for bit."""
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import oracle as orc
from conftest import ROOT
from parity import assert_step_parity, flush, np_state, oracle_step

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
              pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")]

LIB = os.path.join(ROOT, "activation_compression_amd", "libcoat.so")
SRC = os.path.join(ROOT, "tests", "c_abi", "gpu_path.c")
N, G, ROWS, COLS = 32768, 128, 64, 1024


def read_results(path):
    layout = [("theta0", np.float32, N), ("grad", np.uint16, N), ("theta1", np.float32, N),
              ("m_codes", np.uint8, N), ("m_amax", np.float32, N // G), ("m_k", np.float32, N // G),
              ("v_codes", np.uint8, N), ("v_amax", np.float32, N // G), ("v_k", np.float32, N // G),
              ("x", np.uint16, ROWS * COLS), ("partial", np.float32, ROWS * COLS // G), ("amax", np.float32, 1),
              ("codes", np.uint8, ROWS * COLS), ("scale", np.float32, 1), ("gcodes", np.uint8, ROWS * COLS),
              ("gscales", np.float32, ROWS * COLS // G)]
    raw = open(path, "rb").read()
    out, off = {}, 0
    for name, dt, count in layout:
        nbytes = np.dtype(dt).itemsize * count
        out[name] = np.frombuffer(raw, dtype=dt, count=count, offset=off).copy()
        off += nbytes
    assert off == len(raw)
    return out


def norm0(c):
    c = c.copy()
    c[(c & 0x7F) == 0] = 0
    return c


def test_hot_path_from_plain_c(tmp_path):
    exe, out = tmp_path / "gpu_path", tmp_path / "results.bin"
    subprocess.run(["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-o", str(exe), SRC, "-ldl"],
                   check=True, capture_output=True, text=True)
    flush("C driver: coat_adamw_step, coat_group_absmax, coat_quant_per_tensor, coat_quant_group")
    r = subprocess.run([str(exe), LIB, str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    d = read_results(out)

    state = {k: d[k] for k in ("m_codes", "m_amax", "m_k", "v_codes", "v_amax", "v_k")}
    ref = oracle_step(d["theta0"], d["grad"], np_state(N, G), G, "e4m3", 1, threads=1)
    assert_step_parity((d["theta1"], state), ref, "e4m3", "step driven from C")

    x = d["x"].reshape(ROWS, COLS)
    rp, ra = orc.group_absmax(x, G)
    rc, rs = orc.quant_per_tensor(x, ra)
    gc, gs, _ = orc.quant_group(x, G)
    assert (d["partial"] == rp).all() and d["amax"][0] == ra
    assert (norm0(d["codes"]) == rc).all() and d["scale"][0] == rs
    assert (norm0(d["gcodes"]) == gc).all() and (d["gscales"] == gs).all()
