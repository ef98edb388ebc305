"""The boundary from plain C: include/coat.h compiles as strict C99 (gcc
-std=c99 -pedantic -Werror) and a C program that dlopens libcoat.so gets the
documented status from every entry point's host-side validation (no call is
valid, so nothing needs a GPU)."""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

LIB = os.path.join(ROOT, "activation_compression_amd", "libcoat.so")
SRC = os.path.join(ROOT, "tests", "c_abi", "abi_check.c")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.skipif(not os.path.exists(LIB), reason="libcoat.so not built")
def test_header_is_c99_and_validation_answers_from_c(tmp_path):
    exe = tmp_path / "abi_check"
    subprocess.run(["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-o", str(exe), SRC, "-ldl"],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe), LIB], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
