"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of oracle/coat_oracle.c (a dropped
term, a wrong sign, an inverted ratio, a wrong constant, an off-by-one
divisor, a wrong index, a different tie rule), builds it with the oracle's
own flags, and runs the oracle pin tests against that build: at least one
pin must fail.  The unmutated source, built the same way, must pass them.
Everything runs on the CPU."""
import os
import shutil
import subprocess
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
from oracle import build as oracle_build  # noqa: E402

SRC = os.path.join(ROOT, "oracle", "coat_oracle.c")
PINS = [os.path.join(ROOT, "tests", f) for f in (
    "test_oracle_codec.py", "test_oracle_expansion.py", "test_oracle_adamw.py", "test_oracle_group_scaling.py",
    "test_oracle_dequant.py", "test_oracle_swiglu.py", "test_oracle_rmsnorm.py")]

MUTATIONS = {
    "adamw-bias-correction-dropped": ("double mhat = *m1 / c->bc1;", "double mhat = *m1;"),
    "adamw-decay-sign": ("return (1.0 - lr * wd) * theta + dtheta;", "return (1.0 + lr * wd) * theta + dtheta;"),
    "adamw-square-dropped": ("*v1 = b2 * v0 + (1.0 - b2) * g * g;", "*v1 = b2 * v0 + (1.0 - b2) * fabs(g);"),
    "k-inverted": ("k = (float)(log(r_fmt) / log(amax / amin));", "k = (float)(log(amax / amin) / log(r_fmt));"),
    "dequant-power-k-not-inverse": ("pow(fabs(d) / orc_fp8_max(fmt), 1.0 / (double)k)",
                                "pow(fabs(d) / orc_fp8_max(fmt), (double)k)"),
    "cast-wrong-max": ("float y = (float)(x * 448.0 / a);", "float y = (float)(x * 240.0 / a);"),
    "silu-sign": ("return x / (1.0 + exp(-x));", "return x / (1.0 + exp(x));"),
    "rmsnorm-mean-divisor": ("double rs = 1.0 / sqrt(ss / (double)cols + (double)eps);",
                             "double rs = 1.0 / sqrt(ss / (double)(cols - 1) + (double)eps);"),
    "group-row-stride": ("int64_t base = r * cols + j * G;", "int64_t base = r * G + j * G;"),
    "encode-ties-up": ("if (d_hi < d_lo || (d_hi == d_lo && (c & 1u)))", "if (d_hi < d_lo || d_hi == d_lo)"),
}


def _build(tmp_path, name, text):
    src = tmp_path / f"{name}.c"
    src.write_text(text)
    lib = tmp_path / f"{name}.so"
    subprocess.run(["gcc", *oracle_build.FLAGS, "-I", os.path.join(ROOT, "oracle"), "-o", str(lib), str(src), "-lm"],
                   check=True, capture_output=True, text=True)
    return lib


def _run_pins(lib):
    env = dict(os.environ, COAT_ORACLE_LIB=str(lib))
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *PINS],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")


def test_unmutated_build_passes_the_pins(tmp_path):
    r = _run_pins(_build(tmp_path, "unmutated", open(SRC).read()))
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_fails_a_pin(tmp_path, name):
    old, new = MUTATIONS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not found exactly once"
    r = _run_pins(_build(tmp_path, name, text.replace(old, new)))
    assert r.returncode == 1, f"{name}: pins did not fail (exit {r.returncode})\n{r.stdout[-1500:]}"
