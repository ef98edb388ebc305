"""The benchmark's command-line contract, checked without a GPU: more than
one GPU is refused with a message, before anything touches a device."""
import os
import subprocess
import sys

from conftest import ROOT


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_help_lists_the_contract_flags():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup"):
        assert flag in r.stdout


def test_committed_traffic_matches_the_current_kernel_source():
    """The bench reports HBM traffic only from a counter summary taken on the
    kernel source it runs; the committed summary must be that one, and its
    bytes must sit within 1% of the algorithmic bytes it states."""
    sys.path.insert(0, ROOT)
    import bench

    traffic = bench.measured_traffic()
    assert traffic is not None, "profiles/adamw_fp8_step-olmo7b.md was taken on other kernel source"
    from activation_compression_amd import inputs

    alg = inputs.olmo_7b().numel * bench.step_bytes_per_param(128)
    assert abs(traffic / alg - 1.0) < 0.01, (traffic, alg)


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    """A comment or white-space edit keeps the hash (the counters still apply);
    a code edit changes it."""
    sys.path.insert(0, ROOT)
    import shutil

    import bench

    src = os.path.join(ROOT, "activation_compression_amd", "csrc")
    fake = tmp_path / "activation_compression_amd" / "csrc"
    fake.mkdir(parents=True)
    for f in ("adamw_fp8_step.hip", "device.hpp", "kernels.hpp"):
        shutil.copy(os.path.join(src, f), fake / f)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    step = fake / "adamw_fp8_step.hip"
    text = step.read_text()
    step.write_text("// a new comment line\n" + text.replace("\n", "\n   ", 3) + "\n/* trailing */\n")
    assert bench.kernel_source_hash() == h0
    step.write_text(text.replace("kLn2 = 0.693147180559945309417f", "kLn2 = 0.69314718f", 1))
    assert bench.kernel_source_hash() != h0
