"""Quantization-error study of FP8 optimizer states: dynamic-range expansion
vs plain absmax scaling (k = 1), on synthetic AdamW trajectories.

The COAT explainer (blog.daoxuan.cc/posts/57954, section "expansion
function") reports that the expansion lowers the quantization error of the
optimizer states 1.63x against the naive approach, that typical k is 1-3 for
the first moment and 5-15 for the second, and that after expansion E4M3 and
E5M2 are about equally good for the second moment while E4M3 wins without it.
Those figures come from real training states, which are not available; this
study re-measures the same comparisons on synthetic states (parity unpinned):
binary64 AdamW moments of the single 1024x1024 workload (per-row log-normal
gradient scale) after t steps, quantized in 1x128 groups by the oracle.

Error metrics (the explainer does not define its own): relative RMSE
||x' - x|| / ||x|| and the mean relative error |x' - x| / |x| over nonzero x.

  python tests/study_quant_error.py [--steps 1 5 10 50] [--threads 8]
"""
import argparse
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle as orc  # noqa: E402
from activation_compression_amd import inputs  # noqa: E402

G = 128


def trajectory(steps, spec=None):
    """Binary64 AdamW moments after each step in `steps` (oracle, unquantized)."""
    spec = spec or inputs.single_1024()
    f32 = lambda v: float(np.float32(v))
    theta = inputs.gen_params(spec).numpy().astype(np.float64)
    m = np.zeros(spec.numel)
    v = np.zeros(spec.numel)
    out = {}
    for t in range(1, max(steps) + 1):
        g = (inputs.gen_grads(spec, t).numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
        hp = orc.hparams(f32(inputs.LR), f32(inputs.BETA1), f32(inputs.BETA2), f32(inputs.EPS),
                         f32(inputs.WEIGHT_DECAY), t)
        orc.adamw_step_f64(theta, g.astype(np.float64), m, v, hp)
        if t in steps:
            out[t] = (m.copy(), v.copy())
    return out


def quant_error(x64, fmt, expand, threads):
    x = x64.astype(np.float32)
    k_given = None if expand else np.ones(x.size // G, np.float32)
    codes, amax, k = orc.expand_quantize_groups(fmt, x, G, k_given=k_given, threads=threads)
    back = orc.expand_dequantize_groups(fmt, codes, G, amax, k, threads=threads)
    xd = x.astype(np.float64)
    nz = xd != 0
    rrmse = float(np.linalg.norm(back - xd) / np.linalg.norm(xd))
    mre = float(np.mean(np.abs(back[nz] - xd[nz]) / np.abs(xd[nz])))
    return rrmse, mre, k


def study(steps=(1, 5, 10, 50), threads=8):
    res = {}
    for t, (m, v) in trajectory(steps).items():
        row = {}
        for name, x, fmts in (("m", m, ("e4m3", "e5m2")), ("v", v, ("e4m3", "e5m2"))):
            for fmt in fmts:
                e_rmse, e_mre, k = quant_error(x, fmt, True, threads)
                n_rmse, n_mre, _ = quant_error(x, fmt, False, threads)
                row[f"{name}-{fmt}"] = {
                    "expansion": {"rel_rmse": e_rmse, "mean_rel_err": e_mre},
                    "k1": {"rel_rmse": n_rmse, "mean_rel_err": n_mre},
                    "reduction_rel_rmse": n_rmse / e_rmse,
                    "reduction_mean_rel_err": n_mre / e_mre,
                    "k_percentiles_5_50_95": [float(p) for p in np.percentile(k, [5, 50, 95])],
                }
        res[t] = row
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--steps", type=int, nargs="*", default=[1, 5, 10, 50])
    ap.add_argument("--threads", type=int, default=8)
    args = ap.parse_args()
    res = study(tuple(args.steps), args.threads)
    print(json.dumps(res, indent=1))
    print("\nstep  state-fmt   k(5/50/95%)          rel-RMSE k=1 / expansion (x)   mean-rel-err k=1 / expansion (x)")
    for t, row in res.items():
        for key, r in row.items():
            kp = "/".join(f"{x:.2f}" for x in r["k_percentiles_5_50_95"])
            print(f"{t:4d}  {key:9s}  {kp:20s}  {r['k1']['rel_rmse']:.3e} / {r['expansion']['rel_rmse']:.3e} "
                  f"({r['reduction_rel_rmse']:.2f}x)   {r['k1']['mean_rel_err']:.3e} / "
                  f"{r['expansion']['mean_rel_err']:.3e} ({r['reduction_mean_rel_err']:.2f}x)")


if __name__ == "__main__":
    main()
