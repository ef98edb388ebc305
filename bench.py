"""Benchmark: FP8-state AdamW params updated/s and achieved HBM GB/s on one MI355X.

One step is one pass of the whole hot path over synthetic inputs resident in
HBM:
  1. the fused FP8-state AdamW step over the OLMo-7B-shaped parameter arena
     (6 888 095 744 FP32 master weights, BF16 gradients, m and v in E4M3,
     G = 128) -- one coat_adamw_step launch for the whole arena;
  2. Group Scaling of a linear-layer input [16384 x 4096]: the 1x128 E4M3
     group cast writes the per-slice maxima in the same pass (stage 1,
     coat_quant_group), stage 2 reduces them (coat_absmax_reduce), and the
     per-tensor E4M3 cast follows (coat_quant_per_tensor) -- two reads of X;
  3. the 1x128 E4M3 group cast of a SwiGLU input [16384 x 11008].
value = parameters updated per second of whole steps.  The roofline entry is
the dominant kernel, the AdamW step: algorithmic bytes per launch
(14 + 32/G bytes per parameter) over its average launch time, measured with
HIP events on the stream it runs on.  Each activation kernel is also timed
alone after a read-only pass over 1 GiB has evicted the caches, so that its
frac_of_peak is an HBM fraction (in the step the per-tensor cast re-reads X
from the Infinity Cache).  The CPU baseline is the oracle on the host's
cores: the 7B step on a contiguous 1/8 shard of the arena (extrapolated), and
the other workloads in full.

The step is also timed on a second copy of its buffers ("placement"): where
the buffers land in device memory moves the step by several percent, and a
process's first large allocation, which `value` measures, is usually a slow
placement.

Beside the step (not in `value`), "extras" times the other entry points on
the same resident workloads: the step with its BF16 working copy, the step as a
tensor-list launch (one entry per model tensor), the fused SwiGLU and RMSNorm
producers with Group Scaling stage 1 in their epilogues,
and the FP8 -> BF16 activation dequantization.

  python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--cpu-baseline plan|quick|none] [--no-extras]
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
PMC_SUMMARY = os.path.join(ROOT, "profiles", "adamw_fp8_step-olmo7b.md")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def step_bytes_per_param(G):
    # theta r+w 8, grad 2, m codes r+w 2, v codes r+w 2, (amax, k) x 2 states r+w per group
    return 14.0 + 32.0 / G


def kernel_source_hash():
    """Hash of the step kernel's code: its sources with comments removed and
    runs of white space folded, so that a comment edit keeps the counters
    taken on the same code."""
    h = hashlib.sha256()
    for f in ("adamw_fp8_step.hip", "device.hpp", "kernels.hpp"):
        with open(os.path.join(ROOT, "activation_compression_amd", "csrc", f)) as fh:
            code = re.sub(r"/\*.*?\*/", " ", fh.read(), flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it was
    taken on the current kernel source; else None."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    text = open(PMC_SUMMARY).read()
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


CEILING_SRC = os.path.join(ROOT, "bench_ceiling.hip")
CEILING_LIB = os.path.join(ROOT, "_build", "libbench_ceiling.so")


def build_ceiling_lib(force=False):
    """Compile the memory-only reference kernels (bench_ceiling.hip) with hipcc
    for gfx950 into _build/, when forced or when the library is missing or
    older than the source."""
    import subprocess

    if force or not os.path.exists(CEILING_LIB) or os.path.getmtime(CEILING_LIB) < os.path.getmtime(CEILING_SRC):
        os.makedirs(os.path.dirname(CEILING_LIB), exist_ok=True)
        hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
        subprocess.run([hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        "-o", CEILING_LIB + ".tmp", CEILING_SRC], check=True)
        os.replace(CEILING_LIB + ".tmp", CEILING_LIB)
    return CEILING_LIB


def ceiling_lib():
    """The memory-only reference kernels, built first if needed."""
    import ctypes

    L = ctypes.CDLL(build_ceiling_lib())
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.ceiling_step_skeleton.argtypes = [P] * 8 + [i64, i32, i32, P]
    L.ceiling_copy_1r1w.argtypes = [P, P, i64, P]
    L.ceiling_copy_4r3w.argtypes = [P] * 7 + [i64, P]
    return L


def memory_ceiling(theta, grad, st, n, alg_bytes, reps=3):
    """What this device's HBM delivers for the step's own traffic, measured on
    the benchmark's own buffers after the timed region (it overwrites them):
    the memory-only skeleton of the step at residency caps of 2-5 workgroups
    per CU (5 is the step's) and uncapped, with and without the per-group
    metadata traffic; a plain one-read-one-write copy; and an equal-size copy
    of four read and three write streams (the step's stream count)."""
    import ctypes

    import torch

    L = ceiling_lib()
    P = ctypes.c_void_p
    stream = P(torch.cuda.current_stream().cuda_stream)
    ptrs = [P(t.data_ptr()) for t in (theta, grad, st["m_codes"], st["m_amax"], st["m_k"], st["v_codes"],
                                      st["v_amax"], st["v_k"])]

    def timed(fn):
        assert fn() == 0
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    gbs = lambda b, ms: round(b / (ms * 1e-3) / 1e9, 1)
    alg_nometa = n * 14.0
    skel, nometa = {}, {}
    for cap in (2, 3, 4, 5, 0):
        skel[cap] = timed(lambda: L.ceiling_step_skeleton(*ptrs, n, cap, 1, stream))
        nometa[cap] = timed(lambda: L.ceiling_step_skeleton(*ptrs, n, cap, 0, stream))
    b_best = min(skel, key=skel.get)
    nb = grad.numel() * grad.element_size()
    ms_copy = timed(lambda: L.ceiling_copy_1r1w(P(theta.data_ptr()), P(grad.data_ptr()), nb, stream))
    S = theta.numel() * 4 // 7 // 16 * 16
    base = theta.data_ptr()
    streams = [P(base + i * S) for i in range(7)]
    ms_4r3w = timed(lambda: L.ceiling_copy_4r3w(*streams, S, stream))
    name = lambda c: f"cap{c}" if c else "uncapped"
    return {"step_memory_skeleton_gb_per_s": gbs(alg_bytes, skel[5]),
            "best_memory_skeleton_gb_per_s": gbs(alg_bytes, skel[b_best]),
            "best_memory_skeleton_blocks_per_cu": b_best or "uncapped",
            "skeleton_gb_per_s_by_residency": {name(c): gbs(alg_bytes, skel[c]) for c in skel},
            "skeleton_without_metadata_gb_per_s_by_residency": {name(c): gbs(alg_nometa, nometa[c]) for c in nometa},
            "copy_gb_per_s": gbs(2 * nb, ms_copy),
            "copy_4r3w_equal_streams_gb_per_s": gbs(7 * S, ms_4r3w),
            "note": ("skeleton times: the step's bytes with trivial arithmetic; without metadata it moves 14 B per "
                     "parameter and its GB/s counts those")}


def state_diagnostics(st, sample=1 << 22):
    """The expansion exponents of the optimizer state after the timed steps
    (the COAT explainer gives k of 1-3 for m and 5-15 for v on real states):
    percentiles of k over a fixed sample of groups, the share of groups with
    k < 1 (wider than the format) and of all-zero groups."""
    import torch

    out = {}
    ng = st["m_k"].numel()
    count = min(sample, ng)
    # integer stride: every index below ng (a float32 linspace rounds its last
    # index up to ng at this size)
    idx = torch.arange(count, device=st["m_k"].device) * (ng // count)
    assert int(idx[-1]) < ng
    for name in ("m", "v"):
        k = st[f"{name}_k"][idx]
        a = st[f"{name}_amax"][idx]
        q = torch.quantile(k, torch.tensor([0.05, 0.5, 0.95], device=k.device)).tolist()
        out[name] = {"k_p5_p50_p95": [round(x, 3) for x in q],
                     "frac_k_below_1": round(float((k < 1).float().mean()), 5),
                     "frac_zero_groups": round(float((a == 0).float().mean()), 5)}
    return out


def second_allocation_ms(coat, theta, grad, st, G, v_fmt, hp, step0, reps=5):
    """The AdamW step timed again on a second copy of its buffers, allocated
    while the first is still live (HIP events, `reps` launches after one
    warm-up).  The step's time depends on where in device memory the
    buffers land, and a process's first large allocation is usually a slow
    placement; the benchmark's value and roofline keep the first allocation,
    this figure stands beside them."""
    import torch

    th2, g2 = theta.clone(), grad.clone()
    s2 = {k: v.clone() for k, v in st.items()}
    torch.cuda.synchronize()
    ms = time_launches(lambda i: coat.coat_adamw_step(
        th2, g2, s2["m_codes"], s2["m_amax"], s2["m_k"], s2["v_codes"], s2["v_amax"], s2["v_k"],
        group_size=G, v_format=v_fmt, hp=hp(step0 + i)), reps)
    del th2, g2, s2
    torch.cuda.synchronize()
    return ms


def time_launches(fn, reps):
    """Average milliseconds of `fn` (launches on torch's current stream), HIP
    events on that stream around `reps` back-to-back calls after one warm-up."""
    import torch

    fn(0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        fn(i + 1)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def entry(alg_bytes, ms, elems=None):
    d = {"ms": round(ms, 4), "algorithmic_bytes": int(alg_bytes),
         "gb_per_s": round(alg_bytes / (ms * 1e-3) / 1e9, 1),
         "frac_of_peak": round(alg_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    if elems:
        d["elements_per_s"] = elems / (ms * 1e-3)
    return d


def cold_activation_times(coat, xs, partial, amax, codes_pt, scale_pt, gcodes, gscales, G, reps=10):
    """Each activation kernel of the step alone, after a read-only pass over
    1 GiB has evicted the L2s and the 256 MB Infinity Cache: average of `reps`
    launches, HIP events around the kernel only.  Also both stages of Group
    Scaling as one standalone call (coat_group_absmax), cold and warm (right
    after a launch over the same input)."""
    import torch

    evict = torch.ones(1 << 28, device="cuda")   # 1 GiB

    def cold(fn):
        tot = 0.0
        for _ in range(reps):
            evict.amax()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            tot += e0.elapsed_time(e1)
        return tot / reps

    def warm(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    out = {
        "quant_group_stage1_linear": cold(lambda: coat.coat_quant_group(xs[0], gcodes[0], gscales[0], partial,
                                                                        group_size=G)),
        "absmax_reduce": cold(lambda: coat.coat_absmax_reduce(partial, amax)),
        "quant_per_tensor": cold(lambda: coat.coat_quant_per_tensor(xs[0], amax, codes_pt, scale_pt)),
        "quant_group_swiglu": cold(lambda: coat.coat_quant_group(xs[1], gcodes[1], gscales[1], None,
                                                                 group_size=G)),
    }
    N0 = xs[0].numel()
    ga = lambda: coat.coat_group_absmax(xs[0], partial, amax, group_size=G)
    b = N0 * 2 + 2 * 4 * N0 / G
    c_ms, w_ms = cold(ga), warm(ga)
    out["group_absmax_standalone"] = {
        "cold": entry(b, c_ms, N0), "warm_cache_assisted": entry(b, w_ms, N0),
        "note": ("both stages of Group Scaling as one call, outside the step (whose stage 1 comes from the "
                 "1x128 cast's pass); warm: right after a launch over the same input, which the Infinity "
                 "Cache then holds")}
    del evict
    torch.cuda.synchronize()
    return out


def extras(coat, inputs, theta, grad, st, spec, G, step0, reps=10):
    """The entry points beside the timed step, each timed alone on the same
    HBM-resident workloads: the step on the OLMo-1B-shaped set (median of
    steps 2-5); the step with its BF16 working-copy output; the
    step as a tensor-list launch over the model's tensors; the
    fused SwiGLU and RMSNorm producers (stage 1 in the epilogue, with and
    without saving the inputs in 1xG E4M3), against the same op followed by
    a separate stage-1 pass over its output; and the FP8 -> BF16 dequantization of saved activations."""
    import torch

    out = {}
    n = spec.numel
    f = float
    hp = lambda t: coat.adamw_hparams(f(inputs.LR), f(inputs.BETA1), f(inputs.BETA2), f(inputs.EPS),
                                      f(inputs.WEIGHT_DECAY), t)
    wcopy = torch.empty(n, dtype=torch.int16, device="cuda")
    ms = time_launches(lambda i: coat.coat_adamw_step_bf16(
        theta, grad, st["m_codes"], st["m_amax"], st["m_k"], st["v_codes"], st["v_amax"], st["v_k"], wcopy,
        group_size=G, v_format=spec.v_fmt, hp=hp(step0 + i)), 3)
    out["adamw_fp8_step_bf16_copy"] = entry(n * (16.0 + 32.0 / G), ms, n)
    del wcopy

    # the same step through the tensor-list launch: one entry per tensor of
    # the model (views of the arena, so the bytes are the same), one launch
    views = []
    for _, off, m, _ in spec.offsets():
        d = {"param": theta[off:off + m], "grad": grad[off:off + m]}
        for k in ("m_codes", "m_amax", "m_k", "v_codes", "v_amax", "v_k"):
            d[k] = st[k][off:off + m] if k.endswith("codes") else st[k][off // G:(off + m) // G]
        views.append(d)
    tl = coat.AdamWTensorList(views, group_size=G)
    ms = time_launches(lambda i: coat.coat_adamw_step_list(tl, v_format=spec.v_fmt, hp=hp(step0 + 4 + i)), 3)
    out[f"adamw_fp8_step_list_{len(views)}_tensors"] = entry(n * (14.0 + 32.0 / G), ms, n)
    del tl, views

    log("extras: the stress set and the single 1024 x 1024 tensor")
    # the stress set (64 Mi params, gradients over ten decades, 5% zeros) for
    # G in {32, 128, 512} and both v formats, and the single 1024 x 1024 tensor
    # (a launch-bound correctness workload): average of 10 steps after 2
    for sp in [inputs.stress(g_, f_) for g_ in (32, 128, 512) for f_ in ("e4m3", "e5m2")] + [inputs.single_1024()]:
        ns = sp.numel
        ths = inputs.gen_params(sp, device="cuda")
        gs_ = inputs.gen_grads(sp, 1, device="cuda")
        sts = inputs.fresh_state(ns, sp.group_size, device="cuda")
        ms_s = time_launches(lambda i: coat.coat_adamw_step(
            ths, gs_, sts["m_codes"], sts["m_amax"], sts["m_k"], sts["v_codes"], sts["v_amax"], sts["v_k"],
            group_size=sp.group_size, v_format=sp.v_fmt, hp=hp(i + 1)), 10)
        out[f"adamw_fp8_step_{sp.name}"] = entry(ns * (14.0 + 32.0 / sp.group_size), ms_s, ns)
        del ths, gs_, sts

    log("extras: the OLMo-1B-shaped set")
    # the OLMo-1B-shaped parameter set (v in E5M2): five steps from a fresh
    # state, the median of steps 2-5 (each step timed alone)
    s1 = inputs.olmo_1b()
    n1 = s1.numel
    th1 = inputs.gen_params(s1, device="cuda")
    g1 = inputs.gen_grads(s1, 1, device="cuda")
    st1 = inputs.fresh_state(n1, G, device="cuda")
    times = []
    for t in range(1, 6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        coat.coat_adamw_step(th1, g1, st1["m_codes"], st1["m_amax"], st1["m_k"], st1["v_codes"], st1["v_amax"],
                             st1["v_k"], group_size=G, v_format=s1.v_fmt, hp=hp(t))
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms1 = sorted(times[1:])[1:3]
    out["adamw_fp8_step_olmo1b_e5m2"] = entry(n1 * (14.0 + 32.0 / G), sum(ms1) / 2, n1)
    del th1, g1, st1

    log("extras: the fused producers and the dequantizations")
    gs, us = inputs.swiglu_gate(), inputs.swiglu_up()
    N = gs.numel
    gate, up = inputs.gen_activation(gs, device="cuda"), inputs.gen_activation(us, device="cuda")
    h = torch.empty(N, dtype=torch.int16, device="cuda")
    hp_ = torch.empty(N // G, device="cuda")
    saved = (torch.empty(N, dtype=torch.uint8, device="cuda"), torch.empty(N // G, device="cuda"),
             torch.empty(N, dtype=torch.uint8, device="cuda"), torch.empty(N // G, device="cuda"))
    amax = torch.empty(1, device="cuda")
    ms_f = time_launches(lambda i: coat.coat_swiglu_fused(gate, up, h, hp_, None, group_size=G), reps)
    ms_s = time_launches(lambda i: coat.coat_swiglu_fused(gate, up, h, hp_, saved, group_size=G), reps)
    h2 = h.view(gs.rows, gs.cols)
    ms_a = time_launches(lambda i: coat.coat_group_absmax(h2, hp_, amax, group_size=G), reps)
    shape = f"{gs.rows}x{gs.cols}"
    out[f"swiglu_fused_{shape}"] = entry(6 * N + 4 * N / G, ms_f, N)
    out[f"swiglu_fused_save_inputs_{shape}"] = entry(8 * N + 12 * N / G, ms_s, N)
    out[f"swiglu_then_separate_stage1_{shape}"] = {
        "ms": round(ms_f + ms_a, 4), "algorithmic_bytes": int(8 * N + 8 * N / G),
        "stage1_share_fused": round(4 * N / G / (6 * N + 4 * N / G), 4),
        "stage1_share_separate": round(ms_a / (ms_f + ms_a), 4)}

    rs = inputs.rmsnorm_input()
    Nr = rs.numel
    x = inputs.gen_activation(rs, device="cuda")
    w = inputs.gen_norm_weight(rs.cols, device="cuda")
    y = torch.empty(Nr, dtype=torch.int16, device="cuda")
    yp = torch.empty(Nr // G, device="cuda")
    rstd = torch.empty(rs.rows, device="cuda")
    xsave = (torch.empty(Nr, dtype=torch.uint8, device="cuda"), torch.empty(Nr // G, device="cuda"))
    ms_r = time_launches(lambda i: coat.coat_rmsnorm_fused(x, w, y, yp, rstd, None, group_size=G), reps)
    ms_rs = time_launches(lambda i: coat.coat_rmsnorm_fused(x, w, y, yp, rstd, xsave, group_size=G), reps)
    ms_ra = time_launches(lambda i: coat.coat_group_absmax(y.view(rs.rows, rs.cols), yp, amax, group_size=G), reps)
    rshape = f"{rs.rows}x{rs.cols}"
    base_r = 4 * Nr + 4 * Nr / G + 4 * rs.rows + 2 * rs.cols
    out[f"rmsnorm_fused_{rshape}"] = entry(base_r, ms_r, Nr)
    out[f"rmsnorm_fused_save_input_{rshape}"] = entry(base_r + Nr + 4 * Nr / G, ms_rs, Nr)
    out[f"rmsnorm_then_separate_stage1_{rshape}"] = {
        "ms": round(ms_r + ms_ra, 4), "algorithmic_bytes": int(base_r + 2 * Nr + 4 * Nr / G),
        "stage1_share_fused": round(4 * Nr / G / base_r, 4),
        "stage1_share_separate": round(ms_ra / (ms_r + ms_ra), 4)}
    del x, w, y, yp, rstd, xsave

    codes, scales = saved[0], saved[1]
    out16 = h
    ms_dg = time_launches(lambda i: coat.coat_dequant_group(codes, scales, out16, rows=gs.rows, cols=gs.cols,
                                                              group_size=G), reps)
    out[f"dequant_group_{shape}"] = entry(3 * N + 4 * N / G, ms_dg, N)
    ms_dt = time_launches(lambda i: coat.coat_dequant_per_tensor(codes, scales[:1], out16), reps)
    out[f"dequant_per_tensor_{shape}"] = entry(3 * N + 4, ms_dt, N)
    del gate, up, h, hp_, saved
    torch.cuda.synchronize()
    return out


def _oracle_steps(spec, threads, steps=(1, 2), time_steps=(2,), tensors=None):
    """Run the oracle's step on (a prefix of the tensors of) an arena from a
    fresh state; returns (parameters, seconds of each step in time_steps)."""
    import numpy as np

    import oracle as orc
    from activation_compression_amd import inputs

    sub = spec if tensors is None else inputs.ArenaSpec(spec.name + "-shard", spec.config, spec.tensors[:tensors],
                                                        spec.v_fmt, spec.group_size, spec.grad_scale)
    n, G = sub.numel, sub.group_size
    theta = inputs.gen_params(sub).numpy()
    st = {k: v.numpy() for k, v in inputs.fresh_state(n, G).items()}
    f32 = lambda v: float(np.float32(v))
    secs = []
    for t in steps:
        g = inputs.gen_grads(sub, t).numpy().view(np.uint16)
        hp = orc.hparams(f32(inputs.LR), f32(inputs.BETA1), f32(inputs.BETA2), f32(inputs.EPS),
                         f32(inputs.WEIGHT_DECAY), t)
        t0 = time.perf_counter()
        orc.adamw_step(theta, g, st["m_codes"], st["m_amax"], st["m_k"], st["v_codes"], st["v_amax"], st["v_k"],
                       G=G, v_fmt=sub.v_fmt, hp=hp, threads=threads)
        if t in time_steps:
            secs.append(time.perf_counter() - t0)
    return n, secs


def _oracle_activations(acts, G, threads, rows=None):
    """The step's activation pass on the oracle: stage 1 and stage 2 and the
    per-tensor cast of the first tensor, the 1xG cast of both (on the first
    `rows` rows of each when given, scaled to the whole tensors)."""
    import numpy as np

    import oracle as orc
    from activation_compression_amd import inputs

    tot = 0.0
    for i, act in enumerate(acts):
        r = act.rows if rows is None else rows
        x = inputs.gen_activation(inputs.ActivationSpec(act.name, r, act.cols, act.seed)).numpy().view(np.uint16)
        t0 = time.perf_counter()
        if i == 0:
            _, amax = orc.group_absmax(x, G, threads=threads)
            orc.quant_per_tensor(x, amax, threads=threads)
        orc.quant_group(x, G, threads=threads)
        tot += (time.perf_counter() - t0) * act.rows / r
    return tot


def cpu_baseline(spec, acts, G, threads, plan=True):
    """The binary64 C oracle (as it stands) on the host's cores.

    value: params/s of the benchmark's whole step -- the OLMo-7B-shaped AdamW
    step timed on a contiguous 1/8 shard of the arena (its first tensors, the
    largest prefix within n/8; step 2 from the oracle's own step 1, so that the
    dequantized moments are nonzero) and extrapolated linearly to the whole
    arena, plus the activation pass on the full tensors.  plan=True also times
    the other workloads in full: the single 1024x1024 tensor (ten steps), the
    OLMo-1B-shaped set (step 2), the 64 Mi stress set for G in {32, 128, 512}
    x both v formats (its step 1 and step 2), and a single-thread rate."""
    import numpy as np  # noqa: F401

    from activation_compression_amd import inputs

    sizes = [r * c for _, (r, c) in spec.tensors]
    k, acc = 0, 0
    while k < len(sizes) and acc + sizes[k] <= spec.numel // 8:
        acc += sizes[k]
        k += 1
    n_shard, (t_shard,) = _oracle_steps(spec, threads, tensors=k)
    t_step = t_shard * spec.numel / n_shard
    if plan:
        t_act = _oracle_activations(acts, G, threads)
        act_note = "the activation pass on the full tensors"
    else:
        t_act = _oracle_activations(acts, G, threads, rows=2048)
        act_note = "the activation pass on the first 2048 rows of each tensor (scaled)"
    out = {
        "value": spec.numel / (t_step + t_act),
        "unit": "params/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"OLMo-7B-shaped AdamW step 2 on a contiguous shard of the arena (its first {k} tensors, "
                   f"{n_shard} params = 1/{spec.numel / n_shard:.3f} of it), extrapolated x"
                   f"{spec.numel / n_shard:.3f}; {act_note}; binary64 C oracle, {threads} threads"),
        "extrapolated": True,
        "seconds_per_step": t_step + t_act,
        "step_params_per_s": spec.numel / t_step,
        "activation_pass_s": t_act,
    }
    if plan:
        cfg = {}
        s1 = inputs.single_1024()
        n1, secs = _oracle_steps(s1, threads, steps=range(1, 11), time_steps=range(1, 11))
        cfg["single_1024x1024_10_steps"] = {"params": n1, "s_per_step": sum(secs) / 10,
                                            "params_per_s": n1 * 10 / sum(secs)}
        s3 = inputs.olmo_1b()
        n3, (t3,) = _oracle_steps(s3, threads)
        cfg["olmo_1b_shaped_step2"] = {"params": n3, "s_per_step": t3, "params_per_s": n3 / t3}
        for g_ in (32, 128, 512):
            for f_ in ("e4m3", "e5m2"):
                s5 = inputs.stress(g_, f_)
                n5, (a5, b5) = _oracle_steps(s5, threads, time_steps=(1, 2))
                cfg[f"stress_64Mi_G{g_}_{f_}"] = {"params": n5, "s_step1": a5, "s_step2": b5,
                                                   "params_per_s_step1": n5 / a5}
        cfg["activations_full"] = {"s": t_act, "tensors": [[a.rows, a.cols] for a in acts]}
        m1 = 8 << 20
        s1t = inputs.ArenaSpec("single-thread-8Mi", 4, (("w", (m1 // 4096, 4096)),), spec.v_fmt, G, "tensor")
        n1t, (tt,) = _oracle_steps(s1t, 1)
        out["single_thread_step_params_per_s"] = n1t / tt
        out["configs"] = cfg
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-baseline", choices=("plan", "quick", "none"), default="plan",
                    help="plan: the 7B step on a 1/8 shard plus every other workload in full; quick: the shard "
                         "and a sample of the activations only")
    ap.add_argument("--no-extras", action="store_true", help="skip the entry points timed beside the step")
    ap.add_argument("--cpu-threads", type=int, default=0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain device copies of a known size (to scale the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from activation_compression_amd import coat, inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        nbytes = 4 << 30
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read_per_launch": nbytes,
                          "copy_calibration_bytes_written_per_launch": nbytes, "launches": 3}), flush=True)
        return
    coat.lib()
    spec = inputs.olmo_7b()
    G = spec.group_size
    n = spec.numel
    acts = [inputs.linear_input(), inputs.swiglu_input()]

    log(f"allocating {spec.name}: {n} params")
    theta = inputs.gen_params(spec, device="cuda")
    grad = inputs.gen_grads(spec, 1, device="cuda")
    st = inputs.fresh_state(n, G, device="cuda")
    xs = [inputs.gen_activation(a, device="cuda") for a in acts]
    partial = torch.empty(acts[0].numel // G, device="cuda")
    amax = torch.empty(1, device="cuda")
    codes_pt = torch.empty(acts[0].numel, dtype=torch.uint8, device="cuda")
    scale_pt = torch.empty(1, device="cuda")
    gcodes = [torch.empty(a.numel, dtype=torch.uint8, device="cuda") for a in acts]
    gscales = [torch.empty(a.numel // G, device="cuda") for a in acts]
    torch.cuda.synchronize()

    f = lambda v: float(v)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def one_step(t, marks=None):
        hp = coat.adamw_hparams(f(inputs.LR), f(inputs.BETA1), f(inputs.BETA2), f(inputs.EPS),
                                f(inputs.WEIGHT_DECAY), t)
        if marks: marks[0].record()
        coat.coat_adamw_step(theta, grad, st["m_codes"], st["m_amax"], st["m_k"], st["v_codes"], st["v_amax"],
                             st["v_k"], group_size=G, v_format=spec.v_fmt, hp=hp)
        if marks: marks[1].record()
        coat.coat_quant_group(xs[0], gcodes[0], gscales[0], partial, group_size=G)
        if marks: marks[2].record()
        coat.coat_absmax_reduce(partial, amax)
        if marks: marks[3].record()
        coat.coat_quant_per_tensor(xs[0], amax, codes_pt, scale_pt)
        if marks: marks[4].record()
        coat.coat_quant_group(xs[1], gcodes[1], gscales[1], None, group_size=G)
        if marks: marks[5].record()

    step = 0
    for _ in range(args.warmup):
        step += 1
        one_step(step)
    torch.cuda.synchronize()
    log(f"warm-up done ({args.warmup} steps); timing {args.steps} steps")

    marks = [[ev() for _ in range(6)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    start, stop = ev(), ev()
    start.record()
    for i in range(args.steps):
        step += 1
        one_step(step, marks[i])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = start.elapsed_time(stop) / args.steps
    log(f"timed region done: {ms_per_step:.3f} ms per step")

    names = ["adamw_fp8_step", "quant_group_stage1_linear", "absmax_reduce", "quant_per_tensor",
             "quant_group_swiglu"]
    per = {nm: sum(m[j].elapsed_time(m[j + 1]) for m in marks) / args.steps for j, nm in enumerate(names)}
    bpp = step_bytes_per_param(G)
    N0, N1 = acts[0].numel, acts[1].numel
    alg = {
        "adamw_fp8_step": n * bpp,
        "quant_group_stage1_linear": N0 * 3 + 8 * N0 / G,   # codes, scales and stage-1 partials
        "absmax_reduce": 4 * N0 / G + 4,
        "quant_per_tensor": N0 * 3,
        "quant_group_swiglu": N1 * 3 + 4 * N1 / G,
    }
    elems = {"adamw_fp8_step": n, "quant_group_stage1_linear": N0, "absmax_reduce": N0 // G,
             "quant_per_tensor": N0, "quant_group_swiglu": N1}
    # activation kernels: frac_of_peak from launches after a cache eviction (HBM fractions); the
    # in-step times beside them
    log("activation kernels from a cold cache")
    cold = cold_activation_times(coat, xs, partial, amax, codes_pt, scale_pt, gcodes, gscales, G)
    kernels = {"adamw_fp8_step": entry(alg["adamw_fp8_step"], per["adamw_fp8_step"], n)}
    for nm in names[1:]:
        kernels[nm] = entry(alg[nm], cold[nm], elems[nm])
        kernels[nm]["cache"] = "cold: after a read-only pass over 1 GiB"
        kernels[nm]["in_step_ms"] = round(per[nm], 4)
    kernels["quant_per_tensor"]["in_step_note"] = (
        "in the step X was read by the 1x128 cast just before and is served from the Infinity Cache")
    kernels["group_absmax_standalone"] = cold["group_absmax_standalone"]
    step_ms = sorted(m[0].elapsed_time(m[5]) for m in marks)
    ms_median = step_ms[len(step_ms) // 2] if len(step_ms) % 2 else 0.5 * sum(step_ms[len(step_ms) // 2 - 1:][:2])
    achieved = alg["adamw_fp8_step"] / (per["adamw_fp8_step"] * 1e-3) / 1e9
    traffic = measured_traffic()
    diag = state_diagnostics(st)
    log("the step on a second allocation of its buffers")
    hp_at = lambda t: coat.adamw_hparams(f(inputs.LR), f(inputs.BETA1), f(inputs.BETA2), f(inputs.EPS),
                                         f(inputs.WEIGHT_DECAY), t)
    ms_second = second_allocation_ms(coat, theta, grad, st, G, spec.v_fmt, hp_at, step + 1)
    if not args.no_extras:
        log("extras: the other entry points and workloads")
    extra = None if args.no_extras else extras(coat, inputs, theta, grad, st, spec, G, step + 1)
    log("memory ceiling of the step's traffic")
    ceiling = memory_ceiling(theta, grad, st, n, alg["adamw_fp8_step"])
    if ceiling:
        ceiling["frac_of_step_memory_skeleton"] = round(achieved / ceiling["step_memory_skeleton_gb_per_s"], 4)
        ceiling["frac_of_best_memory_skeleton"] = round(achieved / ceiling["best_memory_skeleton_gb_per_s"], 4)

    cpu = None
    if not args.no_cpu_baseline and args.cpu_baseline != "none":
        threads = args.cpu_threads or min(16, len(os.sched_getaffinity(0)))
        log(f"timing the oracle ({args.cpu_baseline}) with {threads} threads")
        del theta, grad, st
        cpu = cpu_baseline(spec, acts, G, threads, plan=args.cpu_baseline == "plan")

    out = {
        "metric": "FP8-state AdamW params updated/s + achieved HBM GB/s (% of peak), 1xMI355X",
        "value": n / (ms_per_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_median": round(ms_median, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; OLMo-7B-shaped parameter arena and activation shapes, no trained weights)",
        "config": {
            "workload": ("olmo-7b-shaped FP8-state AdamW step (6888095744 params, m e4m3, v e4m3, G 128) "
                         "+ Group Scaling and E4M3 casts of [16384x4096] and [16384x11008] BF16 activations"),
            "params": n, "group_size": G, "m_format": "e4m3", "v_format": spec.v_fmt,
            "activations": [[a.rows, a.cols] for a in acts],
        },
        "roofline": {
            "bound": "hbm", "kernel": "adamw_fp8_step",
            "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": int(alg["adamw_fp8_step"]),
            "device_ceiling": ceiling,
        },
        "cpu_baseline": cpu,
        "placement": {
            "first_allocation_adamw_ms": round(per["adamw_fp8_step"], 4),
            "second_allocation_adamw_ms": round(ms_second, 4),
            "second_allocation_frac_of_peak": round(alg["adamw_fp8_step"] / (ms_second * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "note": ("the same step on a second copy of its buffers, allocated while the first is live; "
                     "the step's time depends on where in device memory the buffers land, and value and "
                     "roofline keep the first allocation"),
        },
        "pages_context": {
            "note": ("figures the COAT explainer quotes for its own Hopper-class runs of OLMo training; "
                     "context, not targets, and not measured here"),
            "memory_saving_end_to_end": 1.54, "training_speedup_end_to_end": 1.43,
            "optimizer_state_quant_error_reduction": 1.63,
            "this_workload_optimizer_state_bytes_fp32_over_fp8": round(8.0 / (2.0 + 16.0 / G), 3),
        },
        "gpu_over_cpu_baseline": None if cpu is None else round(n / (ms_per_step * 1e-3) / cpu["value"], 1),
        "kernels": kernels,
        "extras": extra,
        "state_diagnostics": diag,
        "step_hbm_gb_per_s": round(sum(alg.values()) / (ms_per_step * 1e-3) / 1e9, 1),
        "wall_s": round(wall, 3),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
