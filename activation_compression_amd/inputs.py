"""Seeded synthetic workloads for the FP8-state AdamW step and Group Scaling.

This module draws inputs only; it holds none of the method's arithmetic.  The
GPU path and the CPU oracle both receive what it generates.  The pages measure
on OLMo pretraining (the COAT explainer's results section), whose data and
weights are not available; the generators below stand in for them with the
same shapes and plausible value distributions:

* parameters  ~ N(0, 0.02) in FP32;
* gradients   ~ N(0, 1e-3) times a log-normal exp(N(0, 1)) scale per row
  (single 1024x1024 tensor) or per tensor (parameter arenas), rounded to BF16
  with round-to-nearest-even;
* stress      |g| = 10^U(-8, 2), random sign, 5% exact zeros, in BF16;
* activations ~ N(0, 1) in BF16 with max(1, round(1e-4 * cols)) seeded channels
  scaled by 100 (the outlier channels of GLU-type models).

Seeds: a tensor's parameters use ``1000 * config + index``; its gradient at
step t uses that seed plus ``7919 * t``.  The transcendental steps of the
recipes (the log-normal scale, 10^U) run in float64 and are rounded once:
torch's vectorized float32 exp and pow give different last bits on different
x86 CPU generations, which would make the same seed draw different gradients
on different hosts.  Generation runs on whichever device
the caller names (a CPU generator for test-sized inputs, a device generator
for the multi-gigabyte arenas); the two devices draw different streams, so a
test always copies one side's generated tensor to the other.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

# AdamW hyper-parameters of every optimizer workload.
LR, BETA1, BETA2, EPS, WEIGHT_DECAY = 1e-3, 0.9, 0.999, 1e-8, 0.1


@dataclass(frozen=True)
class ArenaSpec:
    """A flat parameter arena: named 2-D tensors laid end to end."""

    name: str
    config: int
    tensors: tuple = field(default_factory=tuple)  # ((name, (rows, cols)), ...)
    v_fmt: str = "e4m3"
    group_size: int = 128
    grad_scale: str = "tensor"  # "row" | "tensor" | "stress"

    @property
    def numel(self) -> int:
        return sum(r * c for _, (r, c) in self.tensors)

    def offsets(self):
        off = 0
        for name, (r, c) in self.tensors:
            yield name, off, r * c, (r, c)
            off += r * c


def single_1024() -> ArenaSpec:
    """One 1024x1024 FP32 tensor, per-row log-normal gradient scale, m/v E4M3."""
    return ArenaSpec("single-1024x1024", 1, (("w", (1024, 1024)),), "e4m3", 128, "row")


def olmo_1b() -> ArenaSpec:
    """OLMo-1B-shaped parameter set: d_model 2048, 16 layers, MLP 8192,
    vocab 50304 with a tied embedding; 1 176 764 416 parameters; v in E5M2."""
    d, L, ff, vocab = 2048, 16, 8192, 50304
    ts = []
    for i in range(L):
        ts += [(f"l{i}.qkv", (3 * d, d)), (f"l{i}.out", (d, d)),
               (f"l{i}.ff_up", (2 * ff, d)), (f"l{i}.ff_down", (d, ff))]
    ts.append(("embed", (vocab, d)))
    return ArenaSpec("olmo-1b-shaped", 3, tuple(ts), "e5m2", 128, "tensor")


def olmo_7b() -> ArenaSpec:
    """OLMo-7B-shaped parameter set: d_model 4096, 32 layers, MLP 11008,
    vocab 50304, untied embedding and head; 6 888 095 744 parameters; v E4M3."""
    d, L, ff, vocab = 4096, 32, 11008, 50304
    ts = []
    for i in range(L):
        ts += [(f"l{i}.qkv", (3 * d, d)), (f"l{i}.out", (d, d)),
               (f"l{i}.ff_up", (2 * ff, d)), (f"l{i}.ff_down", (d, ff))]
    ts += [("embed", (vocab, d)), ("head", (vocab, d))]
    return ArenaSpec("olmo-7b-shaped", 4, tuple(ts), "e4m3", 128, "tensor")


def ragged_list(group_size: int = 128, v_fmt: str = "e4m3") -> ArenaSpec:
    """Nine tensors of G x {1, 2, 7, 8, 9, 64, 100, 513, 1000} parameters: sizes
    below, at and between multiples of the 1024-parameter chunk, for the
    tensor-list step (each tensor in its own allocation there)."""
    ks = (1, 2, 7, 8, 9, 64, 100, 513, 1000)
    return ArenaSpec(f"ragged-list-G{group_size}-{v_fmt}", 6,
                     tuple((f"t{i}", (k, group_size)) for i, k in enumerate(ks)), v_fmt, group_size, "tensor")


def stress(group_size: int = 128, v_fmt: str = "e4m3", numel: int = 64 << 20) -> ArenaSpec:
    """64 Mi parameters with gradients spanning ten decades (and 5% zeros)."""
    cols = 1 << 13
    return ArenaSpec(f"stress-64Mi-G{group_size}-{v_fmt}", 5,
                     (("w", (numel // cols, cols)),), v_fmt, group_size, "stress")


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _bf16_bits(x: torch.Tensor) -> torch.Tensor:
    """Round FP32 to BF16 (RNE, torch's cast) and return the raw 16-bit patterns."""
    return x.to(torch.bfloat16).view(torch.int16)


def gen_params(spec: ArenaSpec, device="cpu", out: torch.Tensor | None = None,
               tensor_range=None) -> torch.Tensor:
    """FP32 parameters ~ N(0, 0.02) for the arena (or a slice of its tensors)."""
    dev = torch.device(device)
    if out is None:
        out = torch.empty(spec.numel, dtype=torch.float32, device=dev)
    for idx, (name, off, n, shape) in enumerate(spec.offsets()):
        if tensor_range is not None and idx not in tensor_range:
            continue
        g = _gen(1000 * spec.config + idx, dev)
        out[off:off + n].copy_(torch.randn(n, generator=g, device=dev).mul_(0.02))
    return out


def _tensor_scale(spec: ArenaSpec, idx: int, rows: int) -> torch.Tensor:
    """Log-normal exp(N(0,1)) gradient scale: one per row or one per tensor.
    Drawn once per tensor on the CPU so that every device agrees on it."""
    g = _gen(1000 * spec.config + 500 + idx, "cpu")
    if spec.grad_scale == "row":
        return torch.randn(rows, generator=g).double().exp().float()
    return torch.randn(1, generator=g).double().exp().float()


def gen_grads(spec: ArenaSpec, step: int, device="cpu", out: torch.Tensor | None = None,
              tensor_range=None, chunk: int = 1 << 28) -> torch.Tensor:
    """BF16 gradients (returned as int16 bit patterns) for update ``step``."""
    dev = torch.device(device)
    if out is None:
        out = torch.empty(spec.numel, dtype=torch.int16, device=dev)
    for idx, (name, off, n, (rows, cols)) in enumerate(spec.offsets()):
        if tensor_range is not None and idx not in tensor_range:
            continue
        g = _gen(1000 * spec.config + idx + 7919 * step, dev)
        if spec.grad_scale == "stress":
            for c0 in range(0, n, chunk):
                c1 = min(n, c0 + chunk)
                m = c1 - c0
                u = torch.rand(m, generator=g, device=dev).double()
                mag = torch.pow(10.0, u * 10.0 - 8.0).float()
                sign = torch.where(torch.rand(m, generator=g, device=dev) < 0.5, -1.0, 1.0)
                zero = torch.rand(m, generator=g, device=dev) < 0.05
                val = torch.where(zero, torch.zeros_like(mag), mag * sign)
                out[off + c0:off + c1].copy_(_bf16_bits(val))
            continue
        scale = _tensor_scale(spec, idx, rows).to(dev)
        r0 = 0
        rows_per_chunk = max(1, chunk // cols)
        while r0 < rows:
            r1 = min(rows, r0 + rows_per_chunk)
            val = torch.randn((r1 - r0, cols), generator=g, device=dev).mul_(1e-3)
            if spec.grad_scale == "row":
                val.mul_(scale[r0:r1, None])
            else:
                val.mul_(scale)
            out[off + r0 * cols:off + r1 * cols].copy_(_bf16_bits(val).reshape(-1))
            r0 = r1
    return out


@dataclass(frozen=True)
class ActivationSpec:
    """A BF16 activation tensor [rows x cols] with seeded outlier channels."""

    name: str
    rows: int
    cols: int
    seed: int
    group_size: int = 128
    outlier_scale: float = 100.0

    @property
    def numel(self) -> int:
        return self.rows * self.cols

    @property
    def n_outlier_channels(self) -> int:
        return max(1, round(1e-4 * self.cols))


def linear_input(rows: int = 16384, cols: int = 4096) -> ActivationSpec:
    """Input of a linear layer, [16384 tokens x 4096]."""
    return ActivationSpec(f"linear-in-{rows}x{cols}", rows, cols, seed=2000)


def swiglu_input(rows: int = 16384, cols: int = 11008) -> ActivationSpec:
    """SwiGLU input, [16384 tokens x 11008]."""
    return ActivationSpec(f"swiglu-in-{rows}x{cols}", rows, cols, seed=2001)


def swiglu_gate(rows: int = 16384, cols: int = 11008) -> ActivationSpec:
    """Gate projection output feeding SwiGLU, [16384 tokens x 11008]."""
    return ActivationSpec(f"swiglu-gate-{rows}x{cols}", rows, cols, seed=2002)


def swiglu_up(rows: int = 16384, cols: int = 11008) -> ActivationSpec:
    """Up projection output feeding SwiGLU, [16384 tokens x 11008]."""
    return ActivationSpec(f"swiglu-up-{rows}x{cols}", rows, cols, seed=2003)


def rmsnorm_input(rows: int = 16384, cols: int = 4096) -> ActivationSpec:
    """Input of the normalization before a linear layer, [16384 tokens x 4096]."""
    return ActivationSpec(f"rmsnorm-in-{rows}x{cols}", rows, cols, seed=2004)


def gen_norm_weight(cols: int, seed: int = 2005, device="cpu") -> torch.Tensor:
    """BF16 normalization gain [cols] as int16 bit patterns: 1 + 0.1 N(0, 1)."""
    g = _gen(seed, torch.device(device))
    w = 1.0 + 0.1 * torch.randn(cols, generator=g, device=torch.device(device))
    return _bf16_bits(w)


def outlier_channels(spec: ActivationSpec) -> torch.Tensor:
    g = _gen(spec.seed + 1, "cpu")
    return torch.randperm(spec.cols, generator=g)[: spec.n_outlier_channels]


def gen_activation(spec: ActivationSpec, device="cpu", chunk_rows: int = 4096) -> torch.Tensor:
    """BF16 activations as int16 bit patterns, shape [rows, cols]."""
    dev = torch.device(device)
    out = torch.empty((spec.rows, spec.cols), dtype=torch.int16, device=dev)
    g = _gen(spec.seed, dev)
    ch = outlier_channels(spec).to(dev)
    for r0 in range(0, spec.rows, chunk_rows):
        r1 = min(spec.rows, r0 + chunk_rows)
        x = torch.randn((r1 - r0, spec.cols), generator=g, device=dev)
        x[:, ch] *= spec.outlier_scale
        out[r0:r1].copy_(_bf16_bits(x))
    return out


def hparams_for_step(step: int) -> dict:
    return dict(lr=LR, beta1=BETA1, beta2=BETA2, eps=EPS, weight_decay=WEIGHT_DECAY, step=int(step))


def fresh_state(n: int, group_size: int, device="cpu"):
    """A never-updated FP8 moment state: codes 0, amax 0, k 1 (both moments)."""
    ng = n // group_size
    dev = torch.device(device)
    z8 = lambda: torch.zeros(n, dtype=torch.uint8, device=dev)
    z32 = lambda: torch.zeros(ng, dtype=torch.float32, device=dev)
    o32 = lambda: torch.ones(ng, dtype=torch.float32, device=dev)
    return dict(m_codes=z8(), m_amax=z32(), m_k=o32(), v_codes=z8(), v_amax=z32(), v_k=o32())

