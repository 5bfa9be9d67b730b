"""Seeded synthetic inputs for normalized Hedgehog linear attention.

This module only draws random numbers and casts them; it holds none of the
method's arithmetic.  Both the CPU oracle (through the tests and the bench)
and the HIP path consume exactly the tensors built here.

Recipe (every case):
  * one ``torch.Generator`` on the CPU, seeded with ``seed`` (default 0);
  * fixed draw order: q, k, v, W_q, W_k, dt, A_log;
  * q, k, v, W drawn as float32 normals, then cast to the case's dtype
    (bfloat16 casts are round-to-nearest-even, done by torch);
  * q, k, v ~ N(0, 1), laid out [B, H, n, d] contiguous (v: [B, H, n, dv]);
  * W_q, W_k are one shared [d, f] matrix each, applied as x @ W, drawn
    N(0, w_std^2) (w_std = 1 for the tiny case, 1/sqrt(d) otherwise);
  * dt ~ N(0, 1) float32 [B, H, n];
  * A_log float32 [H], uniform on [lo, hi]: [0, ln 16] for the Mamba-style
    decay, [ln 2^-9, ln 2^-3] for the mild decay that keeps a_t near 0.99;
  * per-channel-decay cases (make_pc): after W_k, dt float32 [B, H, n, dv] ~ N(0, 1)
    and A_log float32 [H, dv, 2f] ~ U(ln 2^-4, ln 16);
  * the gate branch's pre-activation (when a case has one) comes from its own
    generator, seeded with 7919 * (seed + 1), ~ N(0, 2^2) in o's shape, so that
    both signs and the saturated ends of SiLU are exercised.

The shapes follow the HedgeMamba mixer as the gsyq.cn explainer describes it
(section 5.2: heads of width head_dim; Pythia-1B width H*d = 2048) and the
shape conventions of the cnblogs linear-attention tutorial (Q/K/V [b,h,n,d]).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

LN16 = math.log(16.0)


@dataclass
class Case:
    """One seeded prefill workload (all tensors on the CPU)."""
    name: str
    B: int
    H: int
    n: int
    d: int
    f: int
    dv: int
    dtype: torch.dtype
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    w_q: torch.Tensor
    w_k: torch.Tensor
    dt: torch.Tensor | None = None
    a_log: torch.Tensor | None = None
    meta: dict = field(default_factory=dict)

    @property
    def F(self) -> int:
        return 2 * self.f


def _normal(g, shape, std=1.0):
    x = torch.randn(shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x


def make_prefill(name, B, H, n, d, f, dv, dtype=torch.bfloat16, w_std=None,
                 decay=None, seed=0) -> Case:
    """Draw one prefill case.  ``decay`` is None (a_t = 1), 'mamba' or 'mild'."""
    g = torch.Generator().manual_seed(seed)
    if w_std is None:
        w_std = 1.0 / math.sqrt(d)
    q = _normal(g, (B, H, n, d)).to(dtype)
    k = _normal(g, (B, H, n, d)).to(dtype)
    v = _normal(g, (B, H, n, dv)).to(dtype)
    w_q = _normal(g, (d, f), w_std).to(dtype)
    w_k = _normal(g, (d, f), w_std).to(dtype)
    dt = a_log = None
    if decay is not None:
        dt = _normal(g, (B, H, n))
        u = torch.rand((H,), generator=g, dtype=torch.float64)
        if decay == "mamba":
            lo, hi = 0.0, LN16
        elif decay == "mild":
            lo, hi = -9.0 * math.log(2.0), -3.0 * math.log(2.0)
        else:
            raise ValueError(decay)
        a_log = (lo + (hi - lo) * u).to(torch.float32)
    return Case(name, B, H, n, d, f, dv, dtype, q, k, v, w_q, w_k, dt, a_log,
                {"seed": seed, "decay": decay, "w_std": w_std})


# The five measured workloads plus the parity-only cases.
def tiny(seed=0):
    """B=1, H=2, n=256, d=16, f=16 (phi width 32), fp32, W ~ N(0,1), a_t = 1."""
    return make_prefill("tiny-fp32", 1, 2, 256, 16, 16, 16, torch.float32, 1.0, None, seed)


def pythia1b(seed=0, n=2048, B=8):
    """Pythia-1B-shaped layer: B=8, H=16, d=128, f=64, n=2048, bf16, a_t = 1."""
    return make_prefill("pythia1b-bf16", B, 16, n, 128, 64, 128, torch.bfloat16, None, None, seed)


def mamba_decay(seed=0, n=8192, B=2):
    """Same shapes with Mamba decay: B=2, n=8192, dt ~ N(0,1), A_log ~ U(0, ln 16)."""
    return make_prefill("decay-bf16", B, 16, n, 128, 64, 128, torch.bfloat16, None, "mamba", seed)


def long_context(seed=0, n=131072):
    """B=1, H=16, n=131072, bf16, Mamba decay."""
    return make_prefill("long-bf16", 1, 16, n, 128, 64, 128, torch.bfloat16, None, "mamba", seed)


def mild_decay(seed=0, n=8192, B=2):
    """Decay shapes with A_log ~ U(ln 2^-9, ln 2^-3): a_t ~ 0.99, memory longer than a chunk."""
    return make_prefill("mild-bf16", B, 16, n, 128, 64, 128, torch.bfloat16, None, "mild", seed)


def small(n=37, decay="mamba", dtype=torch.float32, d=16, f=16, dv=16, B=1, H=2, seed=0):
    """Small ragged case for brute-force checks (n not a multiple of any chunk)."""
    return make_prefill(f"small-n{n}", B, H, n, d, f, dv, dtype, None, decay, seed)


def make_pc(name, B, H, n, d, f, dv, dtype=torch.bfloat16, seed=0, shared_a=False) -> Case:
    """Per-channel-decay case: q, k, v, W_q, W_k as in make_prefill (same draw order
    and distributions, W ~ N(0, 1/d)), then dt float32 [B, H, n, dv] ~ N(0, 1) and
    A_log float32 [H, dv, 2f] (or [dv, 2f] when shared_a) ~ U(ln 2^-4, ln 16), so that
    exp(A_log), the per-state decay rate, spans slow and fast states (Mamba-1's own
    initialisation, A_log[c, n] = ln(n + 1), lies in the same range)."""
    g = torch.Generator().manual_seed(seed)
    w_std = 1.0 / math.sqrt(d)
    q = _normal(g, (B, H, n, d)).to(dtype)
    k = _normal(g, (B, H, n, d)).to(dtype)
    v = _normal(g, (B, H, n, dv)).to(dtype)
    w_q = _normal(g, (d, f), w_std).to(dtype)
    w_k = _normal(g, (d, f), w_std).to(dtype)
    dt = _normal(g, (B, H, n, dv))
    shape = (dv, 2 * f) if shared_a else (H, dv, 2 * f)
    lo, hi = -4.0 * math.log(2.0), LN16
    a_log = (lo + (hi - lo) * torch.rand(shape, generator=g, dtype=torch.float64)).to(torch.float32)
    return Case(name, B, H, n, d, f, dv, dtype, q, k, v, w_q, w_k, dt, a_log,
                {"seed": seed, "decay": "per-channel", "w_std": w_std})


@dataclass
class DecodeCase:
    """Decode workload: a prefix that builds the state, then per-step tokens."""
    B: int
    H: int
    d: int
    f: int
    dv: int
    prefix: int
    steps: int
    w_q: torch.Tensor
    w_k: torch.Tensor
    a_log: torch.Tensor | None
    prefix_k: torch.Tensor   # [B, H, prefix, d]
    prefix_v: torch.Tensor   # [B, H, prefix, dv]
    prefix_dt: torch.Tensor | None  # [B, H, prefix]
    seed: int


def decode_setup(B=256, H=16, d=128, f=64, dv=128, prefix=4096, steps=512,
                 decay=True, dtype=torch.bfloat16, seed=0) -> DecodeCase:
    """Decode case: W_q, W_k, A_log, then the prefix k, v, dt (in that order)."""
    g = torch.Generator().manual_seed(seed)
    w_std = 1.0 / math.sqrt(d)
    w_q = _normal(g, (d, f), w_std).to(dtype)
    w_k = _normal(g, (d, f), w_std).to(dtype)
    a_log = None
    if decay:
        u = torch.rand((H,), generator=g, dtype=torch.float64)
        a_log = (LN16 * u).to(torch.float32)
    pk = _normal(g, (B, H, prefix, d)).to(dtype)
    pv = _normal(g, (B, H, prefix, dv)).to(dtype)
    pdt = _normal(g, (B, H, prefix)) if decay else None
    return DecodeCase(B, H, d, f, dv, prefix, steps, w_q, w_k, a_log, pk, pv, pdt, seed)


def decode_step_inputs(dc: DecodeCase, step: int, dtype=torch.bfloat16):
    """Fresh q, k, v [B, H, d|dv] and dt [B, H] for one decode step.

    Each step has its own generator seeded from (seed, step), so any step can be
    regenerated alone (the parity tests sample steps without drawing the rest).
    """
    g = torch.Generator().manual_seed(1_000_003 * (dc.seed + 1) + step)
    q = _normal(g, (dc.B, dc.H, dc.d)).to(dtype)
    k = _normal(g, (dc.B, dc.H, dc.d)).to(dtype)
    v = _normal(g, (dc.B, dc.H, dc.dv)).to(dtype)
    dt = _normal(g, (dc.B, dc.H)) if dc.a_log is not None else None
    return q, k, v, dt


def gate(shape, dtype=torch.bfloat16, seed=0, std=2.0):
    """Gate pre-activation in o's shape (prefill [B, H, n, dv], decode [B, H, dv])."""
    g = torch.Generator().manual_seed(7919 * (seed + 1))
    return _normal(g, tuple(shape), std).to(dtype)


def to_f64(t):
    """Exact conversion of fp32/bf16 tensors to float64 numpy arrays (None passes)."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()
