"""Helpers shared by the GPU parity tests (not a test module)."""
from __future__ import annotations

import numpy as np
import torch

from oracle import hm_oracle as orc
from selective_state_space_hm_amd import hm, inputs

FP32_TOL = 1e-5   # rel-L2 bar for float32 inputs
BF16_TOL = 2e-2   # rel-L2 bar for bf16 inputs with float32 accumulation


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def max_abs(got, ref):
    return float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))))


def tol_for(dtype):
    return FP32_TOL if dtype == torch.float32 else BF16_TOL


def report(name, got, ref):
    r, m = rel_l2(got, ref), max_abs(got, ref)
    print(f"[parity] {name}: rel-L2 {r:.3e}  max-abs {m:.3e}", flush=True)
    return r


def to_dev(case, dev="cuda"):
    d = {}
    for k in ("q", "k", "v", "w_q", "w_k", "dt", "a_log"):
        t = getattr(case, k)
        d[k] = None if t is None else t.to(dev)
    return d


def oracle_heads(case, heads, s_init=None, z_init=None):
    """Oracle recurrent form for a list of (b, h) pairs; returns (o, S, z) stacked
    along a leading axis in the order of `heads`."""
    bs = [b for b, _ in heads]
    hs = [h for _, h in heads]
    f64 = inputs.to_f64
    q = f64(case.q[bs, hs])[:, None]
    k = f64(case.k[bs, hs])[:, None]
    v = f64(case.v[bs, hs])[:, None]
    dt = None if case.dt is None else f64(case.dt[bs, hs])[:, None]
    # per-sample A_log: broadcast through a 1-head axis
    o_l, S_l, z_l = [], [], []
    for i, (b, h) in enumerate(heads):
        a_log = None if case.a_log is None else f64(case.a_log[h:h + 1])
        s0 = None if s_init is None else s_init[i][None, None]
        z0 = None if z_init is None else z_init[i][None, None]
        o, S, z = orc.forward(q[i:i + 1], k[i:i + 1], v[i:i + 1], f64(case.w_q), f64(case.w_k),
                              None if dt is None else dt[i:i + 1], a_log, s0, z0)
        o_l.append(o[0, 0])
        S_l.append(S[0, 0])
        z_l.append(z[0, 0])
    return np.stack(o_l), np.stack(S_l), np.stack(z_l)


def run_fwd(case, dev="cuda", **kw):
    g = to_dev(case, dev)
    return hm.hm_linattn_fwd(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], g["dt"], g["a_log"], **kw)


def with_abs(v):
    """v with |v| appended along the value axis: one oracle pass then yields the
    output over v and the output over |v| (the first-order rounding bound below)."""
    v = np.asarray(v, dtype=np.float64)
    return np.concatenate([v, np.abs(v)], axis=-1)


def check_bound(name, got, ref, ref_abs, tol):
    """Element-wise check of outputs that are convex combinations of the v_j (positive
    features): o_t = sum_j w_tj v_j / sum_j w_tj with every weight carried to a small
    relative error gives |d o_t| <= eps (sum_j w_tj |v_j| / sum_j w_tj + |o_t|), i.e.
    eps times (the output over |v|) + |o_t|.  Asserts every element's error within tol
    times that bound, so a single wrong row or column fails even where it barely moves
    the rel-L2; prints the rel-L2, max-abs and the worst bound ratio."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = np.asarray(ref_abs, dtype=np.float64) + np.abs(ref)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    ratio = np.abs(got - ref) / np.maximum(bound, 1e-300)
    r = report(name, got, ref)
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    print(f"[parity] {name}: max |err| / bound {ratio.max():.3e} at {tuple(int(i) for i in worst)}", flush=True)
    assert ratio.max() <= tol, f"{name}: element {worst} error {ratio.max():.3e} x its bound"
    return r
