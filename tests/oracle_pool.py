"""The float64 oracle over many (b, h) pairs at once, spread over worker processes.

Not a test module.  Workers are started with the "spawn" method and never touch
the HIP library; the forward workers import only numpy and the oracle, the
gradient workers also torch (on the CPU: the autograd oracle).  The work is cut
into groups of a few heads of one batch row; each group runs the oracle
unchanged (the recurrent form, or hm_grad.grads).  At most 12 workers: a process
that loads the ROCm runtime (torch does) counts against the box's limit of 16
processes per GPU, and the test process itself holds the GPU.
"""
from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np


def _group(args):
    from oracle import hm_oracle as orc
    q, k, v, wq, wk, dt, a_log, s0, z0 = args
    return orc.forward(q, k, v, wq, wk, dt, a_log, s0, z0)


def workers() -> int:
    return max(1, min(12, len(os.sched_getaffinity(0))))


def forward_all(q, k, v, wq, wk, dt=None, a_log=None, s_init=None, z_init=None, group=2):
    """orc.forward over every (b, h) of float64 arrays q, k [B,H,n,d], v [B,H,n,dv]
    (W shared [d,f] or per head [H,d,f]; dt [B,H,n], a_log [H]; optional initial
    state S [B,H,F,dv], z [B,H,F]).  Returns (o, S, z) like orc.forward."""
    B, H = q.shape[:2]
    jobs, keys = [], []
    for b in range(B):
        for h0 in range(0, H, group):
            hs = slice(h0, min(H, h0 + group))
            w_of = lambda w: w if w.ndim == 2 else w[hs]
            jobs.append((q[b:b + 1, hs], k[b:b + 1, hs], v[b:b + 1, hs], w_of(wq), w_of(wk),
                         None if dt is None else dt[b:b + 1, hs], None if a_log is None else a_log[hs],
                         None if s_init is None else s_init[b:b + 1, hs],
                         None if z_init is None else z_init[b:b + 1, hs]))
            keys.append((b, hs))
    ctx = mp.get_context("spawn")
    with ctx.Pool(min(workers(), len(jobs))) as pool:
        res = pool.map(_group, jobs)
    n, dv = q.shape[2], v.shape[-1]
    F = 2 * wq.shape[-1]
    o = np.empty((B, H, n, dv))
    S = np.empty((B, H, F, dv))
    z = np.empty((B, H, F))
    for (b, hs), (ob, Sb, zb) in zip(keys, res):
        o[b:b + 1, hs], S[b:b + 1, hs], z[b:b + 1, hs] = ob, Sb, zb
    return o, S, z


def _grad_group(args):
    import torch
    torch.set_num_threads(1)
    from oracle import hm_grad
    kw = args
    return hm_grad.grads(**kw)


def grads_all(q, k, v, wq, wk, d_o, dt=None, a_log=None, group=2):
    """hm_grad.grads over every (b, h), in groups of heads of one batch row (float64
    numpy inputs, W shared [d, f]).  The per-head gradients are placed; the shared
    W's gradient and A_log's (a sum over batch rows) are summed over the groups."""
    B, H = q.shape[:2]
    jobs, keys = [], []
    for b in range(B):
        for h0 in range(0, H, group):
            hs = slice(h0, min(H, h0 + group))
            jobs.append(dict(q=q[b:b + 1, hs], k=k[b:b + 1, hs], v=v[b:b + 1, hs], w_q=wq, w_k=wk,
                             dt=None if dt is None else dt[b:b + 1, hs], a_log=None if a_log is None else a_log[hs],
                             d_o=d_o[b:b + 1, hs]))
            keys.append((b, hs))
    ctx = mp.get_context("spawn")
    with ctx.Pool(min(workers(), len(jobs))) as pool:
        res = pool.map(_grad_group, jobs)
    out = {"q": np.empty(q.shape), "k": np.empty(k.shape), "v": np.empty(v.shape),
           "w_q": np.zeros(wq.shape), "w_k": np.zeros(wk.shape)}
    if dt is not None:
        out["dt"] = np.empty(dt.shape)
        out["a_log"] = np.zeros(a_log.shape)
    for (b, hs), r in zip(keys, res):
        for name in ("q", "k", "v") + (("dt",) if dt is not None else ()):
            out[name][b:b + 1, hs] = r[name]
        out["w_q"] += r["w_q"]
        out["w_k"] += r["w_k"]
        if dt is not None:
            out["a_log"][hs] += r["a_log"]
    return out
