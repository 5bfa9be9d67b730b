"""CPU float64 gradient oracle for causal, normalized Hedgehog linear attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU
baseline may import this module.  It shares no code with the HIP library and
imports nothing from it; the product path never calls it.

The forward pass is written out once more, in plain torch float64 operations
(the masked quadratic form of the cnblogs linear-attention tutorial, part 2,
made causal and decayed as in its part 4.3, with the numerator / denominator
split of the HedgeMamba explainer §2.3 and the Hedgehog map of its §2.1), and
reverse-mode differentiation of those operations gives every gradient.  The
scalar being differentiated is

    loss = sum(o * dO) + sum(S_final * dS_final) + sum(z_final * dz_final),

so the gradients are the vector-Jacobian products a training step needs.  It is
pinned in tests/test_oracle_grad.py by central finite differences of the numpy
oracle (hm_oracle.forward, the recurrent form: an independent implementation).
"""
from __future__ import annotations

import numpy as np
import torch

_F64 = torch.float64


def _t(x, grad=False):
    if x is None:
        return None
    t = torch.tensor(np.asarray(x, dtype=np.float64), dtype=_F64)
    return t.requires_grad_(grad)


def _softplus(x):
    return torch.where(x > 0, x + torch.log1p(torch.exp(-x.abs())), torch.log1p(torch.exp(-x.abs())))


def features(x, w):
    """phi = softmax([x W, -x W]) over the feature axis ([HM] §2.1, §5.3)."""
    u = x @ w if w.dim() == 2 else torch.einsum("bhnd,hdf->bhnf", x, w)
    return torch.softmax(torch.cat([u, -u], dim=-1), dim=-1)


def rotate(phi, pos, dims, base):
    """Rotary encoding of the features ([HM] §5.2 step 3) in the GPT-NeoX rotate-half
    form: pair (i, i + dims/2) turns by pos * base^(-2i/dims); pos [B, n]."""
    h = dims // 2
    inv_freq = torch.pow(torch.tensor(float(base), dtype=_F64), -2.0 * torch.arange(h, dtype=_F64) / dims)
    ang = torch.as_tensor(pos, dtype=_F64)[:, None, :, None] * inv_freq
    c, s = torch.cos(ang), torch.sin(ang)
    x1, x2 = phi[..., :h], phi[..., h:dims]
    return torch.cat([x1 * c - x2 * s, x2 * c + x1 * s, phi[..., dims:]], dim=-1)


def forward_torch(q, k, v, w_q, w_k, dt=None, a_log=None, s_init=None, z_init=None, gate=None,
                  rope_dims=0, rope_base=10000.0, rope_pos0=None):
    """Differentiable forward: returns (o [B,H,n,dv], S_final [B,H,F,dv], z_final [B,H,F]).

    L_t = sum_{s<=t} log a_s with log a_s = -softplus(dt_s) exp(A_log) ([SSM] §3.2);
    o_t = (sum_{j<=t} e^{L_t-L_j} (phiq_t.phik_j) v_j + e^{L_t} phiq_t S_init)
          / (sum_{j<=t} e^{L_t-L_j} (phiq_t.phik_j) + e^{L_t} phiq_t.z_init),
    with phiq, phik rotated at positions rope_pos0[b] + t when rope_dims > 0.
    """
    phiq, phik = features(q, w_q), features(k, w_k)
    B, H, n, F = phiq.shape
    if rope_dims:
        p0 = torch.zeros(B, dtype=_F64) if rope_pos0 is None else torch.as_tensor(
            np.asarray(rope_pos0, dtype=np.float64).reshape(B))
        pos = p0[:, None] + torch.arange(n, dtype=_F64)[None, :]
        phiq, phik = rotate(phiq, pos, rope_dims, rope_base), rotate(phik, pos, rope_dims, rope_base)
    dv = v.shape[-1]
    if dt is None:
        L = torch.zeros((B, H, n), dtype=_F64)
    else:
        L = torch.cumsum(-_softplus(dt) * torch.exp(a_log)[None, :, None], dim=-1)
    mask = torch.tril(torch.ones((n, n), dtype=torch.bool))
    diff = L[..., :, None] - L[..., None, :]
    wgt = torch.where(mask, torch.exp(torch.where(mask, diff, torch.zeros_like(diff))), torch.zeros_like(diff))
    P = (phiq @ phik.transpose(-1, -2)) * wgt
    num = P @ v
    den = P.sum(-1)
    eL = torch.exp(L)
    if s_init is not None:
        num = num + eL[..., None] * (phiq @ s_init)
        den = den + eL * (phiq @ z_init[..., None])[..., 0]
    o = num / den[..., None]
    if gate is not None:
        o = o * (gate * torch.sigmoid(gate))        # the mixer's gate branch, [HM] §5.2 step 6
    if n > 0:
        tail = torch.exp(L[..., -1:] - L)                             # e^{L_{n-1} - L_j}
        S = (phik * tail[..., None]).transpose(-1, -2) @ v
        z = (phik * tail[..., None]).sum(-2)
        carry = torch.exp(L[..., -1])
    else:
        S = torch.zeros((B, H, F, dv), dtype=_F64)
        z = torch.zeros((B, H, F), dtype=_F64)
        carry = torch.ones((B, H), dtype=_F64)
    if s_init is not None:
        S = S + carry[..., None, None] * s_init
        z = z + carry[..., None] * z_init
    return o, S, z


def grads(q, k, v, w_q, w_k, dt=None, a_log=None, s_init=None, z_init=None, d_o=None, ds_final=None,
          dz_final=None, gate=None, rope_dims=0, rope_base=10000.0, rope_pos0=None):
    """Gradients of loss = <o, dO> + <S_final, dS_final> + <z_final, dz_final>.

    Returns a dict with keys q, k, v, w_q, w_k and, when given, dt, a_log,
    s_init, z_init, gate (float64 numpy arrays), plus "o" the forward output
    (after the gate, when there is one).
    """
    args = dict(q=_t(q, True), k=_t(k, True), v=_t(v, True), w_q=_t(w_q, True), w_k=_t(w_k, True),
                dt=_t(dt, dt is not None), a_log=_t(a_log, a_log is not None),
                s_init=_t(s_init, s_init is not None), z_init=_t(z_init, z_init is not None),
                gate=_t(gate, gate is not None))
    o, S, z = forward_torch(**args, rope_dims=rope_dims, rope_base=rope_base, rope_pos0=rope_pos0)
    loss = (o * _t(d_o)).sum()
    if ds_final is not None:
        loss = loss + (S * _t(ds_final)).sum()
    if dz_final is not None:
        loss = loss + (z * _t(dz_final)).sum()
    leaves = {k_: t for k_, t in args.items() if t is not None}
    gs = torch.autograd.grad(loss, list(leaves.values()), allow_unused=True)
    out = {k_: (np.zeros(t.shape) if g is None else g.detach().numpy()) for (k_, t), g in zip(leaves.items(), gs)}
    out["o"] = o.detach().numpy()
    return out
