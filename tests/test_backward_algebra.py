"""CPU check of the chunked backward algebra the gradient kernels implement
(chunk-start states, the reverse state gradient G, the per-chunk products, and
the decay gradient as sums of pair weights over the pairs that span each token),
written out in float64 numpy and compared with the autograd oracle.  No GPU."""
import numpy as np
import pytest

from oracle import hm_grad, hm_oracle as orc


def chunked_backward(q, k, v, w_q, w_k, dt, a_log, S0, z0, dO, dS, dz, C=64):
    """One (b, h); the formulas of the backward kernels, float64."""
    f = w_q.shape[1]
    u = q @ w_q
    phq = np.exp(np.concatenate([u, -u], -1) - np.abs(u).max(-1, keepdims=True))   # unnormalized
    uk = k @ w_k
    phk = np.exp(np.concatenate([uk, -uk], -1) - np.abs(uk).max(-1, keepdims=True))
    phk /= phk.sum(-1, keepdims=True)
    n = q.shape[0]
    la = orc.log_decay(dt[None, None], a_log)[0, 0] if dt is not None else np.zeros(n)
    nch = (n + C - 1) // C
    S, z = S0.copy(), z0.copy()
    Sc, zc, den, o = [], [], np.zeros(n), np.zeros_like(v)
    for c in range(nch):                       # what the training forward saves
        Sc.append(S.copy())
        zc.append(z.copy())
        for t in range(c * C, min(n, c * C + C)):
            S = np.exp(la[t]) * S + np.outer(phk[t], v[t])
            z = np.exp(la[t]) * z + phk[t]
            den[t] = phq[t] @ z
            o[t] = phq[t] @ S / den[t]
    dnum = dO / den[:, None]
    dden = -(dnum * o).sum(-1)
    G, g = dS.copy(), dz.copy()
    Gend, gend = [None] * nch, [None] * nch
    for c in reversed(range(nch)):             # the reverse state-gradient pass
        t0, t1 = c * C, min(n, c * C + C)
        Gend[c], gend[c] = G.copy(), g.copy()
        L = np.cumsum(la[t0:t1])
        G = np.exp(L[-1]) * G + (phq[t0:t1] * np.exp(L)[:, None]).T @ dnum[t0:t1]
        g = np.exp(L[-1]) * g + (phq[t0:t1] * np.exp(L)[:, None]).T @ dden[t0:t1]
    out = {k_: np.zeros_like(x) for k_, x in (("q", q), ("k", k), ("v", v))}
    dwq, dwk, dloga = np.zeros_like(w_q), np.zeros_like(w_k), np.zeros(n)
    for c in range(nch):                       # the per-chunk gradient products
        t0, t1 = c * C, min(n, c * C + C)
        L = np.cumsum(la[t0:t1])
        Lam = L[-1]
        M = np.tril(np.exp(np.minimum(L[:, None] - L[None, :], 0.0)))
        D1 = dnum[t0:t1] @ v[t0:t1].T
        A = M * (D1 + dden[t0:t1, None])
        P = M * (phq[t0:t1] @ phk[t0:t1].T)
        inter_q = np.exp(L)[:, None] * (dnum[t0:t1] @ Sc[c].T + dden[t0:t1, None] * zc[c][None, :])
        dphq = A @ phk[t0:t1] + inter_q
        e = np.exp(Lam - L)
        inter_k = e[:, None] * (v[t0:t1] @ Gend[c].T + gend[c][None, :])
        dphk = A.T @ phq[t0:t1] + inter_k
        out["v"][t0:t1] = P.T @ dnum[t0:t1] + e[:, None] * (phk[t0:t1] @ Gend[c])
        duq = phq[t0:t1] * dphq
        duq = duq[:, :f] - duq[:, f:]
        dot = (phk[t0:t1] * dphk).sum(-1)
        duk = phk[t0:t1] * (dphk - dot[:, None])
        duk = duk[:, :f] - duk[:, f:]
        out["q"][t0:t1] = duq @ w_q.T
        out["k"][t0:t1] = duk @ w_k.T
        dwq += q[t0:t1].T @ duq
        dwk += k[t0:t1].T @ duk
        # decay: pair sums (strictly lower in-chunk pairs, keys before, queries after, spanning)
        W = np.tril(P * (D1 + dden[t0:t1, None]), -1)           # [s][j], j < s
        Q = (phq[t0:t1] * inter_q).sum(-1)
        K = (phk[t0:t1] * inter_k).sum(-1)
        X = np.exp(Lam) * ((Gend[c] * Sc[c]).sum() + gend[c] @ zc[c])
        ev = K + W.sum(0) - W.sum(1) - Q
        dloga[t0:t1] = X + Q.sum() + np.concatenate([[0.0], np.cumsum(ev)[:-1]])
    out["w_q"], out["w_k"] = dwq, dwk
    if dt is not None:
        out["dt"] = dloga * (-(1.0 / (1.0 + np.exp(-dt))) * np.exp(a_log))
        out["a_log"] = np.array([(dloga * la).sum()])
    out["s_init"], out["z_init"] = G, g
    return out


@pytest.mark.parametrize("n,decay", [(150, "fast"), (200, None), (64, "mild"), (1, "fast"), (129, "fast")])
def test_chunked_backward_matches_autograd(n, decay):
    r = np.random.default_rng(n)
    d, f, dv = 12, 6, 10
    q, k, v = r.normal(size=(n, d)), r.normal(size=(n, d)), r.normal(size=(n, dv))
    w_q, w_k = r.normal(size=(d, f)) / 3, r.normal(size=(d, f)) / 3
    dt = None if decay is None else r.normal(size=n) * (2.0 if decay == "fast" else 1.0)
    a_log = None if decay is None else np.array([1.5 if decay == "fast" else -3.0])
    kk = r.random((3, 2 * f))
    kk /= kk.sum(-1, keepdims=True)
    S0, z0 = kk.T @ r.normal(size=(3, dv)), kk.sum(0)
    dO, dS, dz = r.normal(size=(n, dv)), r.normal(size=(2 * f, dv)), r.normal(size=2 * f)
    got = chunked_backward(q, k, v, w_q, w_k, dt, a_log, S0, z0, dO, dS, dz)
    ref = hm_grad.grads(q[None, None], k[None, None], v[None, None], w_q, w_k,
                        None if dt is None else dt[None, None], a_log, S0[None, None], z0[None, None],
                        dO[None, None], dS[None, None], dz[None, None])
    for name in ("q", "k", "v", "w_q", "w_k", "s_init", "z_init") + (("dt", "a_log") if decay else ()):
        r_ = ref[name][0, 0] if ref[name].ndim >= 3 else ref[name]
        np.testing.assert_allclose(got[name], r_, rtol=1e-9, atol=1e-11, err_msg=name)
