"""Pins of the gradient oracle (oracle/hm_grad.py): directional derivatives
against central finite differences of the numpy forward oracle (the recurrent
form, an independent implementation), plus properties the mathematics fixes."""
import numpy as np
import pytest

from oracle import hm_grad, hm_oracle as orc


def case(seed, B=1, H=2, n=9, d=6, f=4, dv=5, decay=True, init=True):
    r = np.random.default_rng(seed)
    c = dict(q=r.normal(size=(B, H, n, d)), k=r.normal(size=(B, H, n, d)), v=r.normal(size=(B, H, n, dv)),
             w_q=r.normal(size=(d, f)) / 2, w_k=r.normal(size=(d, f)) / 2)
    if decay:
        c["dt"] = r.normal(size=(B, H, n))
        c["a_log"] = r.uniform(-2.0, 1.0, size=H)
    if init:
        kk = r.random((B, H, 3, 2 * f))
        kk /= kk.sum(-1, keepdims=True)
        c["s_init"] = np.einsum("bhjf,bhjd->bhfd", kk, r.normal(size=(B, H, 3, dv)))
        c["z_init"] = kk.sum(2)
    return c


def loss_np(c, d_o, ds, dz):
    o, S, z = orc.forward(c["q"], c["k"], c["v"], c["w_q"], c["w_k"], c.get("dt"), c.get("a_log"),
                          c.get("s_init"), c.get("z_init"), gate=c.get("gate"))
    return float((o * d_o).sum() + (S * ds).sum() + (z * dz).sum())


@pytest.mark.parametrize("decay,init,gated", [(True, True, False), (False, False, False), (True, False, True)])
def test_gradients_match_finite_differences(decay, init, gated):
    c = case(1, decay=decay, init=init)
    if gated:
        c["gate"] = np.random.default_rng(11).normal(size=c["v"].shape) * 2
    r = np.random.default_rng(7)
    B, H, n, _ = c["q"].shape
    F, dv = 2 * c["w_q"].shape[1], c["v"].shape[-1]
    d_o = r.normal(size=(B, H, n, dv))
    ds = r.normal(size=(B, H, F, dv))
    dz = r.normal(size=(B, H, F))
    g = hm_grad.grads(**c, d_o=d_o, ds_final=ds, dz_final=dz)
    # the oracle's own forward agrees with the numpy oracle
    o_np = orc.forward(c["q"], c["k"], c["v"], c["w_q"], c["w_k"], c.get("dt"), c.get("a_log"),
                       c.get("s_init"), c.get("z_init"), gate=c.get("gate"))[0]
    np.testing.assert_allclose(g["o"], o_np, rtol=1e-12, atol=1e-12)
    eps = 1e-6
    for name in c:
        direction = r.normal(size=c[name].shape)
        cp = dict(c)
        cm = dict(c)
        cp[name] = c[name] + eps * direction
        cm[name] = c[name] - eps * direction
        fd = (loss_np(cp, d_o, ds, dz) - loss_np(cm, d_o, ds, dz)) / (2 * eps)
        an = float((g[name] * direction).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, fd, an)


def test_value_gradient_is_linear_in_d_o():
    """o is linear in v, so dV is linear in dO (and independent of v)."""
    c = case(2, init=False)
    r = np.random.default_rng(3)
    d1, d2 = r.normal(size=c["v"].shape), r.normal(size=c["v"].shape)
    g1 = hm_grad.grads(**c, d_o=d1)["v"]
    g2 = hm_grad.grads(**c, d_o=d2)["v"]
    g12 = hm_grad.grads(**c, d_o=d1 + 2 * d2)["v"]
    np.testing.assert_allclose(g12, g1 + 2 * g2, rtol=1e-12, atol=1e-12)
    c2 = dict(c, v=r.normal(size=c["v"].shape))
    np.testing.assert_allclose(hm_grad.grads(**c2, d_o=d1)["v"], g1, rtol=1e-12, atol=1e-12)


def test_single_token_depends_on_v_only():
    """With one token and no initial state o_0 = v_0, whatever q, k, W and the
    decay are, so all their gradients vanish."""
    c = case(4, n=1, init=False)
    r = np.random.default_rng(5)
    g = hm_grad.grads(**c, d_o=r.normal(size=c["v"].shape))
    # one token: o_0 = v_0 regardless of q, k, W and the decay
    for name in ("q", "k", "w_q", "w_k", "dt", "a_log"):
        np.testing.assert_allclose(g[name], 0.0, atol=1e-12)
