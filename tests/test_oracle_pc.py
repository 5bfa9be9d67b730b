"""Pins for the oracle's per-channel scan (pc_scan / forward_pc): the decay per
value channel and state that the pages' Mamba-1 wiring implies (HedgeMamba
explainer §2.3 item 3, §5.2 step 4: A, dt and V copied, the V copy set to ones;
Mamba's discretization exp(Delta A) with the input scaled by Delta).

Fixed from outside: the scalar-decay oracle (its own recurrent code) when the
decay is shared by every channel and state, plain linear attention at the
stage-1 identity init, a brute-force double loop over (t, j) with explicit
products of per-channel decays, a hand-computed two-token example, and the
split/handoff property of the state.  CPU only."""
import math

import numpy as np

from oracle import hm_oracle as orc


def case(seed, B=2, H=2, n=13, d=6, f=4, dv=5):
    r = np.random.default_rng(seed)
    return dict(q=r.normal(size=(B, H, n, d)), k=r.normal(size=(B, H, n, d)), v=r.normal(size=(B, H, n, dv)),
                w_q=r.normal(size=(d, f)) / 2, w_k=r.normal(size=(d, f)) / 2,
                dt=r.normal(size=(B, H, n, dv)), a_log=r.uniform(-2.0, 1.0, size=(H, dv, 2 * f)))


def test_two_token_worked_example():
    # one head, one channel, F = 2 states: phik_0 = (1, 0), phik_1 = (0, 1), phiq_1 = (1, 1);
    # Delta = (1, 2), A = (-ln 2, -ln 4): a_1 = (2^-2, 4^-2) = (1/4, 1/16)
    phiq = np.array([[[[1.0, 0.0], [1.0, 1.0]]]])
    phik = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    v = np.array([[[[3.0], [5.0]]]])
    delta = np.array([[[[1.0], [2.0]]]])
    A = np.array([[[-math.log(2.0), -math.log(4.0)]]])
    o, Sn, Sd = orc.pc_scan(phiq, phik, v, delta, A)
    # t = 0: Sn = (3, 0), Sd = (1, 0): o_0 = 3
    # t = 1: Sn = (3/4, 2*5) = (0.75, 10), Sd = (1/4, 2): o_1 = 10.75 / 2.25
    np.testing.assert_allclose(o[0, 0, :, 0], [3.0, 10.75 / 2.25], rtol=1e-15)
    np.testing.assert_allclose(Sn[0, 0, :, 0], [0.75, 10.0], rtol=1e-15)
    np.testing.assert_allclose(Sd[0, 0, :, 0], [0.25, 2.0], rtol=1e-15)


def test_shared_decay_is_the_scalar_path_with_delta_weighted_keys():
    # A_log[c, n] = A_log_h and dt[t, c] = dt_t for every channel: a_t = exp(-softplus(dt_t) e^{A_log_h}),
    # the scalar decay, and the increments carry Delta_t on phik_t for numerator and denominator alike
    c = case(1)
    B, H, n, dv = c["v"].shape
    r = np.random.default_rng(2)
    dt_s = r.normal(size=(B, H, n))
    al_h = r.uniform(-2.0, 1.0, size=H)
    dt = np.repeat(dt_s[..., None], dv, axis=-1)
    F = 2 * c["w_q"].shape[1]
    a_log = np.broadcast_to(al_h[:, None, None], (H, dv, F))
    o, Sn, Sd = orc.forward_pc(c["q"], c["k"], c["v"], c["w_q"], c["w_k"], dt, a_log)
    phiq = orc.hedgehog_features(c["q"], c["w_q"])
    phik = orc.hedgehog_features(c["k"], c["w_k"])
    delta = orc.softplus(dt_s)
    ref, S, z = orc.linattn_recurrent(phiq, phik * delta[..., None], c["v"], orc.log_decay(dt_s, al_h))
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Sn, S, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Sd, np.repeat(z[..., None], dv, axis=-1), rtol=1e-12, atol=1e-13)


def test_constant_step_cancels_and_gives_the_forward_oracle():
    # a step size constant over t and c scales numerator and denominator alike
    c = case(3)
    B, H, n, dv = c["v"].shape
    F = 2 * c["w_q"].shape[1]
    dt = np.full((B, H, n, dv), 0.3)
    al_h = np.array([0.2, -1.0])
    o, _, _ = orc.forward_pc(c["q"], c["k"], c["v"], c["w_q"], c["w_k"], dt, np.broadcast_to(al_h[:, None, None],
                                                                                                (H, dv, F)))
    ref, _, _ = orc.forward(c["q"], c["k"], c["v"], c["w_q"], c["w_k"], np.full((B, H, n), 0.3), al_h)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)


def test_identity_init_is_plain_linear_attention():
    # stage-1 init: lambda = 0 makes the transition the identity (A = 0, A_log = -inf), and a constant step
    c = case(4)
    B, H, n, dv = c["v"].shape
    F = 2 * c["w_q"].shape[1]
    o, _, _ = orc.forward_pc(c["q"], c["k"], c["v"], c["w_q"], c["w_k"], np.full((B, H, n, dv), -1.5),
                             np.full((H, dv, F), -np.inf))
    ref, _, _ = orc.forward(c["q"], c["k"], c["v"], c["w_q"], c["w_k"])
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)


def test_brute_force_double_loop():
    c = case(5, B=1, H=2, n=9, dv=3)
    B, H, n, dv = c["v"].shape
    phiq = orc.hedgehog_features(c["q"], c["w_q"])
    phik = orc.hedgehog_features(c["k"], c["w_k"])
    F = phiq.shape[-1]
    o_ref = np.zeros((B, H, n, dv))
    for h in range(H):
        for ch in range(dv):
            for t in range(n):
                num = den = 0.0
                for j in range(t + 1):
                    dj = math.log1p(math.exp(c["dt"][0, h, j, ch]))
                    for s_ in range(F):
                        A = -math.exp(c["a_log"][h, ch, s_])
                        carry = 1.0
                        for u in range(j + 1, t + 1):
                            carry *= math.exp(math.log1p(math.exp(c["dt"][0, h, u, ch])) * A)
                        w = phiq[0, h, t, s_] * phik[0, h, j, s_] * carry * dj
                        num += w * c["v"][0, h, j, ch]
                        den += w
                o_ref[0, h, t, ch] = num / den
    o, _, _ = orc.forward_pc(c["q"], c["k"], c["v"], c["w_q"], c["w_k"], c["dt"], c["a_log"])
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-13)


def test_split_and_handoff_and_decode_step():
    c = case(6, n=11)
    o, Sn, Sd = orc.forward_pc(**c)
    m = 7
    a = {k: (v[:, :, :m] if k in ("q", "k", "v", "dt") else v) for k, v in c.items()}
    b = {k: (v[:, :, m:] if k in ("q", "k", "v", "dt") else v) for k, v in c.items()}
    oa, Sna, Sda = orc.forward_pc(**a)
    ob, Snb, Sdb = orc.forward_pc(**b, sn0=Sna, sd0=Sda)
    np.testing.assert_allclose(np.concatenate([oa, ob], axis=2), o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Snb, Sn, rtol=1e-12, atol=1e-13)
    # one decode step continues the prefix
    o1, Sn1, Sd1 = orc.step_pc(Sna, Sda, c["q"][:, :, m], c["k"][:, :, m], c["v"][:, :, m], c["w_q"], c["w_k"],
                               c["dt"][:, :, m], c["a_log"])
    np.testing.assert_allclose(o1, o[:, :, m], rtol=1e-12, atol=1e-13)
    flat = orc.pack_state_pc(Sn, Sd)
    F, dv = Sn.shape[2], Sn.shape[3]
    assert flat[1, 0, 3 * F + 2] == Sn[1, 0, 2, 3] and flat[0, 1, F * dv + 4 * F + 1] == Sd[0, 1, 1, 4]  # [dv][F]
    Sn2, Sd2 = orc.unpack_state_pc(flat, Sn.shape[2], Sn.shape[3])
    np.testing.assert_array_equal(Sn2, Sn)
    np.testing.assert_array_equal(Sd2, Sd)


def test_outputs_are_convex_combinations_per_channel():
    c = case(7, n=20)
    o, _, _ = orc.forward_pc(**c)
    v = c["v"]
    for t in range(v.shape[2]):
        lo = v[:, :, : t + 1].min(axis=2)
        hi = v[:, :, : t + 1].max(axis=2)
        assert np.all(o[:, :, t] >= lo - 1e-12) and np.all(o[:, :, t] <= hi + 1e-12)


def test_planted_mistakes_are_caught():
    # (1) input not scaled by Delta: breaks the shared-decay reduction unless Delta is constant
    c = case(8)
    B, H, n, dv = c["v"].shape
    F = 2 * c["w_q"].shape[1]
    dt_s = np.random.default_rng(9).normal(size=(B, H, n))
    al = np.array([0.1, -0.5])
    phiq = orc.hedgehog_features(c["q"], c["w_q"])
    phik = orc.hedgehog_features(c["k"], c["w_k"])
    good, _, _ = orc.linattn_recurrent(phiq, phik * orc.softplus(dt_s)[..., None], c["v"], orc.log_decay(dt_s, al))
    bad, _, _ = orc.linattn_recurrent(phiq, phik, c["v"], orc.log_decay(dt_s, al))
    assert np.abs(good - bad).max() > 1e-3
    # (2) the two-token example with the decay applied to the incoming token too
    a1 = np.array([0.25, 1.0 / 16.0])
    Sn_bad = a1 * (np.array([3.0, 0.0]) + np.array([0.0, 2.0 * 5.0]))
    assert not np.allclose(Sn_bad, [0.75, 10.0])
