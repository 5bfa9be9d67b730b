"""Pins for the CPU oracle: closed forms, library routines, brute force, invariants.

Each test fixes the oracle to something other than itself, so that a plausible
mistake (a dropped term, a wrong sign or index, a transposed operand, a decay
applied at the wrong place) fails at least one of them.  CPU only.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.signal
import scipy.special

from oracle import hm_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def golden():
    with open(GOLDEN) as fh:
        return json.load(fh)


def rng(seed=0):
    return np.random.default_rng(seed)


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


# ----------------------------------------------------------------- features
def test_features_rational_worked_example():
    g = golden()["features_rational"]
    phi = orc.hedgehog_features(np.array([g["x"]]), np.array(g["w"]))
    np.testing.assert_allclose(phi[0], g["phi"], rtol=1e-14, atol=0)


def test_features_two_entries_are_logistic():
    # softmax over [u, -u] equals [sigmoid(2u), sigmoid(-2u)]; scipy's expit is an
    # independent implementation of the logistic function.
    g = golden()["features_two_entry_logistic"]
    phi = orc.hedgehog_features(np.array([g["x"]]), np.array(g["w"]))[0]
    u = g["u"]
    np.testing.assert_allclose(phi, [scipy.special.expit(2 * u), scipy.special.expit(-2 * u)], rtol=1e-14)
    r = rng(1)
    x = r.normal(size=(50, 3))
    w = r.normal(size=(3, 1))
    phi = orc.hedgehog_features(x, w)
    uu = (x @ w)[:, 0]
    np.testing.assert_allclose(phi[:, 0], scipy.special.expit(2 * uu), rtol=1e-13)
    np.testing.assert_allclose(phi[:, 1], scipy.special.expit(-2 * uu), rtol=1e-13)


def test_features_match_library_softmax():
    r = rng(2)
    x = r.normal(size=(2, 3, 40, 16))
    w = r.normal(size=(16, 8))
    u = np.einsum("bhnd,df->bhnf", x, w)
    ref = scipy.special.softmax(np.concatenate([u, -u], axis=-1), axis=-1)
    np.testing.assert_allclose(orc.hedgehog_features(x, w), ref, rtol=1e-13, atol=1e-300)


def test_features_per_head_weights():
    r = rng(3)
    x = r.normal(size=(2, 3, 10, 8))
    w = r.normal(size=(3, 8, 4))
    phi = orc.hedgehog_features(x, w)
    for h in range(3):
        np.testing.assert_allclose(phi[:, h], orc.hedgehog_features(x[:, h], w[h]), rtol=1e-14)


def test_features_positive_rows_sum_to_one_and_extreme_inputs():
    r = rng(4)
    x = r.normal(size=(100, 16)) * 50.0     # large |u|: the max shift must prevent overflow
    w = r.normal(size=(16, 16))
    phi = orc.hedgehog_features(x, w)
    assert np.all(np.isfinite(phi))
    assert np.all(phi >= 0)
    np.testing.assert_allclose(phi.sum(axis=-1), 1.0, rtol=1e-13)
    phi_small = orc.hedgehog_features(r.normal(size=(100, 16)), w * 0.1)
    assert np.all(phi_small > 0)


def test_features_halves_swap_under_negation():
    # phi(-x)[:f] == phi(x)[f:]: the second half is built from -xW.
    r = rng(5)
    x = r.normal(size=(20, 6))
    w = r.normal(size=(6, 5))
    a = orc.hedgehog_features(x, w)
    b = orc.hedgehog_features(-x, w)
    np.testing.assert_allclose(a[:, :5], b[:, 5:], rtol=1e-14)
    np.testing.assert_allclose(a[:, 5:], b[:, :5], rtol=1e-14)


# -------------------------------------------------------------------- decay
def test_softplus_against_library_and_closed_forms():
    x = np.linspace(-800, 800, 20001)
    np.testing.assert_allclose(orc.softplus(x), np.logaddexp(0.0, x), rtol=1e-14, atol=1e-300)
    assert orc.softplus(np.array([0.0]))[0] == pytest.approx(math.log(2.0), rel=1e-16)
    assert orc.softplus(np.array([1000.0]))[0] == 1000.0


def test_log_decay_values_and_identity():
    assert orc.log_decay(None, None) is None
    dt = np.array([[[0.0, 2.0, -3.0]]])
    a_log = np.array([math.log(4.0)])
    la = orc.log_decay(dt, a_log)
    expect = -4.0 * np.logaddexp(0.0, dt)
    np.testing.assert_allclose(la, expect, rtol=1e-14)
    assert np.all(la < 0)


def test_decay_matrix_equals_products():
    r = rng(6)
    la = -r.exponential(size=12)
    G = orc.decay_matrix(la)
    a = np.exp(la)
    for i in range(12):
        for j in range(12):
            ref = 0.0 if j > i else float(np.prod(a[j + 1:i + 1]))
            assert G[i, j] == pytest.approx(ref, rel=1e-12, abs=1e-300)


# ---------------------------------------------------------- worked examples
def _run(ex, form, with_state=False):
    q = np.array(ex["q"])[None, None]
    k = np.array(ex["k"])[None, None]
    v = np.array(ex["v"])[None, None]
    dt = np.array(ex["dt"])[None, None] if "dt" in ex else None
    a_log = np.array(ex["a_log"]) if "a_log" in ex else None
    s0 = np.array(ex["S_init"])[None, None] if with_state else None
    z0 = np.array(ex["z_init"])[None, None] if with_state else None
    return orc.forward(q, k, v, np.array(ex["w_q"]), np.array(ex["w_k"]), dt, a_log, s0, z0, form=form)


@pytest.mark.parametrize("form", ["quadratic", "recurrent"])
def test_worked_examples(form):
    g = golden()
    o, _, _ = _run(g["three_token_identity"], form)
    np.testing.assert_allclose(o[0, 0], g["three_token_identity"]["o"], rtol=1e-14)
    o, S, z = _run(g["two_token_decay"], form)
    np.testing.assert_allclose(o[0, 0], g["two_token_decay"]["o"], rtol=1e-14)
    if form == "recurrent":
        np.testing.assert_allclose(S[0, 0], g["two_token_decay"]["S_final"], rtol=1e-14)
        np.testing.assert_allclose(z[0, 0], g["two_token_decay"]["z_final"], rtol=1e-14)
    o, _, _ = _run(g["initial_state_one_token"], form, with_state=True)
    np.testing.assert_allclose(o[0, 0], g["initial_state_one_token"]["o"], rtol=1e-14)


# --------------------------------------------------------- forms and pins
def random_case(seed=0, B=2, H=3, n=29, d=6, f=4, dv=5, decay=True, state=False, scale=1.0):
    r = rng(seed)
    q = r.normal(size=(B, H, n, d))
    k = r.normal(size=(B, H, n, d))
    v = r.normal(size=(B, H, n, dv))
    wq = r.normal(size=(d, f)) * scale
    wk = r.normal(size=(d, f)) * scale
    dt = r.normal(size=(B, H, n)) if decay else None
    a_log = r.uniform(-3, 1, size=H) if decay else None
    s0 = z0 = None
    if state:
        F = 2 * f
        kk = r.random(size=(B, H, 7, F))
        kk /= kk.sum(-1, keepdims=True)
        s0 = np.einsum("bhjf,bhjd->bhfd", kk, r.normal(size=(B, H, 7, dv)))
        z0 = kk.sum(axis=2)
    return q, k, v, wq, wk, dt, a_log, s0, z0


@pytest.mark.parametrize("decay", [False, True])
@pytest.mark.parametrize("state", [False, True])
def test_quadratic_equals_recurrent(decay, state):
    q, k, v, wq, wk, dt, a_log, s0, z0 = random_case(7, decay=decay, state=state)
    oq, _, _ = orc.forward(q, k, v, wq, wk, dt, a_log, s0, z0, form="quadratic")
    orr, _, _ = orc.forward(q, k, v, wq, wk, dt, a_log, s0, z0, form="recurrent")
    assert rel_l2(oq, orr) < 1e-12


def test_identity_decay_is_three_library_calls():
    # a = 1: o = rownorm(tril(phiQ phiK^T)) V, built here from numpy/scipy calls.
    q, k, v, wq, wk, _, _, _, _ = random_case(8, decay=False)
    uq, uk = q @ wq, k @ wk
    pq = scipy.special.softmax(np.concatenate([uq, -uq], -1), axis=-1)
    pk = scipy.special.softmax(np.concatenate([uk, -uk], -1), axis=-1)
    A = np.tril(pq @ np.swapaxes(pk, -1, -2))
    ref = (A / A.sum(-1, keepdims=True)) @ v
    o, _, _ = orc.forward(q, k, v, wq, wk)
    assert rel_l2(o, ref) < 1e-13


def test_first_output_is_first_value():
    q, k, v, wq, wk, dt, a_log, _, _ = random_case(9)
    for form in ("quadratic", "recurrent"):
        o, _, _ = orc.forward(q, k, v, wq, wk, dt, a_log, form=form)
        np.testing.assert_allclose(o[:, :, 0], v[:, :, 0], rtol=1e-13)


def test_zero_weights_give_running_mean():
    q, k, v, wq, wk, _, _, _, _ = random_case(10, decay=False)
    o, _, _ = orc.forward(q, k, v, wq * 0, wk * 0)
    n = v.shape[2]
    ref = np.cumsum(v, axis=2) / np.arange(1, n + 1)[None, None, :, None]
    np.testing.assert_allclose(o, ref, rtol=1e-12)


@pytest.mark.parametrize("a", [0.9, 0.5, 0.05])
def test_zero_weights_constant_decay_is_iir_filter(a):
    # W = 0: o_t = sum_j a^{t-j} v_j / sum_j a^{t-j}, i.e. the ratio of two
    # first-order IIR filters y_t = a y_{t-1} + x_t (scipy.signal.lfilter).
    r = rng(11)
    n, dv = 40, 3
    v = r.normal(size=(1, 1, n, dv))
    q = r.normal(size=(1, 1, n, 4))
    k = r.normal(size=(1, 1, n, 4))
    w = np.zeros((4, 2))
    a_log = np.array([0.0])
    # choose dt so that softplus(dt) = -log a
    dt = np.full((1, 1, n), math.log(math.expm1(-math.log(a))))
    o, S, z = orc.forward(q, k, v, w, w, dt, a_log)
    num = scipy.signal.lfilter([1.0], [1.0, -a], v[0, 0], axis=0)
    den = scipy.signal.lfilter([1.0], [1.0, -a], np.ones(n))
    np.testing.assert_allclose(o[0, 0], num / den[:, None], rtol=1e-11)
    # the carried state (uniform phi = 1/F) is the filter output itself
    F = 4
    np.testing.assert_allclose(S[0, 0], np.tile(num[-1] / F, (F, 1)), rtol=1e-11)
    np.testing.assert_allclose(z[0, 0], np.full(F, den[-1] / F), rtol=1e-11)


def test_strong_decay_returns_current_value():
    q, k, v, wq, wk, _, _, _, _ = random_case(12)
    dt = np.full(v.shape[:3], 50.0)
    a_log = np.full(v.shape[1], 8.0)      # log a = -50 e^8: state forgotten each step
    for form in ("quadratic", "recurrent"):
        o, _, _ = orc.forward(q, k, v, wq, wk, dt, a_log, form=form)
        np.testing.assert_allclose(o, v, rtol=1e-12)


def test_brute_force_tiny():
    # Nested python loops over the definition, products of a_s taken one by one.
    q, k, v, wq, wk, dt, a_log, _, _ = random_case(13, B=1, H=2, n=6, d=3, f=2, dv=2)
    o, _, _ = orc.forward(q, k, v, wq, wk, dt, a_log)
    for h in range(2):
        a = [math.exp(-math.log1p(math.exp(float(x))) * math.exp(float(a_log[h]))) for x in dt[0, h]]
        def feat(x, w):
            u = [sum(x[i] * w[i][j] for i in range(len(x))) for j in range(len(w[0]))]
            e = [math.exp(t) for t in u] + [math.exp(-t) for t in u]
            s = sum(e)
            return [t / s for t in e]
        for t in range(6):
            fq = feat(q[0, h, t], wq)
            num = [0.0, 0.0]
            den = 0.0
            for j in range(t + 1):
                fk = feat(k[0, h, j], wk)
                wgt = sum(x * y for x, y in zip(fq, fk))
                for s in range(j + 1, t + 1):
                    wgt *= a[s]
                den += wgt
                for c in range(2):
                    num[c] += wgt * v[0, h, j, c]
            np.testing.assert_allclose(o[0, h, t], [num[0] / den, num[1] / den], rtol=1e-12)


def test_convex_combination_bounds_and_den_positive():
    q, k, v, wq, wk, dt, a_log, _, _ = random_case(14, n=64)
    o, S, z = orc.forward(q, k, v, wq, wk, dt, a_log)
    lo = np.minimum.accumulate(v, axis=2)
    hi = np.maximum.accumulate(v, axis=2)
    assert np.all(o >= lo - 1e-12) and np.all(o <= hi + 1e-12)
    assert np.all(z > 0)


def test_constant_and_affine_values():
    q, k, v, wq, wk, dt, a_log, _, _ = random_case(15)
    o, _, _ = orc.forward(q, k, np.full_like(v, 2.5), wq, wk, dt, a_log)
    np.testing.assert_allclose(o, 2.5, rtol=1e-13)
    o1, _, _ = orc.forward(q, k, v, wq, wk, dt, a_log)
    o2, _, _ = orc.forward(q, k, -3.0 * v + 0.75, wq, wk, dt, a_log)
    np.testing.assert_allclose(o2, -3.0 * o1 + 0.75, rtol=1e-12, atol=1e-12)


def test_symmetries():
    q, k, v, wq, wk, dt, a_log, _, _ = random_case(16)
    o, _, _ = orc.forward(q, k, v, wq, wk, dt, a_log)
    o_neg, _, _ = orc.forward(q, k, v, -wq, -wk, dt, a_log)
    np.testing.assert_allclose(o_neg, o, rtol=1e-12)
    perm = np.array([2, 0, 3, 1])
    o_perm, _, _ = orc.forward(q, k, v, wq[:, perm], wk[:, perm], dt, a_log)
    np.testing.assert_allclose(o_perm, o, rtol=1e-12)
    # an unnormalized exp map for q only: a positive per-query scale cancels
    uq = q @ wq
    pq_exp = np.exp(np.concatenate([uq, -uq], -1))
    pk = orc.hedgehog_features(k, wk)
    o_exp = orc.linattn_quadratic(pq_exp, pk, v, orc.log_decay(dt, a_log))
    np.testing.assert_allclose(o_exp, o, rtol=1e-12)
    # but not for k: per-key scales change the weights
    uk = k @ wk
    pk_exp = np.exp(np.concatenate([uk, -uk], -1))
    o_bad = orc.linattn_quadratic(orc.hedgehog_features(q, wq), pk_exp, v, orc.log_decay(dt, a_log))
    assert rel_l2(o_bad, o) > 1e-3


def test_split_and_handoff():
    # fwd[0,n) == fwd[0,m) -> state -> fwd[m,n) == fwd[0,m) -> token-by-token steps
    q, k, v, wq, wk, dt, a_log, _, _ = random_case(17, n=23)
    o, S, z = orc.forward(q, k, v, wq, wk, dt, a_log)
    m = 9
    o1, S1, z1 = orc.forward(q[:, :, :m], k[:, :, :m], v[:, :, :m], wq, wk, dt[:, :, :m], a_log)
    o2, S2, z2 = orc.forward(q[:, :, m:], k[:, :, m:], v[:, :, m:], wq, wk, dt[:, :, m:], a_log, S1, z1)
    np.testing.assert_allclose(np.concatenate([o1, o2], 2), o, rtol=1e-12)
    np.testing.assert_allclose(S2, S, rtol=1e-12)
    Sc, zc = S1, z1
    for t in range(m, 23):
        ot, Sc, zc = orc.step(Sc, zc, q[:, :, t], k[:, :, t], v[:, :, t], wq, wk, dt[:, :, t], a_log)
        np.testing.assert_allclose(ot, o[:, :, t], rtol=1e-12)
    np.testing.assert_allclose(Sc, S, rtol=1e-12)
    np.testing.assert_allclose(zc, z, rtol=1e-12)


def test_prefix_state_closed_form():
    q, k, v, wq, wk, dt, a_log, _, _ = random_case(18, n=31)
    _, S, z = orc.forward(q, k, v, wq, wk, dt, a_log)
    pk = orc.hedgehog_features(k, wk)
    S2, z2 = orc.prefix_state(pk, v, orc.log_decay(dt, a_log))
    np.testing.assert_allclose(S2, S, rtol=1e-11)
    np.testing.assert_allclose(z2, z, rtol=1e-11)
    S3, z3 = orc.prefix_state(pk, v, None)
    np.testing.assert_allclose(S3, np.einsum("bhnf,bhnd->bhfd", pk, v), rtol=1e-13)
    np.testing.assert_allclose(z3, pk.sum(2), rtol=1e-13)


def test_state_pack_roundtrip():
    r = rng(19)
    S = r.normal(size=(2, 3, 8, 5))
    z = r.normal(size=(2, 3, 8))
    flat = orc.pack_state(S, z)
    assert flat.shape == (2, 3, 8 * 5 + 8)
    np.testing.assert_array_equal(flat[0, 1, :5], S[0, 1, 0])
    np.testing.assert_array_equal(flat[0, 1, 40:], z[0, 1])
    S2, z2 = orc.unpack_state(flat, 8, 5)
    np.testing.assert_array_equal(S2, S)
    np.testing.assert_array_equal(z2, z)


# ------------------------------------------------------------------ gate
def test_silu_against_library_sigmoid():
    x = np.concatenate([np.linspace(-40, 40, 801), [-750.0, -80.0, 80.0, 750.0]])
    ref = x * scipy.special.expit(x)
    np.testing.assert_allclose(orc.silu(x), ref, rtol=1e-14, atol=1e-300)
    assert np.all(np.isfinite(orc.silu(x)))
    assert orc.silu(np.array([0.0]))[0] == 0.0


def test_gate_at_identity_init_leaves_output_unchanged():
    # stage-1 init: gate weights 0 and bias SiLU^-1(1), so the gate branch outputs 1
    import scipy.optimize
    c = scipy.optimize.brentq(lambda x: x * scipy.special.expit(x) - 1.0, 0.0, 4.0, xtol=1e-15)
    q, k, v, wq, wk, dt, a_log, s0, z0 = random_case(31, state=True)
    o, S, z = orc.forward(q, k, v, wq, wk, dt, a_log, s0, z0)
    og, Sg, zg = orc.forward(q, k, v, wq, wk, dt, a_log, s0, z0, gate=np.full(v.shape, c))
    assert rel_l2(og, o) < 1e-13
    np.testing.assert_array_equal(Sg, S)       # the gate never touches the state
    np.testing.assert_array_equal(zg, z)


def test_gate_is_elementwise_on_the_output():
    q, k, v, wq, wk, dt, a_log, _, _ = random_case(32)
    g = rng(33).normal(size=v.shape) * 3
    o, _, _ = orc.forward(q, k, v, wq, wk, dt, a_log)
    for form in ("quadratic", "recurrent"):
        og, _, _ = orc.forward(q, k, v, wq, wk, dt, a_log, form=form, gate=g)
        np.testing.assert_allclose(og, o * g * scipy.special.expit(g), rtol=1e-11, atol=1e-14)
    og, _, _ = orc.forward(q, k, v, wq, wk, dt, a_log, gate=np.zeros(v.shape))
    assert np.all(og == 0.0)


def test_gated_step_equals_gated_forward_last_token():
    q, k, v, wq, wk, dt, a_log, _, _ = random_case(34, n=12)
    g = rng(35).normal(size=v.shape)
    o, _, _ = orc.forward(q, k, v, wq, wk, dt, a_log, gate=g)
    _, S, z = orc.forward(q[:, :, :11], k[:, :, :11], v[:, :, :11], wq, wk, dt[:, :, :11], a_log)
    o1, _, _ = orc.step(S, z, q[:, :, 11], k[:, :, 11], v[:, :, 11], wq, wk, dt[:, :, 11], a_log, gate=g[:, :, 11])
    assert rel_l2(o1, o[:, :, 11]) < 1e-12


def test_planted_mistakes_are_caught():
    # Each of these plausible mistakes, planted in a copy of the oracle's
    # arithmetic, must break one of the pins above.
    g = golden()["two_token_decay"]
    ex = {k: np.array(v) for k, v in g.items() if k in ("q", "k", "v", "dt", "a_log", "w_q", "w_k")}
    la = orc.log_decay(ex["dt"][None, None], ex["a_log"])
    phi = orc.hedgehog_features(ex["q"][None, None], ex["w_q"])
    v = ex["v"][None, None]
    # (1) decay applied to the incoming token as well: outputs unchanged but the
    # carried state differs from the worked example's S_final.
    S = np.zeros((2, 1))
    for t in range(2):
        S = np.exp(la[0, 0, t]) * (S + phi[0, 0, t][:, None] * v[0, 0, t][None, :])
    assert not np.allclose(S, g["S_final"])
    # (2) decay index shifted by one (a_{t-1} instead of a_t) on the two-token case
    o_shift = (1.0 * 0.5 * 3 + 0.5 * 6) / (1.0 * 0.5 + 0.5)
    assert o_shift != g["o"][1][0]
    # (3) denominator missing the current token: o_0 would be 0/0
    # (4) sign error in the second half ([u, u]) breaks the rational example
    x = np.array([[1.0]])
    w = np.array(golden()["features_rational"]["w"])
    u = x @ w
    bad = scipy.special.softmax(np.concatenate([u, u], -1), axis=-1)
    assert not np.allclose(bad[0], golden()["features_rational"]["phi"])


# ------------------------------------------------------------ short causal conv
def test_conv_identity_init_is_the_identity():
    """[HM] §3.1: taps [0, ..., 0, 1] with zero bias pass the input through."""
    x = np.random.default_rng(0).normal(size=(2, 3, 11, 8))
    for K in (1, 2, 3, 4):
        w = np.zeros((8, K))
        w[:, -1] = 1.0
        y, fin = orc.causal_conv(x, w, np.zeros(8))
        assert np.array_equal(y, x)
        if K > 1:
            assert np.array_equal(fin, x[:, :, -(K - 1):])


def test_conv_matches_numpy_convolve_per_channel():
    r = np.random.default_rng(1)
    x = r.normal(size=(1, 2, 13, 5))
    w = r.normal(size=(2, 5, 4))          # per-head taps
    b = r.normal(size=(2, 5))
    y, _ = orc.causal_conv(x, w, b)
    for h in range(2):
        for c in range(5):
            ref = np.convolve(x[0, h, :, c], w[h, c, ::-1])[:13] + b[h, c]
            np.testing.assert_allclose(y[0, h, :, c], ref, rtol=1e-13, atol=1e-13)


def test_conv_single_tap_delays():
    """A single tap at position K-1-s delays the stream by s tokens, prev first."""
    r = np.random.default_rng(2)
    x = r.normal(size=(2, 1, 9, 4))
    prev = r.normal(size=(2, 1, 3, 4))
    for s_ in range(4):
        w = np.zeros((4, 4))
        w[:, 3 - s_] = 1.0
        y, _ = orc.causal_conv(x, w, None, prev)
        stream = np.concatenate([prev, x], axis=2)
        np.testing.assert_array_equal(y, stream[:, :, 3 - s_:3 - s_ + 9])


def test_conv_is_causal_and_splits():
    r = np.random.default_rng(3)
    x = r.normal(size=(1, 2, 30, 6))
    w = r.normal(size=(6, 4))
    b = r.normal(size=6)
    prev = r.normal(size=(1, 2, 3, 6))
    y, fin = orc.causal_conv(x, w, b, prev)
    x2 = x.copy()
    x2[:, :, 17] += 5.0
    y2, _ = orc.causal_conv(x2, w, b, prev)
    np.testing.assert_array_equal(y2[:, :, :17], y[:, :, :17])
    assert np.all(y2[:, :, 17:21] != y[:, :, 17:21]) and np.array_equal(y2[:, :, 21:], y[:, :, 21:])
    for m in (0, 1, 2, 5, 29):
        ya, fa = orc.causal_conv(x[:, :, :m], w, b, prev)
        yb, fb = orc.causal_conv(x[:, :, m:], w, b, fa)
        np.testing.assert_allclose(np.concatenate([ya, yb], axis=2), y, rtol=1e-14, atol=1e-14)
        np.testing.assert_array_equal(fb, fin)
    # a stream shorter than the window: final mixes prev and x
    _, f1 = orc.causal_conv(x[:, :, :1], w, b, prev)
    np.testing.assert_array_equal(f1, np.concatenate([prev[:, :, 1:], x[:, :, :1]], axis=2))
