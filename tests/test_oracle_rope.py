"""Pins for the oracle's rotary encoding of the features (HedgeMamba explainer,
§5.2 step 3: RoPE on phi(Q) and phi(K), as in the original Transformer and in
Pythia, i.e. the GPT-NeoX rotate-half form).

The rotation is fixed from outside the oracle by textbook constants (cos and
sin of 1 and 100 radians), by the frequencies 10^-i that base 10^4 gives over
eight features, by a matrix exponential of the rotation generator (scipy), and
by the invariants a rotation must satisfy; the rotated path is then checked by
brute force, across its two forms, across prefill and decode, and across a
change of origin.  CPU only.
"""
import numpy as np
import pytest
import scipy.linalg

from oracle import hm_grad, hm_oracle as orc

COS1, SIN1 = 0.5403023058681398, 0.8414709848078965        # cos(1), sin(1)
COS100, SIN100 = 0.8623188722876839, -0.5063656411097588   # cos(100), sin(100)


def unit(F, i):
    e = np.zeros(F)
    e[i] = 1.0
    return e


def test_worked_example_pairs_and_direction():
    # dims = 4, base 10^4: pairs (0, 2) and (1, 3) turn by pos * 1 and pos * 10^-2.
    out = orc.rope(unit(4, 0)[None], np.array([100.0]), 4)[0]
    np.testing.assert_allclose(out, [COS100, 0.0, SIN100, 0.0], rtol=0, atol=1e-15)
    out = orc.rope(unit(4, 1)[None], np.array([100.0]), 4)[0]
    np.testing.assert_allclose(out, [0.0, COS1, 0.0, SIN1], rtol=0, atol=1e-15)
    # the second member of a pair turns the same way: (0, 1) -> (-sin, cos)
    out = orc.rope(unit(4, 3)[None], np.array([100.0]), 4)[0]
    np.testing.assert_allclose(out, [0.0, -SIN1, 0.0, COS1], rtol=0, atol=1e-15)


def test_frequencies_for_eight_features():
    # base 10^4 over dims = 8: pair i turns by 10^-i per position
    for i in range(4):
        out = orc.rope(unit(8, i)[None], np.array([1.0]), 8)[0]
        assert abs(np.arctan2(out[i + 4], out[i]) - 10.0 ** -i) < 1e-15
        others = np.delete(out, [i, i + 4])
        assert np.all(others == 0.0)
    # another base: pair 1 of dims 4 turns by base^-1/2
    out = orc.rope(unit(4, 1)[None], np.array([3.0]), 4, base=16.0)[0]
    assert abs(np.arctan2(out[3], out[1]) - 3.0 / 4.0) < 1e-15


def test_partial_rotation_leaves_the_tail():
    r = np.random.default_rng(0)
    phi = r.random((5, 16))
    out = orc.rope(phi, np.arange(5.0) * 37, 8)
    np.testing.assert_array_equal(out[:, 8:], phi[:, 8:])
    np.testing.assert_array_equal(orc.rope(phi, np.arange(5.0), 0), phi)
    np.testing.assert_array_equal(out[0], phi[0])  # position 0 is the identity


def test_rotation_matches_matrix_exponential_of_its_generator():
    # R(pos) = expm(pos * J) with J the skew generator that couples i and i + dims/2
    # at rate base^(-2i/dims): an independent construction of the same rotation.
    F, dims, base = 12, 8, 500.0
    J = np.zeros((F, F))
    for i in range(dims // 2):
        th = base ** (-2.0 * i / dims)
        J[i + dims // 2, i] = th
        J[i, i + dims // 2] = -th
    r = np.random.default_rng(1)
    phi = r.normal(size=(6, F))
    pos = np.array([0.0, 1.0, 2.0, 7.0, 31.0, 250.0])
    out = orc.rope(phi, pos, dims, base)
    for t in range(6):
        np.testing.assert_allclose(out[t], scipy.linalg.expm(pos[t] * J) @ phi[t], rtol=1e-12, atol=1e-12)


def test_rotation_is_orthogonal_and_relative():
    r = np.random.default_rng(2)
    a, b = r.normal(size=(1, 32)), r.normal(size=(1, 32))
    for p, pp, shift in ((3.0, 11.0, 1000.0), (0.0, 5.0, 123456.0), (40.0, 2.0, 7.0)):
        ra, rb = orc.rope(a, np.array([p]), 32), orc.rope(b, np.array([pp]), 32)
        np.testing.assert_allclose(np.linalg.norm(ra), np.linalg.norm(a), rtol=1e-14)
        sa, sb = orc.rope(a, np.array([p + shift]), 32), orc.rope(b, np.array([pp + shift]), 32)
        assert abs((ra * rb).sum() - (sa * sb).sum()) < 1e-10


def case(seed, B=2, H=2, n=11, d=6, f=8, dv=5, decay=True):
    r = np.random.default_rng(seed)
    c = dict(q=r.normal(size=(B, H, n, d)), k=r.normal(size=(B, H, n, d)), v=r.normal(size=(B, H, n, dv)),
             w_q=r.normal(size=(d, f)) / 2, w_k=r.normal(size=(d, f)) / 2)
    if decay:
        c["dt"] = r.normal(size=(B, H, n))
        c["a_log"] = r.uniform(-2.0, 0.5, size=H)
    return c


def brute(c, dims, base, pos0):
    """o_t = sum_j w_tj v_j / sum_j w_tj with w_tj = (R_t phiq_t).(R_j phik_j) * prod a,
    rotation matrices built from block 2x2 rotations, double loop over (t, j)."""
    phiq = orc.hedgehog_features(c["q"], c["w_q"])
    phik = orc.hedgehog_features(c["k"], c["w_k"])
    B, H, n, F = phiq.shape
    la = orc.log_decay(c.get("dt"), c.get("a_log"))

    def R(p):
        m = np.eye(F)
        for i in range(dims // 2):
            th = p * base ** (-2.0 * i / dims)
            m[i, i] = m[i + dims // 2, i + dims // 2] = np.cos(th)
            m[i + dims // 2, i] = np.sin(th)
            m[i, i + dims // 2] = -np.sin(th)
        return m

    o = np.zeros(c["v"].shape)
    for b in range(B):
        for h in range(H):
            for t in range(n):
                num, den = np.zeros(c["v"].shape[-1]), 0.0
                qt = R(pos0[b] + t) @ phiq[b, h, t]
                for j in range(t + 1):
                    w = qt @ (R(pos0[b] + j) @ phik[b, h, j])
                    if la is not None:
                        w *= np.exp(la[b, h, j + 1:t + 1].sum())
                    num += w * c["v"][b, h, j]
                    den += w
                o[b, h, t] = num / den
    return o


@pytest.mark.parametrize("dims,decay", [(16, True), (8, False), (16, False)])
def test_forward_matches_brute_force(dims, decay):
    c = case(3, decay=decay)
    pos0 = np.array([0, 29])
    o_ref = brute(c, dims, 10000.0, pos0)
    for form in ("recurrent", "quadratic"):
        o, _, _ = orc.forward(**c, form=form, rope_dims=dims, rope_pos0=pos0)
        np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-12)


def test_zero_dims_is_the_plain_path():
    c = case(4)
    o0, S0, z0 = orc.forward(**c)
    o1, S1, z1 = orc.forward(**c, rope_dims=0, rope_pos0=np.array([5, 9]))
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(S0, S1)


def test_output_depends_on_relative_positions_only():
    # from a zero state every weight is (R_t phiq).(R_j phik) = phiq^T R_{j-t} phik
    c = case(5)
    oa, _, _ = orc.forward(**c, rope_dims=16, rope_pos0=np.array([0, 0]))
    ob, _, _ = orc.forward(**c, rope_dims=16, rope_pos0=np.array([777, 123456]))
    np.testing.assert_allclose(ob, oa, rtol=1e-9, atol=1e-11)
    # while the carried state does change with the origin
    _, Sa, _ = orc.forward(**c, rope_dims=16, rope_pos0=np.array([0, 0]))
    _, Sb, _ = orc.forward(**c, rope_dims=16, rope_pos0=np.array([777, 123456]))
    assert not np.allclose(Sa, Sb)


def test_per_sequence_offsets_and_split():
    c = case(6, n=14)
    pos0 = np.array([3, 40])
    o, S, z = orc.forward(**c, rope_dims=16, rope_pos0=pos0)
    # the second sequence alone, at its own offset
    one = {k: (v[1:2] if k not in ("w_q", "w_k", "a_log") else v) for k, v in c.items()}
    o1, _, _ = orc.forward(**one, rope_dims=16, rope_pos0=pos0[1:])
    np.testing.assert_allclose(o1[0], o[1], rtol=1e-12, atol=1e-13)
    # split at token 9: the second part starts at pos0 + 9 from the carried state
    a = {k: (v[:, :, :9] if k in ("q", "k", "v", "dt") else v) for k, v in c.items()}
    bpart = {k: (v[:, :, 9:] if k in ("q", "k", "v", "dt") else v) for k, v in c.items()}
    oa, Sa, za = orc.forward(**a, rope_dims=16, rope_pos0=pos0)
    ob, Sb, zb = orc.forward(**bpart, s_init=Sa, z_init=za, rope_dims=16, rope_pos0=pos0 + 9)
    np.testing.assert_allclose(np.concatenate([oa, ob], 2), o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(Sb, S, rtol=1e-11, atol=1e-12)


def test_decode_chain_equals_prefill():
    c = case(7, n=9)
    pos0 = np.array([2, 100])
    o, S, z = orc.forward(**c, rope_dims=8, rope_pos0=pos0)
    B, H, n, _ = c["q"].shape
    F, dv = 2 * c["w_q"].shape[1], c["v"].shape[-1]
    Sd, zd = np.zeros((B, H, F, dv)), np.zeros((B, H, F))
    for t in range(n):
        ot, Sd, zd = orc.step(Sd, zd, c["q"][:, :, t], c["k"][:, :, t], c["v"][:, :, t], c["w_q"], c["w_k"],
                              c["dt"][:, :, t], c["a_log"], rope_dims=8, rope_pos=pos0 + t)
        np.testing.assert_allclose(ot, o[:, :, t], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(Sd, S, rtol=1e-11, atol=1e-12)


def test_gradients_with_rotation_match_finite_differences():
    c = case(8, B=1, n=7, f=4)
    r = np.random.default_rng(9)
    kk = r.random((1, 2, 3, 8))
    kk /= kk.sum(-1, keepdims=True)
    c["s_init"] = np.einsum("bhjf,bhjd->bhfd", kk, r.normal(size=(1, 2, 3, 5)))
    c["z_init"] = kk.sum(2)
    d_o = r.normal(size=c["v"].shape)
    ds, dz = r.normal(size=(1, 2, 8, 5)), r.normal(size=(1, 2, 8))
    rp = dict(rope_dims=8, rope_base=100.0, rope_pos0=np.array([11]))
    g = hm_grad.grads(**c, d_o=d_o, ds_final=ds, dz_final=dz, **rp)
    np.testing.assert_allclose(g["o"], orc.forward(**c, **rp)[0], rtol=1e-12, atol=1e-12)

    def loss(cc):
        o, S, z = orc.forward(**cc, **rp)
        return float((o * d_o).sum() + (S * ds).sum() + (z * dz).sum())

    eps = 1e-6
    for name in c:
        u = r.normal(size=c[name].shape)
        fd = (loss(dict(c, **{name: c[name] + eps * u})) - loss(dict(c, **{name: c[name] - eps * u}))) / (2 * eps)
        an = float((g[name] * u).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, fd, an)


def test_planted_rotation_mistakes_are_caught():
    # interleaved pairs (2i, 2i+1) instead of rotate-half: e_0 would move into index 1
    x = unit(4, 0)
    bad = np.array([COS100, SIN100, 0.0, 0.0])
    assert not np.allclose(orc.rope(x[None], np.array([100.0]), 4)[0], bad)
    # exponent -i/dims instead of -2i/dims: pair 1 of eight features would turn by 10^-0.5
    out = orc.rope(unit(8, 1)[None], np.array([1.0]), 8)[0]
    assert abs(np.arctan2(out[5], out[1]) - 10.0 ** -0.5) > 0.1
    # turning the other way (x1 cos + x2 sin, x2 cos - x1 sin): the sign of sin(1) flips
    out = orc.rope(unit(4, 1)[None], np.array([100.0]), 4)[0]
    assert out[3] > 0.8
