"""GPU parity of the rotary encoding of the features (HedgeMamba explainer §5.2
step 3): prefill (every plan), decode, the standalone featurizer and the backward
pass, through the C ABI, against the float64 oracles (oracle/hm_oracle.py's rope
path, oracle/hm_grad.py for gradients, both pinned in tests/test_oracle_rope.py).

Bars as elsewhere: rel-L2 <= 1e-5 for float32 inputs, <= 2e-2 for bf16; max-abs
printed beside every rel-L2.  The turned features are signed, so a denominator
can come near zero, and the output there is ill-conditioned in any arithmetic:
forward outputs are therefore checked element by element against tol times
their first-order rounding bound (see sensitivity), which equals a relative
bound where the denominator is well away from zero."""
import numpy as np
import pytest
import torch

from oracle import hm_grad, hm_oracle as orc
from selective_state_space_hm_amd import hm, inputs
from parity_util import BF16_TOL, FP32_TOL, report, to_dev, tol_for

pytestmark = pytest.mark.gpu
f64 = inputs.to_f64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hm.lib()


def positions(B, base):
    """Start position of each batch row: base, base + 1000, base + 2000, ..."""
    return torch.tensor([base + 1000 * b for b in range(B)], dtype=torch.int64)


def oracle_fwd(c, dims, base, pos0, s_init=None, z_init=None, gate=None):
    return orc.forward(f64(c.q), f64(c.k), f64(c.v), f64(c.w_q), f64(c.w_k), f64(c.dt), f64(c.a_log),
                       s_init, z_init, gate=gate, rope_dims=dims, rope_base=base,
                       rope_pos0=None if pos0 is None else pos0.numpy())


def sensitivity(c, dims, base, pos0, o_ref):
    """First-order rounding bound of each output, from the oracle's turned features:
    o_t = num_t / den_t with every product phiq_t[f] phik_j[f] v_j carried with a small
    relative error gives |d o_t| <= eps * (N_t + |o_t| D_t) / |den_t|, where
    N_t = sum_j a_tj sum_f |phiq_t[f]| |phik_j[f]| |v_j| and D_t likewise without v
    (the magnitudes the chunked sums and the carried state accumulate).  Returns the
    bound per output element (eps = 1) and the smallest den_t / D_t.  A denominator
    that comes near zero (the turned features are signed) makes that output
    ill-conditioned in any arithmetic; the bound says by how much."""
    phq = orc.hedgehog_features(f64(c.q), f64(c.w_q))
    phk = orc.hedgehog_features(f64(c.k), f64(c.w_k))
    pos = orc.rope_positions(c.B, c.n, None if pos0 is None else pos0.numpy())
    phq, phk = orc.rope(phq, pos, dims, base), orc.rope(phk, pos, dims, base)
    la = orc.log_decay(f64(c.dt), f64(c.a_log))
    v = np.abs(f64(c.v))
    bound = np.empty(o_ref.shape)
    margin = np.inf
    for b in range(c.B):
        for h in range(c.H):
            G = np.tril(np.ones((c.n, c.n))) if la is None else orc.decay_matrix(la[b, h])
            Wa = G * (np.abs(phq[b, h]) @ np.abs(phk[b, h]).T)
            den = (G * (phq[b, h] @ phk[b, h].T)).sum(1)
            D = Wa.sum(1)
            bound[b, h] = (Wa @ v[b, h] + np.abs(o_ref[b, h]) * D[:, None]) / np.abs(den)[:, None]
            margin = min(margin, float((den / D).min()))
    return bound, margin


def check_out(name, got, ref, c, dims, base, pos0, tol):
    """Every output's error within tol times its rounding bound; rel-L2 printed too."""
    bound, margin = sensitivity(c, dims, base, pos0, ref)
    got = f64(got) if torch.is_tensor(got) else got
    ratio = np.abs(got - ref) / bound
    r = report(name, got, ref)
    print(f"[parity] {name}: max |err| / bound {ratio.max():.3e}  (min den/D {margin:.3f})", flush=True)
    assert ratio.max() <= tol, name
    return r


# ------------------------------------------------------------------ prefill
@pytest.mark.parametrize("n", [1, 37, 64, 200, 333])
@pytest.mark.parametrize("decay", [None, "mamba", "mild"])
@pytest.mark.parametrize("shape", [(16, 16, 16), (32, 16, 32)])
def test_prefill_fp32(n, decay, shape):
    d, f, dv = shape
    c = inputs.make_prefill("rope", 2, 3, n, d, f, dv, torch.float32, None, decay, seed=n + d)
    pos0 = positions(2, 5)
    g = to_dev(c)
    s_final = torch.full((2, 3, hm.state_numel(f, dv)), float("nan"), device="cuda")
    o = hm.hm_linattn_fwd(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], g["dt"], g["a_log"], s_final=s_final,
                          rope_dims=32, rope_base=10000.0, rope_pos0=pos0.cuda())
    torch.cuda.synchronize()
    ref, S, z = oracle_fwd(c, 32, 10000.0, pos0)
    check_out(f"rope fp32 {shape} n={n} decay={decay} o", o, ref, c, 32, 10000.0, pos0, FP32_TOL)
    # the state is a plain sum of signed terms: its error is relative to the summed magnitudes
    assert report(f"rope fp32 {shape} n={n} decay={decay} S_final", f64(s_final), orc.pack_state(S, z)) <= FP32_TOL


@pytest.mark.parametrize("segments,dsplit", [(1, 1), (3, 1), (4, 2), (0, 0)])
def test_prefill_fp32_plans_and_state_handoff(segments, dsplit):
    """Every plan (segments scanned in parallel, value-column split) and a start
    state carried in from an earlier part of the sequence at a non-zero offset."""
    c = inputs.make_prefill("rope", 2, 2, 700, 32, 16, 32, torch.float32, None, "mild", seed=11)
    pos0 = positions(2, 123)
    g = to_dev(c)
    cut = 300
    s_mid = torch.empty((2, 2, hm.state_numel(16, 32)), device="cuda")
    o1 = hm.hm_linattn_fwd(g["q"][:, :, :cut], g["k"][:, :, :cut], g["v"][:, :, :cut], g["w_q"], g["w_k"],
                           g["dt"][:, :, :cut], g["a_log"], s_final=s_mid, rope_dims=32, rope_pos0=pos0.cuda())
    o2 = hm.hm_linattn_fwd(g["q"][:, :, cut:], g["k"][:, :, cut:], g["v"][:, :, cut:], g["w_q"], g["w_k"],
                           g["dt"][:, :, cut:], g["a_log"], s_init=s_mid, segments=segments, dsplit=dsplit,
                           rope_dims=32, rope_pos0=(pos0 + cut).cuda())
    torch.cuda.synchronize()
    ref, _, _ = oracle_fwd(c, 32, 10000.0, pos0)
    got = np.concatenate([f64(o1), f64(o2)], axis=2)
    check_out(f"rope fp32 plan segments={segments} dsplit={dsplit}", got, ref, c, 32, 10000.0, pos0, FP32_TOL)


@pytest.mark.parametrize("base_pos", [10 ** 6, 2 ** 31 + 12345])
def test_prefill_fp32_far_positions(base_pos):
    """Angles reach ~2e9 radians: the float64 reduction keeps float32 accuracy."""
    c = inputs.make_prefill("rope", 2, 2, 130, 16, 16, 16, torch.float32, None, "mamba", seed=3)
    pos0 = positions(2, base_pos)
    g = to_dev(c)
    o = hm.hm_linattn_fwd(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], g["dt"], g["a_log"],
                          rope_dims=32, rope_base=500.0, rope_pos0=pos0.cuda())
    torch.cuda.synchronize()
    ref, _, _ = oracle_fwd(c, 32, 500.0, pos0)
    check_out(f"rope fp32 positions from {base_pos}", o, ref, c, 32, 500.0, pos0, FP32_TOL)


@pytest.mark.parametrize("dims", [32, 64, 128])
@pytest.mark.parametrize("decay", [None, "mamba"])
def test_prefill_bf16(dims, decay):
    c = inputs.make_prefill("rope", 2, 4, 333, 128, 64, 128, torch.bfloat16, None, decay, seed=dims)
    pos0 = positions(2, 0)
    g = to_dev(c)
    o = hm.hm_linattn_fwd(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], g["dt"], g["a_log"],
                          rope_dims=dims, rope_pos0=pos0.cuda())
    torch.cuda.synchronize()
    ref, _, _ = oracle_fwd(c, dims, 10000.0, pos0)
    r = check_out(f"rope bf16 (128,64,128) dims={dims} decay={decay}", o, ref, c, dims, 10000.0, pos0, BF16_TOL)
    assert r <= BF16_TOL


@pytest.mark.parametrize("segments,dsplit", [(3, 1), (2, 2)])
def test_prefill_bf16_small_head_and_plans(segments, dsplit):
    c = inputs.make_prefill("rope", 2, 3, 400, 64, 32, 64, torch.bfloat16, None, "mild", seed=5)
    g = to_dev(c)
    gate = inputs.gate(c.v.shape, torch.bfloat16, seed=5)
    o = hm.hm_linattn_fwd(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], g["dt"], g["a_log"], gate=gate.cuda(),
                          segments=segments, dsplit=dsplit, rope_dims=64)
    torch.cuda.synchronize()
    ref, _, _ = oracle_fwd(c, 64, 10000.0, None, gate=f64(gate))
    assert report(f"rope bf16 (64,32,64) gated segments={segments} dsplit={dsplit}", f64(o), ref) <= BF16_TOL


# ------------------------------------------------------------------ decode
@pytest.mark.parametrize("dtype,shape", [(torch.float32, (16, 16, 16)), (torch.float32, (32, 16, 32)),
                                         (torch.bfloat16, (128, 64, 128)), (torch.bfloat16, (64, 32, 64))])
def test_decode_chain(dtype, shape):
    """Prefill a prefix, then decode step by step at per-row positions; every step
    against the oracle's step (state and output)."""
    d, f, dv = shape
    B, H, pre, steps = 3, 2, 70, 6
    dims = 2 * f if f <= 16 else f  # full rotation for the small feature maps, half for the wide
    c = inputs.make_prefill("rope", B, H, pre + steps, d, f, dv, dtype, None, "mamba", seed=d)
    pos0 = positions(B, 17)
    g = to_dev(c)
    state = torch.empty((B, H, hm.state_numel(f, dv)), device="cuda")
    hm.hm_linattn_fwd(g["q"][:, :, :pre], g["k"][:, :, :pre], g["v"][:, :, :pre], g["w_q"], g["w_k"],
                      g["dt"][:, :, :pre], g["a_log"], s_final=state, rope_dims=dims, rope_pos0=pos0.cuda())
    ref_all, _, _ = oracle_fwd(c, dims, 10000.0, pos0)
    for s in range(steps):
        t = pre + s
        pos = (pos0 + t).cuda()
        o = hm.hm_linattn_step(g["q"][:, :, t].contiguous(), g["k"][:, :, t].contiguous(),
                               g["v"][:, :, t].contiguous(), g["w_q"], g["w_k"], state,
                               g["dt"][:, :, t].contiguous(), g["a_log"], rope_dims=dims, rope_pos=pos)
        torch.cuda.synchronize()
        assert report(f"rope decode {dtype} {shape} step {s}", f64(o), ref_all[:, :, t]) <= tol_for(dtype)
    _, S, z = oracle_fwd(c, dims, 10000.0, pos0)
    assert report(f"rope decode {dtype} {shape} final state", f64(state), orc.pack_state(S, z)) <= tol_for(dtype)


# ------------------------------------------------------------------ featurize
@pytest.mark.parametrize("dtype,phi_dtype,d,f,dims", [
    (torch.float32, torch.float32, 16, 16, 32), (torch.float32, torch.float32, 64, 64, 96),
    (torch.bfloat16, torch.float32, 128, 64, 128), (torch.bfloat16, torch.bfloat16, 128, 32, 32)])
def test_featurize(dtype, phi_dtype, d, f, dims):
    c = inputs.make_prefill("feat", 2, 3, 77, d, f, 16, dtype, None, None, seed=3)
    pos0 = positions(2, 40)
    phi = hm.hm_featurize(c.q.cuda(), c.w_q.cuda(), phi_dtype=phi_dtype, rope_dims=dims, rope_base=1000.0,
                          rope_pos0=pos0.cuda())
    torch.cuda.synchronize()
    ref = orc.rope(orc.hedgehog_features(f64(c.q), f64(c.w_q)), orc.rope_positions(2, 77, pos0.numpy()), dims,
                   1000.0)
    r = report(f"rope featurize {dtype}->{phi_dtype} d={d} f={f} dims={dims}", f64(phi), ref)
    assert r <= (FP32_TOL if phi_dtype == torch.float32 else 4e-3)


# ------------------------------------------------------------------ backward
def grads_oracle(c, d_o, dims, base, pos0, s_init=None, d_s_final=None, gate=None):
    F, dv = 2 * c.f, c.dv
    S0 = z0 = dS = dz = None
    if s_init is not None:
        S0, z0 = orc.unpack_state(f64(s_init), F, dv)
    if d_s_final is not None:
        dS, dz = orc.unpack_state(f64(d_s_final), F, dv)
    return hm_grad.grads(f64(c.q), f64(c.k), f64(c.v), f64(c.w_q), f64(c.w_k), f64(c.dt), f64(c.a_log), S0, z0,
                         f64(d_o), dS, dz, gate=f64(gate), rope_dims=dims, rope_base=base,
                         rope_pos0=None if pos0 is None else pos0.numpy())


def check(name, got, ref, tol):
    r = report(name, f64(got), ref)
    assert r <= tol, name


@pytest.mark.parametrize("n,decay", [(1, None), (100, None), (100, "mamba"), (160, "mamba")])
@pytest.mark.parametrize("shape", [(16, 16, 16), (32, 16, 32)])
def test_backward_fp32(n, decay, shape):
    """Cases whose denominators stay away from zero (min den / D >= 0.15, D the
    magnitude sum of sensitivity(), checked below): gradients carry the forward's
    conditioning squared, so a near-zero denominator would measure the inputs, not
    the kernels, against the 1e-5 bar."""
    d, f, dv = shape
    c = inputs.make_prefill("bw", 2, 2, n, d, f, dv, torch.float32, None, decay, seed=n + d)
    pos0 = positions(2, 9)
    d_o = torch.randn((2, 2, n, dv), generator=torch.Generator().manual_seed(n))
    g = to_dev(c)
    save = torch.empty(hm.save_size(g["q"], g["v"], g["w_q"]), dtype=torch.uint8, device="cuda")
    rp = dict(rope_dims=32, rope_base=10000.0, rope_pos0=pos0.cuda())
    o = hm.hm_linattn_fwd(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], g["dt"], g["a_log"], save=save, **rp)
    gr = hm.hm_linattn_bwd(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], d_o.cuda(), save, g["dt"], g["a_log"], **rp)
    torch.cuda.synchronize()
    ref = grads_oracle(c, d_o, 32, 10000.0, pos0)
    if n > 1:
        _, margin = sensitivity(c, 32, 10000.0, pos0, ref["o"])
        print(f"[parity] rope bwd fp32 {shape} n={n}: min den/D {margin:.3f}", flush=True)
        assert margin >= 0.15
    assert report(f"rope train-forward fp32 {shape} n={n}", f64(o), ref["o"]) <= FP32_TOL
    if n == 1:
        # one token: o_0 = v_0 whatever the features, so only dv is non-zero
        check(f"rope bwd fp32 {shape} n=1 dv", gr["v"], ref["v"], FP32_TOL)
        for name in ("q", "k", "w_q", "w_k"):
            assert float(np.abs(f64(gr[name])).max()) <= 1e-5, name
        return
    for name in ("q", "k", "v", "w_q", "w_k") + (("dt",) if decay else ()):
        check(f"rope bwd fp32 {shape} n={n} decay={decay} d{name}", gr[name], ref[name], FP32_TOL)


@pytest.mark.parametrize("shape,dims", [((64, 32, 64), 64), ((128, 64, 128), 32), ((128, 64, 128), 128)])
def test_backward_bf16(shape, dims):
    d, f, dv = shape
    B, H, n = 2, 2, 300
    c = inputs.make_prefill("bw", B, H, n, d, f, dv, torch.bfloat16, None, "mamba", seed=dims)
    pos0 = positions(B, 0)
    d_o = torch.randn((B, H, n, dv), generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    gate = inputs.gate(c.v.shape, torch.bfloat16, seed=2)
    g = to_dev(c)
    save = torch.empty(hm.save_size(g["q"], g["v"], g["w_q"]), dtype=torch.uint8, device="cuda")
    rp = dict(rope_dims=dims, rope_pos0=pos0.cuda())
    hm.hm_linattn_fwd(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], g["dt"], g["a_log"], save=save,
                      gate=gate.cuda(), **rp)
    gr = hm.hm_linattn_bwd(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], d_o.cuda(), save, g["dt"], g["a_log"],
                           gate=gate.cuda(), **rp)
    torch.cuda.synchronize()
    ref = grads_oracle(c, d_o, dims, 10000.0, pos0, gate=gate)
    for name in ("q", "k", "v", "w_q", "w_k", "dt", "gate"):
        check(f"rope bwd bf16 {shape} dims={dims} d{name}", gr[name], ref[name], BF16_TOL)
