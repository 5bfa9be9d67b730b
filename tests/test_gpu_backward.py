"""GPU parity of the backward pass (hm_linattn_bwd after a training forward)
against the float64 autograd oracle (oracle/hm_grad.py, pinned by finite
differences of the numpy oracle).  Bars: rel-L2 <= 1e-5 for float32 inputs and
<= 2e-2 for bf16, per gradient; max-abs printed beside every rel-L2."""
import numpy as np
import pytest
import torch

from oracle import hm_grad, hm_oracle as orc
from selective_state_space_hm_amd import hm, inputs
import oracle_pool
from parity_util import BF16_TOL, FP32_TOL, report, to_dev, tol_for

pytestmark = pytest.mark.gpu
f64 = inputs.to_f64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hm.lib()


def run_train(c, s_init=None, segments=0, w=None, gate=None):
    g = to_dev(c)
    wq, wk = (g["w_q"], g["w_k"]) if w is None else (w[0].cuda(), w[1].cuda())
    save = torch.empty(hm.save_size(g["q"], g["v"], wq), dtype=torch.uint8, device="cuda")
    s_final = torch.empty((c.B, c.H, hm.state_numel(c.f, c.dv)), device="cuda")
    o = hm.hm_linattn_fwd(g["q"], g["k"], g["v"], wq, wk, g["dt"], g["a_log"], s_init=s_init, s_final=s_final,
                          save=save, segments=segments, gate=gate)
    return g, wq, wk, o, save, s_final


def check(name, got, ref, tol):
    got = f64(got) if torch.is_tensor(got) else got
    if np.linalg.norm(ref) < 1e-9:
        # the exact gradient is zero (e.g. one token: o_0 = v_0): bound the rounding residue
        m = float(np.max(np.abs(got))) if got.size else 0.0
        print(f"[parity] {name}: exact gradient 0, max-abs {m:.3e}", flush=True)
        assert m <= (1e-5 if tol <= FP32_TOL else 1e-2), name
        return
    r = report(name, got, ref)
    assert r <= tol, name


def check_a_log(name, got, ref, c, tol):
    """dA_log[h] sums d log a_t * log a_t over every (b, t) of head h; bound its error
    by tol times the sum of the terms' magnitudes (the bound for a sum of mixed-sign
    terms), the terms taken from the oracle: d log a_t = d dt_t / (-sigmoid(dt_t) e^{A_log})."""
    dt = f64(c.dt)
    e_a = np.exp(f64(c.a_log))[None, :, None]
    la = -orc.softplus(dt) * e_a
    dla = ref["dt"] / (-(1.0 / (1.0 + np.exp(-dt))) * e_a)
    scale = np.abs(dla * la).sum(axis=(0, 2))
    err = np.abs(f64(got) - ref["a_log"])
    nref = np.linalg.norm(ref["a_log"])
    rel = f"{np.linalg.norm(err) / nref:.3e}" if nref > 0 else "n/a (exact gradient 0)"
    print(f"[parity] {name}: |err| {err.max():.3e}  bound {(tol * scale).min():.3e}  rel {rel}", flush=True)
    assert np.all(err <= tol * scale), name


def oracle_grads(c, d_o, s_init=None, d_s_final=None, w=None, gate=None):
    F, dv = 2 * c.f, c.dv
    S0 = z0 = dS = dz = None
    if s_init is not None:
        S0, z0 = orc.unpack_state(f64(s_init), F, dv)
    if d_s_final is not None:
        dS, dz = orc.unpack_state(f64(d_s_final), F, dv)
    wq, wk = (f64(c.w_q), f64(c.w_k)) if w is None else (f64(w[0]), f64(w[1]))
    return hm_grad.grads(f64(c.q), f64(c.k), f64(c.v), wq, wk, f64(c.dt), f64(c.a_log), S0, z0, f64(d_o), dS, dz,
                         gate=f64(gate))


@pytest.mark.parametrize("n", [1, 64, 100, 200])
@pytest.mark.parametrize("decay", [None, "mild", "mamba"])
@pytest.mark.parametrize("shape", [(16, 16, 16), (32, 16, 32)])
def test_backward_fp32(n, decay, shape):
    d, f, dv = shape
    c = inputs.make_prefill("bw", 2, 2, n, d, f, dv, torch.float32, None, decay, seed=n + d)
    gen = torch.Generator().manual_seed(n)
    d_o = torch.randn((2, 2, n, dv), generator=gen)
    g, wq, wk, o, save, _ = run_train(c)
    gr = hm.hm_linattn_bwd(g["q"], g["k"], g["v"], wq, wk, d_o.cuda(), save, g["dt"], g["a_log"])
    torch.cuda.synchronize()
    ref = oracle_grads(c, d_o)
    for name in ("q", "k", "v", "w_q", "w_k") + (("dt",) if decay else ()):
        check(f"bwd fp32 {shape} n={n} decay={decay} d{name}", gr[name], ref[name], FP32_TOL)
    if decay:
        check_a_log(f"bwd fp32 {shape} n={n} decay={decay} da_log", gr["a_log"], ref, c, FP32_TOL)


@pytest.mark.parametrize("shape", [(128, 64, 128), (64, 32, 64)])
@pytest.mark.parametrize("decay", [None, "mamba"])
def test_backward_bf16_ragged(shape, decay):
    d, f, dv = shape
    c = inputs.make_prefill("bwb", 1, 2, 333, d, f, dv, torch.bfloat16, None, decay, seed=d + 7)
    d_o = torch.randn((1, 2, 333, dv), generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    g, wq, wk, o, save, _ = run_train(c)
    gr = hm.hm_linattn_bwd(g["q"], g["k"], g["v"], wq, wk, d_o.cuda(), save, g["dt"], g["a_log"])
    torch.cuda.synchronize()
    ref = oracle_grads(c, d_o)
    for name in ("q", "k", "v", "w_q", "w_k") + (("dt",) if decay else ()):
        check(f"bwd bf16 {shape} decay={decay} d{name}", gr[name], ref[name], BF16_TOL)
    if decay:
        check_a_log(f"bwd bf16 {shape} decay={decay} da_log", gr["a_log"], ref, c, BF16_TOL)


@pytest.mark.parametrize("segments", [1, 3])
def test_backward_state_gradients_fp32(segments):
    """Initial state in, dloss/ds_final in, dloss/ds_init out; a segmented training forward."""
    c = inputs.small(n=300, decay="mild", dtype=torch.float32, d=32, f=16, dv=32, B=2, H=2, seed=5)
    r = np.random.default_rng(1)
    kk = r.random((2, 2, 5, 32))
    kk /= kk.sum(-1, keepdims=True)
    S0 = np.einsum("bhjf,bhjd->bhfd", kk, r.normal(size=(2, 2, 5, 32)))
    s_init = torch.tensor(orc.pack_state(S0, kk.sum(2)), dtype=torch.float32, device="cuda")
    d_sf = torch.randn((2, 2, hm.state_numel(16, 32)), generator=torch.Generator().manual_seed(9))
    d_o = torch.randn((2, 2, 300, 32), generator=torch.Generator().manual_seed(4))
    g, wq, wk, o, save, s_final = run_train(c, s_init=s_init, segments=segments)
    gr = hm.hm_linattn_bwd(g["q"], g["k"], g["v"], wq, wk, d_o.cuda(), save, g["dt"], g["a_log"],
                           d_s_final=d_sf.cuda(), want_d_s_init=True)
    torch.cuda.synchronize()
    ref = oracle_grads(c, d_o, s_init=s_init.cpu(), d_s_final=d_sf)
    got_S, got_z = orc.unpack_state(f64(gr["s_init"]), 32, 32)
    check(f"bwd segs={segments} d s_init (S)", got_S, ref["s_init"], FP32_TOL)
    check(f"bwd segs={segments} d s_init (z)", got_z, ref["z_init"], FP32_TOL)
    for name in ("q", "k", "v", "w_q", "w_k", "dt"):
        check(f"bwd segs={segments} d{name}", gr[name], ref[name], FP32_TOL)
    check_a_log(f"bwd segs={segments} da_log", gr["a_log"], ref, c, FP32_TOL)


def test_backward_many_heads_whole_gradient_state():
    """B*H = 256: the gradient-state pass runs one workgroup per (b, h) over all
    value columns (below 256 it splits them in two); with dS_final in and
    dS_init out, so the z-gradient path is checked too."""
    c = inputs.make_prefill("bw256", 16, 16, 70, 32, 16, 32, torch.float32, None, "mild", seed=31)
    gen = torch.Generator().manual_seed(31)
    d_o = torch.randn((16, 16, 70, 32), generator=gen)
    d_sf = torch.randn((16, 16, hm.state_numel(16, 32)), generator=gen)
    s_init = torch.zeros((16, 16, hm.state_numel(16, 32)), device="cuda")  # its gradient does not depend on it
    g, wq, wk, o, save, _ = run_train(c, s_init=s_init)
    gr = hm.hm_linattn_bwd(g["q"], g["k"], g["v"], wq, wk, d_o.cuda(), save, g["dt"], g["a_log"],
                           d_s_final=d_sf.cuda(), want_d_s_init=True)
    torch.cuda.synchronize()
    ref = oracle_grads(c, d_o, s_init=s_init.cpu(), d_s_final=d_sf)
    for name in ("q", "k", "v", "w_q", "w_k", "dt"):
        check(f"bwd B*H=256 d{name}", gr[name], ref[name], FP32_TOL)
    got_S, got_z = orc.unpack_state(f64(gr["s_init"]), 32, 32)
    check("bwd B*H=256 d s_init (S)", got_S, ref["s_init"], FP32_TOL)
    check("bwd B*H=256 d s_init (z)", got_z, ref["z_init"], FP32_TOL)


def test_backward_per_head_weights_bf16():
    c = inputs.make_prefill("bwh", 2, 3, 150, 64, 32, 64, torch.bfloat16, None, "mild", seed=12)
    gen = torch.Generator().manual_seed(2)
    w = ((torch.randn((3, 64, 32), generator=gen) / 8).to(torch.bfloat16),
         (torch.randn((3, 64, 32), generator=gen) / 8).to(torch.bfloat16))
    d_o = torch.randn((2, 3, 150, 64), generator=gen).to(torch.bfloat16)
    g, wq, wk, o, save, _ = run_train(c, w=w)
    gr = hm.hm_linattn_bwd(g["q"], g["k"], g["v"], wq, wk, d_o.cuda(), save, g["dt"], g["a_log"])
    torch.cuda.synchronize()
    ref = oracle_grads(c, d_o, w=w)
    assert gr["w_q"].shape == (3, 64, 32)
    for name in ("q", "k", "v", "w_q", "w_k", "dt"):
        check(f"bwd per-head W d{name}", gr[name], ref[name], BF16_TOL)
    check_a_log("bwd per-head W da_log", gr["a_log"], ref, c, BF16_TOL)


def test_backward_empty_sequence():
    c = inputs.make_prefill("bw0", 1, 2, 0, 32, 16, 32, torch.float32, None, "mild", seed=1)
    d_sf = torch.randn((1, 2, hm.state_numel(16, 32)), generator=torch.Generator().manual_seed(1)).cuda()
    g, wq, wk, o, save, s_final = run_train(c)
    gr = hm.hm_linattn_bwd(g["q"], g["k"], g["v"], wq, wk, o, save, g["dt"], g["a_log"], d_s_final=d_sf,
                           want_d_s_init=True)
    torch.cuda.synchronize()
    assert torch.equal(gr["s_init"], d_sf)                       # no token: the gradient passes through
    assert torch.count_nonzero(gr["w_q"]) == 0 and torch.count_nonzero(gr["a_log"]) == 0


@pytest.mark.parametrize("dtype,shape", [(torch.float32, (32, 16, 32)), (torch.bfloat16, (128, 64, 128))])
def test_backward_with_gate(dtype, shape):
    """A gated training forward: d_gate out, and the core's gradients through the gate."""
    d, f, dv = shape
    c = inputs.make_prefill("bwg", 2, 2, 150, d, f, dv, dtype, None, "mild", seed=d + 40)
    gt = inputs.gate(c.v.shape, dtype, seed=4)
    d_o = torch.randn(c.v.shape, generator=torch.Generator().manual_seed(8)).to(dtype)
    g, wq, wk, o, save, _ = run_train(c, gate=gt.cuda())
    gr = hm.hm_linattn_bwd(g["q"], g["k"], g["v"], wq, wk, d_o.cuda(), save, g["dt"], g["a_log"], gate=gt.cuda())
    torch.cuda.synchronize()
    ref = oracle_grads(c, d_o, gate=gt)
    for name in ("gate", "q", "k", "v", "w_q", "w_k", "dt"):
        check(f"bwd gated {dtype} d{name}", gr[name], ref[name], tol_for(dtype))
    check_a_log(f"bwd gated {dtype} da_log", gr["a_log"], ref, c, tol_for(dtype))


@pytest.mark.parametrize("case", ["pythia1b", "decay"])
def test_backward_bf16_full_size(case):
    """bf16 gradients at the measured training shape, every head: the Pythia-1B-shaped layer
    (B=8, H=16, n=2048, identity decay: the bench's training step, a two-segment training
    forward whose slots are composed by combine_kernel) and a Mamba-decay case (B=2, H=8,
    n=2048: eight segments).  dq, dk, dv and d dt per element of every head, dW and
    dA_log (sums over every head) against the autograd oracle run head group by head group."""
    if case == "pythia1b":
        c = inputs.pythia1b()
    else:
        c = inputs.make_prefill("bw-decay", 2, 8, 2048, 128, 64, 128, torch.bfloat16, None, "mamba", seed=11)
    d_o = torch.randn(c.v.shape, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    g, wq, wk, o, save, _ = run_train(c)
    plan = hm.hm_linattn_fwd_plan(g["q"], g["k"], g["v"], wq, wk, g["dt"], g["a_log"])
    print(f"[parity] bwd bf16 full size {case}: forward plan {plan}", flush=True)
    gr = hm.hm_linattn_bwd(g["q"], g["k"], g["v"], wq, wk, d_o.cuda(), save, g["dt"], g["a_log"])
    torch.cuda.synchronize()
    ref = oracle_pool.grads_all(f64(c.q), f64(c.k), f64(c.v), f64(c.w_q), f64(c.w_k), f64(d_o), f64(c.dt),
                                f64(c.a_log))
    names = ("q", "k", "v", "w_q", "w_k") + (("dt",) if c.dt is not None else ())
    for name in names:
        check(f"bwd bf16 full size {case} d{name}", gr[name], ref[name], BF16_TOL)
    for name in ("q", "k", "v") + (("dt",) if c.dt is not None else ()):
        # every head on its own, so that no head can hide in the whole tensor's norm
        got, want = f64(gr[name]), ref[name]
        worst = max(np.linalg.norm(got[b, h] - want[b, h]) / np.linalg.norm(want[b, h])
                    for b in range(c.B) for h in range(c.H))
        print(f"[parity] bwd bf16 full size {case} d{name}: worst head rel-L2 {worst:.3e}", flush=True)
        assert worst <= BF16_TOL, name
    if c.dt is not None:
        check_a_log(f"bwd bf16 full size {case} da_log", gr["a_log"], ref, c, BF16_TOL)
