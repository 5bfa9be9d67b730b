"""GPU parity: the HIP path (through the C ABI) against the CPU float64 oracle.

Bars: rel-L2 <= 1e-5 for float32 inputs, <= 2e-2 for bf16 inputs with float32
accumulation; max-abs is printed beside every rel-L2.  Small cases compare every
output; the full-size workloads compare whole sampled (b, h) rows, which the
oracle computes one by one.
"""
import numpy as np
import pytest
import torch

from oracle import hm_oracle as orc
from selective_state_space_hm_amd import hm, inputs
from parity_util import (BF16_TOL, FP32_TOL, oracle_heads, rel_l2, report, run_fwd, to_dev, tol_for)

pytestmark = pytest.mark.gpu
f64 = inputs.to_f64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hm.lib()


def full_oracle(case, s_init=None, z_init=None, form="recurrent"):
    return orc.forward(f64(case.q), f64(case.k), f64(case.v), f64(case.w_q), f64(case.w_k),
                       f64(case.dt), f64(case.a_log), s_init, z_init, form=form)


# ------------------------------------------------------------------ featurize
@pytest.mark.parametrize("dtype,phi_dtype,d,f,n", [
    (torch.float32, torch.float32, 16, 16, 77), (torch.float32, torch.float32, 128, 64, 77),
    (torch.float32, torch.float32, 64, 32, 77), (torch.bfloat16, torch.bfloat16, 128, 64, 77),
    (torch.bfloat16, torch.float32, 128, 64, 77), (torch.bfloat16, torch.float32, 32, 16, 77),
    # bf16 at d = 16: one MFMA K-step padded past d
    (torch.bfloat16, torch.float32, 16, 16, 77), (torch.bfloat16, torch.bfloat16, 16, 64, 300),
    # several workgroups of four 64-token blocks, the last one ragged
    (torch.bfloat16, torch.bfloat16, 128, 64, 600), (torch.float32, torch.float32, 64, 32, 600)])
def test_featurize(dtype, phi_dtype, d, f, n):
    c = inputs.make_prefill("feat", 2, 3, n, d, f, 16, dtype, None, None, seed=3)
    phi = hm.hm_featurize(c.q.cuda(), c.w_q.cuda(), phi_dtype=phi_dtype)
    torch.cuda.synchronize()
    ref = orc.hedgehog_features(f64(c.q), f64(c.w_q))
    got = f64(phi)
    r = report(f"featurize {dtype} -> {phi_dtype} d={d} f={f} n={n}", got, ref)
    # float32 output: the float32 softmax itself; bf16 output adds one rounding (2^-9)
    assert r <= (FP32_TOL if phi_dtype == torch.float32 else 4e-3)
    np.testing.assert_allclose(got.sum(-1), 1.0, rtol=0, atol=1e-5 if phi_dtype == torch.float32 else 2e-2)
    assert np.all(got >= 0)


def test_featurize_per_head_weights_and_strides():
    c = inputs.make_prefill("feat", 2, 3, 70, 64, 32, 16, torch.float32, None, None, seed=4)
    wh = torch.randn((3, 64, 32), generator=torch.Generator().manual_seed(9)) / 8
    x = c.q.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)  # [B, H, n, d] view of [B, n, H, d]
    phi = hm.hm_featurize(x.cuda(), wh.cuda())
    torch.cuda.synchronize()
    ref = orc.hedgehog_features(f64(c.q), f64(wh))
    assert report("featurize per-head W, strided x", f64(phi), ref) <= FP32_TOL


# ------------------------------------------------------------------ prefill
def test_tiny_fp32_config():
    """B=1, H=2, n=256, d=16, f=16, fp32, a_t = 1: against both oracle forms."""
    c = inputs.tiny()
    o = run_fwd(c)
    torch.cuda.synchronize()
    oq, _, _ = full_oracle(c, form="quadratic")
    orr, _, _ = full_oracle(c)
    assert report("tiny fp32 vs quadratic", f64(o), oq) <= FP32_TOL
    assert report("tiny fp32 vs recurrent", f64(o), orr) <= FP32_TOL


@pytest.mark.parametrize("n", [1, 5, 37, 64, 65, 200, 333])
@pytest.mark.parametrize("decay", [None, "mamba", "mild"])
def test_small_fp32_ragged(n, decay):
    c = inputs.small(n=n, decay=decay, dtype=torch.float32, d=16, f=16, dv=16, B=2, H=3, seed=n)
    s_final = torch.full((2, 3, hm.state_numel(16, 16)), float("nan"), device="cuda")
    o = run_fwd(c, s_final=s_final)
    torch.cuda.synchronize()
    ref, S, z = full_oracle(c)
    assert report(f"fp32 n={n} decay={decay}", f64(o), ref) <= FP32_TOL
    Sg, zg = orc.unpack_state(f64(s_final), 32, 16)
    assert rel_l2(Sg, S) <= FP32_TOL and rel_l2(zg, z) <= FP32_TOL


@pytest.mark.parametrize("dv", [16, 32])
@pytest.mark.parametrize("segments,dsplit", [(1, 1), (2, 1), (3, 1), (1, 2), (2, 2), (4, 2)])
def test_fp32_plans_with_initial_state(dv, segments, dsplit):
    if dsplit == 2 and dv == 16:
        pytest.skip("dv=16 has one value tile")
    c = inputs.small(n=300, decay="mild", dtype=torch.float32, d=32, f=16, dv=dv, B=2, H=2, seed=11)
    r = np.random.default_rng(5)
    kk = r.random((2, 2, 9, 32))
    kk /= kk.sum(-1, keepdims=True)
    S0 = np.einsum("bhjf,bhjd->bhfd", kk, r.normal(size=(2, 2, 9, dv)))
    z0 = kk.sum(2)
    s_init = torch.tensor(orc.pack_state(S0, z0), dtype=torch.float32, device="cuda")
    s_final = torch.empty_like(s_init)
    o = run_fwd(c, s_init=s_init, s_final=s_final, segments=segments, dsplit=dsplit)
    torch.cuda.synchronize()
    ref, S, z = full_oracle(c, S0, z0)
    assert report(f"fp32 dv={dv} segs={segments} dsplit={dsplit} +S_init", f64(o), ref) <= FP32_TOL
    Sg, zg = orc.unpack_state(f64(s_final), 32, dv)
    assert rel_l2(Sg, S) <= FP32_TOL and rel_l2(zg, z) <= FP32_TOL


@pytest.mark.parametrize("f,dv", [(16, 16), (16, 32), (32, 32), (32, 64)])
@pytest.mark.parametrize("segments,dsplit", [(1, 1), (3, 1), (2, 2)])
def test_fp32_d64(f, dv, segments, dsplit):
    """float32 at d = 64: ragged n (five chunks and a tail), Mamba decay, a non-zero
    initial state, segmented and column-split plans, against the oracle (output and
    final state).  Column halves exist where the half width is built."""
    if dsplit == 2 and (f, dv) not in ((16, 32), (32, 64)):
        pytest.skip("no float32 d=64 kernel at half this width")
    c = inputs.small(n=333, decay="mamba", dtype=torch.float32, d=64, f=f, dv=dv, B=2, H=2, seed=f + dv)
    F = 2 * f
    r = np.random.default_rng(7)
    kk = r.random((2, 2, 9, F))
    kk /= kk.sum(-1, keepdims=True)
    S0 = np.einsum("bhjf,bhjd->bhfd", kk, r.normal(size=(2, 2, 9, dv)))
    z0 = kk.sum(2)
    s_init = torch.tensor(orc.pack_state(S0, z0), dtype=torch.float32, device="cuda")
    s_final = torch.empty_like(s_init)
    o = run_fwd(c, s_init=s_init, s_final=s_final, segments=segments, dsplit=dsplit)
    torch.cuda.synchronize()
    ref, S, z = full_oracle(c, S0, z0)
    assert report(f"fp32 d=64 f={f} dv={dv} segs={segments} dsplit={dsplit}", f64(o), ref) <= FP32_TOL
    Sg, zg = orc.unpack_state(f64(s_final), F, dv)
    assert rel_l2(Sg, S) <= FP32_TOL and rel_l2(zg, z) <= FP32_TOL


@pytest.mark.parametrize("decay", ["mild", "mamba"])
@pytest.mark.parametrize("segments,dsplit", [(2, 1), (2, 2), (4, 1), (3, 1)])
def test_fp32_segment_pass_slots(decay, segments, dsplit):
    """n = 500 (8 chunks, ragged tail), B*H = 4: with 2 segments of 4 chunks the
    segment pass cuts segment 0 into 4 one-chunk slots and the full pass composes
    them while loading its start state; with 4 segments of 2 chunks it cuts each
    into 2 slots and the combine pass composes all 6; 3 segments of 3 chunks stay
    whole.  Against the oracle, from a non-zero initial state."""
    c = inputs.small(n=500, decay=decay, dtype=torch.float32, d=32, f=16, dv=32, B=2, H=2, seed=21)
    r = np.random.default_rng(6)
    kk = r.random((2, 2, 9, 32))
    kk /= kk.sum(-1, keepdims=True)
    S0 = np.einsum("bhjf,bhjd->bhfd", kk, r.normal(size=(2, 2, 9, 32)))
    z0 = kk.sum(2)
    s_init = torch.tensor(orc.pack_state(S0, z0), dtype=torch.float32, device="cuda")
    s_final = torch.empty_like(s_init)
    o = run_fwd(c, s_init=s_init, s_final=s_final, segments=segments, dsplit=dsplit)
    torch.cuda.synchronize()
    ref, S, z = full_oracle(c, S0, z0)
    assert report(f"fp32 slots decay={decay} segs={segments} dsplit={dsplit}", f64(o), ref) <= FP32_TOL
    Sg, zg = orc.unpack_state(f64(s_final), 32, 32)
    assert rel_l2(Sg, S) <= FP32_TOL and rel_l2(zg, z) <= FP32_TOL


@pytest.mark.parametrize("shape", [(64, 32, 64), (128, 64, 128), (128, 32, 64), (64, 64, 128), (32, 16, 32),
                                   (64, 32, 32), (128, 64, 32), (32, 16, 64)])
@pytest.mark.parametrize("decay", [None, "mild", "mamba"])
def test_bf16_shapes_ragged(shape, decay):
    d, f, dv = shape
    c = inputs.make_prefill("bf16", 2, 3, 333, d, f, dv, torch.bfloat16, None, decay, seed=d + f)
    s_final = torch.empty((2, 3, hm.state_numel(f, dv)), device="cuda")
    o = run_fwd(c, s_final=s_final)
    torch.cuda.synchronize()
    ref, S, z = full_oracle(c)
    assert report(f"bf16 d={d} f={f} dv={dv} decay={decay}", f64(o), ref) <= BF16_TOL
    Sg, zg = orc.unpack_state(f64(s_final), 2 * f, dv)
    assert report("  state S", Sg, S) <= BF16_TOL
    assert rel_l2(zg, z) <= BF16_TOL


@pytest.mark.parametrize("segments,dsplit", [(1, 1), (1, 2), (2, 1), (5, 2), (16, 2)])
def test_bf16_segment_and_split_invariance(segments, dsplit):
    c = inputs.mild_decay(n=2000, B=1)
    o = run_fwd(c, segments=segments, dsplit=dsplit)
    o_ref = run_fwd(c, segments=1, dsplit=1)
    torch.cuda.synchronize()
    heads = [(0, 0), (0, 7), (0, 15)]
    ref, _, _ = oracle_heads(c, heads)
    got = f64(o)[[0, 0, 0], [0, 7, 15]]
    assert report(f"mild n=2000 segs={segments} dsplit={dsplit}", got, ref) <= BF16_TOL
    # different plans only reorder float32 sums
    assert rel_l2(f64(o), f64(o_ref)) <= 5e-3


def test_deterministic_bitwise():
    c = inputs.mamba_decay(n=1000, B=1)
    a = run_fwd(c, segments=3, dsplit=2)
    b = run_fwd(c, segments=3, dsplit=2)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_outputs_are_convex_combinations():
    c = inputs.make_prefill("cvx", 1, 4, 500, 128, 64, 128, torch.bfloat16, None, "mild", seed=2)
    o = f64(run_fwd(c))
    v = f64(c.v)
    lo = np.minimum.accumulate(v, axis=2)
    hi = np.maximum.accumulate(v, axis=2)
    slack = 1e-2 * (hi - lo) + 1e-2
    assert np.all(o >= lo - slack) and np.all(o <= hi + slack)
    np.testing.assert_allclose(o[:, :, 0], v[:, :, 0], rtol=0, atol=1e-2)  # o_0 = v_0


def test_per_head_weights_and_strided_layout():
    B, H, n, d, f = 2, 4, 150, 64, 32
    c = inputs.make_prefill("ph", B, H, n, d, f, 64, torch.bfloat16, None, "mild", seed=8)
    gw = torch.Generator().manual_seed(3)
    wq = (torch.randn((H, d, f), generator=gw) / 8).to(torch.bfloat16)
    wk = (torch.randn((H, d, f), generator=gw) / 8).to(torch.bfloat16)
    # q, k, v handed over as [B, n, H, d] memory (the mixer's layout), viewed as [B, H, n, d]
    tr = lambda t: t.permute(0, 2, 1, 3).contiguous().cuda().permute(0, 2, 1, 3)
    o = hm.hm_linattn_fwd(tr(c.q), tr(c.k), tr(c.v), wq.cuda(), wk.cuda(), c.dt.cuda(), c.a_log.cuda())
    torch.cuda.synchronize()
    ref, _, _ = orc.forward(f64(c.q), f64(c.k), f64(c.v), f64(wq), f64(wk), f64(c.dt), f64(c.a_log))
    assert report("per-head W, [B,n,H,d] layout", f64(o), ref) <= BF16_TOL


def test_empty_sequence_copies_initial_state():
    c = inputs.make_prefill("e", 1, 2, 0, 64, 32, 64, torch.bfloat16, None, "mamba", seed=1)
    s_init = torch.randn((1, 2, hm.state_numel(32, 64)), device="cuda").abs()
    s_final = torch.zeros_like(s_init)
    o = run_fwd(c, s_init=s_init, s_final=s_final)
    torch.cuda.synchronize()
    assert o.numel() == 0
    assert torch.equal(s_final, s_init)
    s_final.zero_()
    run_fwd(c, s_final=s_final)          # no initial state: zeros
    torch.cuda.synchronize()
    assert torch.count_nonzero(s_final) == 0


@pytest.mark.parametrize("segments,dsplit", [(1, 1), (1, 2), (2, 1), (3, 2)])
def test_split_handoff_with_aliased_state(segments, dsplit):
    """fwd[0,n) == fwd[0,m) -> state -> fwd[m,n), with s_init and s_final the same buffer."""
    c = inputs.make_prefill("h", 1, 2, 700, 128, 64, 128, torch.bfloat16, None, "mild", seed=6)
    m = 260
    g = to_dev(c)
    st = torch.empty((1, 2, hm.state_numel(64, 128)), device="cuda")
    sl = lambda t, a, b: None if t is None else t[:, :, a:b]
    o1 = hm.hm_linattn_fwd(sl(g["q"], 0, m), sl(g["k"], 0, m), sl(g["v"], 0, m), g["w_q"], g["w_k"],
                           sl(g["dt"], 0, m), g["a_log"], s_final=st)
    o2 = hm.hm_linattn_fwd(sl(g["q"], m, 700), sl(g["k"], m, 700), sl(g["v"], m, 700), g["w_q"], g["w_k"],
                           sl(g["dt"], m, 700), g["a_log"], s_init=st, s_final=st, segments=segments, dsplit=dsplit)
    torch.cuda.synchronize()
    ref, S, z = full_oracle(c)
    got = np.concatenate([f64(o1), f64(o2)], axis=2)
    assert report(f"handoff aliased segs={segments} dsplit={dsplit}", got, ref) <= BF16_TOL
    Sg, zg = orc.unpack_state(f64(st), 128, 128)
    assert rel_l2(Sg, S) <= BF16_TOL and rel_l2(zg, z) <= BF16_TOL


# ------------------------------------------------------------------ decode
@pytest.mark.parametrize("dtype,shape", [(torch.float32, (16, 16, 16)), (torch.float32, (32, 16, 32)),
                                         (torch.float32, (64, 32, 64)), (torch.float32, (64, 16, 16)),
                                         (torch.bfloat16, (128, 64, 128)), (torch.bfloat16, (64, 32, 64)),
                                         (torch.bfloat16, (32, 16, 32)), (torch.bfloat16, (128, 64, 32))])
@pytest.mark.parametrize("decay", [True, False])
@pytest.mark.parametrize("per_head", [False, True])
def test_decode_steps(dtype, shape, decay, per_head):
    d, f, dv = shape
    B, H, steps = 3, 2, 40
    dc = inputs.decode_setup(B, H, d, f, dv, prefix=50, steps=steps, decay=decay, dtype=dtype, seed=d)
    if per_head:
        # one W per head ([H, d, f]): the decode step stages each head's own W
        gw = torch.Generator().manual_seed(77)
        dc.w_q = (torch.randn((H, d, f), generator=gw) / d ** 0.5).to(dtype)
        dc.w_k = (torch.randn((H, d, f), generator=gw) / d ** 0.5).to(dtype)
    pk = orc.hedgehog_features(f64(dc.prefix_k), f64(dc.w_k))
    la = orc.log_decay(f64(dc.prefix_dt), f64(dc.a_log)) if decay else None
    S, z = orc.prefix_state(pk, f64(dc.prefix_v), la)
    state = torch.tensor(orc.pack_state(S, z), dtype=torch.float32, device="cuda")
    wq, wk = dc.w_q.cuda(), dc.w_k.cuda()
    a_log = dc.a_log.cuda() if decay else None
    worst = 0.0
    for t in range(steps):
        q, k, v, dt = inputs.decode_step_inputs(dc, t, dtype)
        o = hm.hm_linattn_step(q.cuda(), k.cuda(), v.cuda(), wq, wk, state, dt.cuda() if decay else None, a_log)
        torch.cuda.synchronize()
        ot, S, z = orc.step(S, z, f64(q), f64(k), f64(v), f64(dc.w_q), f64(dc.w_k),
                            f64(dt) if decay else None, f64(dc.a_log) if decay else None)
        worst = max(worst, rel_l2(f64(o), ot))
    Sg, zg = orc.unpack_state(f64(state), 2 * f, dv)
    print(f"[parity] decode {dtype} {shape} decay={decay} per_head={per_head}: worst step rel-L2 {worst:.3e}, "
          f"state rel-L2 {rel_l2(Sg, S):.3e}", flush=True)
    assert worst <= tol_for(dtype)
    assert rel_l2(Sg, S) <= (1e-6 if dtype == torch.float32 else 1e-5)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("f", [16, 32, 64])
@pytest.mark.parametrize("dv", [16, 32, 64, 128])
def test_decode_size_matrix(dtype, d, f, dv):
    """Every (dtype, d, f, dv) of the size matrix: 6 decayed steps from a 30-token
    prefix state, each step's output and the final state against the oracle."""
    B, H, steps = 2, 2, 6
    dc = inputs.decode_setup(B, H, d, f, dv, prefix=30, steps=steps, decay=True, dtype=dtype, seed=d + f + dv)
    pk = orc.hedgehog_features(f64(dc.prefix_k), f64(dc.w_k))
    S, z = orc.prefix_state(pk, f64(dc.prefix_v), orc.log_decay(f64(dc.prefix_dt), f64(dc.a_log)))
    state = torch.tensor(orc.pack_state(S, z), dtype=torch.float32, device="cuda")
    wq, wk, a_log = dc.w_q.cuda(), dc.w_k.cuda(), dc.a_log.cuda()
    worst = 0.0
    for t in range(steps):
        q, k, v, dt = inputs.decode_step_inputs(dc, t, dtype)
        o = hm.hm_linattn_step(q.cuda(), k.cuda(), v.cuda(), wq, wk, state, dt.cuda(), a_log)
        torch.cuda.synchronize()
        ot, S, z = orc.step(S, z, f64(q), f64(k), f64(v), f64(dc.w_q), f64(dc.w_k), f64(dt), f64(dc.a_log))
        worst = max(worst, rel_l2(f64(o), ot))
    Sg, zg = orc.unpack_state(f64(state), 2 * f, dv)
    print(f"[parity] decode {dtype} ({d}, {f}, {dv}): worst step rel-L2 {worst:.3e}, state rel-L2 "
          f"{rel_l2(Sg, S):.3e}", flush=True)
    assert worst <= tol_for(dtype)
    assert rel_l2(Sg, S) <= (1e-6 if dtype == torch.float32 else 1e-5)
    assert rel_l2(zg, z) <= (1e-6 if dtype == torch.float32 else 1e-5)


def test_prefill_then_decode_handoff():
    c = inputs.make_prefill("pd", 2, 2, 300, 128, 64, 128, torch.bfloat16, None, "mamba", seed=12)
    st = torch.empty((2, 2, hm.state_numel(64, 128)), device="cuda")
    run_fwd(c, s_final=st)
    _, S, z = full_oracle(c)
    g = torch.Generator().manual_seed(2)
    for t in range(5):
        q, k, v = (torch.randn((2, 2, 128), generator=g).to(torch.bfloat16) for _ in range(3))
        dt = torch.randn((2, 2), generator=g)
        o = hm.hm_linattn_step(q.cuda(), k.cuda(), v.cuda(), c.w_q.cuda(), c.w_k.cuda(), st, dt.cuda(), c.a_log.cuda())
        torch.cuda.synchronize()
        ot, S, z = orc.step(S, z, f64(q), f64(k), f64(v), f64(c.w_q), f64(c.w_k), f64(dt), f64(c.a_log))
        assert report(f"prefill->decode step {t}", f64(o), ot) <= BF16_TOL


# ------------------------------------------------------------------ gate branch
def gated_oracle(case, gate, s_init=None, z_init=None):
    return orc.forward(f64(case.q), f64(case.k), f64(case.v), f64(case.w_q), f64(case.w_k),
                       f64(case.dt), f64(case.a_log), s_init, z_init, gate=f64(gate))


@pytest.mark.parametrize("n", [1, 63, 200])
@pytest.mark.parametrize("segments,dsplit", [(1, 1), (3, 1), (2, 2)])
def test_gate_fp32(n, segments, dsplit):
    c = inputs.small(n=n, decay="mild", dtype=torch.float32, d=32, f=16, dv=32, B=2, H=3, seed=n + 1)
    gt = inputs.gate(c.v.shape, torch.float32, seed=n)
    s_final = torch.empty((2, 3, hm.state_numel(16, 32)), device="cuda")
    o = run_fwd(c, s_final=s_final, gate=gt.cuda(), segments=segments, dsplit=dsplit)
    o_plain = run_fwd(c, segments=segments, dsplit=dsplit)
    torch.cuda.synchronize()
    ref, S, z = gated_oracle(c, gt)
    assert report(f"gate fp32 n={n} segs={segments} dsplit={dsplit}", f64(o), ref) <= FP32_TOL
    # the gate touches only the output: the state is the ungated one
    Sg, zg = orc.unpack_state(f64(s_final), 32, 32)
    assert rel_l2(Sg, S) <= FP32_TOL and rel_l2(zg, z) <= FP32_TOL
    # and the gated output is the ungated one times SiLU(g), element by element
    np.testing.assert_allclose(f64(o), f64(o_plain) * orc.silu(f64(gt)), rtol=2e-6, atol=1e-7)


@pytest.mark.parametrize("shape", [(128, 64, 128), (64, 32, 64)])
@pytest.mark.parametrize("decay", [None, "mamba"])
def test_gate_bf16_ragged(shape, decay):
    d, f, dv = shape
    c = inputs.make_prefill("gb", 2, 3, 333, d, f, dv, torch.bfloat16, None, decay, seed=d + 3)
    gt = inputs.gate(c.v.shape, torch.bfloat16, seed=d)
    o = run_fwd(c, gate=gt.cuda())
    torch.cuda.synchronize()
    ref, _, _ = gated_oracle(c, gt)
    assert report(f"gate bf16 d={d} f={f} dv={dv} decay={decay}", f64(o), ref) <= BF16_TOL


def test_gate_strided_and_extreme():
    """A gate handed over in [B, n, H, dv] memory, with saturating values (|g| up to 60)."""
    c = inputs.make_prefill("gs", 2, 4, 150, 128, 64, 128, torch.bfloat16, None, "mild", seed=21)
    gt = inputs.gate(c.v.shape, torch.float32, seed=5, std=20.0).to(torch.bfloat16)
    gdev = gt.permute(0, 2, 1, 3).contiguous().cuda().permute(0, 2, 1, 3)
    o = run_fwd(c, gate=gdev, segments=2, dsplit=2)
    torch.cuda.synchronize()
    ref, _, _ = gated_oracle(c, gt)
    assert np.all(np.isfinite(f64(o)))
    assert report("gate bf16 strided, std 20", f64(o), ref) <= BF16_TOL


@pytest.mark.parametrize("dtype,shape", [(torch.float32, (32, 16, 32)), (torch.bfloat16, (128, 64, 128))])
def test_gate_decode_steps(dtype, shape):
    d, f, dv = shape
    B, H, steps = 3, 2, 12
    dc = inputs.decode_setup(B, H, d, f, dv, prefix=40, steps=steps, decay=True, dtype=dtype, seed=d + 1)
    pk = orc.hedgehog_features(f64(dc.prefix_k), f64(dc.w_k))
    S, z = orc.prefix_state(pk, f64(dc.prefix_v), orc.log_decay(f64(dc.prefix_dt), f64(dc.a_log)))
    state = torch.tensor(orc.pack_state(S, z), dtype=torch.float32, device="cuda")
    wq, wk, a_log = dc.w_q.cuda(), dc.w_k.cuda(), dc.a_log.cuda()
    worst = 0.0
    for t in range(steps):
        q, k, v, dt = inputs.decode_step_inputs(dc, t, dtype)
        gt = inputs.gate(v.shape, dtype, seed=100 + t)
        o = hm.hm_linattn_step(q.cuda(), k.cuda(), v.cuda(), wq, wk, state, dt.cuda(), a_log, gate=gt.cuda())
        torch.cuda.synchronize()
        ot, S, z = orc.step(S, z, f64(q), f64(k), f64(v), f64(dc.w_q), f64(dc.w_k), f64(dt), f64(dc.a_log),
                            gate=f64(gt))
        worst = max(worst, rel_l2(f64(o), ot))
    print(f"[parity] gated decode {dtype} {shape}: worst step rel-L2 {worst:.3e}", flush=True)
    assert worst <= tol_for(dtype)
    Sg, _ = orc.unpack_state(f64(state), 2 * f, dv)
    assert rel_l2(Sg, S) <= (1e-6 if dtype == torch.float32 else 1e-5)


# ------------------------------------------------------------------ short causal conv
def conv_inputs(B, H, n, d, K, dtype, seed, per_head=False, with_prev=True):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((B, H, n, d), generator=g).to(dtype)
    w = torch.randn(((H, d, K) if per_head else (d, K)), generator=g) / K
    bias = torch.randn(((H, d) if per_head else (d,)), generator=g) / 4
    prev = torch.randn((B, H, K - 1, d), generator=g).to(dtype) if with_prev and K > 1 else None
    return x, w, bias, prev


def check_conv(got, ref, dtype, name):
    r = report(name, got, ref)
    if dtype == torch.float32:
        assert r <= FP32_TOL
    else:
        # one rounding of a float32 sum to bf16: within 2^-8 relative of the exact value
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("n", [1, 15, 16, 17, 100])
def test_conv_against_oracle(dtype, K, n):
    x, w, bias, prev = conv_inputs(2, 3, n, 64, K, dtype, seed=10 * K + n, per_head=(n % 2 == 1))
    fin = torch.full((2, 3, K - 1, 64), float("nan"), dtype=dtype, device="cuda") if K > 1 else None
    y = hm.hm_causal_conv(x.cuda(), w.cuda(), bias.cuda(), None if prev is None else prev.cuda(), fin)
    torch.cuda.synchronize()
    ref, rfin = orc.causal_conv(f64(x), f64(w), f64(bias), f64(prev))
    check_conv(f64(y), ref, dtype, f"conv {dtype} K={K} n={n}")
    if K > 1:
        assert np.array_equal(f64(fin), rfin)          # rows are copied, bit for bit


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_conv_identity_init_is_exact(dtype):
    x, _, _, _ = conv_inputs(2, 4, 70, 128, 4, dtype, seed=3)
    w = torch.zeros((128, 4))
    w[:, 3] = 1.0
    y = hm.hm_causal_conv(x.cuda(), w.cuda(), torch.zeros(128).cuda())
    torch.cuda.synchronize()
    assert torch.equal(y.cpu(), x)


def test_conv_decode_in_place_matches_prefill():
    """n=1 steps with prev and final_rows the same buffer reproduce one long call."""
    B, H, n, d, K = 3, 2, 40, 128, 4
    x, w, bias, prev = conv_inputs(B, H, n, d, K, torch.bfloat16, seed=8)
    xd, wd, bd = x.cuda(), w.cuda(), bias.cuda()
    y_all = hm.hm_causal_conv(xd, wd, bd, prev.cuda())
    state = prev.cuda().clone()
    ys = []
    for t in range(n):
        ys.append(hm.hm_causal_conv(xd[:, :, t:t + 1], wd, bd, state, state))
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(ys, dim=2), y_all)
    assert torch.equal(state.cpu(), x[:, :, n - 3:])
    # split handoff through a separate final buffer, n = 0 call included
    fin = torch.empty_like(state)
    y1 = hm.hm_causal_conv(xd[:, :, :23], wd, bd, prev.cuda(), fin)
    fin0 = torch.empty_like(state)
    hm.hm_causal_conv(xd[:, :, 23:23], wd, bd, fin, fin0)
    y2 = hm.hm_causal_conv(xd[:, :, 23:], wd, bd, fin0)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([y1, y2], dim=2), y_all)


def test_conv_full_size_strided():
    """q of the B=8 H=16 n=2048 d=128 layer in [B, n, H, d] memory, per-head taps."""
    c = inputs.pythia1b()
    g = torch.Generator().manual_seed(4)
    w = torch.randn((16, 128, 4), generator=g) / 2
    bias = torch.randn((16, 128), generator=g) / 4
    xs = c.q.permute(0, 2, 1, 3).contiguous().cuda().permute(0, 2, 1, 3)
    fin = torch.empty((8, 16, 3, 128), dtype=torch.bfloat16, device="cuda")
    y = hm.hm_causal_conv(xs, w.cuda(), bias.cuda(), None, fin)
    torch.cuda.synchronize()
    ref, rfin = orc.causal_conv(f64(c.q), f64(w), f64(bias))
    check_conv(f64(y), ref, torch.bfloat16, "conv full size, [B,n,H,d] layout")
    assert np.array_equal(f64(fin), rfin)


def test_mixer_path_conv_then_gated_attention():
    """conv(q), conv(k) -> prefill with the gate, against the oracle's same chain."""
    c = inputs.make_prefill("mx", 2, 3, 200, 128, 64, 128, torch.bfloat16, None, "mamba", seed=31)
    g = torch.Generator().manual_seed(6)
    wq, wk = torch.randn((128, 4), generator=g) / 2, torch.randn((128, 4), generator=g) / 2
    gt = inputs.gate(c.v.shape, torch.bfloat16, seed=31)
    d = to_dev(c)
    qc = hm.hm_causal_conv(d["q"], wq.cuda())
    kc = hm.hm_causal_conv(d["k"], wk.cuda())
    o = hm.hm_linattn_fwd(qc, kc, d["v"], d["w_q"], d["w_k"], d["dt"], d["a_log"], gate=gt.cuda())
    torch.cuda.synchronize()
    qr, _ = orc.causal_conv(f64(c.q), f64(wq))
    kr, _ = orc.causal_conv(f64(c.k), f64(wk))
    ref, _, _ = orc.forward(qr, kr, f64(c.v), f64(c.w_q), f64(c.w_k), f64(c.dt), f64(c.a_log), gate=f64(gt))
    assert report("mixer path: conv + gated attention", f64(o), ref) <= BF16_TOL


@pytest.mark.parametrize("dtype,shape", [(torch.float32, (32, 16, 32)), (torch.bfloat16, (128, 64, 128))])
@pytest.mark.parametrize("K", [2, 4])
def test_decode_step_with_fused_conv(dtype, shape, K):
    """The step's fused conv equals hm_causal_conv (n = 1) followed by a plain step,
    bit for bit, and both follow the oracle's conv -> step chain."""
    d, f, dv = shape
    B, H, steps = 3, 2, 6
    dc = inputs.decode_setup(B, H, d, f, dv, prefix=30, steps=steps, decay=True, dtype=dtype, seed=K + d)
    pk = orc.hedgehog_features(f64(dc.prefix_k), f64(dc.w_k))
    S, z = orc.prefix_state(pk, f64(dc.prefix_v), orc.log_decay(f64(dc.prefix_dt), f64(dc.a_log)))
    st_a = torch.tensor(orc.pack_state(S, z), dtype=torch.float32, device="cuda")
    st_b = st_a.clone()
    g = torch.Generator().manual_seed(K)
    cwq, cwk = torch.randn((H, d, K), generator=g) / 2, torch.randn((H, d, K), generator=g) / 2
    cbq, cbk = torch.randn((H, d), generator=g) / 4, torch.randn((H, d), generator=g) / 4
    sq = torch.randn((B, H, K - 1, d), generator=g).to(dtype)
    sk = torch.randn((B, H, K - 1, d), generator=g).to(dtype)
    dev = [t.cuda() for t in (cwq, cwk, cbq, cbk)]
    sq_a, sk_a, sq_b, sk_b = sq.cuda(), sk.cuda(), sq.cuda(), sk.cuda()
    wq, wk, a_log = dc.w_q.cuda(), dc.w_k.cuda(), dc.a_log.cuda()
    prev_q, prev_k = f64(sq), f64(sk)
    worst = 0.0
    for t in range(steps):
        q, k, v, dt = inputs.decode_step_inputs(dc, t, dtype)
        qd, kd, vd, dtd = q.cuda(), k.cuda(), v.cuda(), dt.cuda()
        oa = hm.hm_linattn_step(qd, kd, vd, wq, wk, st_a, dtd, a_log, conv=(*dev, sq_a, sk_a))
        qc = hm.hm_causal_conv(qd[:, :, None], dev[0], dev[2], sq_b, sq_b)[:, :, 0]
        kc = hm.hm_causal_conv(kd[:, :, None], dev[1], dev[3], sk_b, sk_b)[:, :, 0]
        ob = hm.hm_linattn_step(qc, kc, vd, wq, wk, st_b, dtd, a_log)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob) and torch.equal(st_a, st_b)
        assert torch.equal(sq_a, sq_b) and torch.equal(sk_a, sk_b)
        qr, prev_q = orc.causal_conv(f64(q)[:, :, None], f64(cwq), f64(cbq), prev_q)
        kr, prev_k = orc.causal_conv(f64(k)[:, :, None], f64(cwk), f64(cbk), prev_k)
        ot, S, z = orc.step(S, z, qr[:, :, 0], kr[:, :, 0], f64(v), f64(dc.w_q), f64(dc.w_k), f64(dt), f64(dc.a_log))
        worst = max(worst, rel_l2(f64(oa), ot))
    print(f"[parity] decode + fused conv {dtype} {shape} K={K}: worst step rel-L2 {worst:.3e}", flush=True)
    assert worst <= tol_for(dtype)
    assert np.array_equal(f64(sq_a), prev_q) and np.array_equal(f64(sk_a), prev_k)


@pytest.mark.parametrize("dtype,d,f", [(torch.bfloat16, 128, 64), (torch.bfloat16, 16, 16), (torch.float32, 64, 32)])
@pytest.mark.parametrize("K", [1, 2, 4])
@pytest.mark.parametrize("with_prev", [False, True])
def test_featurize_with_fused_conv(dtype, d, f, K, with_prev):
    """hm_featurize with the short causal conv in its load prologue equals hm_causal_conv
    followed by hm_featurize bit for bit (same operation order and rounding), and the
    oracle's conv and features to the dtype's bar; per-head taps and bias, ragged n."""
    B, H, n = 2, 3, 300
    gen = torch.Generator().manual_seed(K * 7 + d + int(with_prev))
    x = torch.randn((B, H, n, d), generator=gen).to(dtype)
    w = (torch.randn((d, f), generator=gen) / d ** 0.5).to(dtype)
    cw = (torch.randn((H, d, K), generator=gen) * 0.6).float()
    cb = (torch.randn((H, d), generator=gen) * 0.1).float()
    prev = torch.randn((B, H, K - 1, d), generator=gen).to(dtype) if with_prev and K > 1 else None
    xd, wd, cwd, cbd = x.cuda(), w.cuda(), cw.cuda(), cb.cuda()
    pd = None if prev is None else prev.cuda()
    fused = hm.hm_featurize(xd, wd, conv_w=cwd, conv_b=cbd, conv_prev=pd)
    y = hm.hm_causal_conv(xd, cwd, cbd, pd)
    sep = hm.hm_featurize(y, wd)
    torch.cuda.synchronize()
    assert torch.equal(fused, sep), "fused conv + featurize differs from conv then featurize"
    yr, _ = orc.causal_conv(f64(x), f64(cw), f64(cb), None if prev is None else f64(prev))
    yr = f64(torch.tensor(yr).to(dtype))  # the conv output rounded as it is stored
    ref = orc.hedgehog_features(yr, f64(w))
    r = report(f"featurize+conv {dtype} d={d} f={f} K={K} prev={with_prev}", f64(fused), ref)
    assert r <= (FP32_TOL if dtype == torch.float32 else 4e-3)
