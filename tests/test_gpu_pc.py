"""GPU parity of the per-channel decay scan (hm_linattn_pc_fwd, hm_linattn_pc_step)
against the float64 oracle (oracle/hm_oracle.py forward_pc / step_pc, pinned in
tests/test_oracle_pc.py): the pages' Mamba-1 wiring with numerator and
denominator channels sharing exp(Delta A) per (channel, state).

Bars: rel-L2 <= 1e-5 for float32 inputs, <= 2e-2 for bf16; max-abs printed
beside every rel-L2.  The features stay float32 inside the scan, so bf16 cases
carry only the inputs' and the output's rounding."""
import numpy as np
import pytest
import torch

from oracle import hm_oracle as orc
from selective_state_space_hm_amd import hm, inputs
from parity_util import BF16_TOL, FP32_TOL, report, tol_for

pytestmark = pytest.mark.gpu
f64 = inputs.to_f64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hm.lib()


def dev(c):
    return {k: getattr(c, k).cuda() for k in ("q", "k", "v", "w_q", "w_k", "dt", "a_log")}


def oracle(c, sn0=None, sd0=None, gate=None, rope=None):
    q, k = f64(c.q), f64(c.k)
    if rope is None:
        return orc.forward_pc(q, k, f64(c.v), f64(c.w_q), f64(c.w_k), f64(c.dt), f64(c.a_log), sn0, sd0, gate)
    dims, pos0 = rope
    phiq = orc.rope(orc.hedgehog_features(q, f64(c.w_q)), orc.rope_positions(c.B, c.n, pos0), dims)
    phik = orc.rope(orc.hedgehog_features(k, f64(c.w_k)), orc.rope_positions(c.B, c.n, pos0), dims)
    o, Sn, Sd = orc.pc_scan(phiq, phik, f64(c.v), orc.softplus(f64(c.dt)), -np.exp(f64(c.a_log)), sn0, sd0)
    return orc.apply_gate(o, gate), Sn, Sd


def pc_bound(c, rope, o_ref):
    """First-order rounding bound of each output of the rotary per-channel scan:
    with every term carrying a small relative error, |d o_t[c]| <= eps (N + |o| D) / |den|,
    N = |phiq_t| . Sn_abs[:, c], D = |phiq_t| . Sd_abs[:, c], the states accumulated from
    |phik| and |v|, den = phiq_t . Sd[:, c] (signed: turned features can cancel).
    Returns the bound per output element (eps = 1) and the smallest den / D."""
    dims, pos0 = rope
    pos = orc.rope_positions(c.B, c.n, pos0)
    phq = orc.rope(orc.hedgehog_features(f64(c.q), f64(c.w_q)), pos, dims)
    phk = orc.rope(orc.hedgehog_features(f64(c.k), f64(c.w_k)), pos, dims)
    dl = orc.softplus(f64(c.dt))
    A = -np.exp(f64(c.a_log))
    At = np.broadcast_to(A if A.ndim == 3 else A[None], (c.H, c.dv, 2 * c.f)).transpose(0, 2, 1)[None]
    v = np.abs(f64(c.v))
    shape = (c.B, c.H, 2 * c.f, c.dv)
    Sn, Sd, S = np.zeros(shape), np.zeros(shape), np.zeros(shape)
    bound = np.empty(o_ref.shape)
    margin = np.inf
    for t in range(c.n):
        a = np.exp(dl[:, :, t, None, :] * At)
        kk = phk[:, :, t, :, None] * dl[:, :, t, None, :]
        Sn = a * Sn + np.abs(kk) * v[:, :, t, None, :]
        Sd = a * Sd + np.abs(kk)
        S = a * S + kk
        qa = np.abs(phq[:, :, t])
        N = np.einsum("bhf,bhfd->bhd", qa, Sn)
        D = np.einsum("bhf,bhfd->bhd", qa, Sd)
        den = np.einsum("bhf,bhfd->bhd", phq[:, :, t], S)
        bound[:, :, t] = (N + np.abs(o_ref[:, :, t]) * D) / np.abs(den)
        margin = min(margin, float((den / D).min()))
    return bound, margin


def check_bound(name, got, ref, bound, tol):
    ratio = np.abs(got - ref) / bound
    report(name, got, ref)
    print(f"[parity] {name}: max |err| / bound {ratio.max():.3e}", flush=True)
    assert ratio.max() <= tol, name


@pytest.mark.parametrize("n", [1, 37, 64, 130])
@pytest.mark.parametrize("shape", [(16, 16, 16), (32, 16, 32)])
@pytest.mark.parametrize("shared_a", [False, True])
def test_prefill_fp32(n, shape, shared_a):
    d, f, dv = shape
    c = inputs.make_pc("pc", 2, 3, n, d, f, dv, torch.float32, seed=n + d, shared_a=shared_a)
    g = dev(c)
    sf = torch.full((2, 3, hm.state_numel_pc(f, dv)), float("nan"), device="cuda")
    o = hm.hm_linattn_pc_fwd(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], g["dt"], g["a_log"], s_final=sf)
    torch.cuda.synchronize()
    ref, Sn, Sd = oracle(c)
    assert report(f"pc fp32 {shape} n={n} shared_a={shared_a} o", f64(o), ref) <= FP32_TOL
    assert report(f"pc fp32 {shape} n={n} shared_a={shared_a} state", f64(sf), orc.pack_state_pc(Sn, Sd)) <= FP32_TOL


@pytest.mark.parametrize("shape", [(16, 16, 16), (32, 16, 32)])
def test_prefill_fp32_handoff_in_place_gate_and_strides(shape):
    """Two calls with the state carried in place (s_init = s_final), the gate, and
    q, k, v read through [B, n, H, d]-ordered views."""
    d, f, dv = shape
    B, H, n, cut = 2, 3, 150, 70
    c = inputs.make_pc("pc", B, H, n, d, f, dv, torch.float32, seed=3)
    g = dev(c)
    for k_ in ("q", "k", "v"):
        g[k_] = g[k_].permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    gate = inputs.gate(c.v.shape, torch.float32, seed=3).cuda()
    st = torch.zeros((B, H, hm.state_numel_pc(f, dv)), device="cuda")
    parts = []
    for a, b in ((0, cut), (cut, n)):
        parts.append(hm.hm_linattn_pc_fwd(g["q"][:, :, a:b], g["k"][:, :, a:b], g["v"][:, :, a:b], g["w_q"], g["w_k"],
                                          g["dt"][:, :, a:b], g["a_log"], s_init=st, s_final=st, gate=gate[:, :, a:b]))
    torch.cuda.synchronize()
    ref, Sn, Sd = oracle(c, gate=f64(gate))
    assert report(f"pc fp32 {shape} handoff+gate o", np.concatenate([f64(p) for p in parts], 2), ref) <= FP32_TOL
    assert report(f"pc fp32 {shape} handoff state", f64(st), orc.pack_state_pc(Sn, Sd)) <= FP32_TOL


def test_empty_sequence_copies_the_state():
    c = inputs.make_pc("pc", 2, 2, 0, 16, 16, 16, torch.float32, seed=1)
    g = dev(c)
    si = torch.randn((2, 2, hm.state_numel_pc(16, 16)), generator=torch.Generator().manual_seed(2)).cuda()
    sf = torch.full_like(si, float("nan"))
    hm.hm_linattn_pc_fwd(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], g["dt"], g["a_log"], s_init=si, s_final=sf)
    torch.cuda.synchronize()
    assert torch.equal(sf, si)


@pytest.mark.parametrize("shape", [(128, 64, 128), (64, 32, 64)])
@pytest.mark.parametrize("extra", [None, "gate", "rope"])
def test_prefill_bf16(shape, extra):
    d, f, dv = shape
    c = inputs.make_pc("pc", 2, 2, 333, d, f, dv, torch.bfloat16, seed=d + f)
    g = dev(c)
    gate = inputs.gate(c.v.shape, torch.bfloat16, seed=4) if extra == "gate" else None
    pos0 = torch.tensor([5, 900], dtype=torch.int64) if extra == "rope" else None
    o = hm.hm_linattn_pc_fwd(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], g["dt"], g["a_log"],
                             gate=None if gate is None else gate.cuda(), rope_dims=32 if extra == "rope" else 0,
                             rope_pos0=None if pos0 is None else pos0.cuda())
    torch.cuda.synchronize()
    ref, _, _ = oracle(c, gate=f64(gate), rope=None if pos0 is None else (32, pos0.numpy()))
    assert report(f"pc bf16 {shape} {extra}", f64(o), ref) <= BF16_TOL
    if pos0 is not None:
        bound, margin = pc_bound(c, (32, pos0.numpy()), ref)
        print(f"[parity] min den/D {margin:.3f}", flush=True)
        check_bound(f"pc bf16 {shape} rope", f64(o), ref, bound, BF16_TOL)


def test_full_size_sampled_heads():
    """The Pythia-1B-shaped layer (B=8, H=16, n=2048, d=128, f=64, dv=128, bf16) in
    the launch configuration the bench times; three sampled (b, h) rows against the
    oracle, computed one by one."""
    c = inputs.make_pc("pc-pythia1b", 8, 16, 2048, 128, 64, 128, torch.bfloat16, seed=0)
    g = dev(c)
    o = hm.hm_linattn_pc_fwd(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], g["dt"], g["a_log"])
    torch.cuda.synchronize()
    for b, h in ((0, 0), (3, 7), (7, 15)):
        sub = inputs.Case("s", 1, 1, c.n, c.d, c.f, c.dv, c.dtype, c.q[b:b + 1, h:h + 1], c.k[b:b + 1, h:h + 1],
                          c.v[b:b + 1, h:h + 1], c.w_q, c.w_k, c.dt[b:b + 1, h:h + 1], c.a_log[h:h + 1])
        ref, _, _ = oracle(sub)
        assert report(f"pc bf16 full size (b={b}, h={h})", f64(o[b:b + 1, h:h + 1]), ref) <= BF16_TOL


@pytest.mark.parametrize("dtype,shape", [(torch.float32, (16, 16, 16)), (torch.float32, (32, 16, 32)),
                                         (torch.bfloat16, (128, 64, 128)), (torch.bfloat16, (64, 32, 64))])
@pytest.mark.parametrize("rope", [False, True])
@pytest.mark.parametrize("per_head", [False, True])
def test_decode_chain(dtype, shape, rope, per_head):
    """Prefill a prefix, then decode step by step, gated; every step against the
    oracle (output and state).  per_head: one W per head ([H, d, f])."""
    d, f, dv = shape
    B, H, pre, steps = 3, 2, 40, 5
    c = inputs.make_pc("pc", B, H, pre + steps, d, f, dv, dtype, seed=d + 1)
    if per_head:
        gw = torch.Generator().manual_seed(78)
        c.w_q = (torch.randn((H, d, f), generator=gw) / d ** 0.5).to(dtype)
        c.w_k = (torch.randn((H, d, f), generator=gw) / d ** 0.5).to(dtype)
    gate = inputs.gate(c.v.shape, dtype, seed=6)
    g = dev(c)
    gg = gate.cuda()
    pos0 = torch.tensor([3, 50, 700], dtype=torch.int64)
    rk = dict(rope_dims=32, rope_pos0=pos0.cuda()) if rope else {}
    state = torch.empty((B, H, hm.state_numel_pc(f, dv)), device="cuda")
    hm.hm_linattn_pc_fwd(g["q"][:, :, :pre], g["k"][:, :, :pre], g["v"][:, :, :pre], g["w_q"], g["w_k"],
                         g["dt"][:, :, :pre], g["a_log"], s_final=state, **rk)
    ref, Sn, Sd = oracle(c, gate=f64(gate), rope=(32, pos0.numpy()) if rope else None)
    if rope:
        # the gate multiplies o and its bound alike; the bound is formed on the pre-gate output
        ref0, _, _ = oracle(c, rope=(32, pos0.numpy()))
        bound, margin = pc_bound(c, (32, pos0.numpy()), ref0)
        bound = bound * np.abs(orc.silu(f64(gate)))
        print(f"[parity] min den/D {margin:.3f}", flush=True)
    for s_ in range(steps):
        t = pre + s_
        kw = dict(rope_dims=32, rope_pos=(pos0 + t).cuda()) if rope else {}
        o = hm.hm_linattn_pc_step(g["q"][:, :, t].contiguous(), g["k"][:, :, t].contiguous(),
                                  g["v"][:, :, t].contiguous(), g["w_q"], g["w_k"], state,
                                  g["dt"][:, :, t].contiguous(), g["a_log"], gate=gg[:, :, t].contiguous(), **kw)
        torch.cuda.synchronize()
        name = f"pc decode {dtype} {shape} rope={rope} step {s_}"
        if rope:
            # the turned features are signed: a channel's denominator can come near zero, so
            # each output is held to tol times its rounding bound
            check_bound(name, f64(o), ref[:, :, t], bound[:, :, t], tol_for(dtype))
        else:
            assert report(name, f64(o), ref[:, :, t]) <= tol_for(dtype)
    assert report(f"pc decode {dtype} {shape} rope={rope} state", f64(state), orc.pack_state_pc(Sn, Sd)) <= FP32_TOL


def test_decode_fused_conv_matches_conv_then_step():
    """The fused short conv in the per-channel step is bit-identical to hm_causal_conv
    (n = 1) followed by a plain per-channel step."""
    B, H, d, f, dv = 4, 2, 128, 64, 128
    c = inputs.make_pc("pc", B, H, 1, d, f, dv, torch.bfloat16, seed=9)
    g = dev(c)
    gen = torch.Generator().manual_seed(10)
    cw = [(torch.randn((d, 4), generator=gen) / 2).cuda() for _ in range(2)]
    cb = [(torch.randn((d,), generator=gen) / 4).cuda() for _ in range(2)]
    cs0 = [torch.randn((B, H, 3, d), generator=gen).to(torch.bfloat16).cuda() for _ in range(2)]
    st0 = torch.randn((B, H, hm.state_numel_pc(f, dv)), generator=gen).abs().cuda()
    q1, k1, v1, dt1 = (g["q"][:, :, 0].contiguous(), g["k"][:, :, 0].contiguous(), g["v"][:, :, 0].contiguous(),
                       g["dt"][:, :, 0].contiguous())
    # fused
    cs = [x.clone() for x in cs0]
    st = st0.clone()
    o_f = hm.hm_linattn_pc_step(q1, k1, v1, g["w_q"], g["w_k"], st, dt1, g["a_log"],
                                conv=(cw[0], cw[1], cb[0], cb[1], cs[0], cs[1]))
    # separate
    qc = hm.hm_causal_conv(q1[:, :, None], cw[0], cb[0], prev=cs0[0])[:, :, 0].contiguous()
    kc = hm.hm_causal_conv(k1[:, :, None], cw[1], cb[1], prev=cs0[1])[:, :, 0].contiguous()
    st2 = st0.clone()
    o_s = hm.hm_linattn_pc_step(qc, kc, v1, g["w_q"], g["w_k"], st2, dt1, g["a_log"])
    torch.cuda.synchronize()
    assert torch.equal(o_f, o_s)
    assert torch.equal(st, st2)


def positive_pc_state(B, H, F, dv, seed):
    """A start state a prefix of tokens could have left: Sd > 0, Sn = sums of phi v."""
    r = np.random.default_rng(seed)
    w = r.random((B, H, 5, F))
    w /= w.sum(-1, keepdims=True)
    vv = r.normal(size=(B, H, 5, dv))
    Sn = np.einsum("bhjf,bhjd->bhfd", w, vv)
    Sd = np.einsum("bhjf,bhjd->bhfd", w, np.ones_like(vv))
    return torch.tensor(orc.pack_state_pc(Sn, Sd), dtype=torch.float32, device="cuda"), Sn, Sd


@pytest.mark.parametrize("segments", [2, 3, 64, 0])
@pytest.mark.parametrize("n", [130, 333, 700])
@pytest.mark.parametrize("shape", [(16, 16, 16), (32, 16, 32)])
def test_prefill_segments_fp32(segments, n, shape):
    """The sequence cut into segments scanned in parallel (segment pass, element-wise
    composition of the start states, full pass) against the oracle, from a start state,
    with s_final; 64 segments cap at one per chunk, 0 is the automatic plan."""
    d, f, dv = shape
    c = inputs.make_pc("pcseg", 2, 3, n, d, f, dv, torch.float32, seed=n + d + segments)
    g = dev(c)
    s0, Sn0, Sd0 = positive_pc_state(2, 3, 2 * f, dv, seed=n)
    sf = torch.full_like(s0, float("nan"))
    plan = hm.hm_linattn_pc_plan(g["q"], g["v"], g["w_q"], segments=segments)
    o = hm.hm_linattn_pc_fwd(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], g["dt"], g["a_log"], s_init=s0,
                             s_final=sf, segments=segments)
    torch.cuda.synchronize()
    assert plan == (min(segments, -(-n // 64)) if segments else plan) and plan >= 1
    ref, Sn, Sd = oracle(c, Sn0, Sd0)
    name = f"pc fp32 {shape} n={n} segments={segments} (plan {plan})"
    assert report(f"{name} o", f64(o), ref) <= FP32_TOL
    assert report(f"{name} state", f64(sf), orc.pack_state_pc(Sn, Sd)) <= FP32_TOL


def test_prefill_segments_in_place_gate_rope():
    """Segments with s_init and s_final the same buffer (zeros), the gate and the rotary
    encoding (positions offset by each segment's first token).  The turned features are
    signed, so each output is held to FP32_TOL times its first-order rounding bound."""
    B, H, n, d, f, dv = 2, 2, 500, 32, 16, 32
    c = inputs.make_pc("pcseg", B, H, n, d, f, dv, torch.float32, seed=21)
    g = dev(c)
    gate = inputs.gate(c.v.shape, torch.float32, seed=8)
    pos0 = torch.tensor([7, 300], dtype=torch.int64)
    st = torch.zeros((B, H, hm.state_numel_pc(f, dv)), device="cuda")
    o = hm.hm_linattn_pc_fwd(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], g["dt"], g["a_log"], s_init=st, s_final=st,
                             gate=gate.cuda(), rope_dims=32, rope_pos0=pos0.cuda(), segments=4)
    torch.cuda.synchronize()
    ref, Sn, Sd = oracle(c, gate=f64(gate), rope=(32, pos0.numpy()))
    ref0, _, _ = oracle(c, rope=(32, pos0.numpy()))
    bound, margin = pc_bound(c, (32, pos0.numpy()), ref0)
    print(f"[parity] min den/D {margin:.3f}", flush=True)
    check_bound("pc fp32 segments in place + gate + rope", f64(o), ref, bound * np.abs(orc.silu(f64(gate))), FP32_TOL)
    assert report("pc fp32 segments in place state", f64(st), orc.pack_state_pc(Sn, Sd)) <= FP32_TOL


@pytest.mark.parametrize("segments", [1, 0, 7])
def test_prefill_segments_bf16_long(segments):
    """A long sequence on few heads (B=1, H=2, n=16384, the Pythia-shaped head): the
    automatic plan cuts it into 64 segments of four chunks; every output against the
    oracle, and the segmented outputs against the unsegmented ones."""
    c = inputs.make_pc("pclong", 1, 2, 16384, 128, 64, 128, torch.bfloat16, seed=5)
    g = dev(c)
    sf = torch.empty((1, 2, hm.state_numel_pc(64, 128)), device="cuda")
    plan = hm.hm_linattn_pc_plan(g["q"], g["v"], g["w_q"], segments=segments)
    assert plan == {1: 1, 0: 64, 7: 7}[segments]
    o = hm.hm_linattn_pc_fwd(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], g["dt"], g["a_log"], s_final=sf,
                             segments=segments)
    torch.cuda.synchronize()
    ref, Sn, Sd = oracle(c)
    assert report(f"pc bf16 long segments={segments} (plan {plan}) o", f64(o), ref) <= BF16_TOL
    assert report(f"pc bf16 long segments={segments} state", f64(sf), orc.pack_state_pc(Sn, Sd)) <= BF16_TOL
