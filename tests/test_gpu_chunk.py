"""GPU parity of the prefill with 128-token chunks (the chunk-wise parallel form of
the cnblogs linear-attention tutorial, part 5, with chunks twice as long: each
chunk's outputs read the state at its start plus the masked, decayed scores of
all its earlier tokens, and the state passes once per chunk).  Against the
float64 oracle element by element (parity_util.check_bound) at ragged lengths,
with segments, column splits and an initial state, and against the 64-token
chunks on the same inputs: the chunk length only reorders the sums."""
import numpy as np
import pytest
import torch

from oracle import hm_oracle as orc
from selective_state_space_hm_amd import hm, inputs
from parity_util import BF16_TOL, FP32_TOL, check_bound, rel_l2, report, run_fwd, to_dev, tol_for, with_abs

pytestmark = pytest.mark.gpu
f64 = inputs.to_f64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hm.lib()


def oracle(c, s_init=None):
    S0 = z0 = None
    if s_init is not None:
        S0, z0 = orc.unpack_state(f64(s_init), c.F, c.dv)
        S0 = np.concatenate([S0, np.abs(S0)], axis=-1)   # the bound's |v| part starts from |S0|
    return orc.forward(f64(c.q), f64(c.k), with_abs(f64(c.v)), f64(c.w_q), f64(c.w_k), f64(c.dt), f64(c.a_log),
                       S0, z0)


def positive_state(B, H, F, dv, seed):
    """An initial state that a prefix of tokens could have left: z > 0, S = sum of phi v."""
    r = np.random.default_rng(seed)
    kk = r.random((B, H, 7, F))
    kk /= kk.sum(-1, keepdims=True)
    S0 = np.einsum("bhjf,bhjd->bhfd", kk, r.normal(size=(B, H, 7, dv)))
    return torch.tensor(orc.pack_state(S0, kk.sum(2)), dtype=torch.float32, device="cuda")


def check_prefill(name, c, o, st, ref, S, z, tol):
    dv = c.dv
    check_bound(name, f64(o), ref[..., :dv], ref[..., dv:], tol)
    Sg, zg = orc.unpack_state(f64(st), c.F, dv)
    assert report(f"{name} S_final", Sg, S[..., :dv]) <= tol
    assert rel_l2(zg, z) <= tol


@pytest.mark.parametrize("n", [1, 37, 64, 65, 127, 128, 129, 200, 333])
@pytest.mark.parametrize("decay", [None, "mamba", "mild"])
@pytest.mark.parametrize("shape", [(16, 16, 16), (32, 16, 32)])
def test_fp32_ragged(n, decay, shape):
    d, f, dv = shape
    c = inputs.make_prefill("c128", 2, 3, n, d, f, dv, torch.float32, None, decay, seed=n + d + 1)
    st = torch.full((2, 3, hm.state_numel(f, dv)), float("nan"), device="cuda")
    o = run_fwd(c, s_final=st, chunk=128)
    torch.cuda.synchronize()
    ref, S, z = oracle(c)
    check_prefill(f"chunk128 fp32 {shape} n={n} decay={decay}", c, o, st, ref, S, z, FP32_TOL)


@pytest.mark.parametrize("segments,dsplit", [(1, 1), (2, 1), (3, 1), (1, 2), (3, 2), (0, 0)])
@pytest.mark.parametrize("decay", ["mild", "mamba"])
def test_fp32_plans_initial_state(segments, dsplit, decay):
    c = inputs.make_prefill("c128p", 2, 2, 700, 32, 16, 32, torch.float32, None, decay, seed=11)
    s0 = positive_state(2, 2, 32, 32, 3)
    st = torch.full_like(s0, float("nan"))
    o = run_fwd(c, s_init=s0, s_final=st, chunk=128, segments=segments, dsplit=dsplit)
    torch.cuda.synchronize()
    ref, S, z = oracle(c, s0)
    plan = hm.hm_linattn_fwd_plan(*(to_dev(c)[k] for k in ("q", "k", "v", "w_q", "w_k", "dt", "a_log")), chunk=128,
                                  segments=segments, dsplit=dsplit)
    check_prefill(f"chunk128 fp32 plan {plan} decay={decay}", c, o, st, ref, S, z, FP32_TOL)


def test_fp32_aliased_handoff():
    """Two calls, the second continuing from the first's state in the same buffer."""
    c = inputs.make_prefill("c128h", 1, 2, 450, 16, 16, 16, torch.float32, None, "mild", seed=5)
    g = to_dev(c)
    st = torch.empty((1, 2, hm.state_numel(16, 16)), device="cuda")
    m = 190
    sl = lambda t, a, b: None if t is None else t[:, :, a:b]
    o1 = hm.hm_linattn_fwd(sl(g["q"], 0, m), sl(g["k"], 0, m), sl(g["v"], 0, m), g["w_q"], g["w_k"],
                           sl(g["dt"], 0, m), g["a_log"], s_final=st, chunk=128)
    o2 = hm.hm_linattn_fwd(sl(g["q"], m, 450), sl(g["k"], m, 450), sl(g["v"], m, 450), g["w_q"], g["w_k"],
                           sl(g["dt"], m, 450), g["a_log"], s_init=st, s_final=st, chunk=128, segments=2)
    torch.cuda.synchronize()
    ref, S, z = oracle(c)
    check_bound("chunk128 handoff", np.concatenate([f64(o1), f64(o2)], axis=2), ref[..., :16], ref[..., 16:], FP32_TOL)
    Sg, zg = orc.unpack_state(f64(st), 32, 16)
    assert rel_l2(Sg, S[..., :16]) <= FP32_TOL and rel_l2(zg, z) <= FP32_TOL


@pytest.mark.parametrize("shape", [(128, 64, 128), (64, 32, 64)])
@pytest.mark.parametrize("decay", [None, "mild", "mamba"])
@pytest.mark.parametrize("dsplit", [1, 2])
def test_bf16_shapes_ragged(shape, decay, dsplit):
    d, f, dv = shape
    c = inputs.make_prefill("c128b", 2, 3, 333, d, f, dv, torch.bfloat16, None, decay, seed=d + 3)
    st = torch.full((2, 3, hm.state_numel(f, dv)), float("nan"), device="cuda")
    o = run_fwd(c, s_final=st, chunk=128, dsplit=dsplit)
    torch.cuda.synchronize()
    ref, S, z = oracle(c)
    check_prefill(f"chunk128 bf16 {shape} decay={decay} dsplit={dsplit}", c, o, st, ref, S, z, BF16_TOL)


@pytest.mark.parametrize("dtype,shape", [(torch.float32, (32, 16, 32)), (torch.bfloat16, (128, 64, 128))])
@pytest.mark.parametrize("decay", [None, "mild"])
def test_chunk_invariance(dtype, shape, decay):
    """64- and 128-token chunks on the same inputs: both match the oracle, and each
    other to the dtype's bar (the chunk length only reorders the sums)."""
    d, f, dv = shape
    c = inputs.make_prefill("cinv", 2, 4, 1000, d, f, dv, dtype, None, decay, seed=9)
    outs, states = [], []
    for ch in (64, 128):
        st = torch.empty((2, 4, hm.state_numel(f, dv)), device="cuda")
        outs.append(f64(run_fwd(c, s_final=st, chunk=ch)))
        states.append(f64(st))
    torch.cuda.synchronize()
    ref, S, z = oracle(c)
    tol = tol_for(dtype)
    for ch, o in zip((64, 128), outs):
        check_bound(f"chunk {ch} {dtype} decay={decay}", o, ref[..., :dv], ref[..., dv:], tol)
    assert report(f"chunk 64 vs 128 {dtype} decay={decay} o", outs[1], outs[0]) <= tol
    assert report(f"chunk 64 vs 128 {dtype} decay={decay} state", states[1], states[0]) <= tol


def test_long_context_chunk128_windows():
    """The 131072-token Mamba-decay workload with 128-token chunks: every head, windows of
    256 tokens at the head, the tail and across every segment boundary of the plan."""
    c = inputs.long_context()
    chunk, segs, _ = hm.hm_linattn_fwd_plan(*(to_dev(c)[k] for k in ("q", "k", "v", "w_q", "w_k", "dt", "a_log")),
                                            chunk=128)
    assert chunk == 128
    nch = -(-c.n // chunk)
    seg_len = -(-nch // segs) * chunk
    w = 256
    starts = sorted({0, c.n - w} | {s * seg_len - w // 2 for s in range(1, segs)})
    st = torch.full((1, 16, hm.state_numel(64, 128)), float("nan"), device="cuda")
    got = f64(run_fwd(c, s_final=st, chunk=128))
    torch.cuda.synchronize()
    wq, wk = f64(c.w_q), f64(c.w_k)
    for h in range(c.H):
        k, v, q = f64(c.k[0:1, h:h + 1]), with_abs(f64(c.v[0:1, h:h + 1])), f64(c.q[0:1, h:h + 1])
        dt, a_log = f64(c.dt[0:1, h:h + 1]), f64(c.a_log[h:h + 1])
        la = orc.log_decay(dt, a_log)
        pk = orc.hedgehog_features(k, wk)
        S, z, at = np.zeros((1, 1, 128, 256)), np.zeros((1, 1, 128)), 0
        refs, gots = [], []
        for p in starts:
            if p > at:
                Sl, zl = orc.prefix_state(pk[:, :, at:p], v[:, :, at:p], la[:, :, at:p])
                carry = np.exp(la[0, 0, at:p].sum())
                S, z = carry * S + Sl, carry * z + zl
            ow, S, z = orc.forward(q[:, :, p:p + w], k[:, :, p:p + w], v[:, :, p:p + w], wq, wk, dt[:, :, p:p + w],
                                   a_log, S, z)
            at = p + w
            refs.append(ow)
            gots.append(got[0:1, h:h + 1, p:p + w])
        ref = np.concatenate(refs, axis=2)
        check_bound(f"long chunk128 h={h} windows", np.concatenate(gots, axis=2), ref[..., :128], ref[..., 128:],
                    BF16_TOL)
        Sg, zg = orc.unpack_state(f64(st[0:1, h:h + 1]), 128, 128)
        assert rel_l2(Sg, S[..., :128]) <= BF16_TOL and rel_l2(zg, z) <= BF16_TOL
