"""GPU parity at the measured workloads' full sizes, in the launch configuration
the bench uses (automatic plan), on EVERY (b, h), element by element.

Each output is checked against its first-order rounding bound (parity_util.check_bound:
the error of o_t within tol times the output over |v| plus |o_t|), so a single wrong
row, column or head fails even where it would barely move a rel-L2; rel-L2 and
max-abs are printed beside it.  The oracle runs in worker processes
(oracle_pool), one group of heads each.  For the 131072-token case the oracle
runs windows of 256 tokens at the head, the tail and across every segment
boundary of the plan, each window starting from the state that the closed form
(one matrix product per range) composes up to it."""
import numpy as np
import pytest
import torch

import oracle_pool
from oracle import hm_oracle as orc
from selective_state_space_hm_amd import hm, inputs
from parity_util import BF16_TOL, check_bound, rel_l2, report, run_fwd, with_abs

pytestmark = pytest.mark.gpu
f64 = inputs.to_f64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def plan_of(c):
    g = [getattr(c, k).cuda() for k in ("q", "k", "v", "w_q", "w_k")]
    dt = None if c.dt is None else c.dt.cuda()
    al = None if c.a_log is None else c.a_log.cuda()
    return hm.hm_linattn_fwd_plan(*g, dt, al)


def check_state(name, st, S, z, f, dv):
    """Final state of every head against the oracle's (rel-L2 per head, the worst reported)."""
    Sg, zg = orc.unpack_state(f64(st), 2 * f, dv)
    worst = max(max(rel_l2(Sg[b, h], S[b, h]), rel_l2(zg[b, h], z[b, h]))
                for b in range(S.shape[0]) for h in range(S.shape[1]))
    print(f"[parity] {name}: worst per-head state rel-L2 {worst:.3e}", flush=True)
    assert worst <= BF16_TOL, name


def run_every_head(c, name):
    plan = plan_of(c)
    print(f"[parity] {name}: plan (chunk, segments, dsplit) = {plan}", flush=True)
    st = torch.full((c.B, c.H, hm.state_numel(c.f, c.dv)), float("nan"), device="cuda")
    o = run_fwd(c, s_final=st)
    torch.cuda.synchronize()
    ref, S, z = oracle_pool.forward_all(f64(c.q), f64(c.k), with_abs(f64(c.v)), f64(c.w_q), f64(c.w_k),
                                        f64(c.dt), f64(c.a_log))
    dv = c.dv
    check_bound(f"{name} every head", f64(o), ref[..., :dv], ref[..., dv:], BF16_TOL)
    check_state(f"{name} s_final", st, S[..., :dv], z, c.f, dv)


def test_pythia1b_layer_every_head():
    run_every_head(inputs.pythia1b(), "pythia1b B=8 H=16 n=2048")


@pytest.mark.parametrize("maker", [inputs.mamba_decay, inputs.mild_decay])
def test_decay_n8192_every_head(maker):
    c = maker()
    run_every_head(c, f"{c.name} B=2 H=16 n=8192")


def test_long_context_windows_every_head():
    c = inputs.long_context()
    chunk, segs, _ = plan_of(c)
    nch = -(-c.n // chunk)
    seg_len = -(-nch // segs) * chunk
    w = 256
    starts = sorted({0, c.n - w} | {s * seg_len - w // 2 for s in range(1, segs)})
    print(f"[parity] long n=131072: {segs} segments of {seg_len} tokens; windows at {starts}", flush=True)
    st = torch.full((1, 16, hm.state_numel(64, 128)), float("nan"), device="cuda")
    o = run_fwd(c, s_final=st)
    torch.cuda.synchronize()
    got = f64(o)
    wq, wk = f64(c.w_q), f64(c.w_k)
    for h in range(c.H):
        k, v = f64(c.k[0:1, h:h + 1]), with_abs(f64(c.v[0:1, h:h + 1]))
        q = f64(c.q[0:1, h:h + 1])
        dt, a_log = f64(c.dt[0:1, h:h + 1]), f64(c.a_log[h:h + 1])
        la = orc.log_decay(dt, a_log)
        pk = orc.hedgehog_features(k, wk)
        S = np.zeros((1, 1, 128, 256))
        z = np.zeros((1, 1, 128))
        at = 0
        refs, gots = [], []
        for p in starts:
            # state at p: the carried state decayed over [at, p) plus that range's closed form
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
        check_bound(f"long n=131072 h={h} windows", np.concatenate(gots, axis=2), ref[..., :128], ref[..., 128:],
                    BF16_TOL)
        Sg, zg = orc.unpack_state(f64(st[0:1, h:h + 1]), 128, 128)
        assert report(f"long n=131072 h={h} final state", Sg, S[..., :128]) <= BF16_TOL
        assert rel_l2(zg, z) <= BF16_TOL


def test_decode_full_batch_every_head():
    """B=256, H=16 (the decode workload's batch): the state comes from a GPU prefill of a
    16-token prefix (the prefill -> decode handoff at full batch), then four decode steps;
    every head's state and every output element checked against the oracle."""
    dc = inputs.decode_setup(prefix=16)
    wq, wk, a_log = dc.w_q.cuda(), dc.w_k.cuda(), dc.a_log.cuda()
    state = torch.full((dc.B, dc.H, hm.state_numel(dc.f, dc.dv)), float("nan"), device="cuda")
    hm.hm_linattn_fwd(dc.prefix_k.cuda(), dc.prefix_k.cuda(), dc.prefix_v.cuda(), wq, wk, dc.prefix_dt.cuda(), a_log,
                      s_final=state)
    torch.cuda.synchronize()
    W = (f64(dc.w_q), f64(dc.w_k))
    pk = orc.hedgehog_features(f64(dc.prefix_k), W[1])
    S, z = orc.prefix_state(pk, with_abs(f64(dc.prefix_v)), orc.log_decay(f64(dc.prefix_dt), f64(dc.a_log)))
    check_state("decode B=256 H=16 prefill handoff", state, S[..., :128], z, dc.f, dc.dv)
    for t in range(4):
        q, k, v, dt = inputs.decode_step_inputs(dc, t)
        o = hm.hm_linattn_step(q.cuda(), k.cuda(), v.cuda(), wq, wk, state, dt.cuda(), a_log)
        torch.cuda.synchronize()
        ot, S, z = orc.step(S, z, f64(q), f64(k), with_abs(f64(v)), *W, f64(dt), f64(dc.a_log))
        check_bound(f"decode B=256 H=16 step {t} every head", f64(o), ot[..., :128], ot[..., 128:], BF16_TOL)
    Sg, zg = orc.unpack_state(f64(state), 128, 128)
    worst = max(rel_l2(Sg[b, h], S[b, h, :, :128]) for b in range(dc.B) for h in range(dc.H))
    print(f"[parity] decode B=256 H=16 after 4 steps: worst per-head state rel-L2 {worst:.3e}", flush=True)
    # the state started from the bf16 prefill (bf16 operands in its products), not from the oracle
    assert worst <= BF16_TOL


def test_decode_full_batch_long_prefix_sampled():
    """The decode workload as measured (4096-token prefix): its states are too costly for
    the oracle at every head, so four heads get the oracle's prefix state and the rest
    start from zero; the outputs of those heads are checked element by element."""
    dc = inputs.decode_setup()          # B=256, H=16, d=128, f=64, prefix 4096, Mamba decay
    heads = [(0, 0), (17, 3), (128, 8), (255, 15)]
    bs, hs = [b for b, _ in heads], [h for _, h in heads]
    state = torch.zeros((dc.B, dc.H, hm.state_numel(dc.f, dc.dv)), device="cuda")
    # the sampled heads side by side on a head axis: [1, 4, ...]
    pk = orc.hedgehog_features(f64(dc.prefix_k[bs, hs])[None], f64(dc.w_k))
    la = orc.log_decay(f64(dc.prefix_dt[bs, hs])[None], f64(dc.a_log[hs]))
    Sc, zc = orc.prefix_state(pk, with_abs(f64(dc.prefix_v[bs, hs])[None]), la)
    for i, (b, h) in enumerate(heads):
        state[b, h] = torch.tensor(orc.pack_state(Sc[:, i:i + 1, :, :128], zc[:, i:i + 1])[0, 0], dtype=torch.float32)
    wq, wk, a_log = dc.w_q.cuda(), dc.w_k.cuda(), dc.a_log.cuda()
    for t in range(6):
        q, k, v, dt = inputs.decode_step_inputs(dc, t)
        o = hm.hm_linattn_step(q.cuda(), k.cuda(), v.cuda(), wq, wk, state, dt.cuda(), a_log)
        torch.cuda.synchronize()
        ot, Sc, zc = orc.step(Sc, zc, f64(q[bs, hs])[None], f64(k[bs, hs])[None], with_abs(f64(v[bs, hs])[None]),
                              f64(dc.w_q), f64(dc.w_k), f64(dt[bs, hs])[None], f64(dc.a_log[hs]))
        check_bound(f"decode B=256 H=16 prefix 4096 step {t}", f64(o[bs, hs]), ot[0, :, :128], ot[0, :, 128:],
                    BF16_TOL)
    for i, (b, h) in enumerate(heads):
        Sg, zg = orc.unpack_state(f64(state[b:b + 1, h:h + 1]), 128, 128)
        assert rel_l2(Sg[0, 0], Sc[0, i, :, :128]) <= 1e-5
