"""GPU parity at the measured workloads' full sizes, in the launch configuration
the bench uses (automatic plan), on sampled (b, h) rows that the oracle computes
one by one.  For the 131072-token case the oracle's state after a long prefix
comes from its closed form (one matrix product) and the recurrent form runs the
head and the tail of the sequence."""
import numpy as np
import pytest
import torch

from oracle import hm_oracle as orc
from selective_state_space_hm_amd import hm, inputs
from parity_util import BF16_TOL, oracle_heads, rel_l2, report, run_fwd, to_dev

pytestmark = pytest.mark.gpu
f64 = inputs.to_f64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def check_heads(name, case, o, heads):
    ref, _, _ = oracle_heads(case, heads)
    bs = [b for b, _ in heads]
    hs = [h for _, h in heads]
    got = f64(o[bs, hs])
    return report(name, got, ref)


def test_pythia1b_layer():
    c = inputs.pythia1b()
    print("[parity] plan", hm.hm_linattn_fwd_plan(*(getattr(c, k).cuda() for k in ("q", "k", "v", "w_q", "w_k"))), flush=True)
    o = run_fwd(c)
    torch.cuda.synchronize()
    assert check_heads("pythia1b B=8 H=16 n=2048", c, o, [(0, 0), (3, 5), (7, 15)]) <= BF16_TOL


@pytest.mark.parametrize("maker", [inputs.mamba_decay, inputs.mild_decay])
def test_decay_n8192(maker):
    c = maker()
    o = run_fwd(c)
    torch.cuda.synchronize()
    assert check_heads(f"{c.name} B=2 H=16 n=8192", c, o, [(0, 0), (1, 9), (1, 15)]) <= BF16_TOL


def test_long_context_head_and_tail():
    c = inputs.long_context()
    st = torch.empty((1, 16, hm.state_numel(64, 128)), device="cuda")
    o = run_fwd(c, s_final=st)
    torch.cuda.synchronize()
    n, w = c.n, 4096
    for h in (3, 12):
        q, k, v = (f64(getattr(c, x)[0:1, h:h + 1]) for x in ("q", "k", "v"))
        dt = f64(c.dt[0:1, h:h + 1])
        a_log = f64(c.a_log[h:h + 1])
        wq, wk = f64(c.w_q), f64(c.w_k)
        # head: tokens [0, w) from a zero state
        ref_head, _, _ = orc.forward(q[:, :, :w], k[:, :, :w], v[:, :, :w], wq, wk, dt[:, :, :w], a_log)
        # tail: closed-form state after [0, n-w), then the recurrent form
        pk = orc.hedgehog_features(k[:, :, :n - w], wk)
        S0, z0 = orc.prefix_state(pk, v[:, :, :n - w], orc.log_decay(dt[:, :, :n - w], a_log))
        ref_tail, S, z = orc.forward(q[:, :, n - w:], k[:, :, n - w:], v[:, :, n - w:], wq, wk, dt[:, :, n - w:],
                                     a_log, S0, z0)
        got = f64(o[0:1, h:h + 1])
        assert report(f"long n=131072 h={h} head", got[:, :, :w], ref_head) <= BF16_TOL
        assert report(f"long n=131072 h={h} tail", got[:, :, n - w:], ref_tail) <= BF16_TOL
        Sg, zg = orc.unpack_state(f64(st[0:1, h:h + 1]), 128, 128)
        assert report(f"long n=131072 h={h} final state", Sg, S) <= BF16_TOL


def test_decode_full_batch_sampled():
    dc = inputs.decode_setup()          # B=256, H=16, d=128, f=64, prefix 4096, Mamba decay
    heads = [(0, 0), (17, 3), (128, 8), (255, 15)]
    state = torch.zeros((dc.B, dc.H, hm.state_numel(dc.f, dc.dv)), device="cuda")
    S0 = np.empty((len(heads), 128, 128))
    z0 = np.empty((len(heads), 128))
    for i, (b, h) in enumerate(heads):
        pk = orc.hedgehog_features(f64(dc.prefix_k[b:b + 1, h:h + 1]), f64(dc.w_k))
        la = orc.log_decay(f64(dc.prefix_dt[b:b + 1, h:h + 1]), f64(dc.a_log[h:h + 1]))
        S, z = orc.prefix_state(pk, f64(dc.prefix_v[b:b + 1, h:h + 1]), la)
        S0[i], z0[i] = S[0, 0], z[0, 0]
        state[b, h] = torch.tensor(orc.pack_state(S, z)[0, 0], dtype=torch.float32)
    wq, wk, a_log = dc.w_q.cuda(), dc.w_k.cuda(), dc.a_log.cuda()
    Sc, zc = S0[:, None], z0[:, None]
    for t in range(6):
        q, k, v, dt = inputs.decode_step_inputs(dc, t)
        o = hm.hm_linattn_step(q.cuda(), k.cuda(), v.cuda(), wq, wk, state, dt.cuda(), a_log)
        torch.cuda.synchronize()
        got, ref = [], []
        for i, (b, h) in enumerate(heads):
            ot, S1, z1 = orc.step(Sc[i:i + 1], zc[i:i + 1], f64(q[b:b + 1, h:h + 1]), f64(k[b:b + 1, h:h + 1]),
                                  f64(v[b:b + 1, h:h + 1]), f64(dc.w_q), f64(dc.w_k), f64(dt[b:b + 1, h:h + 1]),
                                  f64(dc.a_log[h:h + 1]))
            Sc[i:i + 1], zc[i:i + 1] = S1, z1
            got.append(f64(o[b, h]))
            ref.append(ot[0, 0])
        assert report(f"decode B=256 H=16 step {t}", np.stack(got), np.stack(ref)) <= BF16_TOL
    for i, (b, h) in enumerate(heads):
        Sg, zg = orc.unpack_state(f64(state[b:b + 1, h:h + 1]), 128, 128)
        assert rel_l2(Sg[0, 0], Sc[i, 0]) <= 1e-5
