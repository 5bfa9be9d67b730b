"""GPU parity on saturating feature maps: q and k scaled so that |x W| reaches
30 and beyond, where softmax([u, -u]) is nearly one-hot and most of its entries
are below 1e-13 of the largest (the Hedgehog map of the HedgeMamba explainer
§2.1 at its sharp end).  The kernels keep phi(q) unnormalized with its largest
entry 1 and phi(k) normalized; these cases check that the scores, the
denominators and the outputs stay finite and match the float64 oracle element
by element (parity_util.check_bound), and that every output stays inside the
range of the values it averages."""
import numpy as np
import pytest
import torch

from oracle import hm_oracle as orc
from selective_state_space_hm_amd import hm, inputs
from parity_util import check_bound, rel_l2, to_dev, tol_for, with_abs

pytestmark = pytest.mark.gpu
f64 = inputs.to_f64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hm.lib()


def saturate(c, scale):
    """Scale q and k (in float32, then rounded to the case's dtype) so |x W| is large."""
    c.q = (c.q.float() * scale).to(c.dtype)
    c.k = (c.k.float() * scale).to(c.dtype)
    return c


def max_u(c):
    uq = np.abs(f64(c.q) @ f64(c.w_q)).max(-1)
    uk = np.abs(f64(c.k) @ f64(c.w_k)).max(-1)
    return float(np.median(np.minimum(uq, uk))), float(max(uq.max(), uk.max()))


def convex(name, o, v):
    """Every output component lies between the smallest and largest value of its prefix."""
    v = f64(v)
    lo, hi = np.minimum.accumulate(v, axis=2), np.maximum.accumulate(v, axis=2)
    o = f64(o)
    slack = 1e-2 * (np.abs(lo) + np.abs(hi)) + 1e-6
    assert np.all(o >= lo - slack) and np.all(o <= hi + slack), f"{name}: output outside the convex hull"


@pytest.mark.parametrize("dtype,shape,scale", [(torch.bfloat16, (128, 64, 128), 14.0),
                                               (torch.bfloat16, (64, 32, 64), 14.0),
                                               (torch.float32, (16, 16, 16), 12.0),
                                               (torch.float32, (32, 16, 32), 12.0)])
@pytest.mark.parametrize("decay", [None, "mamba", "mild"])
@pytest.mark.parametrize("segments", [1, 3])
def test_prefill_saturating(dtype, shape, scale, decay, segments):
    d, f, dv = shape
    c = saturate(inputs.make_prefill("sat", 2, 3, 333, d, f, dv, dtype, None, decay, seed=d + 3), scale)
    med, top = max_u(c)
    print(f"[parity] saturating {dtype} {shape} decay={decay}: median row max|xW| {med:.1f}, largest {top:.1f}",
          flush=True)
    assert med >= (25.0 if dtype == torch.bfloat16 else 18.0)   # the case does saturate
    g = to_dev(c)
    st = torch.full((2, 3, hm.state_numel(f, dv)), float("nan"), device="cuda")
    o = hm.hm_linattn_fwd(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], g["dt"], g["a_log"], s_final=st,
                          segments=segments)
    torch.cuda.synchronize()
    ref, S, z = orc.forward(f64(c.q), f64(c.k), with_abs(f64(c.v)), f64(c.w_q), f64(c.w_k), f64(c.dt), f64(c.a_log))
    tol = tol_for(dtype)
    check_bound(f"saturating {dtype} {shape} decay={decay} segs={segments}", f64(o), ref[..., :dv], ref[..., dv:], tol)
    convex(f"saturating {dtype} {shape}", o, c.v)
    Sg, zg = orc.unpack_state(f64(st), 2 * f, dv)
    assert np.all(np.isfinite(Sg)) and np.all(zg > 0)
    assert rel_l2(Sg, S[..., :dv]) <= tol and rel_l2(zg, z) <= tol


@pytest.mark.parametrize("dtype,shape,scale", [(torch.bfloat16, (128, 64, 128), 14.0),
                                               (torch.float32, (32, 16, 32), 12.0)])
def test_decode_saturating(dtype, shape, scale):
    d, f, dv = shape
    B, H, steps = 3, 2, 12
    dc = inputs.decode_setup(B, H, d, f, dv, prefix=40, steps=steps, dtype=dtype, seed=d + 5)
    dc.prefix_k = (dc.prefix_k.float() * scale).to(dtype)
    W = (f64(dc.w_q), f64(dc.w_k))
    pk = orc.hedgehog_features(f64(dc.prefix_k), W[1])
    S, z = orc.prefix_state(pk, with_abs(f64(dc.prefix_v)), orc.log_decay(f64(dc.prefix_dt), f64(dc.a_log)))
    state = torch.tensor(orc.pack_state(S[..., :dv], z), dtype=torch.float32, device="cuda")
    wq, wk, a_log = dc.w_q.cuda(), dc.w_k.cuda(), dc.a_log.cuda()
    for t in range(steps):
        q, k, v, dt = inputs.decode_step_inputs(dc, t, dtype)
        q, k = (q.float() * scale).to(dtype), (k.float() * scale).to(dtype)
        o = hm.hm_linattn_step(q.cuda(), k.cuda(), v.cuda(), wq, wk, state, dt.cuda(), a_log)
        torch.cuda.synchronize()
        ot, S, z = orc.step(S, z, f64(q), f64(k), with_abs(f64(v)), *W, f64(dt), f64(dc.a_log))
        check_bound(f"saturating decode {dtype} {shape} step {t}", f64(o), ot[..., :dv], ot[..., dv:], tol_for(dtype))
    Sg, zg = orc.unpack_state(f64(state), 2 * f, dv)
    assert np.all(zg > 0) and rel_l2(Sg, S[..., :dv]) <= (1e-6 if dtype == torch.float32 else 1e-5)
