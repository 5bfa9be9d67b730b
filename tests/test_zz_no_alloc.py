"""hm_linattn_fwd_noalloc (the prefill with the library's per-GPU scratch in place of
a caller workspace) against hm_linattn_fwd, through the C ABI: two calls in a row,
the second on a smaller input, each bit for bit equal to hm_linattn_fwd on the
same inputs (same kernels and plan), and the second also against the float64
oracle.  The first call is the Mamba-decay workload (B=2, H=16, n=8192: eight
segments whose start states pass through the scratch); the second a small
segmented case whose s_init and s_final are one buffer (the scratch then also
holds the copy of s_init).  The same for two chunk-parallel plans (the chunk
states in the scratch)."""
import numpy as np
import pytest
import torch

from oracle import hm_oracle as orc
from selective_state_space_hm_amd import hm, inputs
from parity_util import BF16_TOL, report, to_dev

pytestmark = pytest.mark.gpu
f64 = inputs.to_f64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hm.lib()


def both(c, s0=None, **kw):
    """(o, s_final) from hm_linattn_fwd_noalloc and from hm_linattn_fwd; with s0 the
    state buffer starts as s0 and serves as s_init and s_final at once."""
    g = to_dev(c)
    out = []
    for fn in (hm.hm_linattn_fwd_noalloc, hm.hm_linattn_fwd):
        st = (s0.clone() if s0 is not None else
              torch.full((c.B, c.H, hm.state_numel(c.f, c.dv)), float("nan"), device="cuda"))
        o = fn(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], g["dt"], g["a_log"], s_init=st if s0 is not None else None,
               s_final=st, **kw)
        out.append((o, st))
    torch.cuda.synchronize()
    return out


def test_noalloc_matches_workspace_entry_point_twice():
    big = inputs.mamba_decay()                                           # B=2, H=16, n=8192
    small = inputs.make_prefill("noalloc-small", 1, 4, 700, 128, 64, 128, torch.bfloat16, None, "mild", seed=4)
    plans = [hm.hm_linattn_fwd_plan(*(getattr(c, k).cuda() for k in ("q", "k", "v", "w_q", "w_k", "dt", "a_log")))
             for c in (big, small)]
    print(f"[parity] noalloc plans {plans}", flush=True)
    assert plans[0][1] > 1 and plans[1][1] > 1                           # both use segment states
    # call 1: the large workload
    (o1, s1), (r1, rs1) = both(big)
    assert torch.equal(o1, r1) and torch.equal(s1, rs1)
    # call 2: smaller, s_init aliasing s_final
    gen = torch.Generator().manual_seed(6)
    F, dv = 2 * small.f, small.dv
    S0 = torch.rand((1, 4, F, dv), generator=gen, dtype=torch.float64)
    z0 = torch.rand((1, 4, F), generator=gen, dtype=torch.float64) + 1.0
    s0 = torch.tensor(orc.pack_state(S0.numpy(), z0.numpy()), dtype=torch.float32).cuda()
    (o2, s2), (r2, rs2) = both(small, s0)
    assert torch.equal(o2, r2) and torch.equal(s2, rs2)
    S0f, z0f = orc.unpack_state(f64(s0), F, dv)
    ref, S, z = orc.forward(*(f64(getattr(small, k)) for k in ("q", "k", "v", "w_q", "w_k", "dt", "a_log")), S0f, z0f)
    assert report("noalloc second call o", f64(o2), ref) <= BF16_TOL
    assert report("noalloc second call s_final", f64(s2), orc.pack_state(S, z)) <= BF16_TOL
    # and the first call's result is reproduced after the second one reused the scratch
    (o3, _), _ = both(big)
    assert torch.equal(o3, r1)


def test_noalloc_rejects_oversized_plans_without_launching():
    c = inputs.pythia1b()
    g = to_dev(c)
    o = torch.zeros_like(g["v"])
    with pytest.raises(hm.HMError, match="scratch"):
        hm.hm_linattn_fwd_noalloc(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], o=o, segments=8)
    torch.cuda.synchronize()
    assert torch.count_nonzero(o) == 0


def test_noalloc_chunk_parallel_plans_twice():
    """The chunk-parallel path (chunk 256; float32 at d = 128) through the scratch: two
    calls in a row, the second smaller and with s_init aliasing s_final, each bit for
    bit equal to hm_linattn_fwd; a plan whose chunk states exceed the scratch is
    rejected before any launch."""
    first = inputs.make_prefill("noalloc-cp", 2, 4, 1000, 128, 64, 128, torch.bfloat16, None, "mamba", seed=8)
    second = inputs.make_prefill("noalloc-cp-f32", 1, 2, 300, 128, 64, 128, torch.float32, None, "mild", seed=9)
    (o1, s1), (r1, rs1) = both(first, chunk=256)
    assert torch.equal(o1, r1) and torch.equal(s1, rs1)
    gen = torch.Generator().manual_seed(10)
    S0 = torch.rand((1, 2, 128, 128), generator=gen, dtype=torch.float64)
    z0 = torch.rand((1, 2, 128), generator=gen, dtype=torch.float64) + 1.0
    s0 = torch.tensor(orc.pack_state(S0.numpy(), z0.numpy()), dtype=torch.float32).cuda()
    (o2, s2), (r2, rs2) = both(second, s0)
    assert torch.equal(o2, r2) and torch.equal(s2, rs2)
    S0f, z0f = orc.unpack_state(f64(s0), 128, 128)
    ref, S, z = orc.forward(*(f64(getattr(second, k)) for k in ("q", "k", "v", "w_q", "w_k", "dt", "a_log")), S0f, z0f)
    assert report("noalloc chunk-parallel f32 o", f64(o2), ref) <= 1e-5
    assert report("noalloc chunk-parallel f32 s_final", f64(s2), orc.pack_state(S, z)) <= 1e-5
    c = inputs.long_context()
    g = to_dev(c)
    o = torch.zeros_like(g["v"])
    with pytest.raises(hm.HMError, match="scratch"):
        hm.hm_linattn_fwd_noalloc(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], g["dt"], g["a_log"], o=o, chunk=256)
    torch.cuda.synchronize()
    assert torch.count_nonzero(o) == 0
