"""GPU parity of the chunk-parallel prefill: chunk length 256, and every (dtype, d, f,
dv) of the supported size matrix, including the sizes that have no fused kernel
(float32 at d = 128, bf16 at d = 16, f = 16 at d >= 64).  This is the chunk-wise form of
the cnblogs linear-attention tutorial, part 5: each chunk's outputs read the state
at its start plus the masked, decayed scores of all its earlier tokens, and the
start states come from a scan over the chunks' local states (the quant67 SSM
lecture, §4.2 and §6).  Outputs are checked against the float64 oracle element by
element (parity_util.check_bound), final states by rel-L2, at ragged lengths, with
and without decay, with an initial state and with s_init and s_final in one buffer;
and the chunk lengths 64, 128 and 256 against each other on the same inputs."""
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


def plan_of(c, **kw):
    return hm.hm_linattn_fwd_plan(*(to_dev(c)[k] for k in ("q", "k", "v", "w_q", "w_k", "dt", "a_log")), **kw)


@pytest.mark.parametrize("n", [1, 63, 64, 65, 255, 256, 257, 600])
@pytest.mark.parametrize("decay", [None, "mamba", "mild"])
@pytest.mark.parametrize("shape", [(16, 16, 16), (32, 16, 32)])
def test_fp32_chunk256_ragged(n, decay, shape):
    d, f, dv = shape
    c = inputs.make_prefill("c256", 2, 3, n, d, f, dv, torch.float32, None, decay, seed=n + d + 7)
    st = torch.full((2, 3, hm.state_numel(f, dv)), float("nan"), device="cuda")
    o = run_fwd(c, s_final=st, chunk=256)
    torch.cuda.synchronize()
    ref, S, z = oracle(c)
    check_prefill(f"chunk256 fp32 {shape} n={n} decay={decay}", c, o, st, ref, S, z, FP32_TOL)


@pytest.mark.parametrize("decay", [None, "mild", "mamba"])
@pytest.mark.parametrize("n", [100, 333, 700])
def test_bf16_chunk256_pythia_shape(decay, n):
    c = inputs.make_prefill("c256b", 2, 3, n, 128, 64, 128, torch.bfloat16, None, decay, seed=n + 3)
    st = torch.full((2, 3, hm.state_numel(64, 128)), float("nan"), device="cuda")
    o = run_fwd(c, s_final=st, chunk=256)
    torch.cuda.synchronize()
    ref, S, z = oracle(c)
    check_prefill(f"chunk256 bf16 (128, 64, 128) n={n} decay={decay}", c, o, st, ref, S, z, BF16_TOL)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("f", [16, 32, 64])
@pytest.mark.parametrize("dv", [16, 32, 64, 128])
def test_size_matrix_chunk256(dtype, d, f, dv):
    """Every size of the matrix on the chunk-parallel path (n = 300: a full chunk and a
    ragged one), mild decay, with an initial state."""
    c = inputs.make_prefill("cmat", 1, 2, 300, d, f, dv, dtype, None, "mild", seed=d + 3 * f + 7 * dv)
    s0 = positive_state(1, 2, 2 * f, dv, d + f + dv)
    st = torch.full_like(s0, float("nan"))
    o = run_fwd(c, s_init=s0, s_final=st, chunk=256)
    torch.cuda.synchronize()
    ref, S, z = oracle(c, s0)
    check_prefill(f"chunk256 {dtype} ({d}, {f}, {dv})", c, o, st, ref, S, z, tol_for(dtype))


@pytest.mark.parametrize("dtype,shape", [(torch.float32, (128, 64, 128)), (torch.float32, (64, 64, 64)),
                                         (torch.bfloat16, (16, 16, 16)), (torch.bfloat16, (64, 16, 64)),
                                         (torch.bfloat16, (128, 32, 16))])
@pytest.mark.parametrize("chunk", [0, 128])
@pytest.mark.parametrize("decay", [None, "mamba"])
def test_sizes_without_fused_kernel(dtype, shape, chunk, decay):
    """Sizes with no fused kernel take the chunk-parallel path at chunk 64 (automatic)
    or 128; the plan reports one segment per chunk."""
    d, f, dv = shape
    c = inputs.make_prefill("cnf", 2, 2, 517, d, f, dv, dtype, None, decay, seed=d + f + dv + chunk)
    ch, segs, ds = plan_of(c, chunk=chunk)
    assert ch == (chunk or 64) and segs == -(-517 // ch) and ds == 1
    s0 = positive_state(2, 2, 2 * f, dv, 5)
    st = torch.full_like(s0, float("nan"))
    o = run_fwd(c, s_init=s0, s_final=st, chunk=chunk)
    torch.cuda.synchronize()
    ref, S, z = oracle(c, s0)
    check_prefill(f"chunk-parallel {dtype} {shape} chunk={chunk} decay={decay}", c, o, st, ref, S, z, tol_for(dtype))


@pytest.mark.parametrize("dtype,shape", [(torch.float32, (128, 64, 128)), (torch.bfloat16, (128, 64, 128))])
def test_aliased_handoff(dtype, shape):
    """Two calls, the second continuing from the first's state in the same buffer
    (s_init and s_final alias): the scan reads each element before writing it."""
    d, f, dv = shape
    c = inputs.make_prefill("cph", 1, 2, 700, d, f, dv, dtype, None, "mild", seed=5)
    g = to_dev(c)
    st = torch.empty((1, 2, hm.state_numel(f, dv)), device="cuda")
    m = 300
    sl = lambda t, a, b: None if t is None else t[:, :, a:b]
    o1 = hm.hm_linattn_fwd(sl(g["q"], 0, m), sl(g["k"], 0, m), sl(g["v"], 0, m), g["w_q"], g["w_k"],
                           sl(g["dt"], 0, m), g["a_log"], s_final=st, chunk=256)
    o2 = hm.hm_linattn_fwd(sl(g["q"], m, 700), sl(g["k"], m, 700), sl(g["v"], m, 700), g["w_q"], g["w_k"],
                           sl(g["dt"], m, 700), g["a_log"], s_init=st, s_final=st, chunk=256)
    torch.cuda.synchronize()
    ref, S, z = oracle(c)
    tol = tol_for(dtype)
    check_bound("chunk256 handoff", np.concatenate([f64(o1), f64(o2)], axis=2), ref[..., :dv], ref[..., dv:], tol)
    Sg, zg = orc.unpack_state(f64(st), 2 * f, dv)
    assert rel_l2(Sg, S[..., :dv]) <= tol and rel_l2(zg, z) <= tol


def test_state_only_and_empty():
    """n = 0 copies s_init to s_final (zeros without s_init); B*H = 0 launches nothing."""
    c = inputs.make_prefill("c0", 1, 2, 0, 128, 64, 128, torch.float32, None, None, seed=1)
    s0 = positive_state(1, 2, 128, 128, 2)
    st = torch.full_like(s0, float("nan"))
    run_fwd(c, s_init=s0, s_final=st, chunk=256)
    st2 = torch.full_like(s0, float("nan"))
    run_fwd(c, s_final=st2, chunk=256)
    torch.cuda.synchronize()
    assert torch.equal(st, s0)
    assert torch.count_nonzero(st2).item() == 0


@pytest.mark.parametrize("dtype,shape", [(torch.float32, (32, 16, 32)), (torch.bfloat16, (128, 64, 128))])
@pytest.mark.parametrize("decay", [None, "mild"])
def test_chunk_invariance_64_128_256(dtype, shape, decay):
    """Chunk lengths 64 and 128 (fused kernels) and 256 (chunk-parallel) on the same
    inputs: each matches the oracle, and each other to the dtype's bar."""
    d, f, dv = shape
    c = inputs.make_prefill("cinv3", 2, 4, 1000, d, f, dv, dtype, None, decay, seed=9)
    outs, states = [], []
    for ch in (64, 128, 256):
        st = torch.empty((2, 4, hm.state_numel(f, dv)), device="cuda")
        outs.append(f64(run_fwd(c, s_final=st, chunk=ch)))
        states.append(f64(st))
    torch.cuda.synchronize()
    ref, S, z = oracle(c)
    tol = tol_for(dtype)
    for ch, o in zip((64, 128, 256), outs):
        check_bound(f"chunk {ch} {dtype} decay={decay}", o, ref[..., :dv], ref[..., dv:], tol)
    for i in (1, 2):
        assert report(f"chunk 64 vs {(64, 128, 256)[i]} {dtype} decay={decay} o", outs[i], outs[0]) <= tol
        assert report(f"chunk 64 vs {(64, 128, 256)[i]} {dtype} decay={decay} state", states[i], states[0]) <= tol


def test_long_context_chunk256_windows():
    """The 131072-token Mamba-decay workload with 256-token chunks: every head, windows of
    256 tokens at the head, the tail and across chunk boundaries every 16384 tokens."""
    c = inputs.long_context()
    chunk, segs, _ = plan_of(c, chunk=256)
    assert chunk == 256 and segs == c.n // 256
    w = 256
    starts = sorted({0, c.n - w} | {s * 16384 - w // 2 for s in range(1, c.n // 16384)})
    st = torch.full((1, 16, hm.state_numel(64, 128)), float("nan"), device="cuda")
    got = f64(run_fwd(c, s_final=st, chunk=256))
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
        check_bound(f"long chunk256 h={h} windows", np.concatenate(gots, axis=2), ref[..., :128], ref[..., 128:],
                    BF16_TOL)
        Sg, zg = orc.unpack_state(f64(st[0:1, h:h + 1]), 128, 128)
        assert rel_l2(Sg, S[..., :128]) <= BF16_TOL and rel_l2(zg, z) <= BF16_TOL


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_strided_layouts_and_per_head_weights(dtype):
    """q, k, v as [B, n, H, d] views (token stride H*d), o as a view of a [B, n, H, dv]
    buffer, one W per head ([H, d, f]), chunk 256 and a ragged tail: every stride the
    chunk-parallel kernels take, against the oracle head by head."""
    B, H, n, d, f, dv = 2, 3, 333, 128, 64, 128
    c = inputs.make_prefill("cstr", B, H, n, d, f, dv, dtype, None, "mild", seed=21)
    gw = torch.Generator().manual_seed(22)
    wq = (torch.randn((H, d, f), generator=gw) / d ** 0.5).to(dtype)
    wk = (torch.randn((H, d, f), generator=gw) / d ** 0.5).to(dtype)
    lay = lambda t: t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3).cuda()   # [B, H, n, x] view of [B, n, H, x]
    q, k, v = lay(c.q), lay(c.k), lay(c.v)
    assert q.stride(2) == H * d
    obuf = torch.full((B, n, H, dv), float("nan"), dtype=dtype, device="cuda")
    o = obuf.permute(0, 2, 1, 3)
    st = torch.full((B, H, hm.state_numel(f, dv)), float("nan"), device="cuda")
    hm.hm_linattn_fwd(q, k, v, wq.cuda(), wk.cuda(), c.dt.cuda(), c.a_log.cuda(), s_final=st, o=o, chunk=256)
    torch.cuda.synchronize()
    tol = tol_for(dtype)
    for h in range(H):
        sl = lambda t: f64(t[:, h:h + 1])
        ref, S, z = orc.forward(sl(c.q), sl(c.k), with_abs(sl(c.v)), f64(wq[h]), f64(wk[h]), sl(c.dt),
                                f64(c.a_log[h:h + 1]))
        check_bound(f"chunk256 strided per-head W {dtype} h={h}", f64(o[:, h:h + 1]), ref[..., :dv], ref[..., dv:], tol)
        Sg, zg = orc.unpack_state(f64(st[:, h:h + 1]), 2 * f, dv)
        assert rel_l2(Sg, S[..., :dv]) <= tol and rel_l2(zg, z) <= tol


@pytest.mark.parametrize("chunk", [0, 256])
@pytest.mark.parametrize("decay", ["mild", None])
def test_fp32_long_sequence(chunk, decay):
    """float32 at (128, 64, 128), n = 20000 (313 chunks of 64, or 79 of 256): the scan
    carries float32 states through every chunk; outputs element-wise against the
    float64 oracle at the float32 bar, and the final state."""
    c = inputs.make_prefill("cfp32long", 1, 2, 20000, 128, 64, 128, torch.float32, None, decay, seed=41)
    st = torch.full((1, 2, hm.state_numel(64, 128)), float("nan"), device="cuda")
    o = run_fwd(c, s_final=st, chunk=chunk)
    torch.cuda.synchronize()
    ref, S, z = oracle(c)
    check_prefill(f"chunk-parallel fp32 n=20000 chunk={chunk} decay={decay}", c, o, st, ref, S, z, FP32_TOL)
