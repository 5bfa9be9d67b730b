"""CPU tests of the C ABI: the library loads, exports every entry point that
include/hm.h declares, its struct layouts match the binding, and every invalid
argument is rejected with the documented status before any HIP call (fake,
never-dereferenced device addresses are used, so no GPU is needed)."""
import ctypes as C
import os
import re

import pytest

from selective_state_space_hm_amd import hm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hm.h")

A = 0x7f0000000000  # fake 16-byte aligned device address, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hm_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) == 18
    L = hm.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(hm.EXPORTS)


def test_struct_layouts_match_binding():
    L = hm.lib()
    assert L.hm_args_size(0) == C.sizeof(hm.FeaturizeArgs)
    assert L.hm_args_size(1) == C.sizeof(hm.FwdArgs)
    assert L.hm_args_size(2) == C.sizeof(hm.StepArgs)
    assert L.hm_args_size(3) == C.sizeof(hm.ConvArgs)
    assert L.hm_args_size(4) == C.sizeof(hm.BwdArgs)
    assert L.hm_args_size(5) == C.sizeof(hm.PcArgs)
    assert L.hm_args_size(6) == C.sizeof(hm.PcStepArgs)
    assert L.hm_args_size(7) == 0


def test_version_and_status_strings():
    assert hm.lib().hm_abi_version() == 9 == hm.ABI_VERSION
    with open(os.path.join(ROOT, "include", "hm.h")) as fh:
        assert re.search(r"#define HM_ABI_VERSION (\d+)", fh.read()).group(1) == str(hm.ABI_VERSION)
    for code, name in enumerate(["HM_OK", "HM_ERR_NULL", "HM_ERR_SHAPE", "HM_ERR_DTYPE", "HM_ERR_ALIGN",
                                 "HM_ERR_UNSUPPORTED", "HM_ERR_WORKSPACE", "HM_ERR_HIP"]):
        assert hm.status_string(code) == name
    assert hm.status_string(99) == "HM_ERR_UNKNOWN"


def fwd(B=2, H=16, n=2048, d=128, f=64, dv=128, dtype=hm.HM_BF16, decay=False, **kw):
    a = hm.FwdArgs(q=A, k=A + 0x1000000, v=A + 0x2000000, w_q=A + 0x3000000, w_k=A + 0x3100000,
                   o=A + 0x4000000, dtype=dtype, B=B, H=H, n=n, d=d, f=f, dv=dv,
                   sq_b=H * n * d, sq_h=n * d, sq_t=d, sk_b=H * n * d, sk_h=n * d, sk_t=d,
                   sv_b=H * n * dv, sv_h=n * dv, sv_t=dv, so_b=H * n * dv, so_h=n * dv, so_t=dv)
    if decay:
        a.dt = A + 0x5000000
        a.a_log = A + 0x6000000
        a.sdt_b, a.sdt_h, a.sdt_t = H * n, n, 1
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


def expect(st, code):
    assert st == code, f"{hm.status_string(st)} ({hm.last_error()}) != {hm.status_string(code)}"
    if code != hm.HM_OK:
        assert hm.last_error() != ""


def test_fwd_validation_errors():
    expect(hm.lib().hm_linattn_fwd(None, None), hm.HM_ERR_NULL)
    expect(hm.call_fwd(fwd(q=None)), hm.HM_ERR_NULL)
    expect(hm.call_fwd(fwd(o=None)), hm.HM_ERR_NULL)
    a = fwd()
    a.dt = A
    expect(hm.call_fwd(a), hm.HM_ERR_NULL)            # dt without A_log
    a = fwd(decay=True)
    a.a_log = None
    expect(hm.call_fwd(a), hm.HM_ERR_NULL)            # A_log without dt
    expect(hm.call_fwd(fwd(dtype=7)), hm.HM_ERR_DTYPE)
    expect(hm.call_fwd(fwd(n=-1)), hm.HM_ERR_SHAPE)
    expect(hm.call_fwd(fwd(d=0)), hm.HM_ERR_SHAPE)
    expect(hm.call_fwd(fwd(sq_t=-128)), hm.HM_ERR_SHAPE)
    expect(hm.call_fwd(fwd(so_t=64)), hm.HM_ERR_SHAPE)  # rows of o would overlap
    expect(hm.call_fwd(fwd(q=A + 2)), hm.HM_ERR_ALIGN)
    expect(hm.call_fwd(fwd(sq_t=132)), hm.HM_ERR_ALIGN)  # 264 bytes: not a multiple of 16
    expect(hm.call_fwd(fwd(s_init=A + 4)), hm.HM_ERR_ALIGN)
    expect(hm.call_fwd(fwd(d=96)), hm.HM_ERR_UNSUPPORTED)
    expect(hm.call_fwd(fwd(f=48)), hm.HM_ERR_UNSUPPORTED)
    # sizes without a fused kernel (float32 at d=128, bf16 at d=16) run the chunk-parallel
    # path: one "segment" per 64-token chunk, no column split
    assert hm.call_plan(fwd(dtype=hm.HM_F32)) == (hm.HM_OK, (64, 32, 1))
    assert hm.call_plan(fwd(d=16, f=16, dv=32)) == (hm.HM_OK, (64, 32, 1))
    # the small bf16 shapes have fused kernels
    expect(hm.call_plan(fwd(d=32, f=16, dv=32))[0], hm.HM_OK)
    expect(hm.call_plan(fwd(dv=32))[0], hm.HM_OK)
    assert hm.call_plan(fwd(d=32, f=16, dv=64)) == (hm.HM_OK, (64, 4, 2))  # two 32-column workgroups
    expect(hm.call_fwd(fwd(d=32, f=16, dv=64, dsplit=1)), hm.HM_ERR_UNSUPPORTED)
    # what the chunk-parallel path does not take: gate, rotary, saves, segments, column splits
    G0 = dict(gate=A + 0xa000000, sg_b=16 * 2048 * 128, sg_h=2048 * 128, sg_t=128)
    expect(hm.call_fwd(fwd(dtype=hm.HM_F32, **G0)), hm.HM_ERR_UNSUPPORTED)
    expect(hm.call_fwd(fwd(d=16, f=16, dv=32, segments=2)), hm.HM_ERR_UNSUPPORTED)
    expect(hm.call_fwd(fwd(chunk=96)), hm.HM_ERR_UNSUPPORTED)
    assert hm.call_plan(fwd(chunk=256)) == (hm.HM_OK, (256, 8, 1))
    expect(hm.call_fwd(fwd(chunk=256, **G0)), hm.HM_ERR_UNSUPPORTED)
    expect(hm.call_fwd(fwd(chunk=256, rope_dims=32, rope_base=1e4)), hm.HM_ERR_UNSUPPORTED)
    expect(hm.call_fwd(fwd(chunk=256, segments=4)), hm.HM_ERR_UNSUPPORTED)
    expect(hm.call_fwd(fwd(chunk=256, dsplit=2)), hm.HM_ERR_UNSUPPORTED)
    expect(hm.call_fwd(fwd(chunk=256, d=96)), hm.HM_ERR_UNSUPPORTED)
    expect(hm.call_fwd(fwd(chunk=128, gate=A + 0xa000000, sg_t=128)), hm.HM_ERR_UNSUPPORTED)
    expect(hm.call_fwd(fwd(chunk=128, rope_dims=32, rope_base=1e4)), hm.HM_ERR_UNSUPPORTED)
    expect(hm.call_fwd(fwd(chunk=128, d=16, f=16, dv=16, dtype=hm.HM_F32, save=A + 0xb000000, save_bytes=1 << 30)),
           hm.HM_ERR_UNSUPPORTED)
    expect(hm.call_fwd(fwd(dsplit=3)), hm.HM_ERR_UNSUPPORTED)
    expect(hm.call_fwd(fwd(segments=-2)), hm.HM_ERR_SHAPE)
    G = A + 0xa000000
    g = dict(sg_b=16 * 2048 * 128, sg_h=2048 * 128, sg_t=128)
    expect(hm.call_fwd(fwd(gate=G + 8, **g)), hm.HM_ERR_ALIGN)
    expect(hm.call_fwd(fwd(gate=G, **{**g, "sg_t": 132})), hm.HM_ERR_ALIGN)
    expect(hm.call_fwd(fwd(gate=G, **{**g, "sg_h": -128})), hm.HM_ERR_SHAPE)
    expect(hm.call_fwd(fwd(gate=G, B=0, **g)), hm.HM_OK)     # a read-only input: stride 0 (broadcast) is fine
    expect(hm.call_fwd(fwd(gate=G, B=0, sg_b=0, sg_h=0, sg_t=0)), hm.HM_OK)


def test_fwd_workspace_required_when_segmented():
    a = fwd(B=1, H=16, n=131072, decay=True)
    st, nbytes = hm.call_workspace_size(a)
    expect(st, hm.HM_OK)
    assert nbytes > 0
    expect(hm.call_fwd(a), hm.HM_ERR_WORKSPACE)        # NULL workspace
    a.workspace = A + 0x7000000
    a.workspace_bytes = nbytes - 16
    expect(hm.call_fwd(a), hm.HM_ERR_WORKSPACE)        # too small
    a.workspace_bytes = nbytes
    a.workspace = A + 0x7000004
    expect(hm.call_fwd(a), hm.HM_ERR_ALIGN)


def test_workspace_is_linear_not_quadratic():
    # explicit segment count: the workspace does not depend on n at all
    sizes = [hm.call_workspace_size(fwd(B=1, H=16, n=n, segments=8))[1] for n in (4096, 65536, 1 << 20)]
    assert sizes[0] == sizes[1] == sizes[2]
    # 7 segments before the last; 112 segment-pass items, so each is cut into 2 slots
    F, dv, BH, slots = 128, 128, 16, 14
    assert sizes[0] == slots * BH * (F * dv + F) * 4 + 4 * ((slots * BH + 3) // 4 * 4)
    # automatic plans stay bounded by the segment cap as n grows
    auto = [hm.call_workspace_size(fwd(B=1, H=16, n=n, decay=True))[1] for n in (8192, 131072, 1 << 21)]
    assert max(auto) <= 512 * (F * dv + F) * 4 * 2
    assert hm.call_workspace_size(fwd(B=8, H=16, n=2048, segments=1))[1] == 0


def test_chunk_parallel_workspace():
    # every chunk's state and summed log-decay: O(B*H*(n/C)*F*dv), linear in n
    F, dv = 128, 128
    for n, C in ((2048, 256), (1000, 256), (4096, 64)):
        st, nbytes = hm.call_workspace_size(fwd(B=2, H=16, n=n, chunk=C, decay=True) if C == 256 else
                                            fwd(B=2, H=16, n=n, dtype=hm.HM_F32, decay=True))
        expect(st, hm.HM_OK)
        nc = -(-n // C)
        assert nbytes == 32 * nc * (F * dv + F) * 4 + 4 * ((32 * nc + 3) // 4 * 4)


def test_plans():
    st, plan = hm.call_plan(fwd(B=8, H=16, n=2048))
    expect(st, hm.HM_OK)
    assert plan[0] == 64 and plan[2] in (1, 2)
    # 128-token chunks: segments start on chunk bounds and hold at least four chunks
    st, plan = hm.call_plan(fwd(B=1, H=16, n=131072, decay=True, chunk=128))
    expect(st, hm.HM_OK)
    assert plan == (128, 16, 1)
    st, plan = hm.call_plan(fwd(B=1, H=2, n=300, d=16, f=16, dv=16, dtype=hm.HM_F32, chunk=128, segments=3))
    expect(st, hm.HM_OK)
    assert plan[0] == 128 and plan[1] == 3
    st, plan = hm.call_plan(fwd(B=1, H=16, n=131072, decay=True))
    expect(st, hm.HM_OK)
    assert plan[1] > 1                                  # long context is segmented
    st, plan = hm.call_plan(fwd(B=1, H=16, n=131072, decay=True, segments=4, dsplit=1))
    assert plan == (64, 4, 1)
    st, plan = hm.call_plan(fwd(B=1, H=16, n=100, segments=50))
    assert plan[1] == 2                                 # at most one segment per chunk
    st, plan = hm.call_plan(fwd(B=1, H=2, n=256, d=16, f=16, dv=16, dtype=hm.HM_F32))
    expect(st, hm.HM_OK)
    assert plan[2] == 1                                 # dv=16 cannot be split
    for f_, dv_ in ((16, 16), (16, 32), (32, 32), (32, 64)):   # float32 at d = 64
        st, plan = hm.call_plan(fwd(B=1, H=2, n=256, d=64, f=f_, dv=dv_, dtype=hm.HM_F32))
        expect(st, hm.HM_OK)
    # float32 (64, 64, 64) has no fused kernel: the chunk-parallel path, 4 chunks of 64
    assert hm.call_plan(fwd(B=1, H=2, n=256, d=64, f=64, dv=64, dtype=hm.HM_F32)) == (hm.HM_OK, (64, 4, 1))


def test_alias_needs_init_copy_workspace():
    a = fwd(B=1, H=16, n=4096, dsplit=2, segments=1)
    st, base = hm.call_workspace_size(a)
    a.s_init = A + 0x8000000
    a.s_final = A + 0x8000000
    st, aliased = hm.call_workspace_size(a)
    expect(st, hm.HM_OK)
    assert aliased - base == 16 * (128 * 128 + 128) * 4


def test_zero_sizes_are_valid_without_launch():
    # B*H == 0 and (n == 0 without s_final) return before any HIP call
    expect(hm.call_fwd(fwd(B=0)), hm.HM_OK)
    expect(hm.call_fwd(fwd(n=0)), hm.HM_OK)


def step(B=256, H=16, d=128, f=64, dv=128, dtype=hm.HM_BF16, **kw):
    a = hm.StepArgs(q=A, k=A + 0x100000, v=A + 0x200000, w_q=A + 0x300000, w_k=A + 0x310000,
                    state=A + 0x400000, o=A + 0x9000000, dtype=dtype, B=B, H=H, d=d, f=f, dv=dv,
                    sq_b=H * d, sq_h=d, sk_b=H * d, sk_h=d, sv_b=H * dv, sv_h=dv, so_b=H * dv, so_h=dv)
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


def test_step_validation_errors():
    expect(hm.lib().hm_linattn_step(None, None), hm.HM_ERR_NULL)
    expect(hm.call_step(step(state=None)), hm.HM_ERR_NULL)
    expect(hm.call_step(step(dt=A)), hm.HM_ERR_NULL)
    expect(hm.call_step(step(dtype=5)), hm.HM_ERR_DTYPE)
    expect(hm.call_step(step(B=-1)), hm.HM_ERR_SHAPE)
    expect(hm.call_step(step(state=A + 8)), hm.HM_ERR_ALIGN)
    expect(hm.call_step(step(sq_h=100)), hm.HM_ERR_ALIGN)
    expect(hm.call_step(step(d=48)), hm.HM_ERR_UNSUPPORTED)
    expect(hm.call_step(step(f=48)), hm.HM_ERR_UNSUPPORTED)
    expect(hm.call_step(step(dv=96)), hm.HM_ERR_UNSUPPORTED)
    expect(hm.call_step(step(gate=A + 0xa000008, sg_b=16 * 128, sg_h=128)), hm.HM_ERR_ALIGN)
    expect(hm.call_step(step(gate=A + 0xa000000, sg_b=16 * 128, sg_h=100)), hm.HM_ERR_ALIGN)
    expect(hm.call_step(step(gate=A + 0xa000000, sg_b=-1, sg_h=128)), hm.HM_ERR_SHAPE)
    cv = dict(conv_wq=A + 0xb000000, conv_wk=A + 0xb100000, conv_sq=A + 0xb200000, conv_sk=A + 0xb300000)
    expect(hm.call_step(step(conv_width=5, **cv)), hm.HM_ERR_UNSUPPORTED)
    expect(hm.call_step(step(conv_width=-1, **cv)), hm.HM_ERR_SHAPE)
    expect(hm.call_step(step(conv_width=4, **{**cv, "conv_sk": None})), hm.HM_ERR_NULL)
    # one tap needs no state: the conv checks pass and the size check comes next
    expect(hm.call_step(step(conv_width=1, d=48, **{**cv, "conv_sk": None, "conv_sq": None})), hm.HM_ERR_UNSUPPORTED)
    expect(hm.call_step(step(conv_width=4, B=0, **cv)), hm.HM_OK)
    expect(hm.call_step(step(conv_width=4, **{**cv, "conv_sq": A + 0xb200001})), hm.HM_ERR_ALIGN)
    expect(hm.call_step(step(conv_width=4, **{**cv, "conv_wq": A + 0xb000002})), hm.HM_ERR_ALIGN)
    expect(hm.call_step(step(B=0)), hm.HM_OK)


def feat(B=2, H=16, n=2048, d=128, f=64, dtype=hm.HM_BF16, phi_dtype=hm.HM_BF16, **kw):
    a = hm.FeaturizeArgs(x=A, w=A + 0x1000000, phi=A + 0x2000000, dtype=dtype, phi_dtype=phi_dtype,
                         B=B, H=H, n=n, d=d, f=f, sx_b=H * n * d, sx_h=n * d, sx_t=d,
                         sp_b=H * n * 2 * f, sp_h=n * 2 * f, sp_t=2 * f)
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


def test_featurize_validation_errors():
    expect(hm.lib().hm_featurize(None, None), hm.HM_ERR_NULL)
    expect(hm.call_featurize(feat(phi=None)), hm.HM_ERR_NULL)
    expect(hm.call_featurize(feat(phi_dtype=3)), hm.HM_ERR_DTYPE)
    expect(hm.call_featurize(feat(f=-1)), hm.HM_ERR_SHAPE)
    expect(hm.call_featurize(feat(sp_t=64)), hm.HM_ERR_SHAPE)
    expect(hm.call_featurize(feat(x=A + 6)), hm.HM_ERR_ALIGN)
    expect(hm.call_featurize(feat(d=24)), hm.HM_ERR_UNSUPPORTED)
    # the fused short conv: widths 0..4, taps required, aligned state
    expect(hm.call_featurize(feat(conv_width=5, conv_w=A + 0x5000000)), hm.HM_ERR_UNSUPPORTED)
    expect(hm.call_featurize(feat(conv_width=2)), hm.HM_ERR_NULL)
    expect(hm.call_featurize(feat(conv_width=2, conv_w=A + 0x5000000, scw_h=-1)), hm.HM_ERR_SHAPE)
    expect(hm.call_featurize(feat(conv_width=2, conv_w=A + 0x5000000, conv_prev=A + 0x6000008)), hm.HM_ERR_ALIGN)
    expect(hm.call_featurize(feat(n=0)), hm.HM_OK)


def conv(B=2, H=16, n=2048, d=128, width=4, dtype=hm.HM_BF16, **kw):
    a = hm.ConvArgs(x=A, y=A + 0x1000000, w=A + 0x2000000, bias=A + 0x2100000, dtype=dtype, width=width,
                    B=B, H=H, n=n, d=d, sx_b=H * n * d, sx_h=n * d, sx_t=d, sy_b=H * n * d, sy_h=n * d, sy_t=d)
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


def test_conv_validation_errors():
    L = hm.lib()
    expect(L.hm_causal_conv(None, None), hm.HM_ERR_NULL)
    expect(hm.call_conv(conv(w=None)), hm.HM_ERR_NULL)
    expect(hm.call_conv(conv(dtype=4)), hm.HM_ERR_DTYPE)
    expect(hm.call_conv(conv(width=0)), hm.HM_ERR_SHAPE)
    expect(hm.call_conv(conv(width=5)), hm.HM_ERR_UNSUPPORTED)
    expect(hm.call_conv(conv(n=-3)), hm.HM_ERR_SHAPE)
    expect(hm.call_conv(conv(sy_t=64)), hm.HM_ERR_SHAPE)               # rows of y overlap
    expect(hm.call_conv(conv(d=12)), hm.HM_ERR_UNSUPPORTED)            # 24 bytes per row
    expect(hm.call_conv(conv(x=A + 8)), hm.HM_ERR_ALIGN)
    expect(hm.call_conv(conv(bias=A + 2)), hm.HM_ERR_ALIGN)
    expect(hm.call_conv(conv(sw_h=127)), hm.HM_ERR_ALIGN)
    expect(hm.call_conv(conv(sx_t=132)), hm.HM_ERR_ALIGN)
    expect(hm.call_conv(conv(y=A + 0x100)), hm.HM_ERR_SHAPE)           # y overlaps x
    expect(hm.call_conv(conv(prev=A + 0x3000000, final_rows=A + 0x3000100)), hm.HM_ERR_SHAPE)
    expect(hm.call_conv(conv(B=0)), hm.HM_OK)
    expect(hm.call_conv(conv(n=0)), hm.HM_OK)                           # nothing to write
    expect(hm.call_conv(conv(n=0, width=1, final_rows=A + 0x3000000)), hm.HM_OK)
    expect(hm.call_conv(conv(n=0, x=None, y=None, w=None)), hm.HM_OK)  # nothing is read
    expect(hm.call_conv(conv(n=1, y=None)), hm.HM_ERR_NULL)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(hm, "_lib", None)
    monkeypatch.setattr(hm, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        hm.lib()


def test_null_pointers_allowed_when_nothing_to_compute():
    a = fwd(n=0, q=None, k=None, v=None, o=None, w_q=None, w_k=None)
    expect(hm.call_fwd(a), hm.HM_OK)
    expect(hm.call_fwd(fwd(n=5, q=None)), hm.HM_ERR_NULL)
    expect(hm.call_step(step(B=0, q=None, state=None)), hm.HM_OK)
    expect(hm.call_featurize(feat(n=0, x=None, phi=None)), hm.HM_OK)


def bwd(B=2, H=16, n=2048, d=128, f=64, dv=128, dtype=hm.HM_BF16, decay=False, **kw):
    a = hm.BwdArgs(q=A, k=A + 0x1000000, v=A + 0x2000000, w_q=A + 0x3000000, w_k=A + 0x3100000,
                   d_o=A + 0x4800000, save=A + 0x5000000, save_bytes=1 << 40,
                   d_q=A + 0x6000000, d_k=A + 0x7000000, d_v=A + 0x8000000, d_wq=A + 0x9000000,
                   d_wk=A + 0x9100000, dtype=dtype, B=B, H=H, n=n, d=d, f=f, dv=dv,
                   sq_b=H * n * d, sq_h=n * d, sq_t=d, sk_b=H * n * d, sk_h=n * d, sk_t=d,
                   sv_b=H * n * dv, sv_h=n * dv, sv_t=dv, so_b=H * n * dv, so_h=n * dv, so_t=dv)
    if decay:
        a.dt, a.a_log, a.d_dt, a.d_a_log = A + 0xa000000, A + 0xa100000, A + 0xa200000, A + 0xa300000
        a.sdt_b, a.sdt_h, a.sdt_t = H * n, n, 1
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


def test_backward_validation_and_sizes():
    L = hm.lib()
    expect(L.hm_linattn_bwd(None, None), hm.HM_ERR_NULL)
    expect(hm.call_bwd(bwd(d_o=None)), hm.HM_ERR_NULL)
    expect(hm.call_bwd(bwd(save=None)), hm.HM_ERR_NULL)
    expect(hm.call_bwd(bwd(decay=True, d_dt=None)), hm.HM_ERR_NULL)
    expect(hm.call_bwd(bwd(gate=A + 0xb000000, sg_b=16 * 2048 * 128, sg_h=2048 * 128, sg_t=128)), hm.HM_ERR_NULL)
    expect(hm.call_bwd(bwd(dtype=9)), hm.HM_ERR_DTYPE)
    expect(hm.call_bwd(bwd(n=-1)), hm.HM_ERR_SHAPE)
    expect(hm.call_bwd(bwd(sw_h=7)), hm.HM_ERR_SHAPE)                  # per-head W must be contiguous
    expect(hm.call_bwd(bwd(d_q=A + 0x6000008)), hm.HM_ERR_ALIGN)
    expect(hm.call_bwd(bwd(d=96)), hm.HM_ERR_UNSUPPORTED)
    expect(hm.call_bwd(bwd(f=32)), hm.HM_ERR_UNSUPPORTED)              # (128, 32, 128) has no backward build
    expect(hm.call_bwd(bwd()), hm.HM_ERR_WORKSPACE)                     # no workspace
    expect(hm.call_bwd(bwd(B=0)), hm.HM_OK)
    st, nb = hm.call_bwd_workspace_size(bwd(B=8, H=16, n=2048))
    expect(st, hm.HM_OK)
    F, BH, n = 128, 128, 2048
    # features, dnum and the chunk-end gradient states dominate: O(B*H*n*(2F + dv)), no n^2 term
    assert 2 * (BH * n * (2 * F + 128)) < nb < 2 * (BH * n * (2 * F + 128)) * 2 + 64 << 20
    a = hm.FwdArgs(dtype=hm.HM_BF16, B=8, H=16, n=2048, d=128, f=64, dv=128)
    st, sb = hm.call_save_size(a)
    expect(st, hm.HM_OK)
    # float32 checkpoints at the start of the backward's chunk ranges (256 workgroups over
    # 128 (b, h): 2 ranges of 16 chunks each), denominators, float32 output before the gate
    assert sb == BH * 2 * (F * 128 + F) * 4 + BH * n * 4 + BH * n * 128 * 4
    expect(hm.call_fwd(fwd(B=8, segments=1, save=A + 0xc000000, save_bytes=sb - 1)), hm.HM_ERR_WORKSPACE)
    assert "save" in hm.last_error()
    expect(hm.call_fwd(fwd(save=A + 0xc000000, save_bytes=sb, dsplit=2)), hm.HM_ERR_UNSUPPORTED)
    expect(hm.call_fwd(fwd(save=A + 0xc000004, save_bytes=sb)), hm.HM_ERR_ALIGN)


def test_rotary_field_validation():
    P = A + 0xd000000  # fake int64 position array
    for mk, call in ((fwd, hm.call_fwd), (feat, hm.call_featurize)):
        expect(call(mk(rope_dims=-32, rope_base=1e4)), hm.HM_ERR_SHAPE)
        expect(call(mk(rope_dims=33, rope_base=1e4)), hm.HM_ERR_SHAPE)        # odd
        expect(call(mk(rope_dims=160, rope_base=1e4)), hm.HM_ERR_SHAPE)       # above 2f = 128
        expect(call(mk(rope_dims=48, rope_base=1e4)), hm.HM_ERR_UNSUPPORTED)  # even, not a multiple of 32
        expect(call(mk(rope_dims=64, rope_base=0.0)), hm.HM_ERR_SHAPE)
        expect(call(mk(rope_dims=64, rope_base=-2.0)), hm.HM_ERR_SHAPE)
        expect(call(mk(rope_dims=64, rope_base=float("inf"))), hm.HM_ERR_SHAPE)
        expect(call(mk(rope_dims=64, rope_base=float("nan"))), hm.HM_ERR_SHAPE)
        expect(call(mk(rope_dims=64, rope_base=1e4, rope_pos0=P + 4)), hm.HM_ERR_ALIGN)
        expect(call(mk(rope_dims=64, rope_base=1e4, B=0)), hm.HM_OK)           # nothing to compute
    # with the rotation, prefill kernels exist for (128, 64) and (64, 32) only
    expect(hm.call_fwd(fwd(f=32, rope_dims=32, rope_base=1e4)), hm.HM_ERR_UNSUPPORTED)
    expect(hm.call_fwd(fwd(d=64, f=32, rope_dims=64, rope_base=1e4, B=0)), hm.HM_OK)
    # the training forward too (the size check runs first; B = 0 launches nothing)
    expect(hm.call_fwd(fwd(B=0, rope_dims=128, rope_base=1e4, save=A + 0xc000000, save_bytes=1 << 30)), hm.HM_OK)
    # decode: the positions are required when the rotation is on
    expect(hm.call_step(step(rope_dims=64, rope_base=1e4)), hm.HM_ERR_NULL)
    expect(hm.call_step(step(rope_dims=64, rope_base=1e4, rope_pos=P + 8 + 4)), hm.HM_ERR_ALIGN)
    expect(hm.call_step(step(rope_dims=48, rope_base=1e4, rope_pos=P)), hm.HM_ERR_UNSUPPORTED)
    expect(hm.call_step(step(rope_dims=64, rope_base=1e4, B=0)), hm.HM_OK)
    # backward
    expect(hm.call_bwd(bwd(rope_dims=96, rope_base=0.5, rope_pos0=P + 2)), hm.HM_ERR_ALIGN)
    expect(hm.call_bwd(bwd(rope_dims=200, rope_base=1e4)), hm.HM_ERR_SHAPE)
    expect(hm.call_bwd(bwd(rope_dims=128, rope_base=1e4)), hm.HM_ERR_WORKSPACE)  # valid; no workspace given


def pc(B=2, H=16, n=2048, d=128, f=64, dv=128, dtype=hm.HM_BF16, **kw):
    a = hm.PcArgs(q=A, k=A + 0x1000000, v=A + 0x2000000, w_q=A + 0x3000000, w_k=A + 0x3100000,
                  dt=A + 0x5000000, a_log=A + 0x6000000, o=A + 0x4000000, dtype=dtype, B=B, H=H, n=n, d=d, f=f,
                  dv=dv, sq_b=H * n * d, sq_h=n * d, sq_t=d, sk_b=H * n * d, sk_h=n * d, sk_t=d,
                  sv_b=H * n * dv, sv_h=n * dv, sv_t=dv, so_b=H * n * dv, so_h=n * dv, so_t=dv,
                  sdt_b=H * n * dv, sdt_h=n * dv, sdt_t=dv, sa_h=dv * 2 * f)
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


def pc_step(B=256, H=16, d=128, f=64, dv=128, dtype=hm.HM_BF16, **kw):
    a = hm.PcStepArgs(q=A, k=A + 0x100000, v=A + 0x200000, w_q=A + 0x300000, w_k=A + 0x310000,
                      dt=A + 0x320000, a_log=A + 0x340000, state=A + 0x400000, o=A + 0x9000000, dtype=dtype,
                      B=B, H=H, d=d, f=f, dv=dv, sq_b=H * d, sq_h=d, sk_b=H * d, sk_h=d, sv_b=H * dv, sv_h=dv,
                      so_b=H * dv, so_h=dv, sdt_b=H * dv, sdt_h=dv, sa_h=0)
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


def test_per_channel_segment_plan():
    """Automatic segments only when fewer than 65 workgroups (one per (b, h) and 64
    channels) would run: up to 256 / workgroups segments of at least four chunks."""
    def plan(**kw):
        st, ns = hm.call_pc_plan(pc(**kw))
        expect(st, hm.HM_OK)
        st, nb = hm.call_pc_workspace_size(pc(**kw))
        expect(st, hm.HM_OK)
        return ns, nb
    blk = 2 * 128 * 128 * 4
    ns, nb = plan()                                   # B*H = 32, 2 channel groups: 64 workgroups
    assert ns == 4 and nb == (32 * 4 * blk + 255) // 256 * 256 + 32 * 3 * 128 * 4
    assert plan(B=1, n=131072)[0] == 8                # 32 workgroups: 8 segments of 256 chunks
    assert plan(B=8) == (1, 0)                        # 256 workgroups: one segment, no workspace
    assert plan(B=1, n=256)[0] == 1                   # four chunks: too short to split
    assert plan(segments=3)[0] == 3                   # 11 + 11 + 10 chunks
    assert plan(segments=100)[0] == 32                # at most one segment per chunk
    assert plan(n=100, segments=5)[0] == 2
    assert plan(segments=1) == (1, 0)
    assert plan(n=0) == (1, 0)
    expect(hm.call_pc_plan(pc(segments=-1))[0], hm.HM_ERR_SHAPE)
    expect(hm.call_pc_plan(pc(d=96))[0], hm.HM_ERR_UNSUPPORTED)
    expect(hm.call_pc_fwd(pc(segments=-2)), hm.HM_ERR_SHAPE)
    expect(hm.call_pc_fwd(pc()), hm.HM_ERR_WORKSPACE)                  # 4 segments, no workspace
    assert "workspace" in hm.last_error()
    expect(hm.call_pc_fwd(pc(workspace=A + 0xa000000, workspace_bytes=nb - 1)), hm.HM_ERR_WORKSPACE)
    expect(hm.call_pc_fwd(pc(workspace=A + 0xa000008, workspace_bytes=nb)), hm.HM_ERR_ALIGN)
    expect(hm.call_pc_fwd(pc(B=0, workspace=None)), hm.HM_OK)         # nothing to run


def test_per_channel_validation():
    L = hm.lib()
    expect(L.hm_linattn_pc_fwd(None, None), hm.HM_ERR_NULL)
    expect(hm.call_pc_fwd(pc(dt=None)), hm.HM_ERR_NULL)
    expect(hm.call_pc_fwd(pc(a_log=None)), hm.HM_ERR_NULL)
    expect(hm.call_pc_fwd(pc(q=None)), hm.HM_ERR_NULL)
    expect(hm.call_pc_fwd(pc(n=0, q=None, k=None, v=None, o=None, w_q=None, w_k=None)), hm.HM_OK)  # no token, no s_final
    expect(hm.call_pc_fwd(pc(dtype=4)), hm.HM_ERR_DTYPE)
    expect(hm.call_pc_fwd(pc(dv=-1)), hm.HM_ERR_SHAPE)
    expect(hm.call_pc_fwd(pc(sa_h=7)), hm.HM_ERR_SHAPE)                 # A_log shared or one block per head
    expect(hm.call_pc_fwd(pc(sdt_t=64)), hm.HM_ERR_SHAPE)               # dt rows overlap
    expect(hm.call_pc_fwd(pc(a_log=A + 0x6000004)), hm.HM_ERR_ALIGN)
    expect(hm.call_pc_fwd(pc(dt=A + 0x5000002)), hm.HM_ERR_ALIGN)
    expect(hm.call_pc_fwd(pc(s_final=A + 0x7000008)), hm.HM_ERR_ALIGN)
    expect(hm.call_pc_fwd(pc(d=96)), hm.HM_ERR_UNSUPPORTED)
    expect(hm.call_pc_fwd(pc(f=32)), hm.HM_ERR_UNSUPPORTED)             # (128, 32, 128) is not built
    expect(hm.call_pc_fwd(pc(rope_dims=48, rope_base=1e4)), hm.HM_ERR_UNSUPPORTED)
    blk = 2 * 128 * 128 * 4
    expect(hm.call_pc_fwd(pc(s_init=A + 0x8000000, s_final=A + 0x8000000 + blk)), hm.HM_ERR_SHAPE)  # partial overlap
    expect(hm.call_pc_fwd(pc(B=0, s_init=A + 0x8000000, s_final=A + 0x8000000)), hm.HM_OK)
    expect(L.hm_linattn_pc_step(None, None), hm.HM_ERR_NULL)
    expect(hm.call_pc_step(pc_step(dt=None, a_log=None)), hm.HM_ERR_NULL)
    expect(hm.call_pc_step(pc_step(state=None)), hm.HM_ERR_NULL)
    expect(hm.call_pc_step(pc_step(sa_h=5)), hm.HM_ERR_SHAPE)
    expect(hm.call_pc_step(pc_step(a_log=A + 0x340008)), hm.HM_ERR_ALIGN)
    expect(hm.call_pc_step(pc_step(d=48)), hm.HM_ERR_UNSUPPORTED)
    expect(hm.call_pc_step(pc_step(rope_dims=64, rope_base=1e4)), hm.HM_ERR_NULL)      # positions required
    expect(hm.call_pc_step(pc_step(conv_width=5)), hm.HM_ERR_UNSUPPORTED)
    expect(hm.call_pc_step(pc_step(B=0)), hm.HM_OK)


# ------------------------------------------------------------ binding checks
# The torch binding validates sizes, dtypes and layouts before it marshals a
# pointer: the C ABI only sees raw addresses, so an undersized state or a
# transposed W would otherwise be read or written wrongly on the GPU.  The checks
# run before the device check, so CPU tensors exercise them here; a well-formed
# CPU call stops at "must be on the GPU".
def _cpu_layer(B=2, H=3, n=5, d=32, f=16, dv=32, dtype=None):
    import torch
    dtype = dtype or torch.bfloat16
    g = torch.Generator().manual_seed(0)
    mk = lambda *s: torch.randn(s, generator=g).to(dtype)
    return mk(B, H, n, d), mk(B, H, n, d), mk(B, H, n, dv), mk(d, f), mk(d, f)


def _bad(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


def test_binding_rejects_bad_prefill_tensors():
    import torch
    q, k, v, wq, wk = _cpu_layer()
    B, H, n, d = q.shape
    f, dv = wq.shape[1], v.shape[-1]
    blk = hm.state_numel(f, dv)
    fwd = hm.hm_linattn_fwd
    _bad(lambda: fwd(q, k, v, wq, wk), "on the GPU")                               # well formed
    _bad(lambda: fwd(q, k[:, :, :4], v, wq, wk), "k must have shape")
    _bad(lambda: fwd(q, k, v[:, :, :4], wq, wk), "v must be")
    _bad(lambda: fwd(q, k.float(), v, wq, wk), "k must have q's dtype")
    _bad(lambda: fwd(q, k, v.float(), wq, wk), "v must have q's dtype")
    _bad(lambda: fwd(q, k, v, wq.float(), wk), "w_q must have q's dtype")
    _bad(lambda: fwd(q, k, v, wq, wk, o=torch.empty(B, H, n, dv)), "o must have q's dtype")
    _bad(lambda: fwd(q, k, v, wq, wk, o=torch.empty(B, H, n, dv - 8, dtype=q.dtype)), "o must have shape")
    # a transposed view of a [f, d] weight has the right shape but strides (1, d)
    _bad(lambda: fwd(q, k, v, wq.t().contiguous().t(), wk), "row-major")
    _bad(lambda: fwd(q, k, v, wq[:16], wk), r"w_q must be \[32, 16\]")
    _bad(lambda: fwd(q, k, v, wq.expand(H + 1, d, f), wk.expand(H + 1, d, f)), "3 heads")
    _bad(lambda: fwd(q, k, v, wq.expand(H, d, f).contiguous(), wk), "same layout")
    _bad(lambda: fwd(q, k, v, wq, wk, s_init=torch.zeros(B, H, blk - 1)), "s_init must have shape")
    _bad(lambda: fwd(q, k, v, wq, wk, s_final=torch.zeros(B, H, blk, dtype=torch.bfloat16)), "s_final must be float32")
    _bad(lambda: fwd(q, k, v, wq, wk, s_final=torch.zeros(B, blk, H).transpose(1, 2)), "contiguous")
    _bad(lambda: fwd(q, k, v, wq, wk, gate=torch.zeros(B, H, n, dv + 8, dtype=q.dtype)), "gate must have shape")
    _bad(lambda: fwd(q, k, v, wq, wk, dt=torch.zeros(B, H, n)), "given together")
    _bad(lambda: fwd(q, k, v, wq, wk, dt=torch.zeros(B, H, n + 1), a_log=torch.zeros(H)), "dt must have shape")
    _bad(lambda: fwd(q, k, v, wq, wk, dt=torch.zeros(B, H, n), a_log=torch.zeros(H + 1)), "a_log must have shape")
    _bad(lambda: fwd(q, k, v, wq, wk, dt=torch.zeros(B, H, n, dtype=torch.float64), a_log=torch.zeros(H)), "float32")
    _bad(lambda: hm.hm_linattn_fwd_plan(q, k, v, wq.t().contiguous().t(), wk), "row-major")


def test_binding_rejects_bad_step_and_featurize_tensors():
    import torch
    q, k, v, wq, wk = _cpu_layer()
    B, H, d = q.shape[0], q.shape[1], q.shape[-1]
    f, dv = wq.shape[1], v.shape[-1]
    q1, k1, v1 = q[:, :, 0], k[:, :, 0], v[:, :, 0]
    st = torch.zeros(B, H, hm.state_numel(f, dv))
    step = hm.hm_linattn_step
    _bad(lambda: step(q1, k1, v1, wq, wk, st), "on the GPU")                       # well formed
    _bad(lambda: step(q1, k1, v1, wq, wk, st[:, :, :-4]), "state must have shape")
    _bad(lambda: step(q1, k1, v1, wq, wk, st.to(torch.bfloat16)), "state must be float32")
    _bad(lambda: step(q1, k1, v1, wq, wk, st, dt=torch.zeros(B, H + 1), a_log=torch.zeros(H)), "dt must have shape")
    _bad(lambda: step(q1, k1.float(), v1, wq, wk, st), "k must have q's dtype")
    _bad(lambda: step(q1, k1, v1, wq.t().contiguous().t(), wk, st), "row-major")
    _bad(lambda: step(q1, k1, v1, wq, wk, st, o=torch.empty(B, H, dv + 8, dtype=q.dtype)), "o must have shape")
    _bad(lambda: step(q, k, v, wq, wk, st), "3 dimensions")
    _bad(lambda: hm.hm_featurize(q, wq.t().contiguous().t()), "row-major")
    _bad(lambda: hm.hm_featurize(q, wq.float()), "dtype")
    _bad(lambda: hm.hm_featurize(q, wq, phi=torch.empty(B, H, q.shape[2], f, dtype=q.dtype)), "phi must have shape")
    _bad(lambda: hm.hm_featurize(q, wq), "on the GPU")


def test_binding_rejects_bad_backward_and_per_channel_tensors():
    import torch
    q, k, v, wq, wk = _cpu_layer()
    B, H, n, d = q.shape
    f, dv = wq.shape[1], v.shape[-1]
    save = torch.empty(hm.save_size(q, v, wq), dtype=torch.uint8)
    d_o = torch.randn(B, H, n, dv).to(q.dtype)
    bwd = hm.hm_linattn_bwd
    _bad(lambda: bwd(q, k, v, wq, wk, d_o, save), "on the GPU")                    # well formed
    _bad(lambda: bwd(q, k, v, wq, wk, d_o[:, :, :3], save), "o must have shape")
    _bad(lambda: bwd(q, k, v, wq, wk, d_o, save[:-16]), "save buffer too small")
    _bad(lambda: bwd(q, k, v, wq, wk, d_o, save, d_s_final=torch.zeros(B, H, 7)), "d_s_final must have shape")
    _bad(lambda: bwd(q, k, v, wq.t().contiguous().t(), wk, d_o, save), "row-major")
    F = 2 * f
    dt = torch.zeros(B, H, n, dv)
    al = torch.zeros(H, dv, F)
    pc = hm.hm_linattn_pc_fwd
    _bad(lambda: pc(q, k, v, wq, wk, dt, al), "on the GPU")                        # well formed
    _bad(lambda: pc(q, k, v, wq, wk, dt, al, s_final=torch.zeros(B, H, hm.state_numel(f, dv))), "s_final must have shape")
    _bad(lambda: pc(q, k.float(), v, wq, wk, dt, al), "k must have q's dtype")
    st = torch.zeros(B, H, hm.state_numel_pc(f, dv))
    _bad(lambda: hm.hm_linattn_pc_step(q[:, :, 0], k[:, :, 0], v[:, :, 0], wq, wk, st[..., :-1], dt[:, :, 0], al),
         "state must have shape")


def test_noalloc_rejects_plans_beyond_its_scratch():
    """hm_linattn_fwd_noalloc checks the plan's scratch need against its fixed per-GPU
    array before any HIP call: 7 segment states of 128 heads (59 MB) exceed 40 MiB."""
    a = hm.FwdArgs(q=A, k=A, v=A, w_q=A, w_k=A, o=A, dtype=hm.HM_BF16, B=8, H=16, n=2048, d=128, f=64, dv=128,
                   sq_t=128, sk_t=128, sv_t=128, so_t=128, segments=8)
    st, need = hm.call_workspace_size(a)
    assert st == hm.HM_OK and need > (40 << 20)
    assert hm.call_fwd_noalloc(a) == hm.HM_ERR_WORKSPACE
    assert "40" in hm.last_error() or str(40 << 20) in hm.last_error()
    # invalid arguments are rejected exactly as hm_linattn_fwd rejects them
    a.segments = 0
    a.chunk = 96
    assert hm.call_fwd_noalloc(a) == hm.HM_ERR_UNSUPPORTED
    a.chunk = 0
    a.q = A + 8
    assert hm.call_fwd_noalloc(a) == hm.HM_ERR_ALIGN
