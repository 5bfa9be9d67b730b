"""Thin ctypes binding of libhm.so (the C ABI declared in include/hm.h).

Argument marshalling only: tensors are validated for device/dtype, their
data_ptr() and element strides go into the argument structs, the current torch
stream is passed as the HIP stream, and outputs / workspaces are allocated with
torch.  Every step of the computation runs in the library's HIP kernels; there
is no fallback.  If libhm.so is missing or cannot be loaded, every entry point
raises.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhm.so")

# HM_ABI_VERSION of include/hm.h that the argument structs below are laid out for
ABI_VERSION = 9
HM_OK, HM_ERR_NULL, HM_ERR_SHAPE, HM_ERR_DTYPE, HM_ERR_ALIGN, HM_ERR_UNSUPPORTED, HM_ERR_WORKSPACE, HM_ERR_HIP = range(8)
HM_F32, HM_BF16 = 0, 1
CHUNK = 64

p_void = C.c_void_p
i64 = C.c_int64
i32 = C.c_int32


class FeaturizeArgs(C.Structure):
    _fields_ = [("x", p_void), ("w", p_void), ("phi", p_void), ("dtype", i32), ("phi_dtype", i32),
                ("B", i64), ("H", i64), ("n", i64), ("d", i64), ("f", i64),
                ("sx_b", i64), ("sx_h", i64), ("sx_t", i64), ("sw_h", i64),
                ("sp_b", i64), ("sp_h", i64), ("sp_t", i64),
                ("rope_dims", i32), ("rope_base", C.c_float), ("rope_pos0", p_void),
                ("conv_width", i32), ("reserved", i32), ("conv_w", p_void), ("conv_b", p_void),
                ("conv_prev", p_void), ("scw_h", i64), ("scb_h", i64)]


class FwdArgs(C.Structure):
    _fields_ = [("q", p_void), ("k", p_void), ("v", p_void), ("w_q", p_void), ("w_k", p_void),
                ("dt", p_void), ("a_log", p_void), ("s_init", p_void), ("s_final", p_void), ("o", p_void),
                ("dtype", i32), ("chunk", i32), ("segments", i32), ("dsplit", i32),
                ("B", i64), ("H", i64), ("n", i64), ("d", i64), ("f", i64), ("dv", i64),
                ("sq_b", i64), ("sq_h", i64), ("sq_t", i64), ("sk_b", i64), ("sk_h", i64), ("sk_t", i64),
                ("sv_b", i64), ("sv_h", i64), ("sv_t", i64), ("so_b", i64), ("so_h", i64), ("so_t", i64),
                ("sw_h", i64), ("sdt_b", i64), ("sdt_h", i64), ("sdt_t", i64),
                ("workspace", p_void), ("workspace_bytes", C.c_size_t),
                ("gate", p_void), ("sg_b", i64), ("sg_h", i64), ("sg_t", i64),
                ("save", p_void), ("save_bytes", C.c_size_t),
                ("rope_dims", i32), ("rope_base", C.c_float), ("rope_pos0", p_void)]


class StepArgs(C.Structure):
    _fields_ = [("q", p_void), ("k", p_void), ("v", p_void), ("w_q", p_void), ("w_k", p_void),
                ("dt", p_void), ("a_log", p_void), ("state", p_void), ("o", p_void),
                ("dtype", i32), ("conv_width", i32),
                ("B", i64), ("H", i64), ("d", i64), ("f", i64), ("dv", i64),
                ("sq_b", i64), ("sq_h", i64), ("sk_b", i64), ("sk_h", i64), ("sv_b", i64), ("sv_h", i64),
                ("so_b", i64), ("so_h", i64), ("sw_h", i64), ("sdt_b", i64), ("sdt_h", i64),
                ("gate", p_void), ("sg_b", i64), ("sg_h", i64),
                ("conv_wq", p_void), ("conv_wk", p_void), ("conv_bq", p_void), ("conv_bk", p_void),
                ("conv_sq", p_void), ("conv_sk", p_void), ("scw_h", i64), ("scb_h", i64),
                ("rope_dims", i32), ("rope_base", C.c_float), ("rope_pos", p_void)]


class ConvArgs(C.Structure):
    _fields_ = [("x", p_void), ("y", p_void), ("w", p_void), ("bias", p_void), ("prev", p_void),
                ("final_rows", p_void), ("dtype", i32), ("width", i32),
                ("B", i64), ("H", i64), ("n", i64), ("d", i64),
                ("sx_b", i64), ("sx_h", i64), ("sx_t", i64), ("sy_b", i64), ("sy_h", i64), ("sy_t", i64),
                ("sw_h", i64), ("sb_h", i64)]


class BwdArgs(C.Structure):
    _fields_ = [("q", p_void), ("k", p_void), ("v", p_void), ("w_q", p_void), ("w_k", p_void),
                ("dt", p_void), ("a_log", p_void), ("d_o", p_void), ("gate", p_void),
                ("d_s_final", p_void), ("save", p_void), ("save_bytes", C.c_size_t),
                ("d_q", p_void), ("d_k", p_void), ("d_v", p_void), ("d_gate", p_void), ("d_wq", p_void),
                ("d_wk", p_void), ("d_dt", p_void), ("d_a_log", p_void), ("d_s_init", p_void),
                ("dtype", i32), ("reserved", i32),
                ("B", i64), ("H", i64), ("n", i64), ("d", i64), ("f", i64), ("dv", i64),
                ("sq_b", i64), ("sq_h", i64), ("sq_t", i64), ("sk_b", i64), ("sk_h", i64), ("sk_t", i64),
                ("sv_b", i64), ("sv_h", i64), ("sv_t", i64), ("so_b", i64), ("so_h", i64), ("so_t", i64),
                ("sg_b", i64), ("sg_h", i64), ("sg_t", i64),
                ("sw_h", i64), ("sdt_b", i64), ("sdt_h", i64), ("sdt_t", i64),
                ("workspace", p_void), ("workspace_bytes", C.c_size_t),
                ("rope_dims", i32), ("rope_base", C.c_float), ("rope_pos0", p_void)]


class PcArgs(C.Structure):
    _fields_ = [("q", p_void), ("k", p_void), ("v", p_void), ("w_q", p_void), ("w_k", p_void),
                ("dt", p_void), ("a_log", p_void), ("s_init", p_void), ("s_final", p_void), ("o", p_void),
                ("gate", p_void), ("dtype", i32), ("rope_dims", i32), ("rope_base", C.c_float), ("reserved", i32),
                ("rope_pos0", p_void),
                ("B", i64), ("H", i64), ("n", i64), ("d", i64), ("f", i64), ("dv", i64),
                ("sq_b", i64), ("sq_h", i64), ("sq_t", i64), ("sk_b", i64), ("sk_h", i64), ("sk_t", i64),
                ("sv_b", i64), ("sv_h", i64), ("sv_t", i64), ("so_b", i64), ("so_h", i64), ("so_t", i64),
                ("sg_b", i64), ("sg_h", i64), ("sg_t", i64),
                ("sw_h", i64), ("sdt_b", i64), ("sdt_h", i64), ("sdt_t", i64), ("sa_h", i64),
                ("segments", i32), ("reserved2", i32), ("workspace", p_void), ("workspace_bytes", C.c_size_t)]


class PcStepArgs(C.Structure):
    _fields_ = [("q", p_void), ("k", p_void), ("v", p_void), ("w_q", p_void), ("w_k", p_void),
                ("dt", p_void), ("a_log", p_void), ("state", p_void), ("o", p_void), ("gate", p_void),
                ("dtype", i32), ("conv_width", i32),
                ("B", i64), ("H", i64), ("d", i64), ("f", i64), ("dv", i64),
                ("sq_b", i64), ("sq_h", i64), ("sk_b", i64), ("sk_h", i64), ("sv_b", i64), ("sv_h", i64),
                ("so_b", i64), ("so_h", i64), ("sg_b", i64), ("sg_h", i64),
                ("sw_h", i64), ("sdt_b", i64), ("sdt_h", i64), ("sa_h", i64),
                ("conv_wq", p_void), ("conv_wk", p_void), ("conv_bq", p_void), ("conv_bk", p_void),
                ("conv_sq", p_void), ("conv_sk", p_void), ("scw_h", i64), ("scb_h", i64),
                ("rope_dims", i32), ("rope_base", C.c_float), ("rope_pos", p_void)]


class HMError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status


_lib = None
EXPORTS = ["hm_featurize", "hm_linattn_fwd_workspace_size", "hm_linattn_fwd_plan", "hm_linattn_fwd",
           "hm_linattn_fwd_noalloc",
           "hm_linattn_step", "hm_causal_conv", "hm_linattn_save_size", "hm_linattn_bwd_workspace_size",
           "hm_linattn_bwd", "hm_linattn_pc_fwd", "hm_linattn_pc_fwd_plan", "hm_linattn_pc_fwd_workspace_size",
           "hm_linattn_pc_step", "hm_status_string", "hm_last_error_message", "hm_abi_version", "hm_args_size"]


def lib():
    """Load libhm.so once; raise if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = C.CDLL(LIB_PATH)
        L.hm_featurize.argtypes = [C.POINTER(FeaturizeArgs), p_void]
        L.hm_linattn_fwd_workspace_size.argtypes = [C.POINTER(FwdArgs), C.POINTER(C.c_size_t)]
        L.hm_linattn_fwd_plan.argtypes = [C.POINTER(FwdArgs), C.POINTER(i32), C.POINTER(i32), C.POINTER(i32)]
        L.hm_linattn_fwd.argtypes = [C.POINTER(FwdArgs), p_void]
        L.hm_linattn_fwd_noalloc.argtypes = [C.POINTER(FwdArgs), p_void]
        L.hm_linattn_step.argtypes = [C.POINTER(StepArgs), p_void]
        L.hm_causal_conv.argtypes = [C.POINTER(ConvArgs), p_void]
        L.hm_linattn_save_size.argtypes = [C.POINTER(FwdArgs), C.POINTER(C.c_size_t)]
        L.hm_linattn_bwd_workspace_size.argtypes = [C.POINTER(BwdArgs), C.POINTER(C.c_size_t)]
        L.hm_linattn_bwd.argtypes = [C.POINTER(BwdArgs), p_void]
        L.hm_linattn_pc_fwd.argtypes = [C.POINTER(PcArgs), p_void]
        L.hm_linattn_pc_fwd_plan.argtypes = [C.POINTER(PcArgs), C.POINTER(i32)]
        L.hm_linattn_pc_fwd_workspace_size.argtypes = [C.POINTER(PcArgs), C.POINTER(C.c_size_t)]
        L.hm_linattn_pc_step.argtypes = [C.POINTER(PcStepArgs), p_void]
        for fn in ("hm_featurize", "hm_linattn_fwd_workspace_size", "hm_linattn_fwd_plan", "hm_linattn_fwd",
                   "hm_linattn_fwd_noalloc",
                   "hm_linattn_step", "hm_causal_conv", "hm_linattn_save_size", "hm_linattn_bwd_workspace_size",
                   "hm_linattn_bwd", "hm_linattn_pc_fwd", "hm_linattn_pc_fwd_plan",
                   "hm_linattn_pc_fwd_workspace_size", "hm_linattn_pc_step"):
            getattr(L, fn).restype = C.c_int
        L.hm_status_string.argtypes = [C.c_int]
        L.hm_status_string.restype = C.c_char_p
        L.hm_last_error_message.argtypes = []
        L.hm_last_error_message.restype = C.c_char_p
        L.hm_abi_version.restype = C.c_int
        L.hm_args_size.argtypes = [C.c_int]
        L.hm_args_size.restype = C.c_size_t
        if L.hm_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {L.hm_abi_version()}, this binding {ABI_VERSION}: "
                               "rebuild with __graft_entry__.build()")
        _lib = L
    return _lib


def status_string(st: int) -> str:
    return lib().hm_status_string(st).decode()


def last_error() -> str:
    return lib().hm_last_error_message().decode()


def _check(st):
    if st != HM_OK:
        raise HMError(st, last_error())


# ---------------------------------------------------------------- raw calls
def call_featurize(args: FeaturizeArgs, stream=None) -> int:
    return lib().hm_featurize(C.byref(args), stream)


def call_fwd(args: FwdArgs, stream=None) -> int:
    return lib().hm_linattn_fwd(C.byref(args), stream)


def call_fwd_noalloc(args: FwdArgs, stream=None) -> int:
    return lib().hm_linattn_fwd_noalloc(C.byref(args), stream)


def call_workspace_size(args: FwdArgs):
    n = C.c_size_t(0)
    st = lib().hm_linattn_fwd_workspace_size(C.byref(args), C.byref(n))
    return st, n.value


def call_plan(args: FwdArgs):
    c, s, d = i32(0), i32(0), i32(0)
    st = lib().hm_linattn_fwd_plan(C.byref(args), C.byref(c), C.byref(s), C.byref(d))
    return st, (c.value, s.value, d.value)


def call_step(args: StepArgs, stream=None) -> int:
    return lib().hm_linattn_step(C.byref(args), stream)


def call_conv(args: ConvArgs, stream=None) -> int:
    return lib().hm_causal_conv(C.byref(args), stream)


def call_save_size(args: FwdArgs):
    n = C.c_size_t(0)
    st = lib().hm_linattn_save_size(C.byref(args), C.byref(n))
    return st, n.value


def call_bwd_workspace_size(args: BwdArgs):
    n = C.c_size_t(0)
    st = lib().hm_linattn_bwd_workspace_size(C.byref(args), C.byref(n))
    return st, n.value


def call_pc_fwd(args: PcArgs, stream=None) -> int:
    return lib().hm_linattn_pc_fwd(C.byref(args), stream)


def call_pc_plan(args: PcArgs):
    n = i32(0)
    st = lib().hm_linattn_pc_fwd_plan(C.byref(args), C.byref(n))
    return st, n.value


def call_pc_workspace_size(args: PcArgs):
    n = C.c_size_t(0)
    st = lib().hm_linattn_pc_fwd_workspace_size(C.byref(args), C.byref(n))
    return st, n.value


def call_pc_step(args: PcStepArgs, stream=None) -> int:
    return lib().hm_linattn_pc_step(C.byref(args), stream)


def call_bwd(args: BwdArgs, stream=None) -> int:
    return lib().hm_linattn_bwd(C.byref(args), stream)


# ------------------------------------------------------------ torch-facing
_DT = {torch.float32: HM_F32, torch.bfloat16: HM_BF16}


def _code(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _rope(a, B, rope_dims, rope_base, pos, field="rope_pos0"):
    """Fill the rotary fields of an argument struct; pos is a device int64 [B] tensor or None."""
    if not rope_dims:
        return
    if pos is not None:
        _dev(pos)
        if pos.dtype != torch.int64 or tuple(pos.shape) != (B,) or not pos.is_contiguous():
            raise ValueError("rotary positions are a contiguous int64 tensor [B]")
    a.rope_dims = rope_dims
    a.rope_base = rope_base
    setattr(a, field, _ptr(pos))


def _w_strides(w):
    if w.dim() == 2:
        return 0
    return w.stride(0)


# ------------------------------------------------------------ argument checks
# The C ABI sees raw pointers only, so a tensor of the wrong size, dtype or
# layout would be read or written out of bounds on the GPU.  These checks run
# before anything is marshalled.
def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _check_shape(t, shape, name):
    _need(t is not None and tuple(t.shape) == tuple(shape), f"{name} must have shape {tuple(shape)}, "
          f"got {None if t is None else tuple(t.shape)}")


def _check_same_dtype(ref, *named):
    for name, t in named:
        if t is not None and t.dtype != ref.dtype:
            raise ValueError(f"{name} must have q's dtype {ref.dtype}, got {t.dtype}")


def _check_w(w, d, f, H, name):
    """W is [d, f] (shared) or [H, d, f] (per head), rows contiguous: a transposed
    view (stride (1, d)) would be read as row-major and give wrong results."""
    _need(w.dim() in (2, 3), f"{name} must be [d, f] or [H, d, f], got {tuple(w.shape)}")
    _need(tuple(w.shape[-2:]) == (d, f), f"{name} must be [{d}, {f}] per head, got {tuple(w.shape)}")
    _need(w.dim() == 2 or w.shape[0] == H, f"per-head {name} must have {H} heads, got {w.shape[0]}")
    _need(w.stride(-1) == 1 and (d == 1 or w.stride(-2) == f),
          f"{name} must be row-major with contiguous rows (strides (f, 1)), got strides {tuple(w.stride())}")


def _check_f32(t, shape, name, contiguous=True):
    if t is None:
        return
    _need(t.dtype == torch.float32, f"{name} must be float32, got {t.dtype}")
    _check_shape(t, shape, name)
    _need(not contiguous or t.is_contiguous(), f"{name} must be contiguous")


def _check_decay(dt, a_log, dt_shape, H):
    _need((dt is None) == (a_log is None), "dt and a_log must be given together")
    if dt is None:
        return
    _need(dt.dtype == torch.float32 and a_log.dtype == torch.float32, "dt and a_log are float32")
    _check_shape(dt, dt_shape, "dt")
    _need(dt.stride(-1) == 1 or dt.shape[-1] == 1, "dt must be contiguous along its last axis")
    _check_f32(a_log, (H,), "a_log")


def _check_attn(q, k, v, w_q, w_k, o=None, gate=None, token_axis=True):
    """q, k [B, H, (n,) d]; v, o, gate [B, H, (n,) dv]; one dtype; W [d, f] or [H, d, f]."""
    nd = 4 if token_axis else 3
    _need(q.dim() == nd, f"q must have {nd} dimensions, got {tuple(q.shape)}")
    _check_shape(k, q.shape, "k")
    _need(v.dim() == nd and tuple(v.shape[:-1]) == tuple(q.shape[:-1]),
          f"v must be {tuple(q.shape[:-1]) + ('dv',)}, got {tuple(v.shape)}")
    if o is not None:
        _check_shape(o, v.shape, "o")
    if gate is not None:
        _check_shape(gate, v.shape, "gate")
    _check_same_dtype(q, ("k", k), ("v", v), ("w_q", w_q), ("w_k", w_k), ("o", o), ("gate", gate))
    d, f = q.shape[-1], w_q.shape[-1]
    _check_w(w_q, d, f, q.shape[1], "w_q")
    _check_w(w_k, d, f, q.shape[1], "w_k")
    _need(w_q.dim() == w_k.dim() and (w_q.dim() == 2 or w_q.stride(0) == w_k.stride(0)),
          "w_q and w_k must have the same layout (both shared or both per head, same head stride)")


def hm_featurize(x: torch.Tensor, w: torch.Tensor, phi_dtype=None, phi: torch.Tensor | None = None,
                 rope_dims=0, rope_base=10000.0, rope_pos0=None, conv_w=None, conv_b=None, conv_prev=None):
    """phi = softmax([x W, -x W]) for x [B, H, n, d], W [d, f] or [H, d, f]; with
    rope_dims > 0 turned by the rotary encoding at positions rope_pos0[b] + t; with
    conv_w (float32 [d, K] or [H, d, K]) x first goes through the short causal conv
    (conv_b float32 [d] or [H, d] or None; conv_prev [B, H, K-1, d] or None), fused
    into the featurizer's loads."""
    _need(x.dim() == 4, f"x must be [B, H, n, d], got {tuple(x.shape)}")
    B, H, n, d = x.shape
    f = w.shape[-1]
    _check_same_dtype(x, ("w", w))
    _check_w(w, d, f, H, "w")
    if phi is not None:
        _check_shape(phi, (B, H, n, 2 * f), "phi")
    _dev(x, w, phi)
    if phi is None:
        phi = torch.empty((B, H, n, 2 * f), dtype=phi_dtype or x.dtype, device=x.device)
    a = FeaturizeArgs(x=_ptr(x), w=_ptr(w), phi=_ptr(phi), dtype=_code(x), phi_dtype=_code(phi),
                      B=B, H=H, n=n, d=d, f=f, sx_b=x.stride(0), sx_h=x.stride(1), sx_t=x.stride(2),
                      sw_h=_w_strides(w), sp_b=phi.stride(0), sp_h=phi.stride(1), sp_t=phi.stride(2))
    if x.stride(3) != 1 or phi.stride(3) != 1 or w.stride(-1) != 1:
        raise ValueError("inner dimensions must be contiguous")
    _rope(a, B, rope_dims, rope_base, rope_pos0)
    if conv_w is not None:
        _need(conv_w.dtype == torch.float32 and conv_w.dim() in (2, 3) and conv_w.shape[-2] == d
              and conv_w.is_contiguous(), f"conv_w must be contiguous float32 [d, K] or [H, d, K], got {tuple(conv_w.shape)}")
        K = conv_w.shape[-1]
        _need(conv_w.dim() == 2 or conv_w.shape[0] == H, "conv_w's head dimension must be H")
        if conv_b is not None:
            _need(conv_b.dtype == torch.float32 and conv_b.shape[-1] == d and conv_b.is_contiguous()
                  and (conv_b.dim() == 1 or (conv_b.dim() == 2 and conv_b.shape[0] == H)),
                  "conv_b must be contiguous float32 [d] or [H, d]")
        if conv_prev is not None:
            _need(conv_prev.dtype == x.dtype and tuple(conv_prev.shape) == (B, H, K - 1, d)
                  and conv_prev.is_contiguous(), "conv_prev must be contiguous [B, H, K-1, d] in x's dtype")
        _dev(conv_w, conv_b, conv_prev)
        a.conv_width, a.conv_w, a.conv_b, a.conv_prev = K, _ptr(conv_w), _ptr(conv_b), _ptr(conv_prev)
        a.scw_h = d * K if conv_w.dim() == 3 else 0
        a.scb_h = d if conv_b is not None and conv_b.dim() == 2 else 0
    _check(call_featurize(a, _stream()))
    return phi


def fwd_args(q, k, v, w_q, w_k, dt=None, a_log=None, s_init=None, s_final=None, o=None,
             chunk=0, segments=0, dsplit=0, gate=None) -> FwdArgs:
    B, H, n, d = q.shape
    dv = v.shape[-1]
    f = w_q.shape[-1]
    for t in (q, k, v, o, gate):
        if t is not None and t.stride(3) != 1:
            raise ValueError("inner dimensions must be contiguous")
    return FwdArgs(q=_ptr(q), k=_ptr(k), v=_ptr(v), w_q=_ptr(w_q), w_k=_ptr(w_k), dt=_ptr(dt), a_log=_ptr(a_log),
                   s_init=_ptr(s_init), s_final=_ptr(s_final), o=_ptr(o), dtype=_code(q), chunk=chunk,
                   segments=segments, dsplit=dsplit, B=B, H=H, n=n, d=d, f=f, dv=dv,
                   sq_b=q.stride(0), sq_h=q.stride(1), sq_t=q.stride(2),
                   sk_b=k.stride(0), sk_h=k.stride(1), sk_t=k.stride(2),
                   sv_b=v.stride(0), sv_h=v.stride(1), sv_t=v.stride(2),
                   so_b=o.stride(0) if o is not None else 0, so_h=o.stride(1) if o is not None else 0,
                   so_t=o.stride(2) if o is not None else 0, sw_h=_w_strides(w_q),
                   sdt_b=dt.stride(0) if dt is not None else 0, sdt_h=dt.stride(1) if dt is not None else 0,
                   sdt_t=dt.stride(2) if dt is not None else 0, gate=_ptr(gate),
                   sg_b=gate.stride(0) if gate is not None else 0, sg_h=gate.stride(1) if gate is not None else 0,
                   sg_t=gate.stride(2) if gate is not None else 0)


def hm_linattn_fwd_plan(q, k, v, w_q, w_k, dt=None, a_log=None, chunk=0, segments=0, dsplit=0, o=None,
                        rope_dims=0, rope_base=10000.0, rope_pos0=None):
    _check_attn(q, k, v, w_q, w_k, o)
    _check_decay(dt, a_log, tuple(q.shape[:3]), q.shape[1])
    o = o if o is not None else v
    a = fwd_args(q, k, v, w_q, w_k, dt, a_log, o=o, chunk=chunk, segments=segments, dsplit=dsplit)
    _rope(a, q.shape[0], rope_dims, rope_base, rope_pos0)
    st, plan = call_plan(a)
    _check(st)
    return plan


def hm_linattn_fwd(q, k, v, w_q, w_k, dt=None, a_log=None, s_init=None, s_final=None, o=None,
                   chunk=0, segments=0, dsplit=0, workspace=None, gate=None, save=None,
                   rope_dims=0, rope_base=10000.0, rope_pos0=None):
    """Causal prefill.  Returns o [B, H, n, dv] (v's dtype), times SiLU(gate) when a
    gate [B, H, n, dv] is given.  s_final (if given) receives the float32 state
    [B, H, F*dv + F] after the last token.  rope_dims > 0 turns phi(q) and phi(k)
    by the rotary encoding at positions rope_pos0[b] + t (rope_pos0 int64 [B] on the
    GPU, or None for 0)."""
    _check_attn(q, k, v, w_q, w_k, o, gate)
    B, H, n, _ = q.shape
    _check_decay(dt, a_log, (B, H, n), H)
    blk = state_numel(w_q.shape[-1], v.shape[-1])
    _check_f32(s_init, (B, H, blk), "s_init")
    _check_f32(s_final, (B, H, blk), "s_final")
    _dev(q, k, v, w_q, w_k, dt, a_log, s_init, s_final, o, gate, save, workspace)
    if o is None:
        o = torch.empty(v.shape, dtype=v.dtype, device=v.device)
    a = fwd_args(q, k, v, w_q, w_k, dt, a_log, s_init, s_final, o, chunk, segments, dsplit, gate)
    _rope(a, q.shape[0], rope_dims, rope_base, rope_pos0)
    if save is not None:
        if save.numel() * save.element_size() < save_size(q, v, w_q):
            raise ValueError("save buffer too small (see save_size)")
        a.save = save.data_ptr()
        a.save_bytes = save.numel() * save.element_size()
    st, nbytes = call_workspace_size(a)
    _check(st)
    if nbytes:
        if workspace is None or workspace.numel() * workspace.element_size() < nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    _check(call_fwd(a, _stream()))
    return o


def hm_linattn_step(q, k, v, w_q, w_k, state, dt=None, a_log=None, o=None, gate=None, conv=None,
                    rope_dims=0, rope_base=10000.0, rope_pos=None):
    """One decode token per (b, h): q, k [B, H, d], v [B, H, dv]; state [B, H, F*dv+F]
    float32 is updated in place.  Returns o [B, H, dv], times SiLU(gate) when a gate
    [B, H, dv] is given.  conv = (w_q, w_k, b_q, b_k, state_q, state_k) runs q and k
    through the short causal conv first (taps float32 [d, K] or [H, d, K], bias
    float32 [d] / [H, d] or None, states [B, H, K-1, d] updated in place).  rope_dims > 0
    turns phi(q) and phi(k) by the rotary encoding at position rope_pos[b] (int64 [B]
    on the GPU, required)."""
    _check_attn(q, k, v, w_q, w_k, o, gate, token_axis=False)
    B, H, d = q.shape
    dv = v.shape[-1]
    f = w_q.shape[-1]
    _check_decay(dt, a_log, (B, H), H)
    _check_f32(state, (B, H, state_numel(f, dv)), "state")
    _dev(q, k, v, w_q, w_k, state, dt, a_log, o, gate, *(conv or ()))
    if o is None:
        o = torch.empty((B, H, dv), dtype=v.dtype, device=v.device)
    a = StepArgs(q=_ptr(q), k=_ptr(k), v=_ptr(v), w_q=_ptr(w_q), w_k=_ptr(w_k), dt=_ptr(dt), a_log=_ptr(a_log),
                 state=_ptr(state), o=_ptr(o), dtype=_code(q), B=B, H=H, d=d, f=f, dv=dv,
                 sq_b=q.stride(0), sq_h=q.stride(1), sk_b=k.stride(0), sk_h=k.stride(1),
                 sv_b=v.stride(0), sv_h=v.stride(1), so_b=o.stride(0), so_h=o.stride(1), sw_h=_w_strides(w_q),
                 sdt_b=dt.stride(0) if dt is not None else 0, sdt_h=dt.stride(1) if dt is not None else 0,
                 gate=_ptr(gate), sg_b=gate.stride(0) if gate is not None else 0,
                 sg_h=gate.stride(1) if gate is not None else 0)
    if gate is not None and gate.stride(2) != 1:
        raise ValueError("inner dimensions must be contiguous")
    if conv is not None:
        cwq, cwk, cbq, cbk, csq, csk = conv
        K = cwq.shape[-1]
        for t in (cwq, cwk):
            if t.dtype != torch.float32 or t.shape[-2:] != (d, K) or t.stride(-1) != 1 or t.stride(-2) != K:
                raise ValueError("conv taps are float32 [d, K] (or [H, d, K]) with contiguous rows")
        for t in (cbq, cbk):
            if t is not None and (t.dtype != torch.float32 or t.stride(-1) != 1):
                raise ValueError("conv bias is float32, contiguous along d")
        for t in (csq, csk):
            if t is not None and (tuple(t.shape) != (B, H, K - 1, d) or not t.is_contiguous() or t.dtype != q.dtype):
                raise ValueError("conv states are contiguous [B, H, K-1, d] in q's dtype")
        a.conv_width = K
        a.conv_wq, a.conv_wk, a.conv_bq, a.conv_bk = _ptr(cwq), _ptr(cwk), _ptr(cbq), _ptr(cbk)
        a.conv_sq, a.conv_sk = _ptr(csq), _ptr(csk)
        a.scw_h = cwq.stride(0) if cwq.dim() == 3 else 0
        a.scb_h = cbq.stride(0) if cbq is not None and cbq.dim() == 2 else 0
        if (cwk.dim() == 3) != (cwq.dim() == 3) or (cbq is None) != (cbk is None) or \
                (cbk is not None and cbk.dim() != cbq.dim()):
            raise ValueError("conv taps and biases of q and k must have the same layout")
    _rope(a, B, rope_dims, rope_base, rope_pos, "rope_pos")
    _check(call_step(a, _stream()))
    return o


def hm_causal_conv(x, w, bias=None, prev=None, final_rows=None, y=None):
    """Short causal conv over the token axis of x [B, H, n, d]: w float32 [d, K]
    (or [H, d, K]), bias float32 [d] (or [H, d]) or None; prev [B, H, K-1, d] the rows
    before token 0 (None = zeros); final_rows [B, H, K-1, d] (optional, may be prev)
    receives the last K-1 rows of prev ++ x.  Returns y (x's shape and dtype)."""
    _dev(x, w, bias, prev, final_rows, y)
    B, H, n, d = x.shape
    K = w.shape[-1]
    if w.dtype != torch.float32 or (bias is not None and bias.dtype != torch.float32):
        raise TypeError("conv taps and bias are float32")
    if w.shape[-2] != d or w.stride(-1) != 1 or w.stride(-2) != K:
        raise ValueError("w must be [d, K] (or [H, d, K]) with contiguous rows")
    for t in (prev, final_rows):
        if t is not None and (tuple(t.shape) != (B, H, K - 1, d) or not t.is_contiguous() or t.dtype != x.dtype):
            raise ValueError("prev and final_rows are contiguous [B, H, K-1, d] in x's dtype")
    if bias is not None and bias.stride(-1) != 1:
        raise ValueError("bias must be contiguous along d")
    if y is None:
        y = torch.empty(x.shape, dtype=x.dtype, device=x.device)
    if x.stride(3) != 1 or y.stride(3) != 1:
        raise ValueError("inner dimensions must be contiguous")
    a = ConvArgs(x=_ptr(x), y=_ptr(y), w=_ptr(w), bias=_ptr(bias), prev=_ptr(prev), final_rows=_ptr(final_rows),
                 dtype=_code(x), width=K, B=B, H=H, n=n, d=d,
                 sx_b=x.stride(0), sx_h=x.stride(1), sx_t=x.stride(2), sy_b=y.stride(0), sy_h=y.stride(1),
                 sy_t=y.stride(2), sw_h=w.stride(0) if w.dim() == 3 else 0,
                 sb_h=bias.stride(0) if bias is not None and bias.dim() == 2 else 0)
    _check(call_conv(a, _stream()))
    return y


def hm_linattn_fwd_noalloc(q, k, v, w_q, w_k, dt=None, a_log=None, s_init=None, s_final=None, o=None,
                           chunk=0, segments=0, dsplit=0, gate=None, save=None, rope_dims=0, rope_base=10000.0,
                           rope_pos0=None):
    """hm_linattn_fwd without a workspace: the library's per-GPU scratch stands in
    for it (see include/hm.h).  Calls that overlap on one GPU race.  o is allocated
    here only when not given."""
    _check_attn(q, k, v, w_q, w_k, o, gate)
    B, H, n, _ = q.shape
    _check_decay(dt, a_log, (B, H, n), H)
    blk = state_numel(w_q.shape[-1], v.shape[-1])
    _check_f32(s_init, (B, H, blk), "s_init")
    _check_f32(s_final, (B, H, blk), "s_final")
    _dev(q, k, v, w_q, w_k, dt, a_log, s_init, s_final, o, gate, save)
    if o is None:
        o = torch.empty(v.shape, dtype=v.dtype, device=v.device)
    a = fwd_args(q, k, v, w_q, w_k, dt, a_log, s_init, s_final, o, chunk, segments, dsplit, gate)
    _rope(a, B, rope_dims, rope_base, rope_pos0)
    if save is not None:
        if save.numel() * save.element_size() < save_size(q, v, w_q):
            raise ValueError("save buffer too small (see save_size)")
        a.save = save.data_ptr()
        a.save_bytes = save.numel() * save.element_size()
    _check(call_fwd_noalloc(a, _stream()))
    return o


def save_size(q, v, w_q) -> int:
    """Bytes of the buffer a training forward fills for hm_linattn_bwd."""
    B, H, n, d = q.shape
    a = FwdArgs(dtype=_code(q), B=B, H=H, n=n, d=d, f=w_q.shape[-1], dv=v.shape[-1])
    st, nb = call_save_size(a)
    _check(st)
    return nb


def hm_linattn_bwd(q, k, v, w_q, w_k, d_o, save, dt=None, a_log=None, gate=None, d_s_final=None,
                   want_d_s_init=False, workspace=None, rope_dims=0, rope_base=10000.0, rope_pos0=None):
    """Gradients of the prefill from d_o = dloss/do (save: what the training forward
    saved; gate: the forward's gate; d_s_final: dloss/ds_final).  Returns a dict: q,
    k, v (dtype of q), w_q, w_k (float32, [d, f] or [H, d, f]), and gate, dt, a_log,
    s_init when applicable.  The rotary fields are the forward's."""
    _check_attn(q, k, v, w_q, w_k, d_o, gate)
    B, H, n, d = q.shape
    dv = v.shape[-1]
    f = w_q.shape[-1]
    _check_decay(dt, a_log, (B, H, n), H)
    _check_f32(d_s_final, (B, H, state_numel(f, dv)), "d_s_final")
    _need(save.numel() * save.element_size() >= save_size(q, v, w_q), "save buffer too small (see save_size)")
    _dev(q, k, v, w_q, w_k, d_o, save, dt, a_log, gate, d_s_final, workspace)
    for t in (q, k, v, d_o, gate):
        if t is not None and t.stride(3) != 1:
            raise ValueError("inner dimensions must be contiguous")
    if w_q.dim() == 3 and not (w_q.is_contiguous() and w_k.is_contiguous()):
        raise ValueError("per-head W must be contiguous [H, d, f]")
    dq = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    dk = torch.empty_strided(k.shape, k.stride(), dtype=k.dtype, device=k.device)
    dvv = torch.empty_strided(v.shape, v.stride(), dtype=v.dtype, device=v.device)
    dwq = torch.empty(w_q.shape, dtype=torch.float32, device=q.device)
    dwk = torch.empty(w_k.shape, dtype=torch.float32, device=q.device)
    ddt = torch.empty_strided(dt.shape, dt.stride(), dtype=torch.float32, device=q.device) if dt is not None else None
    dal = torch.empty_like(a_log) if a_log is not None else None
    F = 2 * f
    dsi = torch.empty((B, H, F * dv + F), dtype=torch.float32, device=q.device) if want_d_s_init else None
    dg = torch.empty_strided(gate.shape, gate.stride(), dtype=gate.dtype, device=q.device) if gate is not None else None
    a = BwdArgs(q=_ptr(q), k=_ptr(k), v=_ptr(v), w_q=_ptr(w_q), w_k=_ptr(w_k), dt=_ptr(dt), a_log=_ptr(a_log),
                d_o=_ptr(d_o), gate=_ptr(gate), d_s_final=_ptr(d_s_final), save=_ptr(save),
                save_bytes=save.numel() * save.element_size(), d_q=_ptr(dq), d_k=_ptr(dk), d_v=_ptr(dvv),
                d_gate=_ptr(dg), d_wq=_ptr(dwq), d_wk=_ptr(dwk), d_dt=_ptr(ddt), d_a_log=_ptr(dal),
                d_s_init=_ptr(dsi), dtype=_code(q), B=B, H=H, n=n, d=d, f=f, dv=dv,
                sq_b=q.stride(0), sq_h=q.stride(1), sq_t=q.stride(2), sk_b=k.stride(0), sk_h=k.stride(1),
                sk_t=k.stride(2), sv_b=v.stride(0), sv_h=v.stride(1), sv_t=v.stride(2),
                so_b=d_o.stride(0), so_h=d_o.stride(1), so_t=d_o.stride(2),
                sg_b=gate.stride(0) if gate is not None else 0, sg_h=gate.stride(1) if gate is not None else 0,
                sg_t=gate.stride(2) if gate is not None else 0, sw_h=_w_strides(w_q),
                sdt_b=dt.stride(0) if dt is not None else 0, sdt_h=dt.stride(1) if dt is not None else 0,
                sdt_t=dt.stride(2) if dt is not None else 0)
    _rope(a, B, rope_dims, rope_base, rope_pos0)
    st, nbytes = call_bwd_workspace_size(a)
    _check(st)
    if workspace is None or workspace.numel() * workspace.element_size() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    a.workspace = workspace.data_ptr()
    a.workspace_bytes = workspace.numel() * workspace.element_size()
    _check(call_bwd(a, _stream()))
    out = {"q": dq, "k": dk, "v": dvv, "w_q": dwq, "w_k": dwk}
    if dg is not None:
        out["gate"] = dg
    if dt is not None:
        out["dt"], out["a_log"] = ddt, dal
    if dsi is not None:
        out["s_init"] = dsi
    return out


def _a_log_stride(a_log, dv, F):
    if a_log.dtype != torch.float32 or tuple(a_log.shape[-2:]) != (dv, F) or not a_log.is_contiguous():
        raise ValueError("a_log is contiguous float32 [dv, 2f] (shared) or [H, dv, 2f]")
    return a_log.stride(0) if a_log.dim() == 3 else 0


def hm_linattn_pc_plan(q, v, w_q, segments=0) -> int:
    """The number of sequence segments hm_linattn_pc_fwd runs for these sizes."""
    B, H, n, d = q.shape
    a = PcArgs(dtype=_code(q), B=B, H=H, n=n, d=d, f=w_q.shape[-1], dv=v.shape[-1], segments=segments)
    st, ns = call_pc_plan(a)
    _check(st)
    return ns


def hm_linattn_pc_fwd(q, k, v, w_q, w_k, dt, a_log, s_init=None, s_final=None, o=None, gate=None,
                      rope_dims=0, rope_base=10000.0, rope_pos0=None, segments=0, workspace=None):
    """Prefill with a decay per value channel and state (the pages' Mamba-1 wiring):
    dt float32 [B, H, n, dv] (the step size before softplus), a_log float32 [dv, 2f] or
    [H, dv, 2f].  Returns o [B, H, n, dv]; s_final (if given) receives the float32
    state [B, H, 2*dv*2f] (Sn [dv][2f] then Sd [dv][2f]).  segments: 0 = automatic,
    else the number of sequence segments scanned in parallel; workspace: a uint8
    device buffer (allocated here when None or too small)."""
    _check_attn(q, k, v, w_q, w_k, o, gate)
    B, H, n, d = q.shape
    dv = v.shape[-1]
    f = w_q.shape[-1]
    _check_f32(s_init, (B, H, state_numel_pc(f, dv)), "s_init")
    _check_f32(s_final, (B, H, state_numel_pc(f, dv)), "s_final")
    _dev(q, k, v, w_q, w_k, dt, a_log, s_init, s_final, o, gate)
    if dt.dtype != torch.float32 or tuple(dt.shape) != (B, H, n, dv) or dt.stride(3) != 1:
        raise ValueError("dt is float32 [B, H, n, dv] with contiguous channels")
    for t in (q, k, v, o, gate):
        if t is not None and t.stride(3) != 1:
            raise ValueError("inner dimensions must be contiguous")
    if o is None:
        o = torch.empty(v.shape, dtype=v.dtype, device=v.device)
    a = PcArgs(q=_ptr(q), k=_ptr(k), v=_ptr(v), w_q=_ptr(w_q), w_k=_ptr(w_k), dt=_ptr(dt), a_log=_ptr(a_log),
               s_init=_ptr(s_init), s_final=_ptr(s_final), o=_ptr(o), gate=_ptr(gate), dtype=_code(q),
               B=B, H=H, n=n, d=d, f=f, dv=dv,
               sq_b=q.stride(0), sq_h=q.stride(1), sq_t=q.stride(2), sk_b=k.stride(0), sk_h=k.stride(1),
               sk_t=k.stride(2), sv_b=v.stride(0), sv_h=v.stride(1), sv_t=v.stride(2),
               so_b=o.stride(0), so_h=o.stride(1), so_t=o.stride(2),
               sg_b=gate.stride(0) if gate is not None else 0, sg_h=gate.stride(1) if gate is not None else 0,
               sg_t=gate.stride(2) if gate is not None else 0, sw_h=_w_strides(w_q),
               sdt_b=dt.stride(0), sdt_h=dt.stride(1), sdt_t=dt.stride(2), sa_h=_a_log_stride(a_log, dv, 2 * f),
               segments=segments)
    _rope(a, B, rope_dims, rope_base, rope_pos0)
    st, nbytes = call_pc_workspace_size(a)
    _check(st)
    if nbytes > 0:
        if workspace is None or workspace.numel() * workspace.element_size() < nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    _check(call_pc_fwd(a, _stream()))
    return o


def hm_linattn_pc_step(q, k, v, w_q, w_k, state, dt, a_log, o=None, gate=None, conv=None,
                       rope_dims=0, rope_base=10000.0, rope_pos=None):
    """One decode token per (b, h) of the per-channel scan: q, k [B, H, d], v [B, H, dv],
    dt float32 [B, H, dv]; state float32 [B, H, 2*dv*2f] updated in place.  conv and
    the rotary fields as in hm_linattn_step."""
    _check_attn(q, k, v, w_q, w_k, o, gate, token_axis=False)
    B, H, d = q.shape
    dv = v.shape[-1]
    f = w_q.shape[-1]
    _check_f32(state, (B, H, state_numel_pc(f, dv)), "state")
    _dev(q, k, v, w_q, w_k, state, dt, a_log, o, gate, *(conv or ()))
    if dt.dtype != torch.float32 or tuple(dt.shape) != (B, H, dv) or dt.stride(2) != 1:
        raise ValueError("dt is float32 [B, H, dv] with contiguous channels")
    if o is None:
        o = torch.empty((B, H, dv), dtype=v.dtype, device=v.device)
    a = PcStepArgs(q=_ptr(q), k=_ptr(k), v=_ptr(v), w_q=_ptr(w_q), w_k=_ptr(w_k), dt=_ptr(dt), a_log=_ptr(a_log),
                   state=_ptr(state), o=_ptr(o), gate=_ptr(gate), dtype=_code(q), B=B, H=H, d=d, f=f, dv=dv,
                   sq_b=q.stride(0), sq_h=q.stride(1), sk_b=k.stride(0), sk_h=k.stride(1),
                   sv_b=v.stride(0), sv_h=v.stride(1), so_b=o.stride(0), so_h=o.stride(1),
                   sg_b=gate.stride(0) if gate is not None else 0, sg_h=gate.stride(1) if gate is not None else 0,
                   sw_h=_w_strides(w_q), sdt_b=dt.stride(0), sdt_h=dt.stride(1), sa_h=_a_log_stride(a_log, dv, 2 * f))
    if conv is not None:
        cwq, cwk, cbq, cbk, csq, csk = conv
        a.conv_width = cwq.shape[-1]
        a.conv_wq, a.conv_wk, a.conv_bq, a.conv_bk = _ptr(cwq), _ptr(cwk), _ptr(cbq), _ptr(cbk)
        a.conv_sq, a.conv_sk = _ptr(csq), _ptr(csk)
        a.scw_h = cwq.stride(0) if cwq.dim() == 3 else 0
        a.scb_h = cbq.stride(0) if cbq is not None and cbq.dim() == 2 else 0
    _rope(a, B, rope_dims, rope_base, rope_pos, "rope_pos")
    _check(call_pc_step(a, _stream()))
    return o


def state_numel_pc(f: int, dv: int) -> int:
    """float32 elements of one (b, h) per-channel state block: Sn and Sd, [dv][2f] each."""
    return 2 * dv * 2 * f


def state_numel(f: int, dv: int) -> int:
    """float32 elements of one (b, h) state block: S [2f][dv] then z [2f]."""
    return 2 * f * dv + 2 * f
