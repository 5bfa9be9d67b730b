"""CPU float64 oracle for causal, normalized Hedgehog linear attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU
baseline may import this module.  It shares no code with the HIP library and
imports nothing from it; the product path never calls it.

Pages cited (by title and section):
  [HM]  "HedgeMamba：融合线性注意力与状态空间模型的高效序列建模" (gsyq.cn news 1418924)
        §2.1 Hedgehog feature map, §2.3 state expansion and normalization,
        §3.1 stage-1 identity initialisation, §5.2 HedgeMambaMixer,
        §5.3 HedgehogProjection.
  [LA]  "线性注意力（Linear Attention）详解" (cnblogs ying-chease 22790249)
        part 2 (kernel form of normalized attention, associativity),
        part 3 (recurrent form), part 4.3 (RetNet scalar decay),
        part 5 (chunk-wise parallel vs recurrent modes).
  [SSM] "状态空间模型：Mamba、S4 的线性复杂度路径" (quant67.com, lecture 56)
        §3.2 (softplus on the step size), §4.2 (associative affine scan).

What is computed, per (batch b, head h), for tokens t = 0..n-1:
  phi(x)  = softmax([x W, -x W]) over the feature axis          [HM §2.1, §5.3]
  log a_t = -softplus(dt_t) * exp(A_log[h]);  a_t = 1 without dt [SSM §3.2; HM §3.1]
  S_t = a_t S_{t-1} + phi(k_t) v_t^T,  z_t = a_t z_{t-1} + phi(k_t)
  o_t = phi(q_t)^T S_t / phi(q_t)^T z_t                          [LA parts 2-3, 4.3; HM §2.3]
  optionally o_t <- o_t * SiLU(g_t) with the gate branch's g    [HM §5.2 step 6]
  optionally phi(q_t), phi(k_t) turned by rotary position encoding before
  both sums, so numerator and denominator see the rotated features
                                                                 [HM §5.2 step 3]
as a variant, a decay per value channel and state (pc_scan): the A / dt / V
copies of the pages' Mamba-1 wiring, a numerator and a denominator channel per
value channel with Delta-scaled input                            [HM §2.3, §5.2]
and, as a separate step ahead of the featurizer, Mamba's short causal conv
(depthwise over time, K taps per channel, identity at the stage-1 init)
[HM §2.2, §2.3 item 4, §3.1].
S_{-1}, z_{-1} are the given initial state (zeros when absent); a_t scales the
carried state only, never the current token (the RetNet form, [LA] 4.3).

Readings where the pages are silent (listed with reasons in the design notes):
one shared W per projection applied as x @ W with no bias or temperature;
separate W_q, W_k; the u half precedes the -u half; no epsilon in the
denominator; the denominator state is one F-vector because the decay is a
per-head scalar.  Rotary encoding follows GPT-NeoX (the architecture Pythia
uses, which [HM §5.2] names): feature i of the leading `dims` pairs with feature
i + dims/2 and turns by pos * base^(-2i/dims); features past `dims` pass
through; positions count from a start offset per sequence.

Every function here is pinned by tests/test_oracle.py (the rotary encoding by
tests/test_oracle_rope.py, the per-channel scan by tests/test_oracle_pc.py)
against closed forms, library routines, brute force and invariants; there is no
parity-unpinned function in this module.
"""
from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------------
# A2: Hedgehog feature map  [HM §2.1 (linear map, concat with its negation,
# softmax over the feature axis), §5.3 HedgehogProjection.forward]
# --------------------------------------------------------------------------
def hedgehog_features(x, w):
    """phi(x) = softmax([x W, -x W], axis=-1) in float64.

    x: [..., d];  w: [d, f] shared, or [H, d, f] per head with x [B, H, n, d].
    Returns [..., 2f]: the first f entries come from +xW, the last f from -xW.
    The max shift is M = max|u| (the largest of u and -u); it cancels exactly.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    if w.ndim == 2:
        u = x @ w
    else:  # per-head weights
        u = np.einsum("bhnd,hdf->bhnf", x, w)
    both = np.concatenate([u, -u], axis=-1)
    m = np.max(np.abs(u), axis=-1, keepdims=True)
    e = np.exp(both - m)
    return e / np.sum(e, axis=-1, keepdims=True)


# --------------------------------------------------------------------------
# A1: per-head decay  [SSM §3.2: the step size passes through softplus;
# decay a_t = exp(-softplus(dt_t) * exp(A_log)); HM §3.1: stage-1 init a = 1]
# --------------------------------------------------------------------------
def softplus(x):
    """log(1 + e^x) without overflow: x + log1p(e^-x) for x > 0, log1p(e^x) otherwise."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x > 0
    out[pos] = x[pos] + np.log1p(np.exp(-x[pos]))
    out[~pos] = np.log1p(np.exp(x[~pos]))
    return out


def log_decay(dt, a_log):
    """log a_t = -softplus(dt[b,h,t]) * exp(A_log[h]).  Returns [B, H, n] float64.

    With dt absent the decay is the identity (log a_t = 0) and None is returned.
    """
    if dt is None:
        return None
    dt = np.asarray(dt, dtype=np.float64)
    a_log = np.asarray(a_log, dtype=np.float64)
    return -softplus(dt) * np.exp(a_log)[None, :, None]


# --------------------------------------------------------------------------
# Quadratic form: explicit causal n x n weights  [LA part 2: normalized kernel
# attention o_i = sum_j sim(q_i,k_j) v_j / sum_j sim(q_i,k_j) with
# sim = phi(q).phi(k); made causal and decayed as in LA 4.3]
# --------------------------------------------------------------------------
def decay_matrix(log_a_row):
    """G[i, j] = prod_{s=j+1..i} a_s for j <= i, else 0, from one head's log a [n].

    Formed as exp(L_i - L_j) with L the inclusive cumulative sum of log a.
    """
    n = log_a_row.shape[0]
    L = np.cumsum(log_a_row)
    diff = L[:, None] - L[None, :]
    G = np.zeros((n, n))
    mask = np.tril(np.ones((n, n), dtype=bool))
    G[mask] = np.exp(diff[mask])
    return G


def linattn_quadratic(phiq, phik, v, log_a=None, s_init=None, z_init=None):
    """Output o [B, H, n, dv] from explicit masked n x n weights, per (b, h).

    phiq, phik: [B, H, n, F]; v: [B, H, n, dv]; log_a: [B, H, n] or None;
    s_init: [B, H, F, dv] or None; z_init: [B, H, F] or None.
    """
    B, H, n, F = phiq.shape
    dv = v.shape[-1]
    o = np.empty((B, H, n, dv))
    for b in range(B):
        for h in range(H):
            scores = phiq[b, h] @ phik[b, h].T                     # [n, n]
            if log_a is None:
                G = np.tril(np.ones((n, n)))
                carry = np.ones(n)
            else:
                G = decay_matrix(log_a[b, h])
                carry = np.exp(np.cumsum(log_a[b, h]))             # prod_{s<=i} a_s
            wgt = G * scores
            num = wgt @ v[b, h]
            den = wgt.sum(axis=1)
            if s_init is not None:
                num = num + carry[:, None] * (phiq[b, h] @ s_init[b, h])
                den = den + carry * (phiq[b, h] @ z_init[b, h])
            o[b, h] = num / den[:, None]
    return o


# --------------------------------------------------------------------------
# Recurrent form  [LA part 3: S_i = S_{i-1} + phi(k_i) v_i^T, o_i = phi(q_i)^T S_i;
# LA 4.3: S_i = gamma S_{i-1} + ...; HM §2.3: numerator / denominator split]
# --------------------------------------------------------------------------
def linattn_recurrent(phiq, phik, v, log_a=None, s_init=None, z_init=None):
    """Token-by-token scan, vectorized over (b, h).

    Returns (o [B,H,n,dv], S [B,H,F,dv], z [B,H,F]): the outputs and the state
    after the last token.
    """
    B, H, n, F = phiq.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, F, dv)) if s_init is None else np.array(s_init, dtype=np.float64)
    z = np.zeros((B, H, F)) if z_init is None else np.array(z_init, dtype=np.float64)
    o = np.empty((B, H, n, dv))
    for t in range(n):
        if log_a is not None:
            a = np.exp(log_a[:, :, t])
            S *= a[:, :, None, None]
            z *= a[:, :, None]
        S += phik[:, :, t, :, None] * v[:, :, t, None, :]
        z += phik[:, :, t, :]
        num = np.einsum("bhf,bhfd->bhd", phiq[:, :, t, :], S)
        den = np.einsum("bhf,bhf->bh", phiq[:, :, t, :], z)
        o[:, :, t, :] = num / den[:, :, None]
    return o, S, z


def prefix_state(phik, v, log_a=None):
    """Closed form of the state after a prefix: S = sum_j (prod_{s>j} a_s) phi(k_j) v_j^T.

    One matrix product per (b, h); z is the same sum with v_j replaced by 1.
    """
    B, H, n, F = phik.shape
    dv = v.shape[-1]
    S = np.empty((B, H, F, dv))
    z = np.empty((B, H, F))
    for b in range(B):
        for h in range(H):
            if log_a is None:
                wgt = np.ones(n)
            else:
                tail = np.cumsum(log_a[b, h][::-1])[::-1]       # sum_{s>=j} log a_s
                wgt = np.exp(tail - log_a[b, h])                 # sum_{s>j}
            kw = phik[b, h] * wgt[:, None]
            S[b, h] = kw.T @ v[b, h]
            z[b, h] = kw.sum(axis=0)
    return S, z


# --------------------------------------------------------------------------
# Gate branch of the mixer  [HM §1 (Mamba's gate branch), §3.1, §5.2 step 6]
# --------------------------------------------------------------------------
def silu(x):
    """SiLU(x) = x * sigmoid(x), the gate branch's activation.  Evaluated as
    x / (1 + e^-x) for x >= 0 and x e^x / (1 + e^x) for x < 0, so that no
    exponential overflows."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, x / (1.0 + e), x * e / (1.0 + e))


def apply_gate(o, gate):
    """The normalized output multiplied element-wise by the gate branch's output
    SiLU(g) ([HM] §5.2 step 6); gate None leaves o unchanged."""
    if gate is None:
        return o
    return o * silu(gate)


# --------------------------------------------------------------------------
# Short causal conv of the mixer  [HM §2.2 (local mixing by a light conv),
# §2.3 item 4 (kept in HedgeMamba), §3.1 (init: taps [0, ..., 0, 1], bias 0)]
# --------------------------------------------------------------------------
def causal_conv(x, w, bias=None, prev=None):
    """Depthwise causal convolution over the token axis.

    x [B,H,n,d]; w [d,K] (one set of K taps per channel, shared by the heads) or
    [H,d,K]; bias [d] or [H,d] or None; prev [B,H,K-1,d] = the K-1 input rows that
    precede token 0 (None = zeros).  Tap K-1 multiplies the current token, tap j
    the token K-1-j steps earlier:
        y_t[c] = bias[c] + sum_j w[c, j] * x_{t-K+1+j}[c].
    Returns (y [B,H,n,d], final [B,H,K-1,d]) where final holds the last K-1 rows
    of the stream prev ++ x, i.e. the prev of a call that continues the sequence.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, H, n, d = x.shape
    K = w.shape[-1]
    wh = np.broadcast_to(w if w.ndim == 3 else w[None], (H, d, K))
    if prev is None:
        prev = np.zeros((B, H, K - 1, d))
    stream = np.concatenate([np.asarray(prev, dtype=np.float64), x], axis=2)  # row K-1+t is token t
    y = np.zeros((B, H, n, d))
    if bias is not None:
        bh = np.asarray(bias, dtype=np.float64)
        y += (bh if bh.ndim == 2 else bh[None])[None, :, None, :]
    for j in range(K):
        # stream rows j .. j+n-1 are tokens t-K+1+j for t = 0..n-1
        y += wh[None, :, None, :, j] * stream[:, :, j:j + n, :]
    return y, stream[:, :, n:n + K - 1, :].copy()


# --------------------------------------------------------------------------
# Rotary position encoding of the features  [HM §5.2 step 3: RoPE on phi(Q)
# and phi(K), as in the original Transformer and Pythia]
# --------------------------------------------------------------------------
def rope_angles(pos, dims, base=10000.0):
    """theta[..., i] = pos * base^(-2i/dims) for the dims/2 rotation pairs (float64)."""
    i = np.arange(dims // 2, dtype=np.float64)
    inv_freq = np.power(float(base), -2.0 * i / dims)
    return np.asarray(pos, dtype=np.float64)[..., None] * inv_freq


def rope(phi, pos, dims, base=10000.0):
    """Turn each pair (phi_i, phi_{i+dims/2}), i < dims/2, by the angle
    pos * base^(-2i/dims):  (x1, x2) -> (x1 cos - x2 sin, x2 cos + x1 sin)
    (the rotate-half form of GPT-NeoX); features at index >= dims are unchanged.

    phi [..., n, F]; pos broadcasts against phi's [..., n] (e.g. [n] or [B, 1, n]);
    dims is even and at most F; dims = 0 returns phi unchanged.
    """
    phi = np.asarray(phi, dtype=np.float64)
    if dims == 0:
        return phi.copy()
    h = dims // 2
    ang = rope_angles(pos, dims, base)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = phi[..., :h], phi[..., h:dims]
    out = phi.copy()
    out[..., :h] = x1 * c - x2 * s
    out[..., h:dims] = x2 * c + x1 * s
    return out


def rope_positions(B, n, pos0=None):
    """Positions [B, 1, n] of a prefill: pos0[b] + t (pos0 None = 0)."""
    p0 = np.zeros(B) if pos0 is None else np.asarray(pos0, dtype=np.float64).reshape(B)
    return (p0[:, None] + np.arange(n, dtype=np.float64)[None, :])[:, None, :]


# --------------------------------------------------------------------------
# Whole path and decode step
# --------------------------------------------------------------------------
def forward(q, k, v, w_q, w_k, dt=None, a_log=None, s_init=None, z_init=None, form="recurrent", gate=None,
            rope_dims=0, rope_base=10000.0, rope_pos0=None):
    """Featurize q and k, then run the chosen form; a gate [B,H,n,dv] (pre-activation)
    multiplies the output by SiLU(gate).  With rope_dims > 0 both feature maps are
    rotated at positions rope_pos0[b] + t before the sums.  Returns (o, S_final,
    z_final); the quadratic form returns None for the state."""
    phiq = hedgehog_features(q, w_q)
    phik = hedgehog_features(k, w_k)
    if rope_dims:
        pos = rope_positions(phiq.shape[0], phiq.shape[2], rope_pos0)
        phiq = rope(phiq, pos, rope_dims, rope_base)
        phik = rope(phik, pos, rope_dims, rope_base)
    v = np.asarray(v, dtype=np.float64)
    la = log_decay(dt, a_log)
    if form == "quadratic":
        return apply_gate(linattn_quadratic(phiq, phik, v, la, s_init, z_init), gate), None, None
    if form == "recurrent":
        o, S, z = linattn_recurrent(phiq, phik, v, la, s_init, z_init)
        return apply_gate(o, gate), S, z
    raise ValueError(form)


def step(S, z, q, k, v, w_q, w_k, dt=None, a_log=None, gate=None, rope_dims=0, rope_base=10000.0,
         rope_pos=None):
    """One decode step from state (S [B,H,F,dv], z [B,H,F]) with one token per
    (b, h): q, k [B,H,d], v [B,H,dv], dt [B,H], gate [B,H,dv] or None, and with
    rope_dims > 0 the token's position rope_pos [B].
    Returns (o [B,H,dv], S', z').  This is the recurrent form advanced by a single
    token  [LA part 5]."""
    q = np.asarray(q, dtype=np.float64)[:, :, None, :]
    k = np.asarray(k, dtype=np.float64)[:, :, None, :]
    v = np.asarray(v, dtype=np.float64)[:, :, None, :]
    dt3 = None if dt is None else np.asarray(dt, dtype=np.float64)[:, :, None]
    o, S2, z2 = forward(q, k, v, w_q, w_k, dt3, a_log, S, z, rope_dims=rope_dims, rope_base=rope_base,
                        rope_pos0=rope_pos)
    return apply_gate(o[:, :, 0, :], gate), S2, z2


# --------------------------------------------------------------------------
# Per-channel decay: the scan the way the pages wire it through Mamba-1's
# selective scan  [HM §2.3 item 3 and §5.2 step 4: A, dt and V are copied and
# concatenated, the V copy replaced by ones, so every value channel has a
# numerator and a denominator channel with the same A row and step size;
# Mamba's discretization (HM §2.2, SSM §3.2): a = exp(Delta A) with
# Delta = softplus(dt), input scaled by Delta]
# --------------------------------------------------------------------------
def pc_scan(phiq, phik, v, delta, A, sn0=None, sd0=None):
    """Per (b, h), value channel c and state n (n runs over the F features):
        a_t[c, n] = exp(delta_t[c] * A[c, n])
        Sn_t[c, n] = a_t[c, n] Sn_{t-1}[c, n] + delta_t[c] phik_t[n] v_t[c]
        Sd_t[c, n] = a_t[c, n] Sd_{t-1}[c, n] + delta_t[c] phik_t[n]
        o_t[c] = sum_n phiq_t[n] Sn_t[c, n] / sum_n phiq_t[n] Sd_t[c, n]
    phiq, phik [B,H,n,F]; v, delta [B,H,n,dv]; A [H,dv,F] (or [dv,F] shared);
    sn0, sd0 [B,H,F,dv] initial states (None = zeros).  Token by token,
    vectorized over (b, h, c, n).  Returns (o [B,H,n,dv], Sn, Sd) with the
    states laid out [B,H,F,dv]."""
    phiq = np.asarray(phiq, dtype=np.float64)
    phik = np.asarray(phik, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    delta = np.asarray(delta, dtype=np.float64)
    B, H, n, F = phiq.shape
    dv = v.shape[-1]
    A = np.asarray(A, dtype=np.float64)
    At = np.broadcast_to(A if A.ndim == 3 else A[None], (H, dv, F)).transpose(0, 2, 1)   # [H, F, dv]
    Sn = np.zeros((B, H, F, dv)) if sn0 is None else np.array(sn0, dtype=np.float64)
    Sd = np.zeros((B, H, F, dv)) if sd0 is None else np.array(sd0, dtype=np.float64)
    o = np.empty((B, H, n, dv))
    for t in range(n):
        dl = delta[:, :, t, None, :]                       # [B,H,1,dv]
        a = np.exp(dl * At[None])                          # [B,H,F,dv]
        kk = phik[:, :, t, :, None] * dl                   # [B,H,F,dv]
        Sn = a * Sn + kk * v[:, :, t, None, :]
        Sd = a * Sd + kk
        num = np.einsum("bhf,bhfd->bhd", phiq[:, :, t], Sn)
        den = np.einsum("bhf,bhfd->bhd", phiq[:, :, t], Sd)
        o[:, :, t] = num / den
    return o, Sn, Sd


def forward_pc(q, k, v, w_q, w_k, dt, a_log, sn0=None, sd0=None, gate=None):
    """Featurize q and k, then the per-channel scan with Delta = softplus(dt)
    (dt [B,H,n,dv]) and A = -exp(A_log) (A_log [H,dv,F] or [dv,F]); the gate as in
    forward.  Returns (o, Sn_final, Sd_final)."""
    phiq = hedgehog_features(q, w_q)
    phik = hedgehog_features(k, w_k)
    delta = softplus(dt)
    A = -np.exp(np.asarray(a_log, dtype=np.float64))
    o, Sn, Sd = pc_scan(phiq, phik, v, delta, A, sn0, sd0)
    return apply_gate(o, gate), Sn, Sd


def step_pc(Sn, Sd, q, k, v, w_q, w_k, dt, a_log, gate=None):
    """One decode step of the per-channel scan: q, k [B,H,d], v, dt [B,H,dv]."""
    o, Sn2, Sd2 = forward_pc(np.asarray(q, dtype=np.float64)[:, :, None], np.asarray(k, dtype=np.float64)[:, :, None],
                             np.asarray(v, dtype=np.float64)[:, :, None], w_q, w_k,
                             np.asarray(dt, dtype=np.float64)[:, :, None], a_log, Sn, Sd)
    return apply_gate(o[:, :, 0], gate), Sn2, Sd2


def pack_state_pc(Sn, Sd):
    """Boundary layout of the per-channel state, channel-major like A_log: per (b, h)
    Sn [dv][F] then Sd [dv][F] (the oracle's arrays are [B,H,F,dv])."""
    B, H, F, dv = Sn.shape
    return np.concatenate([Sn.transpose(0, 1, 3, 2).reshape(B, H, F * dv),
                           Sd.transpose(0, 1, 3, 2).reshape(B, H, F * dv)], axis=-1)


def unpack_state_pc(flat, F, dv):
    flat = np.asarray(flat, dtype=np.float64)
    B, H, _ = flat.shape
    return (flat[:, :, : F * dv].reshape(B, H, dv, F).transpose(0, 1, 3, 2),
            flat[:, :, F * dv:].reshape(B, H, dv, F).transpose(0, 1, 3, 2))


# --------------------------------------------------------------------------
# State buffer layout used at the library boundary: per (b, h) one contiguous
# block of F*dv + F float32 values, the numerator S [F][dv] row-major followed
# by the denominator state z [F].
# --------------------------------------------------------------------------
def pack_state(S, z):
    B, H, F, dv = S.shape
    return np.concatenate([S.reshape(B, H, F * dv), z.reshape(B, H, F)], axis=-1)


def unpack_state(flat, F, dv):
    flat = np.asarray(flat, dtype=np.float64)
    B, H, _ = flat.shape
    return flat[:, :, : F * dv].reshape(B, H, F, dv), flat[:, :, F * dv:]
