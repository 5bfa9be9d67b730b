/*
 * hm.h — C ABI of the MI355X (gfx950) library for causal, normalized Hedgehog
 * linear attention, the hot path of the HedgeMamba mixer.
 *
 * Pages that define the operations:
 *   [HM]  "HedgeMamba：融合线性注意力与状态空间模型的高效序列建模" (gsyq.cn):
 *         §2.1 Hedgehog feature map, §2.3 state expansion with a numerator and
 *         a denominator, §3.1 stage-1 identity init (a_t = 1), §5.2 the mixer's
 *         [batch, seq_len, num_heads, head_dim] tensors, §5.3 HedgehogProjection.
 *   [LA]  "线性注意力（Linear Attention）详解" (cnblogs): part 2 normalized kernel
 *         attention, part 3 recurrent state S_i = S_{i-1} + phi(k_i) v_i^T,
 *         part 4.3 scalar decay, part 5 chunk-parallel and recurrent modes,
 *         "Q、K、V 的维度详解" (Q,K [b,h,n,d], V [b,h,n,d_v], S [b,h,d,d_v]).
 *   [SSM] "状态空间模型：Mamba、S4 的线性复杂度路径" (quant67.com): §3.2 softplus on
 *         the step size, §4.2 associative composition of affine maps.
 *
 * The computation, per batch b, head h and token t (F = 2f is the feature width):
 *   phi(x)  = softmax([x W, -x W])                       (feature axis)
 *   log a_t = -softplus(dt[b,h,t]) * exp(A_log[h])       (a_t = 1 when dt is NULL)
 *   S_t = a_t S_{t-1} + phi(k_t) v_t^T   [F x dv]
 *   z_t = a_t z_{t-1} + phi(k_t)         [F]
 *   o_t = phi(q_t)^T S_t / phi(q_t)^T z_t
 *   o_t <- o_t * SiLU(g_t)  when a gate g is given (the mixer's gate branch,
 *                           [HM] §5.2 step 6; SiLU(x) = x / (1 + e^-x))
 * and, when rope_dims > 0, phi(q_t) and phi(k_t) are first turned by the rotary
 * position encoding ([HM] §5.2 step 3, in the GPT-NeoX rotate-half form, the
 * architecture of the Pythia models the page builds on): for i < rope_dims/2 the
 * pair (phi_i, phi_{i + rope_dims/2}) becomes
 *   (phi_i cos(p w_i) - phi_{i+r/2} sin(p w_i),  phi_{i+r/2} cos(p w_i) + phi_i sin(p w_i))
 * with w_i = rope_base^(-2i/rope_dims) and p the token's position; entries from
 * rope_dims on are unchanged.  Numerator and denominator both use the turned
 * features.  They are signed, so the denominator is no longer positive by
 * construction; no epsilon is added (o = num / den as defined).
 *
 * Rotary fields, shared by hm_featurize, hm_linattn_fwd, hm_linattn_bwd and
 * hm_linattn_step: rope_dims 0 = off, else a multiple of 32, at most 2f
 * (HM_ERR_SHAPE if negative, above 2f or odd; HM_ERR_UNSUPPORTED if even but not a
 * multiple of 32); rope_base > 0 and finite (HM_ERR_SHAPE otherwise; 10000 in
 * GPT-NeoX); positions: device int64, one per batch row, 8-byte aligned
 * (HM_ERR_ALIGN): rope_pos0[b] is the position of token 0 of a prefill (NULL =
 * 0 for every row), rope_pos[b] the position of a decode step's token (required).
 * Each angle is formed and reduced to one turn in float64, then a float32 sine and
 * cosine are taken: the angle's error is about p * 2^-52 radians (below 1e-6 for
 * positions under 2^32).
 *
 * Conventions shared by every entry point:
 *   - Every data pointer is DEVICE memory owned by the caller.  The library never
 *     allocates, frees, copies to the host or synchronizes; all work is enqueued on
 *     `stream` (a hipStream_t; NULL means the default stream).
 *   - Strides are in ELEMENTS; the last (feature) dimension is always contiguous.
 *     Base pointers must be 16-byte aligned, and every stride times the element
 *     size must be a multiple of 16 bytes.
 *   - W is [d, f] row-major and applied as x @ W (no bias, no temperature).  One W
 *     may serve all heads (sw_h = 0) or each head may have its own (sw_h = d*f).
 *   - dt is float32 [B, H, n] (strides sdt_*), A_log float32 [H] contiguous.  Both
 *     NULL selects the identity decay; exactly one NULL is HM_ERR_NULL.
 *   - State buffers are float32, one contiguous block of F*dv + F values per
 *     (b, h), blocks at stride (F*dv + F), [b][h] order: the numerator S [F][dv]
 *     row-major followed by the denominator state z [F].
 *   - All arguments are checked on the host before any HIP call.  A failed check
 *     returns its code, launches nothing and sets hm_last_error_message().  A
 *     launch failure returns HM_ERR_HIP.  Device faults surface at the caller's
 *     next synchronization.  NaN/Inf in the inputs are not checked; they
 *     propagate to the outputs.
 *   - Supported sizes (anything else is HM_ERR_UNSUPPORTED):
 *       hm_linattn_fwd, hm_linattn_step: d in {16, 32, 64, 128}, f in {16, 32, 64},
 *         dv in {16, 32, 64, 128}, bf16 and f32.  The prefill runs fused kernels
 *         (chunk 64 or 128; segments, column splits, gate, rotary, saves) at
 *           bf16:  d in {64, 128}, f in {32, 64}, dv in {64, 128}; (d, f, dv) =
 *                  (32, 16, 32); dv = 32 at every (d, f) of this line; and
 *                  (32, 16, 64) as two 32-column workgroups (dsplit 2)
 *           f32:   d in {16, 32}, f = 16, dv in {16, 32}; and d = 64 with
 *                  (f, dv) in {(16, 16), (16, 32), (32, 32), (32, 64)}
 *         and every other size, and chunk 256 at every size, on the
 *         chunk-parallel path (see hm_linattn_fwd): the plain prefill only (no
 *         gate, rotary encoding or training saves; segments 0; dsplit 0 or 1).
 *         The fused kernels hold W_q^T, W_k^T, phi(q), phi(k)^T, the score tile
 *         and the output rows of a 64-token chunk in LDS (157 KB at bf16, d = 128,
 *         f = 64), which float32 at that size would double; bf16 d = 16 is below
 *         one 32-deep bf16 MFMA step; f = 16 at the larger d and dv is not
 *         instantiated.  The decode step is built at every size and dtype.
 *       hm_featurize:
 *         bf16 x: d in {16, 32, 64, 128}, f in {16, 32, 64} (phi bf16 or f32)
 *         f32 x:  d in {16, 32, 64, 128}, f in {16, 32, 64}
 *       with rope_dims > 0, hm_linattn_fwd is built for bf16 (d, f) in
 *       {(128, 64), (64, 32)} and f32 (d, f) in {(16, 16), (32, 16)}; the step and
 *       the featurizer for every size above.
 *     B, H, n may be 0 (nothing to compute; s_final is still written).
 */
#ifndef HM_H
#define HM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HM_ABI_VERSION 9

typedef enum {
  HM_OK = 0,
  HM_ERR_NULL = 1,        /* a required pointer is NULL (or dt/A_log given alone) */
  HM_ERR_SHAPE = 2,       /* negative size, or a stride that makes rows overlap   */
  HM_ERR_DTYPE = 3,       /* unknown dtype code                                    */
  HM_ERR_ALIGN = 4,       /* pointer or stride not 16-byte aligned                 */
  HM_ERR_UNSUPPORTED = 5, /* valid but not built: see the size table above         */
  HM_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required            */
  HM_ERR_HIP = 7          /* a HIP launch failed                                   */
} hm_status;

typedef enum { HM_F32 = 0, HM_BF16 = 1 } hm_dtype;

/*
 * hm_featurize — the Hedgehog feature map alone ([HM] §2.1, §5.3):
 *   phi[b,h,t,:] = softmax([x[b,h,t,:] W_h, -x[b,h,t,:] W_h]),  F = 2f entries,
 *   the +xW half first.
 * x: [B, H, n, d] in `dtype` (strides sx_*); w: [d, f] in `dtype` (head stride
 * sw_h); phi: [B, H, n, 2f] in `phi_dtype` (strides sp_*).  The projection is
 * accumulated in float32, the softmax is evaluated in float32.
 * With conv_width K > 0 the mixer's short causal conv (the one hm_causal_conv
 * computes, [HM] §2.3 item 4) is applied to x in the featurizer's load prologue:
 * each loaded row slice becomes bias + sum_j w[c][j] x[t-K+1+j][c] (float32, bias
 * then taps oldest first, rows before token 0 from conv_prev or zero), rounded to
 * `dtype`, before the projection: phi equals hm_featurize of hm_causal_conv's
 * output bit for bit, without writing the convolved x.  conv_width above 4 is
 * HM_ERR_UNSUPPORTED; K > 0 with conv_w NULL is HM_ERR_NULL.
 */
typedef struct {
  const void *x;
  const void *w;
  void *phi;
  int32_t dtype;      /* hm_dtype of x and w */
  int32_t phi_dtype;  /* hm_dtype of phi     */
  int64_t B, H, n, d, f;
  int64_t sx_b, sx_h, sx_t;
  int64_t sw_h;
  int64_t sp_b, sp_h, sp_t;
  int32_t rope_dims;        /* 0 = off (see the rotary fields above) */
  float rope_base;
  const int64_t *rope_pos0; /* [B] position of token 0 of each row, or NULL */
  /* optional short causal conv applied to x as it is loaded (conv_width 0 = none) */
  int32_t conv_width;       /* K taps, 0..4 */
  int32_t reserved;
  const float *conv_w;      /* float32 [d][K] (head stride scw_h), tap K-1 on the current token */
  const float *conv_b;      /* float32 [d] (head stride scb_h) or NULL */
  const void *conv_prev;    /* [B, H, K-1, d] in dtype, contiguous: the rows before token 0, or NULL (zeros) */
  int64_t scw_h, scb_h;
} hm_featurize_args;

hm_status hm_featurize(const hm_featurize_args *args, void *stream);

/*
 * hm_linattn_fwd — causal prefill over n tokens (the chunk-parallel mode of
 * [LA] part 5): featurize q and k, run the decayed state scan with the
 * numerator/denominator split of [HM] §2.3, write o.
 *   q, k: [B, H, n, d]; v: [B, H, n, dv]; o: [B, H, n, dv] — all in `dtype`
 *   (strides s*_b, s*_h, s*_t; inner dimension contiguous).
 *   w_q, w_k: [d, f] each (head stride sw_h).
 *   s_init: optional initial state (NULL = zeros); s_final: optional, receives the
 *   state after token n-1.  They may point to the same buffer.
 *   chunk: the chunk length of the chunk-wise form, 0 = automatic (64), 64, 128
 *   or 256.  A chunk's outputs read the state at the chunk's start plus the
 *   masked, decayed scores of all its earlier tokens, and the state passes once
 *   per chunk.  128 runs the fused kernels for the plain prefill (no `save`, gate
 *   or rotary encoding: HM_ERR_UNSUPPORTED).  256, and every size without a fused
 *   kernel, run the chunk-parallel path: one pass writes every chunk's local end
 *   state and summed log-decay to the workspace, a scan over the chunks turns
 *   them into start states (and s_final), and a last pass forms each 64-query
 *   block's outputs from its chunk's start state and the chunk's earlier keys.
 *   That path takes the plain prefill only, segments = 0 and dsplit 0 or 1
 *   (else HM_ERR_UNSUPPORTED); its workspace is B*H*ceil(n/chunk)*(F*dv + F + 1)
 *   floats (rounded up), linear in n, and the plan reports one segment per chunk.
 *   segments: 0 = automatic, else the number of sequence segments scanned in
 *   parallel (their start states are joined by the affine composition of
 *   [SSM] §4.2).  dsplit: 0 = automatic, 1 or 2 = number of workgroups that
 *   share one (b, h), each owning dv/dsplit value columns.
 *   workspace: device scratch of at least hm_linattn_fwd_workspace_size() bytes
 *   (it may be NULL when that size is 0).  On the fused kernels its size grows
 *   with B*H*segments (up to 4 state blocks per segment: the segment pass may cut
 *   a segment into equal pieces when that fills more of the GPU); on the
 *   chunk-parallel path with B*H*chunks; never with n^2.
 *   save: optional (NULL = inference), hm_linattn_save_size() bytes: the forward
 *   also keeps what hm_linattn_bwd reads (a float32 state checkpoint at the start
 *   of each of the backward's chunk ranges, at most 256 / (B*H) of them per
 *   (b, h), the denominators and the float32 output before the gate); it then
 *   runs with dsplit 1.  Built for the sizes hm_linattn_bwd lists.
 *   gate: optional [B, H, n, dv] in `dtype` (strides sg_*), the pre-activation of
 *   the mixer's gate branch; when given, o = (normalized output) * SiLU(gate),
 *   rounded once to `dtype` after the normalized output was rounded (NULL = no
 *   gate).
 * Accumulation is float32 and the carried state is float32; bf16 operands of the
 * matrix products (phi, the masked score tile, the state copy used for the
 * read-out) are rounded to nearest even.
 */
typedef struct {
  const void *q, *k, *v, *w_q, *w_k;
  const float *dt, *a_log;
  const float *s_init;
  float *s_final;
  void *o;
  int32_t dtype;
  int32_t chunk;
  int32_t segments;
  int32_t dsplit;
  int64_t B, H, n, d, f, dv;
  int64_t sq_b, sq_h, sq_t;
  int64_t sk_b, sk_h, sk_t;
  int64_t sv_b, sv_h, sv_t;
  int64_t so_b, so_h, so_t;
  int64_t sw_h;
  int64_t sdt_b, sdt_h, sdt_t;
  void *workspace;
  size_t workspace_bytes;
  const void *gate;
  int64_t sg_b, sg_h, sg_t;
  void *save;
  size_t save_bytes;
  int32_t rope_dims;        /* 0 = off (see the rotary fields above) */
  float rope_base;
  const int64_t *rope_pos0; /* [B] position of token 0 of each row, or NULL */
} hm_linattn_fwd_args;

hm_status hm_linattn_fwd_workspace_size(const hm_linattn_fwd_args *args, size_t *bytes);

/* The (chunk, segments, dsplit) that hm_linattn_fwd will use for these args. */
hm_status hm_linattn_fwd_plan(const hm_linattn_fwd_args *args, int32_t *chunk,
                              int32_t *segments, int32_t *dsplit);

hm_status hm_linattn_fwd(const hm_linattn_fwd_args *args, void *stream);

/*
 * hm_linattn_fwd_noalloc — hm_linattn_fwd for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same prefill, kernels and plan, with the workspace taken from a
 * scratch array the library holds on each GPU instead of from the caller.
 * `workspace` and `workspace_bytes` are ignored; every other field is as for
 * hm_linattn_fwd (the caller still passes all inputs and outputs, `save` included).
 *   - The scratch is HM_NOALLOC_SCRATCH_BYTES (40 MiB) per GPU, a static device
 *     array that each GPU the library runs on holds until the process ends.  Every
 *     automatic plan of the fused kernels fits (its segment states stay within 256
 *     state blocks plus a copy of s_init); a plan that needs more (many explicit
 *     `segments` with many heads, or a chunk-parallel plan whose B*H*chunks state
 *     blocks exceed it) returns HM_ERR_WORKSPACE and launches nothing.
 *   - The first call with a device current looks up that device's scratch address
 *     (hipGetSymbolAddress); a failure there returns HM_ERR_HIP.  No call allocates
 *     or frees memory.
 *   - Every call on one GPU shares that GPU's scratch: calls that may overlap on one
 *     GPU (other streams, other threads) race and must be ordered by the caller.
 *     Nothing in the scratch needs to start at zero: each call writes every value
 *     it later reads.
 */
#define HM_NOALLOC_SCRATCH_BYTES (40 << 20)
hm_status hm_linattn_fwd_noalloc(const hm_linattn_fwd_args *args, void *stream);

/* Bytes of the `save` buffer a training forward needs (only B, H, n, f, dv and
 * dtype of args are read). */
hm_status hm_linattn_save_size(const hm_linattn_fwd_args *args, size_t *bytes);

/*
 * hm_linattn_bwd — gradients of the prefill (training: [HM] §3 trains the mixer;
 * the chunk-wise form of [LA] part 5 run backwards).  For a scalar loss with
 * d_o = dloss/do (and optionally d_s_final = dloss/ds_final) it writes
 *   d_q, d_k: [B, H, n, d] in `dtype`, strides of q / k;  d_v: like v;
 *   d_wq, d_wk: float32 [d][f] (one W) or [H][d][f] (sw_h = d*f), overwritten;
 *   d_dt: float32 with dt's strides and d_a_log: float32 [H], when dt is given;
 *   d_s_init: optional float32 state-layout gradient of s_init.
 * Inputs: the forward's q, k, v, w_q, w_k, dt, a_log (same strides), d_o (strides
 * so_*), and `save`: the buffer the forward filled when it was called with a
 * non-NULL `save` (hm_linattn_save_size bytes; that forward runs with dsplit 1;
 * it holds the float32 output before the gate, so o itself is not an input).
 * gate: the forward's gate or NULL; with it, d_gate (strides sg_*, like gate)
 * receives d_o * o * SiLU'(g) and the core sees d_o * SiLU(g).  d_s_final: optional
 * dloss/ds_final (float32, state layout).  Outputs must not overlap inputs.
 * Math: with dnum_t = dO_t / den_t and dden_t = -(dO_t . o_t) / den_t, the gradient
 * of the state at each chunk end, G <- e^{Lam} G + sum_t e^{L_t} phi(q_t) dnum_t^T,
 * runs from the last chunk back.  The state at every chunk start is recomputed
 * from the nearest checkpoint in `save` (the forward's state update, one pass per
 * chunk range, the ranges in parallel); d log a_t is the sum, over
 * the (query, key) pairs whose decay product contains a_t, of their weight times
 * its loss gradient, taken per chunk without differences of nearly equal terms.
 * Products in the dtype on MFMA with float32 accumulation; the decay gradient's
 * per-chunk sums in float64.
 * Built: bf16 (d, f, dv) = (64, 32, 64), (128, 64, 128); f32 (16, 16, 16), (32, 16, 32).
 * workspace: hm_linattn_bwd_workspace_size() bytes (O(B*H*n*(2F+dv))).
 */
typedef struct {
  const void *q, *k, *v, *w_q, *w_k;
  const float *dt, *a_log;
  const void *d_o;
  const void *gate;
  const float *d_s_final;
  const void *save;
  size_t save_bytes;
  void *d_q, *d_k, *d_v, *d_gate;
  float *d_wq, *d_wk, *d_dt, *d_a_log, *d_s_init;
  int32_t dtype;
  int32_t reserved;
  int64_t B, H, n, d, f, dv;
  int64_t sq_b, sq_h, sq_t, sk_b, sk_h, sk_t, sv_b, sv_h, sv_t, so_b, so_h, so_t, sg_b, sg_h, sg_t;
  int64_t sw_h, sdt_b, sdt_h, sdt_t;
  void *workspace;
  size_t workspace_bytes;
  int32_t rope_dims;        /* the forward's rotary fields */
  float rope_base;
  const int64_t *rope_pos0;
} hm_linattn_bwd_args;

hm_status hm_linattn_bwd_workspace_size(const hm_linattn_bwd_args *args, size_t *bytes);
hm_status hm_linattn_bwd(const hm_linattn_bwd_args *args, void *stream);

/*
 * hm_linattn_step — one decode token per (b, h) (the recurrent mode of [LA]
 * part 5): featurize q_t, k_t, then S <- a_t S + phi(k_t) v_t^T,
 * z <- a_t z + phi(k_t), o_t = phi(q_t)^T S / phi(q_t)^T z.  The state is read and
 * written in place.
 *   q, k: [B, H, d]; v, o: [B, H, dv] in `dtype` (strides s*_b, s*_h);
 *   dt: [B, H] float32 (strides sdt_b, sdt_h) or NULL; state: see above.
 *   gate: optional [B, H, dv] in `dtype` (strides sg_b, sg_h): o_t is multiplied
 *   by SiLU(gate) (NULL = no gate).
 *   conv_width: 0 = no conv; 1..4 = q_t and k_t first pass through the mixer's
 *   short causal conv, exactly as hm_causal_conv with n = 1 would compute it (same
 *   order of operations, result rounded to `dtype`), with taps conv_wq / conv_wk
 *   float32 [d][K] (head stride scw_h), bias conv_bq / conv_bk float32 [d] (head
 *   stride scb_h) or NULL, and conv states conv_sq / conv_sk [B, H, K-1, d] in
 *   `dtype`, contiguous: the K-1 previous input rows, read and shifted in place
 *   (hm_causal_conv's final_rows after a prefill is this state).
 */
typedef struct {
  const void *q, *k, *v, *w_q, *w_k;
  const float *dt, *a_log;
  float *state;
  void *o;
  int32_t dtype;
  int32_t conv_width;
  int64_t B, H, d, f, dv;
  int64_t sq_b, sq_h, sk_b, sk_h, sv_b, sv_h, so_b, so_h;
  int64_t sw_h;
  int64_t sdt_b, sdt_h;
  const void *gate;
  int64_t sg_b, sg_h;
  const float *conv_wq, *conv_wk, *conv_bq, *conv_bk;
  void *conv_sq, *conv_sk;
  int64_t scw_h, scb_h;
  int32_t rope_dims;        /* 0 = off (see the rotary fields above) */
  float rope_base;
  const int64_t *rope_pos;  /* [B] position of each row's token (required when on) */
} hm_linattn_step_args;

hm_status hm_linattn_step(const hm_linattn_step_args *args, void *stream);

/*
 * hm_causal_conv — the mixer's short causal convolution ([HM] §2.2: Mamba's light
 * conv mixes neighbouring tokens; §2.3 item 4: HedgeMamba keeps it; §3.1: taps
 * [0, ..., 0, 1] and zero bias make it the identity at the stage-1 init).  Applied
 * to q and to k ahead of hm_linattn_fwd / hm_linattn_step, one call per tensor.
 * Depthwise over the token axis, K = width taps per channel:
 *   y[b,h,t,c] = bias[c] + sum_{j<K} w[c][j] * x[b,h,t-K+1+j,c]
 * where rows t < 0 come from `prev` (the K-1 rows before token 0; NULL = zeros).
 *   x, y: [B, H, n, d] in `dtype` (strides s*_b, s*_h, s*_t); y must not overlap x,
 *   prev or final_rows.
 *   w: float32 [d][K] (each channel's K taps, tap K-1 on the current token), head
 *   stride sw_h (0 = shared by the heads); bias: float32 [d] (head stride sb_h) or
 *   NULL.
 *   prev, final_rows: [B, H, K-1, d] in `dtype`, contiguous, optional.  final_rows
 *   receives the last K-1 rows of the stream prev ++ x (the prev of a call that
 *   continues the sequence); it may be the same buffer as prev, so a decode step
 *   (n = 1) keeps its conv state in place.  With n = 0 only final_rows is written
 *   and x, y, w may be NULL.
 * Products and sums in float32, y rounded to `dtype` to nearest even.
 * Built: width 1..4; d times the element size a multiple of 16 bytes; one thread
 * per 8 tokens and 16 bytes of channels, fewer than 2^31 threads (B*H*n*d below
 * about 2^37 elements for bf16, 2^36 for f32).
 */
typedef struct {
  const void *x;
  void *y;
  const float *w, *bias;
  const void *prev;
  void *final_rows;
  int32_t dtype;
  int32_t width;
  int64_t B, H, n, d;
  int64_t sx_b, sx_h, sx_t;
  int64_t sy_b, sy_h, sy_t;
  int64_t sw_h, sb_h;
} hm_causal_conv_args;

hm_status hm_causal_conv(const hm_causal_conv_args *args, void *stream);

/*
 * hm_linattn_pc_fwd — prefill with a decay per value channel and state: the
 * scan as the pages wire the mixer through Mamba-1's selective scan ([HM] §2.3
 * item 3 and §5.2 step 4: A, dt and V are copied and concatenated, the V copy
 * set to ones, so each value channel c has a numerator and a denominator channel
 * sharing its A row and step size; Mamba's discretization, [SSM] §3.2).  Per
 * (b, h), channel c < dv and state n < F = 2f (the feature index):
 *   Delta_t[c] = softplus(dt[b,h,t,c]),   a_t[c,n] = exp(-Delta_t[c] exp(A_log[h,c,n]))
 *   Sn[c,n] <- a_t[c,n] Sn[c,n] + Delta_t[c] phi(k_t)[n] v_t[c]
 *   Sd[c,n] <- a_t[c,n] Sd[c,n] + Delta_t[c] phi(k_t)[n]
 *   o_t[c]  = sum_n phi(q_t)[n] Sn[c,n] / sum_n phi(q_t)[n] Sd[c,n]
 * then the optional gate (o *= SiLU(gate)) and, when rope_dims > 0, phi(q) and
 * phi(k) turned first exactly as in hm_linattn_fwd.
 *   q, k: [B, H, n, d]; v, o (and gate): [B, H, n, dv] in `dtype` (strides s*_*).
 *   w_q, w_k: [d, f] (head stride sw_h).
 *   dt: float32 [B, H, n, dv] (strides sdt_b, sdt_h, sdt_t; channels contiguous).
 *   a_log: float32 [dv][F] per head, head stride sa_h (0 = shared, dv*F = per head).
 *   s_init, s_final: optional float32 state, per (b, h) one block of 2*dv*F values:
 *   Sn [dv][F] then Sd [dv][F]; they may be the same buffer.
 * The scan is element-wise (a decay per (c, n) does not factor into the chunked
 * matrix products of hm_linattn_fwd): one exponential per token, channel and state,
 * float32 throughout, phi kept in float32.  q, k, v, w_q, w_k, o, dt and a_log
 * are required whenever B*H*n > 0 (with n = 0 only the state is copied or zeroed).
 * segments: 0 = automatic, else the number of sequence segments scanned in
 * parallel (at most one per 64-token chunk).  A segment pass scans every segment
 * but the last from a zero state; the start states then follow by the
 * element-wise affine composition (a segment's decay product is
 * exp(-exp(A_log[c,n]) * sum of Delta_t[c] over it), [SSM] §4.2), and the full
 * pass scans every segment from its start state.  This doubles the scan work of
 * all segments but the last, so the automatic plan splits only when fewer than 65
 * workgroups (one per (b, h) and 64 channels) would cover the GPU's 256 compute
 * units: then into up to 256 / workgroups segments of at least four chunks.
 * workspace: hm_linattn_pc_fwd_workspace_size() bytes, 16-byte aligned (NULL when
 * that size is 0): per (b, h) one state block per segment and dv floats per
 * segment boundary.
 * Built: bf16 (d, f, dv) = (128, 64, 128), (64, 32, 64); f32 (16, 16, 16), (32, 16, 32).
 */
typedef struct {
  const void *q, *k, *v, *w_q, *w_k;
  const float *dt, *a_log;
  const float *s_init;
  float *s_final;
  void *o;
  const void *gate;
  int32_t dtype;
  int32_t rope_dims;        /* 0 = off (see the rotary fields above) */
  float rope_base;
  int32_t reserved;
  const int64_t *rope_pos0; /* [B] position of token 0 of each row, or NULL */
  int64_t B, H, n, d, f, dv;
  int64_t sq_b, sq_h, sq_t, sk_b, sk_h, sk_t, sv_b, sv_h, sv_t, so_b, so_h, so_t, sg_b, sg_h, sg_t;
  int64_t sw_h, sdt_b, sdt_h, sdt_t, sa_h;
  int32_t segments;         /* 0 = automatic (see above) */
  int32_t reserved2;
  void *workspace;
  size_t workspace_bytes;
} hm_linattn_pc_args;

hm_status hm_linattn_pc_fwd(const hm_linattn_pc_args *args, void *stream);
/* The segment count hm_linattn_pc_fwd will use for these sizes, and the workspace
 * bytes it needs (0 when it runs as one segment).  Only the sizes, dtype and
 * segments of args are read. */
hm_status hm_linattn_pc_fwd_plan(const hm_linattn_pc_args *args, int32_t *segments);
hm_status hm_linattn_pc_fwd_workspace_size(const hm_linattn_pc_args *args, size_t *bytes);

/*
 * hm_linattn_pc_step — one decode token per (b, h) of the per-channel scan above
 * (the state of hm_linattn_pc_fwd, updated in place): q, k [B, H, d], v, o, gate
 * [B, H, dv] in `dtype`, dt float32 [B, H, dv] (strides sdt_b, sdt_h), a_log as
 * above, state float32 [B*H] blocks of 2*dv*F.  The short conv and the rotary
 * fields work as in hm_linattn_step.  Same sizes as hm_linattn_pc_fwd.
 */
typedef struct {
  const void *q, *k, *v, *w_q, *w_k;
  const float *dt, *a_log;
  float *state;
  void *o;
  const void *gate;
  int32_t dtype;
  int32_t conv_width;
  int64_t B, H, d, f, dv;
  int64_t sq_b, sq_h, sk_b, sk_h, sv_b, sv_h, so_b, so_h, sg_b, sg_h;
  int64_t sw_h, sdt_b, sdt_h, sa_h;
  const float *conv_wq, *conv_wk, *conv_bq, *conv_bk;
  void *conv_sq, *conv_sk;
  int64_t scw_h, scb_h;
  int32_t rope_dims;
  float rope_base;
  const int64_t *rope_pos;
} hm_linattn_pc_step_args;

hm_status hm_linattn_pc_step(const hm_linattn_pc_step_args *args, void *stream);

const char *hm_status_string(int status);
/* Detail of the last failure on the calling thread ("" if none). */
const char *hm_last_error_message(void);
int hm_abi_version(void);
/* sizeof of the argument structs (0: featurize, 1: fwd, 2: step, 3: causal conv, 4: bwd, 5: pc fwd,
 * 6: pc step), for bindings. */
size_t hm_args_size(int which);

#ifdef __cplusplus
}
#endif

#endif /* HM_H */
