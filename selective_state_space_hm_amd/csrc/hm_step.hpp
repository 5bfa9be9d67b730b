// Decode step and standalone featurizer.
//
// Decode (the recurrent mode of the cnblogs linear-attention tutorial, part 5;
// per-step cost is the fixed-size state, quant67 SSM lecture §5.1): one
// workgroup per (b, h).  The kernel is bound by HBM traffic on the state
// (F*dv + F floats read and written once), so it is organised around that:
// W and the token's q, k values are fetched first (W straight into LDS), then
// every thread issues all of its 16-byte state loads, computes the two Hedgehog
// features and the decay from LDS and registers while they are in flight, then
// updates, reads out and stores its slice with 16-byte accesses.  (Loads retire
// in order, so a global load issued after the state loads and waited for during
// the featurization would wait for the whole state.)
#pragma once

#include "hm_device.hpp"

namespace hm {

struct StepParams {
  const void *q, *k, *v, *wq, *wk;
  const float *dt, *a_log;
  float *state;
  void *o;
  int64_t B, H;
  int64_t sq_b, sq_h, sk_b, sk_h, sv_b, sv_h, so_b, so_h, sw_h, sdt_b, sdt_h;
  const void *gate;  // optional gate pre-activation [B, H, dv] (NULL = none)
  int64_t sg_b, sg_h;
  // optional short causal conv on q and k (width 0 = none): taps [d][K], bias [d]
  // (head strides scw_h, scb_h), conv states [B, H, K-1, d] in the input dtype
  const float *cwq, *cwk, *cbq, *cbk;
  void *csq, *csk;
  int cwidth;
  int64_t scw_h, scb_h;
  // optional rotary encoding of phi(q) and phi(k) (dims 0 = off) at rope_pos[b]
  int rope_dims;
  float rope_base;
  const int64_t *rope_pos;
};

template <typename T> __device__ __forceinline__ float ldf(const T *p) { return (float)*p; }

// Channel c of the token row of projection proj (0 = q, 1 = k) of (b, h) as a
// float: through the mixer's short causal conv when one is given (in the order of
// the standalone conv: bias, then taps oldest first, rounded to the input type; the
// conv state shifts by one row in place), else the input value.  xpre, when given,
// is the already loaded input value.
template <typename T, int DK>
__device__ __forceinline__ float step_input(const StepParams &p, int64_t b, int64_t h, int proj, int c,
                                            const T *xpre) {
  const int64_t bh = b * p.H + h;
  const T *xq = (const T *)p.q + b * p.sq_b + h * p.sq_h;
  const T *xk = (const T *)p.k + b * p.sk_b + h * p.sk_h;
  const T xt = xpre ? *xpre : (proj == 0 ? xq : xk)[c];
  float xv = (float)xt;
  if (p.cwidth > 0) {
    const int K = p.cwidth;
    const float *w = (proj == 0 ? p.cwq : p.cwk) + h * p.scw_h + (int64_t)c * K;
    const float *bias = proj == 0 ? p.cbq : p.cbk;
    T *cs = (T *)(proj == 0 ? p.csq : p.csk) + bh * (int64_t)(K - 1) * DK + c;
    T prev[3];
    for (int r = 0; r < K - 1; ++r) prev[r] = cs[r * DK];
    float acc = bias ? bias[h * p.scb_h + c] : 0.f;
    for (int r = 0; r < K - 1; ++r) acc = __builtin_fmaf(w[r], (float)prev[r], acc);
    acc = __builtin_fmaf(w[K - 1], xv, acc);
    for (int r = 0; r + 1 < K - 1; ++r) cs[r * DK] = prev[r + 1];
    if (K > 1) cs[(K - 2) * DK] = xt;
    xv = (float)to_elem<T>(acc);
  }
  return xv;
}

// phi(q_t) and phi(k_t) of one (b, h) into sphi[0], sphi[1], worked by the first
// 256 threads of the workgroup: the token rows are staged as floats (through the
// short causal conv when one is given), projected by W split over PARTS threads
// per output, and turned into softmax rows by waves 0 (q) and 1 (k); with
// rope_dims > 0 both rows are then turned by the rotary encoding.  Every thread
// of the workgroup must call it (it holds barriers); it ends with a barrier,
// after which sphi is complete.  Given sW (an LDS copy of W_q then W_k, complete
// for every thread) and xpre (this thread's token value), it reads no global
// memory unless the short conv or the rotary encoding is on.
template <typename T, int DK, int FH>
__device__ __forceinline__ void step_features(const StepParams &p, int64_t b, int64_t h, float (*sx)[DK],
                                              float (*su)[2 * FH], float (*sphi)[2 * FH], const T *sW = nullptr,
                                              const T *xpre = nullptr) {
  constexpr int NT = 256;
  constexpr int PARTS = NT / (2 * FH);       // threads per projection output
  constexpr int DPART = DK / PARTS;
  static_assert(NT % (2 * FH) == 0 && DK % PARTS == 0, "step mapping");
  const int tid = threadIdx.x;
  for (int i = tid; i < 2 * DK; i += NT) {
    const int proj = i / DK, c = i % DK;
    sx[proj][c] = step_input<T, DK>(p, b, h, proj, c, xpre);
  }
  __syncthreads();
  if (tid < NT) {
    const int o = tid % (2 * FH), part = tid / (2 * FH);
    const int proj = o / FH, j = o % FH;
    const T *W = sW ? sW + proj * (DK * FH) : (const T *)(proj == 0 ? p.wq : p.wk) + h * p.sw_h;
    float acc = 0.f;
#pragma unroll 8
    for (int i = part * DPART; i < (part + 1) * DPART; ++i) acc += sx[proj][i] * ldf(W + i * FH + j);
    su[part][o] = acc;
  }
  __syncthreads();
  // softmax over [u, -u]: wave 0 handles q, wave 1 handles k (FH <= 64 lanes)
  {
    const int w = tid >> 6, lane = tid & 63;
    if (w < 2) {
      float u = 0.f;
      if (lane < FH) {
#pragma unroll
        for (int part = 0; part < PARTS; ++part) u += su[part][w * FH + lane];
      }
      float m = lane < FH ? fabsf(u) : 0.f;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
      const float ep = lane < FH ? __expf(u - m) : 0.f, em = lane < FH ? __expf(-u - m) : 0.f;
      float sum = ep + em;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
      const float inv = 1.f / sum;
      if (lane < FH) {
        sphi[w][lane] = ep * inv;
        sphi[w][FH + lane] = em * inv;
      }
    }
  }
  __syncthreads();
  if (p.rope_dims > 0) {
    // rotary encoding (HedgeMamba explainer §5.2 step 3): thread (row w, pair i)
    // turns features i and i + dims/2 of phi(q) (w = 0) or phi(k) (w = 1)
    const int hr = p.rope_dims / 2;
    if (tid < 2 * hr) {
      const int w = tid / hr, i = tid % hr;
      float c, s, x1 = sphi[w][i], x2 = sphi[w][i + hr];
      rope_cs(rope_rev(i, p.rope_dims, p.rope_base), (double)p.rope_pos[b], c, s);
      rope_turn<false>(x1, x2, c, s);
      sphi[w][i] = x1;
      sphi[w][i + hr] = x2;
    }
    __syncthreads();
  }
}

// W_q then W_k of head h into LDS (sW: [2][DK*FH]) with asynchronous 16-byte
// global-to-LDS loads by the first 256 threads; piece i lands at sW + i*EP
// elements.  Complete for every thread after the next barrier.
template <typename T, int DK, int FH>
__device__ __forceinline__ void stage_w_lds(const StepParams &p, int64_t h, T *sW) {
  constexpr int EP = 16 / (int)sizeof(T), PER_MAT = DK * FH / EP, NP = 2 * PER_MAT, NIT = (NP + 255) / 256;
  // every wave loads 64 whole pieces (a wave may take the end of W_q and the start of W_k)
  static_assert(NP % 64 == 0, "whole waves of pieces");
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (tid >= 256) return;
#pragma unroll
  for (int m = 0; m < NIT; ++m) {
    const int wbase = m * 256 + w * 64;  // first piece of this wave's load
    if (wbase < NP) {
      const int piece = wbase + lane;
      const T *src = (const T *)(piece < PER_MAT ? p.wq : p.wk) + h * p.sw_h + (piece % PER_MAT) * EP;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                       (__attribute__((address_space(3))) void *)(sW + wbase * EP), 16, 0, 0);
    }
  }
}

template <typename T, int DK, int FH, int DV, bool DECAY>
__global__ __launch_bounds__(256) void step_kernel(const StepParams p) {
  constexpr int NT = 256;
  constexpr int F = 2 * FH;
  constexpr int RV = DV / 4;                 // float4 per state row
  constexpr int NS4 = F * RV;                // float4 in S
  constexpr int PER = (NS4 + NT - 1) / NT;   // float4 per thread
  constexpr int GROUPS = NT / RV;            // threads sharing one column group
  constexpr int PARTS = NT / (2 * FH);
  static_assert(NT % RV == 0, "step mapping");

  __shared__ float sx[2][DK];
  __shared__ float su[PARTS][2 * FH];
  __shared__ __align__(16) float sphi[2][F];  // [0] = phi(q), [1] = phi(k)
  __shared__ __align__(16) float sred[GROUPS][DV];
  __shared__ float sden[F / 4 > 0 ? F / 4 : 1];
  __shared__ float sa;
  __shared__ __align__(16) T sW[2 * DK * FH];  // W_q, W_k of the head

  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x;
  const int64_t b = bh / p.H, h = bh % p.H;
  constexpr int64_t BLK = (int64_t)F * DV + F;
  float *st = p.state + bh * BLK;

  // 0. W into LDS and this thread's token value (q or k channel), and the decay's
  //    inputs, before anything else: with them in hand the featurization below
  //    needs no global memory (without the short conv or the rotary encoding) and
  //    runs while the state loads are in flight
  static_assert(2 * DK <= NT, "one token value per thread");
  stage_w_lds<T, DK, FH>(p, h, sW);
  T xpre{};
  if (tid < 2 * DK) xpre = ((const T *)(tid < DK ? p.q : p.k) + b * (tid < DK ? p.sq_b : p.sk_b) +
                            h * (tid < DK ? p.sq_h : p.sk_h))[tid % DK];
  float dtv = 0.f, alog = 0.f;
  if constexpr (DECAY) {
    if (tid == 0) {
      dtv = p.dt[b * p.sdt_b + h * p.sdt_h];
      alog = p.a_log[h];
    }
  }
  __syncthreads();

  // 1. issue the state loads
  f32x4 sv[PER];
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int idx = tid + NT * m;
    if (idx < NS4) sv[m] = reinterpret_cast<const f32x4 *>(st)[idx];
  }
  f32x4 zv = zero4();
  if (tid < F / 4) zv = reinterpret_cast<const f32x4 *>(st + F * DV)[tid];

  // 2. the decay, and phi(q), phi(k) while the loads are in flight
  if (tid == 0) {
    float a = 1.f;
    if constexpr (DECAY) a = __expf(-softplus_f32(dtv) * expf(alog));
    sa = a;
  }
  step_features<T, DK, FH>(p, b, h, sx, su, sphi, sW, &xpre);
  // 3. update, read out, store.  Thread tid owns column group c4 = tid % RV and
  //    rows f = tid / RV + GROUPS * m.
  const float a = sa;
  const int c4 = tid % RV;
  const T *vp = (const T *)p.v + b * p.sv_b + h * p.sv_h + 4 * c4;
  const f32x4 v4 = f32x4{ldf(vp), ldf(vp + 1), ldf(vp + 2), ldf(vp + 3)};
  f32x4 num = zero4();
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int idx = tid + NT * m;
    if (idx < NS4) {
      const int f = idx / RV;
      const f32x4 s = a * sv[m] + sphi[1][f] * v4;
      num += sphi[0][f] * s;
      reinterpret_cast<f32x4 *>(st)[idx] = s;
    }
  }
  *reinterpret_cast<f32x4 *>(&sred[tid / RV][4 * c4]) = num;
  if (tid < F / 4) {
    const f32x4 pk = *reinterpret_cast<const f32x4 *>(&sphi[1][4 * tid]);
    const f32x4 pq = *reinterpret_cast<const f32x4 *>(&sphi[0][4 * tid]);
    const f32x4 z = a * zv + pk;
    reinterpret_cast<f32x4 *>(st + F * DV)[tid] = z;
    sden[tid] = pq[0] * z[0] + pq[1] * z[1] + pq[2] * z[2] + pq[3] * z[3];
  }
  __syncthreads();
  if (tid < DV) {
    float nsum = 0.f, den = 0.f;
#pragma unroll
    for (int gi = 0; gi < GROUPS; ++gi) nsum += sred[gi][tid];
#pragma unroll
    for (int i = 0; i < F / 4; ++i) den += sden[i];
    T *op = (T *)p.o + b * p.so_b + h * p.so_h;
    float o = nsum / den;
    if (p.gate) o = (float)to_elem<T>(o) * silu_f32(ldf((const T *)p.gate + b * p.sg_b + h * p.sg_h + tid));
    op[tid] = to_elem<T>(o);
  }
}

struct FeatParams {
  const void *x, *w;
  void *phi;
  int64_t B, H, n;
  int64_t sx_b, sx_h, sx_t, sw_h, sp_b, sp_h, sp_t;
  int rope_dims;              // rotary encoding of phi (0 = off)
  float rope_base;
  const int64_t *rope_pos0;   // position of token 0 per batch row (NULL = 0)
  // optional short causal conv on x (cwidth 0 = none): taps [d][K] (head stride
  // scw_h), bias [d] (scb_h) or NULL, rows before token 0 [B, H, K-1, d] or NULL
  int cwidth;
  const float *cw, *cb;
  const void *cprev;
  int64_t scw_h, scb_h;
};

// Hedgehog features of 16 tokens per wave (gsyq.cn HedgeMamba explainer §2.1,
// §5.3): U^T = W^T X^T on the MFMA from the token rows' operand fragments xf
// (lane (g, col) holds row col's K-slices) and W^T in LDS (rows f, stride LDW),
// then exp([u, -u] - max|u|) per token.  On return lane (g, col) holds feature
// 16t + 4g + r of token col in ph[t][r] (the +u half in tiles t < FH/16), not
// yet divided by the row sum, which is returned.
template <typename T, int DK, int FH>
__device__ __forceinline__ float feature_tiles(const typename Mma<T>::frag *xf, const T *sW, f32x4 *ph) {
  using M = Mma<T>;
  // K padded to one MFMA step when d is shorter (bf16 d = 16: W^T columns and operand slices past d are zero)
  constexpr int DKP = DK < M::KS ? M::KS : DK, NFH = FH / 16, KD = DKP / M::KS, LDW = DKP + M::PAD;
  const int lane = threadIdx.x & 63, col = lane & 15, g = lane >> 4;
  f32x4 u[NFH];
#pragma unroll
  for (int t = 0; t < NFH; ++t) {
    u[t] = zero4();
#pragma unroll
    for (int s = 0; s < KD; ++s) u[t] = M::mma(M::ld_contig(sW + (16 * t + col) * LDW + s * M::KS, g), xf[s], u[t]);
  }
  float m = 0.f;
#pragma unroll
  for (int t = 0; t < NFH; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(u[t][r]));
  m = group_max(m);
  float sum = 0.f;
#pragma unroll
  for (int t = 0; t < NFH; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float ep = __expf(u[t][r] - m), em = __expf(-u[t][r] - m);
      ph[t][r] = ep;
      ph[NFH + t][r] = em;
      sum += ep + em;
    }
  return group_sum(sum);
}

// Standalone Hedgehog featurizer: phi = softmax([x W, -x W]).  One workgroup =
// kFeatBlocks 64-token blocks of one (b, h), so that W^T is staged once per 256
// tokens; wave w featurizes token tile w of each block, the next block's x rows in
// flight meanwhile, and stores phi rows with 8/16-byte vector stores.
constexpr int kFeatBlocks = 4;
template <typename T, typename TO, int DK, int FH, bool CONV>
__global__ __launch_bounds__(256) void featurize_kernel(const FeatParams p) {
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int DKP = DK < M::KS ? M::KS : DK;  // K padded to one MFMA step (bf16 d = 16)
  constexpr int NFH = FH / 16, NFT = 2 * NFH, KD = DKP / M::KS, LDW = DKP + M::PAD;
  __shared__ __align__(16) T sW[FH * LDW];
  __shared__ double sRev[FH];
  __shared__ float sCw[CONV ? DK * 4 : 1], sCb[CONV ? DK : 1];  // conv taps [d][K] and bias of the head
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, col = lane & 15, g = lane >> 4;
  const int64_t bh = blockIdx.y, b = bh / p.H, h = bh % p.H;
  const int64_t c0 = (int64_t)blockIdx.x * 64 * kFeatBlocks + 16 * wv + col;  // this lane's token in block 0
  const T *X0 = (const T *)p.x + b * p.sx_b + h * p.sx_h;
  frag xf[KD], xn[KD];
  const int K = CONV ? p.cwidth : 0;
  const T *CP = CONV && p.cprev ? (const T *)p.cprev + bh * (int64_t)(K - 1) * DK : nullptr;
  auto load_x = [&](frag *x, int64_t c) {
    if constexpr (!CONV) {
#pragma unroll
      for (int s = 0; s < KD; ++s)
        x[s] = c < p.n && s * M::KS + (M::EPL == 8 ? 8 * g : g) < DK ? M::ld_contig(X0 + c * p.sx_t + s * M::KS, g)
                                                                     : frag{};
    } else {
    // the short causal conv in the load prologue: the lane's channels of rows c-K+1 .. c
    // (rows before token 0 from the conv state), bias then taps oldest first in float32,
    // rounded to T as the standalone conv stores it
#pragma unroll
    for (int s = 0; s < KD; ++s) {
      const int ch0 = s * M::KS + (M::EPL == 8 ? 8 * g : g);  // first channel of this lane's slice
      frag out{};
      if (c < p.n && ch0 < DK) {
        frag rows[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t t = c - (K - 1) + j;
          rows[j] = frag{};
          if (j < K) {
            if (t >= 0) rows[j] = M::ld_contig(X0 + t * p.sx_t + s * M::KS, g);
            else if (CP) rows[j] = M::ld_contig(CP + (K - 1 + t) * DK + s * M::KS, g);
          }
        }
        const float *wt = sCw + ch0 * K;
#pragma unroll
        for (int e = 0; e < M::EPL; ++e) {
          float acc = sCb[ch0 + e];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (j < K) {
              float xv;
              if constexpr (M::EPL == 8) xv = (float)rows[j][e];
              else xv = (float)rows[j];
              acc = __builtin_fmaf(wt[e * K + j], xv, acc);
            }
          }
          if constexpr (M::EPL == 8) out[e] = (T)acc;
          else out = (T)acc;
        }
      }
      x[s] = out;
    }
    }
  };
  if constexpr (CONV) {  // the head's conv taps and bias into LDS (read by every load below)
    for (int i = tid; i < DK * K; i += 256) sCw[i] = p.cw[h * p.scw_h + i];
    for (int i = tid; i < DK; i += 256) sCb[i] = p.cb ? p.cb[h * p.scb_h + i] : 0.f;
  } else {
    load_x(xf, c0);  // the first block's rows go out before W^T is staged
  }
  {
    // W^T: sW[f][d] = W[d][f], W read as 16-byte vectors, all issued before the first LDS write
    constexpr int EP = 16 / (int)sizeof(T), NV = DK * FH / EP, VPT = (NV + 255) / 256;
    typedef T tvec __attribute__((ext_vector_type(EP)));
    const T *W = (const T *)p.w + h * p.sw_h;
    tvec wv4[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int v = tid + 256 * i;
      if (v < NV) wv4[i] = *reinterpret_cast<const tvec *>(W + v * EP);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int v = tid + 256 * i;
      if (v < NV) {
        const int d = v * EP / FH, f0 = v * EP % FH;
#pragma unroll
        for (int e = 0; e < EP; ++e) sW[(f0 + e) * LDW + d] = wv4[i][e];
      }
    }
    if constexpr (DKP > DK) {
      for (int i = tid; i < FH * (DKP - DK); i += 256) sW[(i / (DKP - DK)) * LDW + DK + i % (DKP - DK)] = (T)0.f;
    }
  }
  if (tid < p.rope_dims / 2) sRev[tid] = rope_rev(tid, p.rope_dims, p.rope_base);
  __syncthreads();
  if constexpr (CONV) load_x(xf, c0);
  for (int r = 0; r < kFeatBlocks; ++r) {
    const int64_t c = c0 + 64 * r;
    if (c - 16 * wv - col >= p.n) break;  // the workgroup's last block (uniform over the workgroup)
    if (r + 1 < kFeatBlocks) load_x(xn, c + 64);
    f32x4 ph[NFT];
    const float inv = 1.f / feature_tiles<T, DK, FH>(xf, sW, ph);
    if (p.rope_dims > 0) {
      const double pos = (double)((p.rope_pos0 ? p.rope_pos0[b] : 0) + c);
      rope_apply<NFT>(ph, sRev, g, pos, p.rope_dims);
    }
    if (c < p.n) {
      TO *P = (TO *)p.phi + b * p.sp_b + h * p.sp_h + c * p.sp_t;
#pragma unroll
      for (int t = 0; t < NFT; ++t) store4(P + 16 * t + 4 * g, ph[t] * inv);
    }
#pragma unroll
    for (int s = 0; s < KD; ++s) xf[s] = xn[s];
  }
}

}  // namespace hm
