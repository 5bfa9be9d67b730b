// Per-channel decay: the scan the way the HedgeMamba explainer (gsyq.cn, §2.3
// item 3 and §5.2 step 4) wires the mixer through Mamba-1's selective scan.
// A, dt and V are copied and the V copy is set to ones, so every value channel c
// of a head has a numerator and a denominator channel that share one decay per
// state n (n runs over the F Hedgehog features):
//   Delta_t[c] = softplus(dt_t[c]),  a_t[c, n] = exp(Delta_t[c] A[c, n]),  A = -exp(A_log)
//   Sn[c, n] <- a Sn[c, n] + Delta_t[c] phik_t[n] v_t[c]
//   Sd[c, n] <- a Sd[c, n] + Delta_t[c] phik_t[n]
//   o_t[c] = sum_n phiq_t[n] Sn[c, n] / sum_n phiq_t[n] Sd[c, n]
// (Mamba's discretization, quant67 SSM lecture §3.2: the input is scaled by Delta.)
// With a decay per (c, n) the chunked matrix form of the scalar-decay kernels does
// not apply (the in-chunk weights no longer factor into phiq . phik times one
// decay), so this is an element-wise scan: one exponential per (token, channel,
// state), shared by the two copies, and the kernels are bound by that VALU and
// transcendental issue, not by HBM.
//
// State per (b, h): Sn [dv][F] then Sd [dv][F], float32, channel-major like A_log.
#pragma once

#include "hm_step.hpp"

namespace hm {

struct PcParams {
  const void *q, *k, *v, *wq, *wk;
  const float *dt;       // [B, H, n, dv] (strides sdt_*; channels contiguous)
  const float *a_log;    // [H][dv][F] (head stride sa_h; 0 = shared)
  const float *s_init;   // [B*H][2][dv][F] or NULL
  float *s_final;        // same layout, or NULL
  void *o;
  const void *gate;      // o's shape or NULL
  int64_t B, H, n;
  int64_t sq_b, sq_h, sq_t, sk_b, sk_h, sk_t, sv_b, sv_h, sv_t, so_b, so_h, so_t, sg_b, sg_h, sg_t;
  int64_t sw_h, sdt_b, sdt_h, sdt_t, sa_h;
  int rope_dims;             // rotary encoding of the features (0 = off)
  float rope_base;
  const int64_t *rope_pos0;  // position of token 0 per batch row (NULL = 0)
  // Segments: the sequence is cut into nseg segments of seg_len tokens (a multiple
  // of the 64-token chunk; nseg = 1: one segment, seg_len >= n).  With nseg > 1 the
  // workspace holds, per (b, h), slots [nseg][2][dv][F] (slot s: the start state of
  // segment s; the segment pass first leaves the end state of segment s - 1, from a
  // zero start, in slot s) and dsum [nseg - 1][dv] (the sum of Delta_t[c] over
  // segment s).
  int64_t seg_len;
  int nseg;
  float *slots;
  float *dsum;
};

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}
// Sum over aligned groups of L consecutive lanes (L = 2, 4, 8 or 16), every lane
// of a group ending with the group's sum: quad permutations, then the half-row
// and row mirrors (lane i with 7 - i, then with 15 - i).
template <int L>
__device__ __forceinline__ float group_lanes_sum(float v) {
  if constexpr (L >= 2) v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
  if constexpr (L >= 4) v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
  if constexpr (L >= 8) v += dpp_f32<0x141>(v);  // row_half_mirror
  if constexpr (L >= 16) v += dpp_f32<0x140>(v); // row_mirror
  return v;
}

// ---------------------------------------------------------------- prefill
// One workgroup per (b, h, segment, group of CPW channels), CPW x LPC threads: thread
// (channel cl, lane nb of LPC) holds the NPL = F/LPC states n0 .. n0+NPL-1 of its
// channel for both copies, in registers, for the whole sequence.  Per chunk of 64
// tokens the waves featurize q and k on the MFMA into LDS (float32 rows, each
// thread's NPL features padded by 4 so that the LPC distinct 16-byte reads of a
// wave fall in distinct banks), stage Delta and v, then scan the chunk token by
// token: NPL exponentials and FMAs per thread, the readout summed over the LPC
// lanes of a channel with DPP.  LOCAL: the segment pass (segments 0 .. nseg-2 from
// a zero state; end state and the segment's Delta sums to the workspace, no
// read-out).  Otherwise every segment from its start state (s_init or its slot).
template <typename T, int DK, int FH, int DV, int CPW, int LPC, bool LOCAL>
__global__ __launch_bounds__(CPW * LPC) void pc_fwd_kernel(const PcParams p) {
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int NT = CPW * LPC, NW = NT / 64, F = 2 * FH, NPL = F / LPC, BLK = NPL + 4, ROW = LPC * BLK;
  constexpr int C = 64, NFH = FH / 16, NFT = 2 * NFH, KD = DK / M::KS, LDW = DK + M::PAD;
  constexpr float L2E = 1.4426950408889634f;
  static_assert(NT % 64 == 0 && NPL >= 4 && NPL % 4 == 0 && LPC <= 16 && DV % CPW == 0, "pc mapping");
  __shared__ __align__(16) T sW[2][FH * LDW];   // W_q^T, W_k^T
  __shared__ __align__(16) float sPh[2][C * ROW];  // phi(q) (unnormalized), phi(k) of the chunk
  __shared__ float sD[C * CPW];                 // Delta of the chunk
  __shared__ float sVO[C * CPW];                // v of the chunk, then o
  __shared__ double sRev[FH];                   // rotary rate of each feature pair

  const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, g = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int NG = DV / CPW;
  const int nrun = LOCAL ? p.nseg - 1 : p.nseg;  // segments of this launch
  const int64_t item = blockIdx.x / NG, bh = item / nrun, b = bh / p.H, h = bh % p.H;
  const int seg = (int)(item % nrun);
  const int grp = (int)(blockIdx.x % NG);
  const int cl = tid / LPC, nb = tid % LPC, c = grp * CPW + cl, n0 = nb * NPL;
  const int64_t ts = seg * p.seg_len;                                   // first token of the segment
  const int64_t nloc = p.n - ts < p.seg_len ? p.n - ts : p.seg_len;     // its tokens
  constexpr int64_t SB = 2 * (int64_t)DV * F;                           // state block
  // where the segment starts from and where its end state goes
  const float *sbase = nullptr;
  float *fbase = nullptr;
  if (LOCAL) {
    fbase = p.slots + (bh * p.nseg + seg + 1) * SB;
  } else if (p.nseg > 1) {
    sbase = p.slots + (bh * p.nseg + seg) * SB;
    fbase = seg == p.nseg - 1 && p.s_final ? p.s_final + bh * SB : nullptr;
  } else {
    sbase = p.s_init ? p.s_init + bh * SB : nullptr;
    fbase = p.s_final ? p.s_final + bh * SB : nullptr;
  }

  // the thread's A row (times log2 e) and states; with no token W and A are not read
  float A2[NPL], hn[NPL], hd[NPL];
  if (nloc > 0) {
    const T *wq = (const T *)p.wq + h * p.sw_h, *wk = (const T *)p.wk + h * p.sw_h;
    for (int i = tid; i < DK * FH; i += NT) {
      sW[0][(i % FH) * LDW + i / FH] = wq[i];
      sW[1][(i % FH) * LDW + i / FH] = wk[i];
    }
    if (tid < p.rope_dims / 2) sRev[tid] = rope_rev(tid, p.rope_dims, p.rope_base);
    const float *al = p.a_log + h * p.sa_h + (int64_t)c * F + n0;
#pragma unroll
    for (int k = 0; k < NPL; k += 4) {
      const f32x4 a4 = *reinterpret_cast<const f32x4 *>(al + k);
#pragma unroll
      for (int e = 0; e < 4; ++e) A2[k + e] = -expf(a4[e]) * L2E;
    }
  }
  {
    const float *si = sbase ? sbase + (int64_t)c * F + n0 : nullptr;
#pragma unroll
    for (int k = 0; k < NPL; k += 4) {
      const f32x4 sn = si ? *reinterpret_cast<const f32x4 *>(si + k) : zero4();
      const f32x4 sd = si ? *reinterpret_cast<const f32x4 *>(si + DV * F + k) : zero4();
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hn[k + e] = sn[e];
        hd[k + e] = sd[e];
      }
    }
  }
  const T *Q = (const T *)p.q + b * p.sq_b + h * p.sq_h + ts * p.sq_t;
  const T *K = (const T *)p.k + b * p.sk_b + h * p.sk_h + ts * p.sk_t;
  const T *V = (const T *)p.v + b * p.sv_b + h * p.sv_h + ts * p.sv_t + grp * CPW;
  const float *DT = p.dt + b * p.sdt_b + h * p.sdt_h + ts * p.sdt_t + grp * CPW;
  T *O = (T *)p.o + b * p.so_b + h * p.so_h + ts * p.so_t + grp * CPW;
  const T *G = p.gate ? (const T *)p.gate + b * p.sg_b + h * p.sg_h + ts * p.sg_t + grp * CPW : nullptr;

  // A chunk's q, k rows, dt and v are loaded into registers one chunk ahead, during
  // the previous chunk's scan: with one workgroup per compute unit nothing else
  // would cover their latency.
  constexpr int TPW = (8 + NW - 1) / NW;  // featurize tasks per wave
  constexpr int IT = (C * CPW + NT - 1) / NT;  // staged (token, channel) items per thread
  frag xn[TPW][KD];
  float dtn[IT], vnx[IT];
  auto prefetch = [&](int64_t tc) {
    const int nvc = (int)(nloc - tc < C ? nloc - tc : C);
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int task = wv + u * NW;
      const int proj = task >> 2, tok = 16 * (task & 3) + col;
      if (LOCAL && proj == 0) continue;  // the segment pass needs no phi(q)
      const T *X = (proj == 0 ? Q + (tc + tok) * p.sq_t : K + (tc + tok) * p.sk_t);
#pragma unroll
      for (int s = 0; s < KD; ++s) xn[u][s] = task < 8 && tok < nvc ? M::ld_contig(X + s * M::KS, g) : frag{};
    }
#pragma unroll
    for (int m = 0; m < IT; ++m) {
      const int i = tid + m * NT, tt = i / CPW, cc = i % CPW;
      const bool ok = i < C * CPW && tt < nvc;
      dtn[m] = ok ? DT[(tc + tt) * p.sdt_t + cc] : 0.f;
      vnx[m] = ok ? (float)V[(tc + tt) * p.sv_t + cc] : 0.f;
    }
  };
  if (nloc > 0) prefetch(0);
  double dsum = 0.0;  // LOCAL: the segment's sum of Delta_t[c]

  for (int64_t t0 = 0; t0 < nloc; t0 += C) {
    const int nv = (int)(nloc - t0 < C ? nloc - t0 : C);
    __syncthreads();  // W staged; the previous chunk's o rows are stored
    // featurize: eight 16-token tasks (q tiles 0-3, k tiles 0-3) over the waves
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int task = wv + u * NW;
      if (task >= 8) continue;
      const int proj = task >> 2, tok = 16 * (task & 3) + col;
      if (LOCAL && proj == 0) continue;
      const frag *xf = xn[u];
      f32x4 ph[NFT];
      const float sum = feature_tiles<T, DK, FH>(xf, sW[proj], ph);
      const float inv = proj == 1 ? __builtin_amdgcn_rcpf(sum) : 1.f;  // phi(q)'s scale cancels in o
      if (p.rope_dims > 0) {
        const double pos = (double)((p.rope_pos0 ? p.rope_pos0[b] : 0) + ts + t0 + tok);
        rope_apply<NFT>(ph, sRev, g, pos, p.rope_dims);
      }
      float *row = sPh[proj] + tok * ROW;
#pragma unroll
      for (int t = 0; t < NFT; ++t) {
        const int f = 16 * t + 4 * g;
        *reinterpret_cast<f32x4 *>(row + (f / NPL) * BLK + f % NPL) = ph[t] * inv;
      }
    }
#pragma unroll
    for (int m = 0; m < IT; ++m) {
      const int i = tid + m * NT, tt = i / CPW;
      if (i < C * CPW) {
        sD[i] = tt < nv ? softplus_f32(dtn[m]) : 0.f;
        sVO[i] = vnx[m];
      }
    }
    __syncthreads();
    if (t0 + C < nloc) prefetch(t0 + C);
    for (int t = 0; t < nv; ++t) {
      const float dl = sD[t * CPW + cl], dlv = dl * sVO[t * CPW + cl];
      if constexpr (LOCAL) dsum += (double)dl;
      const float *pk = sPh[1] + t * ROW + nb * BLK, *pq = sPh[0] + t * ROW + nb * BLK;
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int k = 0; k < NPL; k += 4) {
        const f32x4 k4 = *reinterpret_cast<const f32x4 *>(pk + k);
        const f32x4 q4 = *reinterpret_cast<const f32x4 *>(pq + k);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = __builtin_amdgcn_exp2f(dl * A2[k + e]);
          // s <- k dl v + a s with the decayed state as the addend: the product
          // takes the state's register and v_fmac's tied addend is that register.
          // Written as fma(a, s, k dl v) the tie fell on k dl v, and the
          // loop-carried state cost two register moves per element (measured:
          // 12.9 VALU instructions per (token, channel, state), 8 of arithmetic)
          hn[k + e] = __builtin_fmaf(k4[e], dlv, a * hn[k + e]);
          hd[k + e] = __builtin_fmaf(k4[e], dl, a * hd[k + e]);
          if constexpr (!LOCAL) {
            num = __builtin_fmaf(q4[e], hn[k + e], num);
            den = __builtin_fmaf(q4[e], hd[k + e], den);
          }
        }
      }
      if constexpr (!LOCAL) {
        num = group_lanes_sum<LPC>(num);
        den = group_lanes_sum<LPC>(den);
        if (nb == 0) sVO[t * CPW + cl] = num / den;  // v[t][cl] was read by every lane of the channel above
      }
    }
    __syncthreads();
    for (int i = tid; !LOCAL && i < nv * CPW; i += NT) {
      const int tt = i / CPW, cc = i % CPW;
      float o = sVO[i];
      if (G) o = (float)to_elem<T>(o) * silu_f32((float)G[(t0 + tt) * p.sg_t + cc]);
      O[(t0 + tt) * p.so_t + cc] = to_elem<T>(o);
    }
  }
  if constexpr (LOCAL) {
    if (nb == 0) p.dsum[(bh * (p.nseg - 1) + seg) * DV + c] = (float)dsum;
  }
  if (fbase) {
    float *sf = fbase + (int64_t)c * F + n0;
#pragma unroll
    for (int k = 0; k < NPL; k += 4) {
      *reinterpret_cast<f32x4 *>(sf + k) = f32x4{hn[k], hn[k + 1], hn[k + 2], hn[k + 3]};
      *reinterpret_cast<f32x4 *>(sf + DV * F + k) = f32x4{hd[k], hd[k + 1], hd[k + 2], hd[k + 3]};
    }
  }
}

// Start states of the segments from the segment pass: slot 0 gets s_init (or zero),
// then for s = 0 .. nseg-2
//   slot[s+1] <- D_s * slot[s] + slot[s+1],   D_s[c][n] = 2^(A2[c][n] dsum_s[c]),
// with A2 = -exp(A_log) log2(e) as in the scan: the product of the segment's per-token
// decays a_t[c][n] = 2^(A2[c][n] Delta_t[c]) (the affine composition of the
// associative scan, quant67 SSM lecture §4.2, element by element).  One thread per
// (b, h, state element); the chain over the segments is short.
template <int DV, int F>
__global__ __launch_bounds__(256) void pc_combine_kernel(const PcParams p) {
  constexpr int64_t SB = 2 * (int64_t)DV * F;
  constexpr float L2E = 1.4426950408889634f;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x, bh = idx / SB, e = idx % SB;
  if (bh >= p.B * p.H) return;
  const int64_t h = bh % p.H, cn = e % (DV * F), c = cn / F;
  const float A2 = -expf(p.a_log[h * p.sa_h + cn]) * L2E;
  float *slot = p.slots + bh * p.nseg * SB + e;
  float s = p.s_init ? p.s_init[bh * SB + e] : 0.f;
  slot[0] = s;
  for (int sg = 0; sg + 1 < p.nseg; ++sg) {
    const float d = __builtin_amdgcn_exp2f(A2 * p.dsum[(bh * (p.nseg - 1) + sg) * DV + c]);
    s = __builtin_fmaf(d, s, slot[(sg + 1) * SB]);
    slot[(sg + 1) * SB] = s;
  }
}

// ---------------------------------------------------------------- decode step
struct PcStepParams {
  StepParams s;          // q, k, v, w, o, gate, conv, rotary fields and strides (s.dt, s.a_log unused)
  const float *dt;       // [B, H, dv] (strides sdt_b, sdt_h)
  const float *a_log;    // [H][dv][F] (head stride sa_h)
  float *state;          // [B*H][2][dv][F], in place
  int64_t sdt_b, sdt_h, sa_h;
};

// phi(q_t) and phi(k_t) of (b, h) into sphi[0] and sphi[1], worked by all 256
// threads: the token rows are staged as floats (through the short causal conv when
// one is given), then thread (part, group) multiplies its DPART rows of W, read as
// 16-byte pieces of EPL consecutive outputs, into partial sums; the parts are added
// in LDS and waves 0 (q) and 1 (k) turn the projections into softmax rows (and,
// with rope_dims > 0, the rotary encoding turns both).  Ends with a barrier.
template <typename T, int DK, int FH>
struct PcFeat {
  static constexpr int NT = 256, EPL = 16 / (int)sizeof(T), G = 2 * FH / EPL;  // G output groups
  static constexpr int P = NT / G < DK ? NT / G : DK, DPART = DK / P;          // P parts of DK
  static_assert(FH % EPL == 0 && DK % P == 0 && FH <= 64 && G * P <= NT, "feature mapping");
};
template <typename T, int DK, int FH>
__device__ __forceinline__ void pc_step_features(const StepParams &p, int64_t b, int64_t h, float (*sx)[DK],
                                                 float *su, float (*sphi)[2 * FH]) {
  using PF = PcFeat<T, DK, FH>;
  constexpr int NT = PF::NT, EPL = PF::EPL, G = PF::G, P = PF::P, DPART = PF::DPART;
  const int tid = threadIdx.x;
  for (int i = tid; i < 2 * DK; i += NT) sx[i / DK][i % DK] = step_input<T, DK>(p, b, h, i / DK, i % DK, nullptr);
  __syncthreads();
  if (tid < G * P) {
    const int grp = tid % G, part = tid / G;
    const int proj = grp * EPL / FH, j0 = grp * EPL % FH;
    const T *W = (const T *)(proj == 0 ? p.wq : p.wk) + h * p.sw_h + j0;
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    // W rows in batches of WB pieces
    constexpr int WB = DPART < 4 ? DPART : 4;
#pragma unroll
    for (int i0 = 0; i0 < DPART; i0 += WB) {
      f32x4 wr[WB];
#pragma unroll
      for (int i = 0; i < WB; ++i)
        wr[i] = *reinterpret_cast<const f32x4 *>(W + (int64_t)(part * DPART + i0 + i) * FH);
#pragma unroll
      for (int i = 0; i < WB; ++i) {
        const T *wv = reinterpret_cast<const T *>(&wr[i]);
        const float x = sx[proj][part * DPART + i0 + i];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = __builtin_fmaf(x, (float)wv[e], acc[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < EPL; e += 4)
      *reinterpret_cast<f32x4 *>(&su[part * 2 * FH + proj * FH + j0 + e]) =
          f32x4{acc[e], acc[e + 1], acc[e + 2], acc[e + 3]};
  }
  __syncthreads();
  {
    const int w = tid >> 6, lane = tid & 63;
    if (w < 2) {
      float u = 0.f;
      if (lane < FH) {
#pragma unroll 8
        for (int part = 0; part < P; ++part) u += su[part * 2 * FH + w * FH + lane];
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

// One workgroup of 256 threads per (b, h, group of CPS channels): every thread
// issues the loads of its PER (channel, 4 states) items of both copies (non-temporal:
// the state streams through once per step) and of A (temporal: every batch row of the
// head reads it) first, featurizes while they are in flight (each group recomputes phi(q), phi(k)
// of its (b, h), reading W as 16-byte pieces), then updates, reads out (sum over
// the QPC lanes of a channel) and stores in place.  Small workgroups let four share
// a CU, so one group's featurization overlaps another's state traffic.  Bound by
// the state's HBM traffic.
template <typename T, int DK, int FH, int DV, int CPS>
// At least five waves per SIMD (80 VGPRs, six waves, at bf16 (128, 64, 128)): with the
// state streamed non-temporally the extra workgroups per CU keep more state loads in flight (0.1952 -> 0.1891 ms at B=256,
// H=16; it measured slower with cached state accesses).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5))) void pc_step_kernel(const PcStepParams pp) {
  constexpr int NT = 256, F = 2 * FH, QPC = F / 4;  // float4 per channel row
  constexpr int ITEMS = CPS * QPC, PER = (ITEMS + NT - 1) / NT, NG = DV / CPS;
  constexpr float L2E = 1.4426950408889634f;
  static_assert(QPC == 32 || QPC == 16 || QPC == 8, "lanes per channel");
  static_assert(DV % CPS == 0 && 64 % QPC == 0, "channel groups");
  const StepParams &p = pp.s;
  __shared__ float sx[2][DK];
  __shared__ __align__(16) float su[PcFeat<T, DK, FH>::P * F];
  __shared__ __align__(16) float sphi[2][F];
  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x / NG, b = bh / p.H, h = bh % p.H;
  const int c0 = (int)(blockIdx.x % NG) * CPS;
  float *Sn = pp.state + bh * (2 * (int64_t)DV * F) + (int64_t)c0 * F;
  float *Sd = Sn + DV * F;
  const float *AL = pp.a_log + h * pp.sa_h + (int64_t)c0 * F;
  f32x4 vn[PER], vd[PER], va[PER];
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int idx = tid + NT * m;
    if (idx < ITEMS) {
      vn[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(Sn) + idx);
      vd[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(Sd) + idx);
      va[m] = reinterpret_cast<const f32x4 *>(AL)[idx];
    }
  }
  pc_step_features<T, DK, FH>(p, b, h, sx, su, sphi);
  const T *vp = (const T *)p.v + b * p.sv_b + h * p.sv_h + c0;
  const float *dtp = pp.dt + b * pp.sdt_b + h * pp.sdt_h + c0;
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int idx = tid + NT * m;
    const int c = idx / QPC, n = 4 * (idx % QPC);
    float num = 0.f, den = 0.f;
    if (idx < ITEMS) {
      const float dl = softplus_f32(dtp[c]), dlv = dl * (float)vp[c];
      const f32x4 k4 = *reinterpret_cast<const f32x4 *>(&sphi[1][n]);
      const f32x4 q4 = *reinterpret_cast<const f32x4 *>(&sphi[0][n]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = __builtin_amdgcn_exp2f(-dl * __builtin_amdgcn_exp2f(va[m][e] * L2E) * L2E);
        vn[m][e] = __builtin_fmaf(a, vn[m][e], k4[e] * dlv);
        vd[m][e] = __builtin_fmaf(a, vd[m][e], k4[e] * dl);
        num = __builtin_fmaf(q4[e], vn[m][e], num);
        den = __builtin_fmaf(q4[e], vd[m][e], den);
      }
      __builtin_nontemporal_store(vn[m], reinterpret_cast<f32x4 *>(Sn) + idx);
      __builtin_nontemporal_store(vd[m], reinterpret_cast<f32x4 *>(Sd) + idx);
    }
    // the QPC lanes of channel c are consecutive and aligned
    if constexpr (QPC == 32) {
      num = xor16_pair(group_lanes_sum<16>(num), false);
      den = xor16_pair(group_lanes_sum<16>(den), false);
    } else {
      num = group_lanes_sum<QPC>(num);
      den = group_lanes_sum<QPC>(den);
    }
    if (idx < ITEMS && idx % QPC == 0) {
      float o = num / den;
      const int64_t cg = c0 + c;
      T *op = (T *)p.o + b * p.so_b + h * p.so_h;
      if (p.gate) o = (float)to_elem<T>(o) * silu_f32((float)((const T *)p.gate)[b * p.sg_b + h * p.sg_h + cg]);
      op[cg] = to_elem<T>(o);
    }
  }
}

}  // namespace hm
