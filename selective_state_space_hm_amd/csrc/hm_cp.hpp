// Chunk-parallel prefill: the chunk-wise form of causal, normalized Hedgehog
// linear attention (cnblogs linear-attention tutorial, part 5; the SSD chunking of
// the quant67 SSM lecture, §6) run as three passes, for any chunk length that is a
// multiple of 64 tokens and any supported (d, f, dv):
//   1. cp_local_kernel, one workgroup per (b, h, chunk c): the chunk's local end
//      state dS_c = sum_s e^{Lam_c - L_s} phiK_s v_s^T (F x dv), dz_c likewise, and
//      its summed log-decay Lam_c, with L the inclusive log-decay prefix from the
//      chunk's start;
//   2. cp_scan_kernel, per (b, h) and state element: the start state of every chunk,
//      S(c+1) = e^{Lam_c} S(c) + dS_c from S(0) = s_init (the composition of affine
//      maps, quant67 SSM lecture §4.2), and s_final;
//   3. cp_out_kernel, one workgroup per (b, h, chunk, 64-query block): for query t,
//        O_t = e^{L_t} phiQ_t S(c) + sum_{s <= t in the chunk} e^{L_t - L_s} (phiQ_t . phiK_s) v_s,
//        den_t = e^{L_t} phiQ_t . z(c) + sum_{s <= t} e^{L_t - L_s} (phiQ_t . phiK_s),
//      o_t = O_t / den_t (HedgeMamba explainer §2.3: numerator over denominator).
// phi = softmax([x W, -x W]) (HedgeMamba explainer §2.1, §5.3); log a_t =
// -softplus(dt_t) exp(A_log[h]) (quant67 §3.2), and a_t = 1 without dt.
// Every product (projections, scores, the masked and decayed score tiles times V,
// the read-out of the start state, the local state) is a 16x16 MFMA tile, its
// operands read from LDS rows or kept in registers in the same K order; for bf16
// inputs the MFMA operands (phi, the weighted scores, the start state's read-out
// copy) are rounded to bf16 and accumulated in float32.  The carried states are
// float32 in the workspace.
#pragma once

#include "hm_device.hpp"

namespace hm {

struct CpParams {
  const void *q, *k, *v, *wq, *wk;
  const float *dt, *a_log;  // both NULL: a_t = 1
  const float *s_init;      // [B*H][F*dv + F] or NULL
  float *s_final;           // same layout, or NULL (may alias s_init)
  void *o;
  float *ws_state;          // [B*H][nc][dv*F + F]: local states, then start states, S^T [dv][F] then z [F]
  float *ws_lam;            // [B*H][nc]: summed log-decay of each chunk
  int64_t B, H, n, nc;
  int d, chunk;
  int64_t sq_b, sq_h, sq_t, sk_b, sk_h, sk_t, sv_b, sv_h, sv_t, so_b, so_h, so_t;
  int64_t sw_h, sdt_b, sdt_h, sdt_t;
};

constexpr int CP_DKMAX = 128;  // largest head dim (LDS rows of W^T are sized for it)
constexpr int CP_BLK = 64;     // tokens per block: four 16-token tiles, one per wave
constexpr int CP_CHMAX = 256;  // longest chunk

template <typename T> struct CpLds {
  static constexpr int PAD = Mma<T>::PAD;
  static constexpr int LDW = CP_DKMAX + PAD;  // W^T rows
  static constexpr int LDB = CP_BLK + PAD;    // rows over a block's tokens
};

// The dt values of tokens t0 .. t0+cnt-1 of one (b, h) for one wave (lane + 64 i),
// requested together; then their inclusive log-decay prefix from t0 on, into
// sL[0 .. cnt), in float64 (differences of large prefix sums lose ~|L| 2^-24 in
// float32); tokens at or past n add 0.
struct CpDt {
  float v[CP_CHMAX / 64];
};
__device__ __forceinline__ void cp_load_dt(const CpParams &p, int64_t b, int64_t h, int64_t t0, int cnt, CpDt &r,
                                           int lane) {
  const bool decay = p.dt != nullptr;
  const float *DT = decay ? p.dt + b * p.sdt_b + h * p.sdt_h : nullptr;
#pragma unroll
  for (int i = 0; i < CP_CHMAX / 64; ++i) {
    const int64_t t = t0 + 64 * i + lane;
    r.v[i] = decay && 64 * i + lane < cnt && t < p.n ? DT[t * p.sdt_t] : 0.f;
  }
}
__device__ __forceinline__ void cp_decay_scan(const CpParams &p, int64_t h, int64_t t0, int cnt, const CpDt &r,
                                              double *sL, int lane) {
  const bool decay = p.dt != nullptr;
  const float expA = decay ? expf(p.a_log[h]) : 0.f;
  double carry = 0.0;
#pragma unroll
  for (int i = 0; i < CP_CHMAX / 64; ++i) {
    if (64 * i < cnt) {
      const int64_t t = t0 + 64 * i + lane;
      const bool valid = decay && 64 * i + lane < cnt && t < p.n;
      const double x = valid ? (double)(-softplus_f32(r.v[i]) * expA) : 0.0;
      const double L = wave_inclusive_scan(x) + carry;
      if (64 * i + lane < cnt) sL[64 * i + lane] = L;
      carry = lane63(L);
    }
  }
}

// W (W is [d][FH] row-major, head stride sw_h) as 16-byte pieces, one per thread and
// NI rounds (consecutive threads read consecutive pieces of a row) ...
template <typename T, int FH> struct CpW {
  static constexpr int EPL = 16 / (int)sizeof(T), PR = FH / EPL, NI = (CP_DKMAX * PR + 255) / 256;
  f32x4 raw[NI];
};
template <typename T, int FH>
__device__ __forceinline__ void cp_load_w(const T *W, int d, CpW<T, FH> &r) {
  using WW = CpW<T, FH>;
#pragma unroll
  for (int m = 0; m < WW::NI; ++m) {
    const int i = threadIdx.x + 256 * m;
    if (i < d * WW::PR)
      r.raw[m] = *reinterpret_cast<const f32x4 *>(W + (int64_t)(i / WW::PR) * FH + (i % WW::PR) * WW::EPL);
  }
}
// ... into sW as W^T (rows of LDW elements), columns d .. KS-1 zero when d is below
// one MFMA K-step.
template <typename T, int FH>
__device__ __forceinline__ void cp_write_wt(const CpW<T, FH> &r, int d, T *sW) {
  using WW = CpW<T, FH>;
  using L = CpLds<T>;
#pragma unroll
  for (int m = 0; m < WW::NI; ++m) {
    const int i = threadIdx.x + 256 * m;
    if (i < d * WW::PR) {
      const int dd = i / WW::PR, j0 = (i % WW::PR) * WW::EPL;
      const T *e = reinterpret_cast<const T *>(&r.raw[m]);
#pragma unroll
      for (int x = 0; x < WW::EPL; ++x) sW[(j0 + x) * L::LDW + dd] = e[x];
    }
  }
  const int dpad = d < Mma<T>::KS ? Mma<T>::KS : d;
  for (int i = threadIdx.x; i < FH * (dpad - d); i += 256) sW[(i / (dpad - d)) * L::LDW + d + i % (dpad - d)] = (T)0.f;
}

// The token row of token tile `wv` of the block at token tb (token tb + 16 wv + col
// for lane (col, g)) as the MFMA B operands of the projection, every K-step
// requested at once; zeros at or past n and past d.
template <typename T> struct CpX {
  typename Mma<T>::frag x[CP_DKMAX / Mma<T>::KS];
  bool ok;
};
template <typename T>
__device__ __forceinline__ void cp_load_x(const T *X, int64_t sx_t, int64_t tb, int64_t n, int d, CpX<T> &r, int wv,
                                          int lane) {
  using M = Mma<T>;
  const int col = lane & 15, g = lane >> 4;
  const int64_t t = tb + 16 * wv + col;
  r.ok = t < n;
  const T *row = X + (r.ok ? t : 0) * sx_t;
#pragma unroll
  for (int i = 0; i < CP_DKMAX / M::KS; ++i) {
    const int k0 = i * M::KS;
    r.x[i] = r.ok && k0 + (M::EPL == 8 ? 8 * g : g) < d ? M::ld_contig(row + k0, g) : typename M::frag{};
  }
}

// Features of the loaded token tile: lane (col, g) gets ph[t][r] = phi at feature
// 16t + 4g + r of the u half (t < FH/16) or of the -u half (t >= FH/16), normalized
// (softmax over both halves), or 0 for tokens at or past n.  The projection U^T =
// W^T X^T runs on the MFMA.
template <typename T, int FH>
__device__ __forceinline__ void cp_features(const CpX<T> &xr, int d, const T *sW, f32x4 *ph, int lane) {
  using M = Mma<T>;
  using L = CpLds<T>;
  constexpr int NFH = FH / 16;
  constexpr float L2E = 1.4426950408889634f;
  const int col = lane & 15, g = lane >> 4;
  f32x4 u[NFH];
#pragma unroll
  for (int ft = 0; ft < NFH; ++ft) u[ft] = zero4();
#pragma unroll
  for (int i = 0; i < CP_DKMAX / M::KS; ++i) {
    const int k0 = i * M::KS;
    if (k0 < d) {
#pragma unroll
      for (int ft = 0; ft < NFH; ++ft)
        u[ft] = M::mma(M::ld_contig(sW + (16 * ft + col) * L::LDW + k0, g), xr.x[i], u[ft]);
    }
  }
  float m = 0.f;
#pragma unroll
  for (int ft = 0; ft < NFH; ++ft)
#pragma unroll
    for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(u[ft][r]));
  const float ml = group_max(m) * L2E;
  float sum = 0.f;
#pragma unroll
  for (int ft = 0; ft < NFH; ++ft)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float ep = __builtin_amdgcn_exp2f(__builtin_fmaf(u[ft][r], L2E, -ml));
      const float em = __builtin_amdgcn_exp2f(__builtin_fmaf(-u[ft][r], L2E, -ml));
      ph[ft][r] = ep;
      ph[NFH + ft][r] = em;
      sum += ep + em;
    }
  const float inv = xr.ok ? 1.f / group_sum(sum) : 0.f;
#pragma unroll
  for (int ft = 0; ft < 2 * NFH; ++ft) ph[ft] *= inv;
}

// v rows [tb, tb+64) of one (b, h) in 16-byte pieces, one per thread and NI rounds: a
// wave's lanes take the 64 tokens of one piece (so the transposed LDS writes of a
// wave fill one row); zeros past n.
template <typename T, int DV> struct CpV {
  static constexpr int EPL = 16 / (int)sizeof(T), PR = DV / EPL, NI = CP_BLK * PR / 256 > 0 ? CP_BLK * PR / 256 : 1;
  f32x4 raw[NI];
};
template <typename T, int DV>
__device__ __forceinline__ void cp_load_v(const T *V, int64_t sv_t, int64_t tb, int64_t n, CpV<T, DV> &r) {
  using VV = CpV<T, DV>;
#pragma unroll
  for (int m = 0; m < VV::NI; ++m) {
    const int i = threadIdx.x + 256 * m, tt = i % CP_BLK, c0 = (i / CP_BLK) * VV::EPL;
    r.raw[m] = i < CP_BLK * VV::PR && tb + tt < n ? *reinterpret_cast<const f32x4 *>(V + (tb + tt) * sv_t + c0)
                                                  : zero4();
  }
}
// ... into sVt[c][t] (transposed, LDB elements per row), the keys in tile order
// (TILE) or in order.
template <typename T, int DV, bool TILE>
__device__ __forceinline__ void cp_write_vt(const CpV<T, DV> &r, T *sVt) {
  using VV = CpV<T, DV>;
  using L = CpLds<T>;
#pragma unroll
  for (int m = 0; m < VV::NI; ++m) {
    const int i = threadIdx.x + 256 * m, tt = i % CP_BLK, c0 = (i / CP_BLK) * VV::EPL;
    const int tp = TILE ? Mma<T>::tpos(tt) : tt;
    if (i < CP_BLK * VV::PR) {
      const T *e = reinterpret_cast<const T *>(&r.raw[m]);
#pragma unroll
      for (int x = 0; x < VV::EPL; ++x) sVt[(c0 + x) * L::LDB + tp] = e[x];
    }
  }
}

// Pass 1: one workgroup (4 waves) per (b, h, chunk).
template <typename T, int FH, int DV>
__global__ __launch_bounds__(256) void cp_local_kernel(const CpParams p) {
  using M = Mma<T>;
  using L = CpLds<T>;
  constexpr int F = 2 * FH, NFT = F / 16, NCT = DV / 16, NTL = NFT * NCT, TPW = (NTL + 3) / 4;
  __shared__ __align__(16) T sW[FH * L::LDW];
  __shared__ __align__(16) T sKt[F * L::LDB];
  __shared__ __align__(16) T sVt[DV * L::LDB];
  __shared__ double sL[CP_CHMAX];
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, col = lane & 15, g = lane >> 4;
  const int64_t bh = blockIdx.x / p.nc, c = blockIdx.x % p.nc, b = bh / p.H, h = bh % p.H;
  const int64_t t0 = c * p.chunk;
  const int cnt = (int)(p.n - t0 < p.chunk ? p.n - t0 : p.chunk);
  const T *K = (const T *)p.k + b * p.sk_b + h * p.sk_h;
  const T *V = (const T *)p.v + b * p.sv_b + h * p.sv_h;
  // every load of the setup is requested before the first is used: dt (wave 0), W_k,
  // the first block's k rows and v pieces
  CpDt dtr;
  if (wv == 0) cp_load_dt(p, b, h, t0, cnt, dtr, lane);
  CpW<T, FH> wk;
  cp_load_w<T, FH>((const T *)p.wk + h * p.sw_h, p.d, wk);
  CpX<T> xk;
  CpV<T, DV> vr;
  cp_load_x<T>(K, p.sk_t, t0, p.n, p.d, xk, wv, lane);
  cp_load_v<T, DV>(V, p.sv_t, t0, p.n, vr);
  if (wv == 0) cp_decay_scan(p, h, t0, cnt, dtr, sL, lane);
  cp_write_wt<T, FH>(wk, p.d, sW);
  __syncthreads();
  const double lam = sL[cnt - 1];
  f32x4 acc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) acc[i] = zero4();
  float zsum = 0.f;  // thread f < F: dz[f]
  for (int kb = 0; kb * CP_BLK < cnt; ++kb) {
    const int64_t tb = t0 + kb * CP_BLK;
    {
      f32x4 ph[2 * (FH / 16)];
      cp_features<T, FH>(xk, p.d, sW, ph, lane);
      const int lt = kb * CP_BLK + 16 * wv + col;  // token within the chunk
      const float w = lt < cnt ? __expf((float)(lam - sL[lt])) : 0.f;
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
        for (int r = 0; r < 4; ++r) sKt[(16 * ft + 4 * g + r) * L::LDB + 16 * wv + col] = (T)(ph[ft][r] * w);
    }
    cp_write_vt<T, DV, false>(vr, sVt);
    // the next block's rows are in flight during this block's products
    if ((kb + 1) * CP_BLK < cnt) {
      cp_load_x<T>(K, p.sk_t, tb + CP_BLK, p.n, p.d, xk, wv, lane);
      cp_load_v<T, DV>(V, p.sv_t, tb + CP_BLK, p.n, vr);
    }
    __syncthreads();
    // dS^T[c][f] += sum_t Vt[c][t] Kt[f][t]: tile i of this wave is (value tile, feature tile)
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tile = 4 * i + wv;
      if (tile < NTL) {
        const int ft = tile % NFT, ct = tile / NFT;
#pragma unroll
        for (int k0 = 0; k0 < CP_BLK; k0 += M::KS)
          acc[i] = M::mma(M::ld_contig(sVt + (16 * ct + col) * L::LDB + k0, g),
                          M::ld_contig(sKt + (16 * ft + col) * L::LDB + k0, g), acc[i]);
      }
    }
    if (tid < F) {
      constexpr int EPL = 16 / (int)sizeof(T);
#pragma unroll
      for (int t = 0; t < CP_BLK; t += EPL) {
        const f32x4 raw = *reinterpret_cast<const f32x4 *>(&sKt[tid * L::LDB + t]);
        const T *e = reinterpret_cast<const T *>(&raw);
#pragma unroll
        for (int x = 0; x < EPL; ++x) zsum += (float)e[x];
      }
    }
    __syncthreads();
  }
  const int64_t BLK = (int64_t)F * DV + F;
  float *st = p.ws_state + (bh * p.nc + c) * BLK;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int tile = 4 * i + wv;
    if (tile < NTL) {
      const int ft = tile % NFT, ct = tile / NFT;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        __builtin_nontemporal_store(acc[i][r], st + (int64_t)(16 * ct + 4 * g + r) * F + 16 * ft + col);
    }
  }
  if (tid < F) st[(int64_t)F * DV + tid] = zsum;
  if (tid == 0) p.ws_lam[bh * p.nc + c] = (float)lam;
}

// Pass 2: thread e of (b, h) walks the chunks, replacing each local state by the
// chunk's start state; s_init is read before s_final is written (same element,
// same thread), so the two may alias.
// The workspace holds S^T: its element e = c*F + f is S[f][c], at f*dv + c in the
// state layout of s_init and s_final.
static __global__ __launch_bounds__(256) void cp_scan_kernel(const CpParams p, int64_t BLK, int F, int dv) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x, bh = blockIdx.y;
  if (e >= BLK) return;
  const int64_t es = e < (int64_t)F * dv ? (e % F) * dv + e / F : e;  // the same element in the state layout
  float s = p.s_init ? p.s_init[bh * BLK + es] : 0.f;
  float *st = p.ws_state + bh * p.nc * BLK + e;
  const float *lam = p.ws_lam + bh * p.nc;
  // the local states of UNR chunks are requested together, so only the carry is serial; the
  // states stream through once (non-temporal: no cache level holds B*H*chunks of them)
  constexpr int UNR = 16;
  for (int64_t c0 = 0; c0 < p.nc; c0 += UNR) {
    float loc[UNR], dec[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      loc[u] = c0 + u < p.nc ? __builtin_nontemporal_load(st + (c0 + u) * BLK) : 0.f;
      dec[u] = c0 + u < p.nc ? lam[c0 + u] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      if (c0 + u < p.nc) {
        __builtin_nontemporal_store(s, st + (c0 + u) * BLK);
        s = __builtin_fmaf(__expf(dec[u]), s, loc[u]);
      }
    }
  }
  if (p.s_final) p.s_final[bh * BLK + es] = s;
}

// Four consecutive values of an accumulator column as T, at p (8 or 16 bytes).
__device__ __forceinline__ void cp_store4(bf16 *p, f32x4 v) {
  *reinterpret_cast<bf16x4 *>(p) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}
__device__ __forceinline__ void cp_store4(float *p, f32x4 v) { *reinterpret_cast<f32x4 *>(p) = v; }

// Pass 3: one workgroup (4 waves) per (b, h, chunk, 64-query block); wave w owns
// query tile w (16 tokens, one per lane column).  The products run transposed, with
// the queries as MFMA columns, so phi(q) and the weighted scores stay in registers as
// B operands (tile order) and each lane ends with its token's outputs, numerator
// and denominator:
//   O^T = e^{L} S^T phiQ^T + V^T Pt,   Pt[s][t] = e^{L_t - L_s} [s <= t] phiK_s . phiQ_t,
//   den_t = e^{L_t} phiQ_t . z + sum_s Pt[s][t].
template <typename T, int FH, int DV>
__global__ __launch_bounds__(256) void cp_out_kernel(const CpParams p) {
  using M = Mma<T>;
  using frag = typename M::frag;
  using L = CpLds<T>;
  constexpr int F = 2 * FH, NFT = F / 16, NCT = DV / 16, LDF = F + L::PAD;
  constexpr int KF = M::steps(NFT), KB = M::steps(4);  // K-steps over the features, over a block's keys
  // LDS: W_q^T, W_k^T; the start state's read-out copy S^T (dv rows of F, features in
  // tile order) shares space with one key block's phi(k) rows and v^T, used after it
  constexpr int KV = CP_BLK * LDF + DV * L::LDB, ST = DV * LDF;
  constexpr int NS = (DV * F / 4 + 255) / 256;  // 16-byte pieces of S^T per thread
  __shared__ __align__(16) T sWq[FH * L::LDW];
  __shared__ __align__(16) T sWk[FH * L::LDW];
  __shared__ __align__(16) T sU[KV > ST ? KV : ST];
  __shared__ __align__(16) float sZ[F];
  __shared__ double sL[CP_CHMAX];
  T *sSt = sU, *sK = sU, *sVt = sU + CP_BLK * LDF;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, col = lane & 15, g = lane >> 4;
  // workgroup -> (chunk, query block): consecutive workgroups go to different XCDs (bid % 8), so the nqb
  // query blocks of chunk ci = 8m + x take workgroups 8 (m nqb + qb) + x, all on XCD x, where they share
  // the chunk's start state, k and v through that XCD's L2
  const int nqb = p.chunk / CP_BLK;
  const int64_t x8 = blockIdx.x % 8, r8 = blockIdx.x / 8, qb = r8 % nqb, ci = (r8 / nqb) * 8 + x8;
  if (ci >= p.B * p.H * p.nc) return;  // grid padding (uniform)
  const int64_t c = ci % p.nc, bh = ci / p.nc;
  const int64_t b = bh / p.H, h = bh % p.H, t0 = c * p.chunk, tq = t0 + qb * CP_BLK;
  if (tq >= p.n) return;  // the whole block is past the sequence's end (uniform)
  const int cnt = (int)((qb + 1) * CP_BLK);  // chunk tokens up to this block's end
  const int64_t BLK = (int64_t)F * DV + F;
  const float *st = p.ws_state + (bh * p.nc + c) * BLK;  // start state: S^T [DV][F], then z [F]
  // every load of the setup is requested before the first is used: dt (wave 0), the
  // query rows, W_q and W_k, the start state
  CpDt dtr;
  if (wv == 0) cp_load_dt(p, b, h, t0, cnt, dtr, lane);
  CpX<T> xq;
  cp_load_x<T>((const T *)p.q + b * p.sq_b + h * p.sq_h, p.sq_t, tq, p.n, p.d, xq, wv, lane);
  CpW<T, FH> wq, wk;
  cp_load_w<T, FH>((const T *)p.wq + h * p.sw_h, p.d, wq);
  cp_load_w<T, FH>((const T *)p.wk + h * p.sw_h, p.d, wk);
  f32x4 sr[NS];
#pragma unroll
  for (int m = 0; m < NS; ++m) {
    const int i = tid + 256 * m;
    if (i < DV * F / 4) sr[m] = *reinterpret_cast<const f32x4 *>(st + 4 * i);
  }
  const f32x4 zr = tid < F / 4 ? *reinterpret_cast<const f32x4 *>(st + (int64_t)F * DV + 4 * tid) : zero4();
  if (wv == 0) cp_decay_scan(p, h, t0, cnt, dtr, sL, lane);
  cp_write_wt<T, FH>(wq, p.d, sWq);
  cp_write_wt<T, FH>(wk, p.d, sWk);
#pragma unroll
  for (int m = 0; m < NS; ++m) {
    const int i = tid + 256 * m;  // S^T[cc][f0 .. f0+3] -> its tile-order place in row cc
    if (i < DV * F / 4) cp_store4(&sSt[(i / (F / 4)) * LDF + M::tpos(4 * (i % (F / 4)))], sr[m]);
  }
  if (tid < F / 4) *reinterpret_cast<f32x4 *>(&sZ[4 * tid]) = zr;
  __syncthreads();
  // the first key block's rows are in flight during the query features and the read-out
  const T *K = (const T *)p.k + b * p.sk_b + h * p.sk_h;
  const T *V = (const T *)p.v + b * p.sv_b + h * p.sv_h;
  CpX<T> xk;
  CpV<T, DV> vr;
  cp_load_x<T>(K, p.sk_t, t0, p.n, p.d, xk, wv, lane);
  cp_load_v<T, DV>(V, p.sv_t, t0, p.n, vr);
  const int lq = (int)qb * CP_BLK + 16 * wv + col;  // this lane's query within the chunk
  frag qf[KF];
  float den;
  {
    f32x4 ph[NFT];
    cp_features<T, FH>(xq, p.d, sWq, ph, lane);
#pragma unroll
    for (int s = 0; s < KF; ++s) qf[s] = M::from_acc(ph, s);
    // e^{L} phiQ . z on the rounded features the products use
    float dz = 0.f;
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft) {
      const f32x4 z4 = *reinterpret_cast<const f32x4 *>(&sZ[16 * ft + 4 * g]);
#pragma unroll
      for (int r = 0; r < 4; ++r) dz = __builtin_fmaf((float)(T)ph[ft][r], z4[r], dz);
    }
    den = group_sum(dz);
  }
  const float eLq = __expf((float)sL[lq]);
  den *= eLq;
  // inter-chunk read-out: O^T[c][t] = e^{L_t} sum_f S^T[c][f] phiQ[t][f]
  f32x4 O[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    O[ct] = zero4();
#pragma unroll
    for (int s = 0; s < KF; ++s) O[ct] = M::mma(M::ld_tile(sSt + (16 * ct + col) * LDF, s, g), qf[s], O[ct]);
    O[ct] *= eLq;
  }
  __syncthreads();  // the read-out copy's space goes to the key blocks
  for (int kb = 0; kb <= qb; ++kb) {
    const int64_t tb = t0 + kb * CP_BLK;
    {
      f32x4 ph[NFT];
      cp_features<T, FH>(xk, p.d, sWk, ph, lane);
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft) cp_store4(&sK[(16 * wv + col) * LDF + M::tpos(16 * ft + 4 * g)], ph[ft]);
    }
    cp_write_vt<T, DV, true>(vr, sVt);
    // the next key block's rows are in flight during this block's products
    if (kb < qb) {
      cp_load_x<T>(K, p.sk_t, tb + CP_BLK, p.n, p.d, xk, wv, lane);
      cp_load_v<T, DV>(V, p.sv_t, tb + CP_BLK, p.n, vr);
    }
    __syncthreads();
    // weighted scores Pt[s][t] of the block's four key tiles against this wave's queries
    f32x4 pt[4];
    float dsum = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x4 a = zero4();
#pragma unroll
      for (int s = 0; s < KF; ++s) a = M::mma(M::ld_tile(sK + (16 * j + col) * LDF, s, g), qf[s], a);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ls = kb * CP_BLK + 16 * j + 4 * g + r;  // key within the chunk
        const float w = ls <= lq ? a[r] * __expf((float)(sL[lq] - sL[ls])) : 0.f;
        pt[j][r] = (float)(T)w;  // the weight as the product with V sees it
        dsum += pt[j][r];
      }
    }
    den += group_sum(dsum);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int s = 0; s < KB; ++s)
        O[ct] = M::mma(M::ld_tile(sVt + (16 * ct + col) * L::LDB, s, g), M::from_acc(pt, s), O[ct]);
    __syncthreads();
  }
  // lane (col, g) holds columns 16ct + 4g .. +3 of query tq + 16 wv + col
  const int64_t t = tq + 16 * wv + col;
  if (t < p.n) {
    const float inv = 1.f / den;
    T *orow = (T *)p.o + b * p.so_b + h * p.so_h + t * p.so_t;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) cp_store4(orow + 16 * ct + 4 * g, O[ct] * inv);
  }
}

}  // namespace hm
