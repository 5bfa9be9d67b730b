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
// the read-out of the start state, the local state) is a 16x16 MFMA tile on LDS
// rows that are contiguous in K; for bf16 inputs the MFMA operands (phi, the
// weighted scores, the start state's read-out copy) are rounded to bf16 and
// accumulated in float32.  The carried states are float32 in the workspace.
#pragma once

#include "hm_device.hpp"

namespace hm {

struct CpParams {
  const void *q, *k, *v, *wq, *wk;
  const float *dt, *a_log;  // both NULL: a_t = 1
  const float *s_init;      // [B*H][F*dv + F] or NULL
  float *s_final;           // same layout, or NULL (may alias s_init)
  void *o;
  float *ws_state;          // [B*H][nc][F*dv + F]: local states, then start states
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

// The inclusive log-decay prefix over tokens t0 .. t0+cnt-1 of one (b, h), from t0
// on, into sL[0 .. cnt), by one wave, in float64 (differences of large prefix sums
// lose ~|L| 2^-24 in float32); tokens at or past n add 0.
__device__ __forceinline__ void cp_decay_prefix(const CpParams &p, int64_t b, int64_t h, int64_t t0, int cnt,
                                                double *sL, int lane) {
  const bool decay = p.dt != nullptr;
  const float *DT = decay ? p.dt + b * p.sdt_b + h * p.sdt_h : nullptr;
  const float expA = decay ? expf(p.a_log[h]) : 0.f;
  double carry = 0.0;
  for (int i0 = 0; i0 < cnt; i0 += 64) {
    const int64_t t = t0 + i0 + lane;
    const bool valid = decay && i0 + lane < cnt && t < p.n;
    const double x = valid ? (double)(-softplus_f32(DT[t * p.sdt_t]) * expA) : 0.0;
    const double L = wave_inclusive_scan(x) + carry;
    if (i0 + lane < cnt) sL[i0 + lane] = L;
    carry = lane63(L);
  }
}

// W^T (W is [d][FH] row-major, head stride sw_h) into sW rows of LDW elements,
// columns past d up to one MFMA K-step zero-filled; all threads.
template <typename T, int FH>
__device__ __forceinline__ void cp_stage_wt(const T *W, int d, T *sW) {
  using L = CpLds<T>;
  const int dpad = d < Mma<T>::KS ? Mma<T>::KS : d;
  for (int i = threadIdx.x; i < FH * dpad; i += blockDim.x) {
    const int j = i / dpad, dd = i % dpad;
    sW[j * L::LDW + dd] = dd < d ? W[(int64_t)dd * FH + j] : (T)0.f;
  }
}

// Features of token tile `wv` of the block at token tb: the wave's lane (col, g)
// gets, for token tb + 16 wv + col, ph[t][r] = phi at feature 16t + 4g + r of the u
// half (t < FH/16) or of the -u half (t >= FH/16), normalized (softmax over both
// halves), or 0 for tokens at or past n.  The projection U^T = W^T X^T runs on the
// MFMA with the token rows read from global memory straight into B operands.
template <typename T, int FH>
__device__ __forceinline__ void cp_features(const T *X, int64_t sx_t, int64_t tb, int64_t n, int d, const T *sW,
                                            f32x4 *ph, int wv, int lane) {
  using M = Mma<T>;
  using frag = typename M::frag;
  using L = CpLds<T>;
  constexpr int NFH = FH / 16;
  constexpr float L2E = 1.4426950408889634f;
  const int col = lane & 15, g = lane >> 4;
  const int64_t t = tb + 16 * wv + col;
  const bool ok = t < n;
  const T *row = X + (ok ? t : 0) * sx_t;
  f32x4 u[NFH];
#pragma unroll
  for (int ft = 0; ft < NFH; ++ft) u[ft] = zero4();
  for (int k0 = 0; k0 < d; k0 += M::KS) {
    const bool in = ok && k0 + (M::EPL == 8 ? 8 * g : g) < d;
    const frag xb = in ? M::ld_contig(row + k0, g) : frag{};
#pragma unroll
    for (int ft = 0; ft < NFH; ++ft) u[ft] = M::mma(M::ld_contig(sW + (16 * ft + col) * L::LDW + k0, g), xb, u[ft]);
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
  const float inv = ok ? 1.f / group_sum(sum) : 0.f;
#pragma unroll
  for (int ft = 0; ft < 2 * NFH; ++ft) ph[ft] *= inv;
}

// v rows [tb, tb+64) of one (b, h) into sVt[c][t] (transposed, LDB elements per
// row), zeros past n; all threads, 16-byte loads.
template <typename T, int DV>
__device__ __forceinline__ void cp_stage_vt(const T *V, int64_t sv_t, int64_t tb, int64_t n, T *sVt) {
  using L = CpLds<T>;
  constexpr int EPL = 16 / (int)sizeof(T), PR = DV / EPL;  // 16-byte pieces per row
  for (int i = threadIdx.x; i < CP_BLK * PR; i += blockDim.x) {
    const int tt = i / PR, c0 = (i % PR) * EPL;
    const int64_t t = tb + tt;
    f32x4 raw = zero4();
    if (t < n) raw = *reinterpret_cast<const f32x4 *>(V + t * sv_t + c0);
    const T *e = reinterpret_cast<const T *>(&raw);
#pragma unroll
    for (int x = 0; x < EPL; ++x) sVt[(c0 + x) * L::LDB + tt] = e[x];
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
  if (wv == 0) cp_decay_prefix(p, b, h, t0, cnt, sL, lane);
  cp_stage_wt<T, FH>((const T *)p.wk + h * p.sw_h, p.d, sW);
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
      cp_features<T, FH>(K, p.sk_t, tb, p.n, p.d, sW, ph, wv, lane);
      const int lt = kb * CP_BLK + 16 * wv + col;  // token within the chunk
      const float w = lt < cnt ? __expf((float)(lam - sL[lt])) : 0.f;
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
        for (int r = 0; r < 4; ++r) sKt[(16 * ft + 4 * g + r) * L::LDB + 16 * wv + col] = (T)(ph[ft][r] * w);
    }
    cp_stage_vt<T, DV>(V, p.sv_t, tb, p.n, sVt);
    __syncthreads();
    // dS[f][c] += sum_t Kt[f][t] Vt[c][t]: tile i of this wave is (tile row, tile column)
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tile = 4 * i + wv;
      if (tile < NTL) {
        const int ft = tile / NCT, ct = tile % NCT;
#pragma unroll
        for (int k0 = 0; k0 < CP_BLK; k0 += M::KS)
          acc[i] = M::mma(M::ld_contig(sKt + (16 * ft + col) * L::LDB + k0, g),
                          M::ld_contig(sVt + (16 * ct + col) * L::LDB + k0, g), acc[i]);
      }
    }
    if (tid < F) {
#pragma unroll 8
      for (int t = 0; t < CP_BLK; ++t) zsum += (float)sKt[tid * L::LDB + t];
    }
    __syncthreads();
  }
  const int64_t BLK = (int64_t)F * DV + F;
  float *st = p.ws_state + (bh * p.nc + c) * BLK;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int tile = 4 * i + wv;
    if (tile < NTL) {
      const int ft = tile / NCT, ct = tile % NCT;
#pragma unroll
      for (int r = 0; r < 4; ++r) st[(int64_t)(16 * ft + 4 * g + r) * DV + 16 * ct + col] = acc[i][r];
    }
  }
  if (tid < F) st[(int64_t)F * DV + tid] = zsum;
  if (tid == 0) p.ws_lam[bh * p.nc + c] = (float)lam;
}

// Pass 2: thread e of (b, h) walks the chunks, replacing each local state by the
// chunk's start state; s_init is read before s_final is written (same element,
// same thread), so the two may alias.
static __global__ __launch_bounds__(256) void cp_scan_kernel(const CpParams p, int64_t BLK) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x, bh = blockIdx.y;
  if (e >= BLK) return;
  float s = p.s_init ? p.s_init[bh * BLK + e] : 0.f;
  float *st = p.ws_state + bh * p.nc * BLK + e;
  const float *lam = p.ws_lam + bh * p.nc;
  for (int64_t c = 0; c < p.nc; ++c) {
    const float loc = st[c * BLK];
    st[c * BLK] = s;
    s = __builtin_fmaf(__expf(lam[c]), s, loc);
  }
  if (p.s_final) p.s_final[bh * BLK + e] = s;
}

// Pass 3: one workgroup (4 waves) per (b, h, chunk, 64-query block); wave w owns
// query tile w (16 tokens) and all dv columns of its output.
template <typename T, int FH, int DV>
__global__ __launch_bounds__(256) void cp_out_kernel(const CpParams p) {
  using M = Mma<T>;
  using L = CpLds<T>;
  constexpr int F = 2 * FH, NFT = F / 16, NCT = DV / 16, LDF = F + L::PAD;
  // the read-out copy of the start state (S^T, dv rows of F) shares space with the
  // key block's phi(k) rows, v^T and the weighted score rows, used after it
  constexpr int KV = CP_BLK * LDF + DV * L::LDB + CP_BLK * L::LDB, ST = DV * LDF;
  __shared__ __align__(16) T sW[FH * L::LDW];
  __shared__ __align__(16) T sQ[CP_BLK * LDF];
  __shared__ __align__(16) T sU[KV > ST ? KV : ST];
  __shared__ float sZ[F];
  __shared__ float sDen[CP_BLK];
  __shared__ double sL[CP_CHMAX];
  T *sSt = sU, *sK = sU, *sVt = sU + CP_BLK * LDF, *sP = sVt + DV * L::LDB;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, col = lane & 15, g = lane >> 4;
  const int nqb = p.chunk / CP_BLK;
  const int64_t qb = blockIdx.x % nqb, c = (blockIdx.x / nqb) % p.nc, bh = blockIdx.x / nqb / p.nc;
  const int64_t b = bh / p.H, h = bh % p.H, t0 = c * p.chunk, tq = t0 + qb * CP_BLK;
  if (tq >= p.n) return;  // the whole block is past the sequence's end (uniform)
  const int cnt = (int)((qb + 1) * CP_BLK);  // chunk tokens up to this block's end
  const int64_t BLK = (int64_t)F * DV + F;
  const float *st = p.ws_state + (bh * p.nc + c) * BLK;
  if (wv == 0) cp_decay_prefix(p, b, h, t0, cnt, sL, lane);
  cp_stage_wt<T, FH>((const T *)p.wq + h * p.sw_h, p.d, sW);
  for (int i = tid; i < F * DV / 4; i += 256) {  // S^T, rounded to the operand type
    const int f = i / (DV / 4), c4 = 4 * (i % (DV / 4));
    const f32x4 s4 = *reinterpret_cast<const f32x4 *>(st + (int64_t)f * DV + c4);
#pragma unroll
    for (int x = 0; x < 4; ++x) sSt[(c4 + x) * LDF + f] = (T)s4[x];
  }
  for (int i = tid; i < F; i += 256) sZ[i] = st[(int64_t)F * DV + i];
  __syncthreads();
  // phi(q) rows of the block
  {
    f32x4 ph[NFT];
    cp_features<T, FH>((const T *)p.q + b * p.sq_b + h * p.sq_h, p.sq_t, tq, p.n, p.d, sW, ph, wv, lane);
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
      for (int r = 0; r < 4; ++r) sQ[(16 * wv + col) * LDF + 16 * ft + 4 * g + r] = (T)ph[ft][r];
  }
  __syncthreads();
  // inter-chunk read-out: O = diag(e^{L}) phiQ S, den = e^{L} phiQ . z
  f32x4 O[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    O[ct] = zero4();
#pragma unroll
    for (int k0 = 0; k0 < F; k0 += M::KS)
      O[ct] = M::mma(M::ld_contig(sQ + (16 * wv + col) * LDF + k0, g), M::ld_contig(sSt + (16 * ct + col) * LDF + k0, g),
                     O[ct]);
  }
  float eL[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) eL[r] = __expf((float)sL[qb * CP_BLK + 16 * wv + 4 * g + r]);
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) O[ct][r] *= eL[r];
  float den = 0.f;  // thread t < 64: query t's denominator
  if (tid < CP_BLK) {
    for (int f = 0; f < F; ++f) den = __builtin_fmaf((float)sQ[tid * LDF + f], sZ[f], den);
    den *= __expf((float)sL[qb * CP_BLK + tid]);
  }
  __syncthreads();  // the start state's copy is done with; W^T of k replaces W^T of q
  cp_stage_wt<T, FH>((const T *)p.wk + h * p.sw_h, p.d, sW);
  const T *K = (const T *)p.k + b * p.sk_b + h * p.sk_h;
  const T *V = (const T *)p.v + b * p.sv_b + h * p.sv_h;
  __syncthreads();
  for (int kb = 0; kb <= qb; ++kb) {
    const int64_t tb = t0 + kb * CP_BLK;
    {
      f32x4 ph[NFT];
      cp_features<T, FH>(K, p.sk_t, tb, p.n, p.d, sW, ph, wv, lane);
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
        for (int r = 0; r < 4; ++r) sK[(16 * wv + col) * LDF + 16 * ft + 4 * g + r] = (T)ph[ft][r];
    }
    cp_stage_vt<T, DV>(V, p.sv_t, tb, p.n, sVt);
    __syncthreads();
    // weighted scores of query tile wv against the block's four key tiles
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x4 s = zero4();
#pragma unroll
      for (int k0 = 0; k0 < F; k0 += M::KS)
        s = M::mma(M::ld_contig(sQ + (16 * wv + col) * LDF + k0, g), M::ld_contig(sK + (16 * j + col) * LDF + k0, g), s);
      const int ls = kb * CP_BLK + 16 * j + col;  // key within the chunk
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int lq = qb * CP_BLK + 16 * wv + 4 * g + r;  // query within the chunk
        const float w = ls <= lq ? s[r] * __expf((float)(sL[lq] - sL[ls])) : 0.f;
        sP[(16 * wv + 4 * g + r) * L::LDB + 16 * j + col] = (T)w;
      }
    }
    __syncthreads();
    if (tid < CP_BLK) {
#pragma unroll 8
      for (int s = 0; s < CP_BLK; ++s) den += (float)sP[tid * L::LDB + s];
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int k0 = 0; k0 < CP_BLK; k0 += M::KS)
        O[ct] = M::mma(M::ld_contig(sP + (16 * wv + col) * L::LDB + k0, g), M::ld_contig(sVt + (16 * ct + col) * L::LDB + k0, g),
                       O[ct]);
    __syncthreads();
  }
  if (tid < CP_BLK) sDen[tid] = den;
  __syncthreads();
  T *Ob = (T *)p.o + b * p.so_b + h * p.so_h;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int lt = 16 * wv + 4 * g + r;
    const int64_t t = tq + lt;
    if (t < p.n) {
      const float inv = 1.f / sDen[lt];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) Ob[t * p.so_t + 16 * ct + col] = (T)(O[ct][r] * inv);
    }
  }
}

}  // namespace hm
