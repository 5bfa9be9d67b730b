// Chunked prefill of causal, normalized Hedgehog linear attention on gfx950.
//
// What one workgroup computes (pages: [HM] = the gsyq.cn HedgeMamba explainer,
// [LA] = the cnblogs linear-attention tutorial, [SSM] = the quant67 SSM lecture):
// one (b, h), one sequence segment [t0, t1), the value columns [n0, n0 + DW).
// It walks the segment in chunks of C = 64 tokens and keeps the carried state
// (numerator S [F x DW] in MFMA accumulators, denominator z [F] in LDS) on chip
// the whole time.  Per chunk, with L_c the inclusive cumulative log-decay inside
// the chunk ([SSM] §3.2 decay, [LA] 4.3 scalar decay on the carried state):
//   featurize ([HM] §2.1, §5.3):  phiQ, phiK = softmax([x W, -x W])
//   scores:      Pt[c'][c] = phiK_c' . phiQ_c * exp(L_c - L_c') * [c' <= c]
//   inter-chunk: O^T  = S^T phiQ^T * diag(e^{L_c}),  den_c = e^{L_c} phiQ_c . z
//   intra-chunk: O^T += V^T Pt,                    den_c += sum_c' Pt[c'][c]
//   output:      o_c = O_c / den_c          ([HM] §2.3 numerator / denominator)
//   state:       S = e^{L_last} S + (phiK * e^{L_last - L})^T V,  z likewise
//                ([LA] part 3 recurrence applied to a whole chunk at once).
// This is the chunk-parallel mode of [LA] part 5; chunking only reorders the sums
// of the recurrent definition.
//
// Layout choices (all matrix products are 16x16 MFMA tiles, wave w owns value
// tile w, i.e. columns n0 + 16w .. n0 + 16w + 15):
//   * q and k rows are read from HBM straight into B-operand fragments (no LDS);
//   * v rows are read into A-operand fragments and turned into the
//     accumulator layout by one MFMA against a 0/1 selector, which is the
//     tile-order operand layout both V products need: v never touches LDS;
//   * phiK is likewise re-laid out by selector MFMAs into phiK^T for the state
//     update; all LDS traffic is 8- or 16-byte vectors;
//   * the state S stays in accumulators and is fed back as the A operand of the
//     read-out in tile order (see hm_device.hpp);
//   * the next chunk's q, k, v, dt are loaded into registers while the current
//     chunk computes.
#pragma once

#include "hm_device.hpp"

namespace hm {

constexpr int CHUNK = 64;
enum { MODE_FULL = 0, MODE_LOCAL = 1 };

struct FwdParams {
  const void *q, *k, *v, *wq, *wk;
  const float *dt, *a_log;
  const float *s_start0;  // start state of segment 0 (NULL = zeros)
  float *s_final;         // written by the last segment (NULL = not written)
  void *o;
  float *ws_state;        // [nseg-1][B*H][F*dv+F]: local end states, then start states
  float *ws_lam;          // [nseg-1][B*H]: summed log-decay of each segment
  int64_t B, H, n, dv;
  int64_t sq_b, sq_h, sq_t, sk_b, sk_h, sk_t, sv_b, sv_h, sv_t, so_b, so_h, so_t;
  int64_t sw_h, sdt_b, sdt_h, sdt_t;
  int64_t seg_len;        // tokens per segment, a multiple of CHUNK
  int64_t nitems;         // (b,h,segment) items in this launch
  int nseg;               // segments of the whole sequence
  int nseg_run;           // segments covered by this launch (nseg, or nseg-1 for MODE_LOCAL)
  int dsplit;             // workgroups per item, each owning dv/dsplit columns
};

template <typename F> __device__ __forceinline__ F zfrag() { return F{}; }

// Workgroup layout: 4 feature waves (featurize, score tiles, denominators, decay)
// and NS state waves (value columns, state, read-out), the two roles one chunk
// apart so that the softmax VALU work of one overlaps the MFMA work of the other.
constexpr int fwd_state_waves(int DW) { return DW >= 32 ? DW / 32 : 1; }
constexpr int fwd_waves(int DW) { return 4 + fwd_state_waves(DW); }

// Element pointer `base` (wave-uniform) plus a per-lane 32-bit byte offset: lets
// the compiler address global memory as scalar base + vector offset.
template <typename T>
__device__ __forceinline__ const T *at(const T *base, uint32_t byte_off) {
  return reinterpret_cast<const T *>(reinterpret_cast<const char *>(base) + byte_off);
}

template <typename T, int DK, int FH, int DW, bool DECAY, int MODE>
__global__ __launch_bounds__(fwd_waves(DW) * 64) void fwd_kernel(const FwdParams p) {
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int C = CHUNK;
  constexpr int F = 2 * FH;
  constexpr int NS = fwd_state_waves(DW);  // state waves
  constexpr int NTW = DW / (16 * NS);      // value tiles per state wave
  constexpr int NT = fwd_waves(DW) * 64;
  constexpr int NCT = C / 16;              // token tiles per chunk (4)
  constexpr int NFH = FH / 16;             // feature tiles per half of phi
  constexpr int NFT = F / 16;              // feature tiles
  constexpr int KD = DK / M::KS;           // featurize K-steps (contiguous order)
  constexpr int KF = M::steps(NFT);        // K-steps over F (tile order)
  constexpr int KC = M::steps(NCT);        // K-steps over the chunk (tile order)
  constexpr int EPL = M::EPL;              // operand elements per lane
  constexpr int PAD = M::PAD;
  constexpr int LDW = DK + PAD, LDQ = F + PAD, LDC = C + PAD;
  constexpr bool FULL = MODE == MODE_FULL;
  constexpr int TPF_ = FULL ? 2 : 1;       // featurize tasks per feature wave
  constexpr int KVL = EPL == 8 ? 1 : 4;    // K-steps of the v re-layout per tile
  constexpr float L2E = 1.4426950408889634f;
  static_assert(NCT == 4, "four token tiles per chunk");
  static_assert(NTW >= 1 && NTW <= 2 && NTW * 16 * NS == DW, "value tile split");
  static_assert(DK % M::KS == 0 && F % M::KS == 0, "K multiples");

  __shared__ __align__(16) T sWq[FULL ? FH * LDW : 8];    // W^T: sW[f][d] = W[d][f]
  __shared__ __align__(16) T sWk[FH * LDW];
  __shared__ __align__(16) T sKt[2][F * LDC];               // decay-weighted phi(k)^T, tile order
  __shared__ __align__(16) T sQ[FULL ? 2 : 1][FULL ? C * LDQ : 8];  // phi(q) (unnormalized)
  __shared__ __align__(16) T sP[FULL ? 2 : 1][FULL ? C * LDC : 8];  // masked decayed scores
  __shared__ __align__(16) double sL[3][C];                 // inclusive log-decay prefix, float64
  __shared__ __align__(16) float seL[3][C];
  __shared__ __align__(16) float seK[3][C];
  __shared__ float sLast[3];
  __shared__ __align__(16) float sDenPart[2][NCT][C];
  __shared__ __align__(16) float sDenInter[2][C];

  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, col = lane & 15, g = lane >> 4;
  const bool fwave = wv < 4;
  const int sw = wv - 4;  // state wave index

  // Workgroup -> (item, half).  Consecutive workgroups go to different XCDs
  // (bid % 8); the dsplit halves of one item share an XCD so the second half
  // finds q, k in that XCD's L2.
  const int64_t bid = blockIdx.x;
  const int xcd = (int)(bid & 7);
  const int64_t rnd = bid >> 3;
  const int half = (int)(rnd % p.dsplit);
  const int64_t item = (rnd / p.dsplit) * 8 + xcd;
  if (item >= p.nitems) return;
  const int64_t BH = p.B * p.H;
  const int64_t bh = item / p.nseg_run;
  const int seg = (int)(item % p.nseg_run);
  const int64_t b = bh / p.H, h = bh % p.H;
  const int64_t t0 = (int64_t)seg * p.seg_len;
  const int64_t t1 = t0 + p.seg_len < p.n ? t0 + p.seg_len : p.n;
  const int ncol = half * DW + 16 * NTW * (fwave ? 0 : sw);  // first value column (state waves)
  const int64_t BLK = (int64_t)F * p.dv + F;

  const T *Q = (const T *)p.q + b * p.sq_b + h * p.sq_h;
  const T *K = (const T *)p.k + b * p.sk_b + h * p.sk_h;
  const T *V = (const T *)p.v + b * p.sv_b + h * p.sv_h;
  T *O = (T *)p.o + b * p.so_b + h * p.so_h;
  const float *DT = DECAY ? p.dt + b * p.sdt_b + h * p.sdt_h : nullptr;
  const float expA = DECAY ? expf(p.a_log[h]) : 1.f;

  // W^T into LDS: sW[f][d] = W[d][f]
  {
    const T *wk = (const T *)p.wk + h * p.sw_h;
    for (int i = tid; i < DK * FH; i += NT) sWk[(i % FH) * LDW + i / FH] = wk[i];
    if constexpr (FULL) {
      const T *wq = (const T *)p.wq + h * p.sw_h;
      for (int i = tid; i < DK * FH; i += NT) sWq[(i % FH) * LDW + i / FH] = wq[i];
    }
  }

  const float *st = nullptr;
  if constexpr (FULL) {
    if (seg == 0) st = p.s_start0 ? p.s_start0 + bh * BLK : nullptr;
    else st = p.ws_state + ((int64_t)(seg - 1) * BH + bh) * BLK;
  }
  const int64_t nch = t1 > t0 ? (t1 - t0 + C - 1) / C : 0;
  float *dst = nullptr;  // end state destination
  if constexpr (FULL) {
    if (seg == p.nseg - 1) dst = p.s_final ? p.s_final + bh * BLK : nullptr;
  } else {
    dst = p.ws_state + ((int64_t)seg * BH + bh) * BLK;
  }

  // The two roles run separate loops with the same two barriers per iteration:
  // iteration j, half A: feature waves featurize chunk j while state waves read
  // out and advance the state over chunk j-1; half B: feature waves form chunk
  // j's score tiles and denominators while state waves finish chunk j-1.
  if (fwave) {
    // ---------------------------------------------------------------- feature waves
    // Feature-wave tasks.  FULL: waves 0, 1 featurize q tiles {0,1}, {2,3}; waves
    // 2, 3 featurize k tiles {0,3}, {1,2} (their score-tile rows balance: 4+1, 3+2).
    // LOCAL: wave w featurizes k tile w.
    const bool isq = FULL && wv < 2;
    int tile[TPF_];
#pragma unroll
    for (int i = 0; i < TPF_; ++i) {
      if constexpr (!FULL) tile[i] = wv;
      else tile[i] = wv < 2 ? 2 * wv + i : (wv == 2 ? (i == 0 ? 0 : 3) : (i == 0 ? 1 : 2));
    }
    uint32_t xoff[TPF_];
#pragma unroll
    for (int i = 0; i < TPF_; ++i)
      xoff[i] = (uint32_t)(((int64_t)(16 * tile[i] + col) * (isq ? p.sq_t : p.sk_t) + EPL * g) * sizeof(T));

    // z (feature wave 0): first column of an [F x 16] accumulator block
    f32x4 Z[NFT];
#pragma unroll
    for (int t = 0; t < NFT; ++t) Z[t] = zero4();
    if (st && wv == 0 && col == 0) {
#pragma unroll
      for (int t = 0; t < NFT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) Z[t][r] = st[(int64_t)F * p.dv + 16 * t + 4 * g + r];
    }

    frag xf[TPF_][KD];
    auto load_x = [&](int64_t tc) {
      const T *base = (isq ? Q : K) + tc * (isq ? p.sq_t : p.sk_t);
#pragma unroll
      for (int i = 0; i < TPF_; ++i) {
        const bool ok = tc + 16 * tile[i] + col < t1;
#pragma unroll
        for (int s = 0; s < KD; ++s) xf[i][s] = ok ? M::ld_contig(at(base, xoff[i]) + s * M::KS, 0) : zfrag<frag>();
      }
    };
    float dtn = 0.f;
    auto load_dt = [&](int64_t tc) {
      if constexpr (DECAY) dtn = tc + lane < t1 ? DT[(tc + lane) * p.sdt_t] : 0.f;
    };
    // Wave 1: decay factors of the chunk starting at tc into buffer `bufi`.  The
    // prefix sums are carried in float64: differences L_c - L_c' of large prefix
    // sums would lose ~|L| * 2^-24 in float32, and |L| reaches the thousands.
    double lam = 0.0;
    auto decay = [&](int64_t tc, int bufi) {
      const bool valid = tc + lane < t1;
      if constexpr (DECAY) {
        const double L = wave_inclusive_scan(valid ? (double)(-softplus_f32(dtn) * expA) : 0.0);
        const double Ll = lane63(L);
        sL[bufi][lane] = L;
        seL[bufi][lane] = __expf((float)L);
        seK[bufi][lane] = valid ? __expf((float)(Ll - L)) : 0.f;
        if (lane == 0) sLast[bufi] = __expf((float)Ll);
        lam += Ll;
      } else {
        if (lane == 0) sLast[bufi] = 1.f;
      }
    };
    constexpr int NKS = EPL == 8 ? 2 : 4;
    frag ksel[NKS];
#pragma unroll
    for (int x = 0; x < NKS; ++x) {
      if constexpr (EPL == 8) ksel[x] = M::select([&](int e) { return 16 * (e >> 2) + 4 * g + (e & 3) == 16 * x + col; });
      else ksel[x] = M::select([&](int) { return 4 * g + x == col; });
    }
    const frag ones = M::select([&](int) { return col == 0; });  // column 0 of a K x 16 block

    if (nch > 0) {
      load_x(t0);
      if (wv == 1) {
        load_dt(t0);
        decay(t0, 0);
        if (nch > 1) load_dt(t0 + C);
      }
    }
    __syncthreads();

    frag kf[TPF_][KF];  // phi(k) of the current chunk, tile order
    for (int64_t j = 0; j <= nch; ++j) {
      const int64_t tf = t0 + j * C;
      const int bf = (int)(j & 1);
      const int df = (int)(j % 3);
      // ---- half A: featurize chunk j
      if (j < nch) {
        f32x4 u[TPF_][NFH];
        const T *sW = isq ? sWq : sWk;
#pragma unroll
        for (int t = 0; t < NFH; ++t) {
          frag wa[KD];  // W^T fragments of feature tile t, shared by the wave's tiles
#pragma unroll
          for (int s = 0; s < KD; ++s) wa[s] = M::ld_contig(sW + (16 * t + col) * LDW + s * M::KS, g);
#pragma unroll
          for (int i = 0; i < TPF_; ++i) {
            u[i][t] = zero4();
#pragma unroll
            for (int s = 0; s < KD; ++s) u[i][t] = M::mma(wa[s], xf[i][s], u[i][t]);
          }
        }
        if (j + 1 < nch) load_x(tf + C);
#pragma unroll
        for (int i = 0; i < TPF_; ++i) {
          const int bt = tile[i];
          float m = 0.f;
#pragma unroll
          for (int t = 0; t < NFH; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(u[i][t][r]));
          const float ml = group_max(m) * L2E;
          f32x4 ph[NFT];
          float sum = 0.f;
#pragma unroll
          for (int t = 0; t < NFH; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float x = u[i][t][r];
              const float ep = __builtin_amdgcn_exp2f(__builtin_fmaf(x, L2E, -ml));
              const float em = __builtin_amdgcn_exp2f(__builtin_fmaf(-x, L2E, -ml));
              ph[t][r] = ep;
              ph[NFH + t][r] = em;
              sum += ep + em;
            }
          if (isq) {
            // phi(q) unnormalized: a positive per-query factor cancels in o's ratio
            const int cr = 16 * bt + col;
#pragma unroll
            for (int t = 0; t < NFT; ++t) store4(&sQ[bf][cr * LDQ + M::tpos(16 * t + 4 * g)], ph[t]);
          } else {
            float inv = 1.f / group_sum(sum);
            if constexpr (!DECAY) {
              if (tf + 16 * bt + col >= t1) inv = 0.f;  // rows past the end contribute nothing
            }
#pragma unroll
            for (int t = 0; t < NFT; ++t) ph[t] *= inv;
#pragma unroll
            for (int s = 0; s < KF; ++s) kf[i][s] = M::from_acc(ph, s);
            f32x4 w4;
            if constexpr (DECAY) w4 = *reinterpret_cast<const f32x4 *>(&seK[df][16 * bt + 4 * g]);
            // phiK^T tile uo (decay-weighted): lane (g, col f') gets phiK[16bt+4g+r][16uo+f']
#pragma unroll
            for (int uo = 0; uo < NFT; ++uo) {
              f32x4 acc = zero4();
              if constexpr (EPL == 8) {
                acc = M::mma(kf[i][uo >> 1], ksel[uo & 1], acc);
              } else {
#pragma unroll
                for (int s = 4 * uo; s < 4 * uo + 4; ++s) acc = M::mma(kf[i][s], ksel[s & 3], acc);
              }
              if constexpr (DECAY) acc *= w4;
              store4(&sKt[bf][(16 * uo + col) * LDC + M::tpos(16 * bt + 4 * g)], acc);
            }
          }
        }
      }
      __syncthreads();
      // ---- half B: score tiles, denominators and z for chunk j; decay of chunk j+1
      if (j < nch) {
        if constexpr (FULL) {
          if (wv >= 2) {
            // score tiles of rows a (this wave's k tiles) -> sP, row sums -> sDenPart
#pragma unroll
            for (int i = 0; i < TPF_; ++i) {
              const int a = tile[i];
#pragma unroll
              for (int bt = 0; bt < NCT; ++bt) {
                const int cc = 16 * bt + col;
                if (bt < a) {
                  store4(&sP[bf][cc * LDC + M::tpos(16 * a + 4 * g)], zero4());
                  continue;
                }
                frag bq[KF];
#pragma unroll
                for (int s = 0; s < KF; ++s) bq[s] = M::ld_tile(&sQ[bf][cc * LDQ], s, g);
                f32x4 acc = zero4();
#pragma unroll
                for (int s = 0; s < KF; ++s) acc = M::mma(kf[i][s], bq[s], acc);
                f32x4 w;
                double lc = 0.0;
                if constexpr (DECAY) lc = sL[df][cc];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                  const int cp = 16 * a + 4 * g + r;
                  float x = cp <= cc ? acc[r] : 0.f;
                  if constexpr (DECAY) {
                    if (cp <= cc) x *= __expf((float)(lc - sL[df][cp]));
                  }
                  w[r] = x;
                }
                w = round4(w, T{});
                store4(&sP[bf][cc * LDC + M::tpos(16 * a + 4 * g)], w);
                const float dsum = group_sum(w[0] + w[1] + w[2] + w[3]);
                if (g == 0) sDenPart[bf][a][cc] = dsum;
              }
            }
          } else if (wv == 0) {
            // den_inter = e^{L_c} z . phi(q_c): z as row 0 of the A operand
            frag zf[KF];
#pragma unroll
            for (int s = 0; s < KF; ++s) zf[s] = M::from_acc(Z, s);
#pragma unroll
            for (int bt = 0; bt < NCT; ++bt) {
              const int cc = 16 * bt + col;
              f32x4 acc = zero4();
#pragma unroll
              for (int s = 0; s < KF; ++s) acc = M::mma(zf[s], M::ld_tile(&sQ[bf][cc * LDQ], s, g), acc);
              if (g == 0) sDenInter[bf][cc] = DECAY ? acc[0] * seL[df][cc] : acc[0];
            }
          }
        }
        if (wv == 0) {
          // z <- e^{L_last} z + sum_c' phi~(k_c'): phi~(k)^T times a ones column
          if constexpr (DECAY) {
            const float el = sLast[df];
#pragma unroll
            for (int t = 0; t < NFT; ++t) Z[t] *= el;
          }
#pragma unroll
          for (int t = 0; t < NFT; ++t)
#pragma unroll
            for (int s = 0; s < KC; ++s) Z[t] = M::mma(M::ld_tile(&sKt[bf][(16 * t + col) * LDC], s, g), ones, Z[t]);
        }
        if (wv == 1 && j + 1 < nch) {
          decay(tf + C, (int)((j + 1) % 3));
          if (j + 2 < nch) load_dt(tf + 2 * C);
        }
      }
      __syncthreads();
    }
    if (!FULL && half == 0 && wv == 1 && lane == 0) p.ws_lam[(int64_t)seg * BH + bh] = (float)lam;
    if (dst && wv == 0 && col == 0 && half == 0) {
#pragma unroll
      for (int t = 0; t < NFT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(int64_t)F * p.dv + 16 * t + 4 * g + r] = Z[t][r];
    }
  } else {
    // ---------------------------------------------------------------- state waves
    f32x4 S[NTW][NFT];
#pragma unroll
    for (int jj = 0; jj < NTW; ++jj)
#pragma unroll
      for (int t = 0; t < NFT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          S[jj][t][r] = st ? st[(int64_t)(16 * t + 4 * g + r) * p.dv + ncol + 16 * jj + col] : 0.f;
    uint32_t voff[NTW];
#pragma unroll
    for (int jj = 0; jj < NTW; ++jj)
      voff[jj] = (uint32_t)(((int64_t)col * p.sv_t + ncol + 16 * jj + (EPL == 8 ? 8 * g : g)) * sizeof(T));
    frag vf[NTW][NCT][KVL];
    auto load_v = [&](int64_t tc) {
#pragma unroll
      for (int bt = 0; bt < NCT; ++bt) {
        const T *base = V + (tc + 16 * bt) * p.sv_t;
        const bool ok = tc + 16 * bt + col < t1;
#pragma unroll
        for (int jj = 0; jj < NTW; ++jj) {
          if constexpr (EPL == 8) {
            vf[jj][bt][0] = (ok && g < 2) ? M::ld_contig(at(base, voff[jj]), 0) : zfrag<frag>();
          } else {
#pragma unroll
            for (int s = 0; s < KVL; ++s) vf[jj][bt][s] = ok ? at(base, voff[jj])[4 * s] : 0.f;
          }
        }
      }
    };
    frag vsel[KVL];
#pragma unroll
    for (int s = 0; s < KVL; ++s) {
      if constexpr (EPL == 8) vsel[s] = M::select([&](int e) { return 8 * g + e == col; });
      else vsel[s] = M::select([&](int) { return 4 * s + g == col; });
    }

    if (nch > 0) load_v(t0);
    __syncthreads();

    frag vfr[NTW][KC];  // v of the chunk being read out, tile order
    f32x4 oacc[NTW][NCT];
    for (int64_t j = 0; j <= nch; ++j) {
      const int64_t ts = t0 + (j - 1) * C;  // chunk read out in this iteration (j >= 1)
      const int bs = (int)((j + 1) & 1);
      const int ds = (int)((j + 2) % 3);
      // ---- half A: inter read-out and state update over chunk j-1
      if (j >= 1) {
        // v of chunk ts -> accumulator layout: lane (g, col n) holds v[16bt + 4g + r][n]
#pragma unroll
        for (int jj = 0; jj < NTW; ++jj) {
          f32x4 vacc[NCT];
#pragma unroll
          for (int bt = 0; bt < NCT; ++bt) {
            vacc[bt] = zero4();
#pragma unroll
            for (int s = 0; s < KVL; ++s) vacc[bt] = M::mma(vf[jj][bt][s], vsel[s], vacc[bt]);
          }
#pragma unroll
          for (int s = 0; s < KC; ++s) vfr[jj][s] = M::from_acc(vacc, s);
        }
        if (j < nch) load_v(ts + C);
        if constexpr (FULL) {
          frag sfr[NTW][KF];
#pragma unroll
          for (int jj = 0; jj < NTW; ++jj)
#pragma unroll
            for (int s = 0; s < KF; ++s) sfr[jj][s] = M::from_acc(S[jj], s);
#pragma unroll
          for (int bt = 0; bt < NCT; ++bt) {
            const int cc = 16 * bt + col;
            frag bq[KF];
#pragma unroll
            for (int s = 0; s < KF; ++s) bq[s] = M::ld_tile(&sQ[bs][cc * LDQ], s, g);
#pragma unroll
            for (int jj = 0; jj < NTW; ++jj) {
              oacc[jj][bt] = zero4();
#pragma unroll
              for (int s = 0; s < KF; ++s) oacc[jj][bt] = M::mma(sfr[jj][s], bq[s], oacc[jj][bt]);
              if constexpr (DECAY) oacc[jj][bt] *= seL[ds][cc];
            }
          }
        }
        if constexpr (DECAY) {
          const float el = sLast[ds];
#pragma unroll
          for (int jj = 0; jj < NTW; ++jj)
#pragma unroll
            for (int t = 0; t < NFT; ++t) S[jj][t] *= el;
        }
#pragma unroll
        for (int t = 0; t < NFT; ++t) {
          frag ak[KC];
#pragma unroll
          for (int s = 0; s < KC; ++s) ak[s] = M::ld_tile(&sKt[bs][(16 * t + col) * LDC], s, g);
#pragma unroll
          for (int jj = 0; jj < NTW; ++jj)
#pragma unroll
            for (int s = 0; s < KC; ++s) S[jj][t] = M::mma(ak[s], vfr[jj][s], S[jj][t]);
        }
      }
      __syncthreads();
      // ---- half B: intra read-out of chunk j-1, normalize, store
      if constexpr (FULL) {
        if (j >= 1) {
#pragma unroll
          for (int bt = 0; bt < NCT; ++bt) {
            const int cc = 16 * bt + col;
            frag bp[M::steps_upto(NCT - 1)];
#pragma unroll
            for (int s = 0; s < M::steps_upto(bt); ++s) bp[s] = M::ld_tile(&sP[bs][cc * LDC], s, g);
#pragma unroll
            for (int jj = 0; jj < NTW; ++jj)
#pragma unroll
              for (int s = 0; s < M::steps_upto(bt); ++s) oacc[jj][bt] = M::mma(vfr[jj][s], bp[s], oacc[jj][bt]);
            const int64_t c = ts + cc;
            if (c < t1) {
              float den = sDenInter[bs][cc];
#pragma unroll
              for (int a = 0; a <= bt; ++a) den += sDenPart[bs][a][cc];
              const float inv = 1.f / den;
#pragma unroll
              for (int jj = 0; jj < NTW; ++jj) store4(O + c * p.so_t + ncol + 16 * jj + 4 * g, oacc[jj][bt] * inv);
            }
          }
        }
      }
      __syncthreads();
    }
    if (dst) {
#pragma unroll
      for (int jj = 0; jj < NTW; ++jj)
#pragma unroll
        for (int t = 0; t < NFT; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) dst[(int64_t)(16 * t + 4 * g + r) * p.dv + ncol + 16 * jj + col] = S[jj][t][r];
    }
  }
}

// Start states of segments 1..nseg-1 from the local end states (in place):
//   start(s) = e^{lam(s-1)} start(s-1) + local(s-1),  start(0) = s_init,
// the composition of affine maps of [SSM] §4.2 with a scalar decay.  Optionally
// copies s_init to `init_copy` first (used when s_init aliases s_final).
static __global__ __launch_bounds__(256) void combine_kernel(float *ws_state, const float *ws_lam, const float *s_init,
                                                      float *init_copy, int64_t BH, int64_t BLK, int nseg) {
  const int64_t bh = blockIdx.y;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= BLK) return;
  float cur = s_init ? s_init[bh * BLK + e] : 0.f;
  if (init_copy) init_copy[bh * BLK + e] = cur;
  for (int s = 1; s < nseg; ++s) {
    const int64_t slot = (int64_t)(s - 1) * BH + bh;
    const float loc = ws_state[slot * BLK + e];
    cur = expf(ws_lam[slot]) * cur + loc;
    ws_state[slot * BLK + e] = cur;
  }
}

}  // namespace hm
