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

// One wave per 16-column value tile.
constexpr int fwd_waves(int DW) { return DW / 16; }

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
  constexpr int NW = fwd_waves(DW);   // waves; wave w owns value tile w
  constexpr int NT = NW * 64;
  constexpr int NCT = C / 16;         // token tiles per chunk
  constexpr int NFH = FH / 16;        // feature tiles per half of phi
  constexpr int NFT = F / 16;         // feature tiles
  constexpr int KD = DK / M::KS;      // featurize K-steps (contiguous order)
  constexpr int KF = M::steps(NFT);   // K-steps over F (tile order)
  constexpr int KC = M::steps(NCT);   // K-steps over the chunk (tile order)
  constexpr int EPL = M::EPL;         // operand elements per lane
  constexpr int PAD = M::PAD;
  constexpr int LDW = DK + PAD, LDQ = F + PAD, LDC = C + PAD;
  constexpr bool FULL = MODE == MODE_FULL;
  constexpr int NTASK = FULL ? 2 * NCT : NCT;  // featurize tasks: (q|k, token tile)
  constexpr int TPW = (NTASK + NW - 1) / NW;   // consecutive tasks per wave
  constexpr int KVL = EPL == 8 ? 1 : 4;        // K-steps of the v re-layout per tile
  constexpr int TPF = NT >= F ? NT / F : 1;    // threads per feature row in the z update
  constexpr float L2E = 1.4426950408889634f;
  static_assert(DW % 16 == 0 && NW >= 1 && NW <= 8, "value tile split");
  static_assert(DK % M::KS == 0 && F % M::KS == 0, "K multiples");
  static_assert(C % TPF == 0, "z update mapping");

  __shared__ __align__(16) T sWq[FULL ? FH * LDW : 8];  // W^T: sW[f][d] = W[d][f]
  __shared__ __align__(16) T sWk[FH * LDW];
  __shared__ __align__(16) T sKt[F * LDC];                // decay-weighted phi(k)^T, tile order
  __shared__ __align__(16) T sQ[FULL ? C * LDQ : 8];      // phi(q) (unnormalized), tile order
  __shared__ __align__(16) T sP[FULL ? C * LDC : 8];      // masked decayed scores, tile order
  __shared__ __align__(16) double sL[2][C];               // inclusive log-decay prefix, float64
  __shared__ __align__(16) float seL[2][C];
  __shared__ __align__(16) float seK[2][C];
  __shared__ float sLast[2];
  __shared__ __align__(16) float sDenPart[NCT][C];
  __shared__ __align__(16) float sDenInter[C];
  __shared__ __align__(16) float sZ[F];

  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, col = lane & 15, g = lane >> 4;

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
  const int ncol = half * DW + 16 * wv;  // first value column of this wave
  const int64_t BLK = (int64_t)F * p.dv + F;

  const T *Q = (const T *)p.q + b * p.sq_b + h * p.sq_h;
  const T *K = (const T *)p.k + b * p.sk_b + h * p.sk_h;
  const T *V = (const T *)p.v + b * p.sv_b + h * p.sv_h;
  T *O = (T *)p.o + b * p.so_b + h * p.so_h;
  const float *DT = DECAY ? p.dt + b * p.sdt_b + h * p.sdt_h : nullptr;
  const float expA = DECAY ? expf(p.a_log[h]) : 1.f;

  // Featurize tasks of this wave: tasks wv*TPW .. wv*TPW+TPW-1 (q tiles first).
  auto task_ok = [&](int i) { return wv * TPW + i < NTASK; };
  auto task_isq = [&](int i) { return FULL && wv * TPW + i < NCT; };
  auto task_tile = [&](int i) { return (wv * TPW + i) % NCT; };

  // W^T into LDS: sW[f][d] = W[d][f]
  {
    const T *wk = (const T *)p.wk + h * p.sw_h;
    for (int i = tid; i < DK * FH; i += NT) sWk[(i % FH) * LDW + i / FH] = wk[i];
    if constexpr (FULL) {
      const T *wq = (const T *)p.wq + h * p.sw_h;
      for (int i = tid; i < DK * FH; i += NT) sWq[(i % FH) * LDW + i / FH] = wq[i];
    }
  }

  // Start state.
  f32x4 S[NFT];
  {
    const float *st = nullptr;
    if constexpr (FULL) {
      if (seg == 0) st = p.s_start0 ? p.s_start0 + bh * BLK : nullptr;
      else st = p.ws_state + ((int64_t)(seg - 1) * BH + bh) * BLK;
    }
#pragma unroll
    for (int t = 0; t < NFT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        S[t][r] = st ? st[(int64_t)(16 * t + 4 * g + r) * p.dv + ncol + col] : 0.f;
    for (int i = tid; i < F; i += NT) sZ[i] = st ? st[(int64_t)F * p.dv + i] : 0.f;
  }

  // Per-lane byte offsets of the global rows this lane reads (32-bit; the chunk
  // and tile bases are wave-uniform).
  uint32_t xoff[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i)
    xoff[i] = (uint32_t)(((int64_t)(16 * task_tile(i) + col) * (task_isq(i) ? p.sq_t : p.sk_t) + EPL * g) * sizeof(T));
  const uint32_t voff = (uint32_t)(((int64_t)col * p.sv_t + ncol + (EPL == 8 ? 8 * g : g)) * sizeof(T));
  const int64_t vtile = 16 * p.sv_t;  // elements between token tiles of v

  // Prefetch registers for one chunk.
  frag xf[TPW][KD];
  frag vf[NCT][KVL];
  float dtn = 0.f;
  auto load_chunk = [&](int64_t tc) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      if (!task_ok(i)) continue;
      const bool isq = task_isq(i);
      const T *base = (isq ? Q : K) + tc * (isq ? p.sq_t : p.sk_t);
      const bool ok = tc + 16 * task_tile(i) + col < t1;
#pragma unroll
      for (int s = 0; s < KD; ++s)
        xf[i][s] = ok ? M::ld_contig(at(base, xoff[i]) + s * M::KS, 0) : zfrag<frag>();
    }
#pragma unroll
    for (int bt = 0; bt < NCT; ++bt) {
      const T *base = V + (tc * p.sv_t + bt * vtile);
      const bool ok = tc + 16 * bt + col < t1;
      if constexpr (EPL == 8) {
        vf[bt][0] = (ok && g < 2) ? M::ld_contig(at(base, voff), 0) : zfrag<frag>();
      } else {
#pragma unroll
        for (int s = 0; s < KVL; ++s) vf[bt][s] = ok ? at(base, voff)[4 * s] : 0.f;
      }
    }
    if constexpr (DECAY) {
      if (wv == 0) dtn = tc + lane < t1 ? DT[(tc + lane) * p.sdt_t] : 0.f;
    }
  };

  // Wave 0: decay factors of one chunk into buffer `bufi`.  The prefix sums are
  // carried in float64: differences L_c - L_c' of large prefix sums would lose
  // ~|L| * 2^-24 in float32, and |L| reaches the thousands under strong decay.
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

  // Loop-invariant selector operands of the re-layout products.
  frag vsel[KVL];
#pragma unroll
  for (int s = 0; s < KVL; ++s) {
    if constexpr (EPL == 8) vsel[s] = M::select([&](int e) { return 8 * g + e == col; });
    else vsel[s] = M::select([&](int) { return 4 * s + g == col; });
  }
  constexpr int NKS = EPL == 8 ? 2 : 4;
  frag ksel[NKS];
#pragma unroll
  for (int x = 0; x < NKS; ++x) {
    if constexpr (EPL == 8) ksel[x] = M::select([&](int e) { return 16 * (e >> 2) + 4 * g + (e & 3) == 16 * x + col; });
    else ksel[x] = M::select([&](int) { return 4 * g + x == col; });
  }

  const int64_t nch = t1 > t0 ? (t1 - t0 + C - 1) / C : 0;
  if (nch > 0) {
    load_chunk(t0);
    if (wv == 0) decay(t0, 0);
  }

  for (int64_t ci = 0; ci < nch; ++ci) {
    const int buf = (int)(ci & 1);
    const int64_t tc = t0 + ci * C;
    __syncthreads();  // decay[buf] visible; previous chunk's LDS readers done

    // v tile rows -> accumulator layout: lane (g, col n) holds v[16bt + 4g + r][n]
    frag vfr[KC];
    {
      f32x4 vacc[NCT];
#pragma unroll
      for (int bt = 0; bt < NCT; ++bt) {
        vacc[bt] = zero4();
#pragma unroll
        for (int s = 0; s < KVL; ++s) vacc[bt] = M::mma(vf[bt][s], vsel[s], vacc[bt]);
      }
#pragma unroll
      for (int s = 0; s < KC; ++s) vfr[s] = M::from_acc(vacc, s);
    }

    // ---- phase A: featurize (q tasks -> sQ, den_inter; k tasks -> kf, sKt)
    f32x4 u[TPW][NFH];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      if (!task_ok(i)) continue;
      const T *sW = task_isq(i) ? sWq : sWk;
#pragma unroll
      for (int t = 0; t < NFH; ++t) {
        frag wa[KD];
#pragma unroll
        for (int s = 0; s < KD; ++s) wa[s] = M::ld_contig(sW + (16 * t + col) * LDW + s * M::KS, g);
        u[i][t] = zero4();
#pragma unroll
        for (int s = 0; s < KD; ++s) u[i][t] = M::mma(wa[s], xf[i][s], u[i][t]);
      }
    }
    if (ci + 1 < nch) load_chunk(tc + C);  // next chunk's q, k, v, dt (registers now free)

    frag kf[TPW][KF];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      if (!task_ok(i)) continue;
      const int bt = task_tile(i);
      // softmax over [u, -u] for token column col; max|u| is the max of both halves
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
      if (task_isq(i)) {
        // phi(q) is used unnormalized: a positive per-query factor multiplies both
        // o's numerator and denominator and cancels exactly.
        const int cr = 16 * bt + col;
        float dz = 0.f;
#pragma unroll
        for (int t = 0; t < NFT; ++t) {
          ph[t] = round4(ph[t], T{});
          store4(&sQ[cr * LDQ + M::tpos(16 * t + 4 * g)], ph[t]);
          const f32x4 z4 = *reinterpret_cast<const f32x4 *>(&sZ[16 * t + 4 * g]);
          dz += ph[t][0] * z4[0] + ph[t][1] * z4[1] + ph[t][2] * z4[2] + ph[t][3] * z4[3];
        }
        dz = group_sum(dz);
        if (g == 0) sDenInter[cr] = DECAY ? dz * seL[buf][cr] : dz;
      } else {
        float inv = 1.f / group_sum(sum);
        if constexpr (!DECAY) {
          if (tc + 16 * bt + col >= t1) inv = 0.f;  // rows past the end contribute nothing
        }
#pragma unroll
        for (int t = 0; t < NFT; ++t) ph[t] *= inv;
#pragma unroll
        for (int s = 0; s < KF; ++s) kf[i][s] = M::from_acc(ph, s);
        f32x4 w4;
        if constexpr (DECAY) w4 = *reinterpret_cast<const f32x4 *>(&seK[buf][16 * bt + 4 * g]);
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
          store4(&sKt[(16 * uo + col) * LDC + M::tpos(16 * bt + 4 * g)], acc);
        }
      }
    }
    __syncthreads();

    // ---- phase B: score tiles (k-task owners), z update, inter read-out, state update
    if constexpr (FULL) {
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        if (!task_ok(i) || task_isq(i)) continue;
        const int a = task_tile(i);  // rows c' of this wave's tiles
#pragma unroll
        for (int bt = 0; bt < NCT; ++bt) {
          const int cc = 16 * bt + col;
          if (bt < a) {
            store4(&sP[cc * LDC + M::tpos(16 * a + 4 * g)], zero4());
            continue;
          }
          frag bq[KF];
#pragma unroll
          for (int s = 0; s < KF; ++s) bq[s] = M::ld_tile(&sQ[cc * LDQ], s, g);
          f32x4 acc = zero4();
#pragma unroll
          for (int s = 0; s < KF; ++s) acc = M::mma(kf[i][s], bq[s], acc);
          f32x4 w;
          double lc = 0.0;
          if constexpr (DECAY) lc = sL[buf][cc];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int cp = 16 * a + 4 * g + r;
            float x = cp <= cc ? acc[r] : 0.f;
            if constexpr (DECAY) {
              if (cp <= cc) x *= __expf((float)(lc - sL[buf][cp]));
            }
            w[r] = x;
          }
          w = round4(w, T{});
          store4(&sP[cc * LDC + M::tpos(16 * a + 4 * g)], w);
          const float ds = group_sum(w[0] + w[1] + w[2] + w[3]);
          if (g == 0) sDenPart[a][cc] = ds;
        }
      }
    }
    {
      const float el = sLast[buf];
      for (int f = tid / TPF; f < F; f += NT / TPF) {
        const int part = tid % TPF;
        float zs = 0.f;
        const T *row = &sKt[f * LDC + part * (C / TPF)];
#pragma unroll
        for (int c = 0; c < C / TPF; ++c) zs += (float)row[c];
#pragma unroll
        for (int off = 1; off < TPF; off <<= 1) zs += __shfl_xor(zs, off);
        if (part == 0) sZ[f] = DECAY ? el * sZ[f] + zs : sZ[f] + zs;
      }
    }
    f32x4 oacc[NCT];
    if constexpr (FULL) {
      frag sfr[KF];
#pragma unroll
      for (int s = 0; s < KF; ++s) sfr[s] = M::from_acc(S, s);
      frag bq[NCT][KF];
#pragma unroll
      for (int bt = 0; bt < NCT; ++bt)
#pragma unroll
        for (int s = 0; s < KF; ++s) bq[bt][s] = M::ld_tile(&sQ[(16 * bt + col) * LDQ], s, g);
#pragma unroll
      for (int bt = 0; bt < NCT; ++bt) {
        oacc[bt] = zero4();
#pragma unroll
        for (int s = 0; s < KF; ++s) oacc[bt] = M::mma(sfr[s], bq[bt][s], oacc[bt]);
        if constexpr (DECAY) oacc[bt] *= seL[buf][16 * bt + col];
      }
    }
    if constexpr (DECAY) {
      const float el = sLast[buf];
#pragma unroll
      for (int t = 0; t < NFT; ++t) S[t] *= el;
    }
    {
      frag ak[NFT][KC];
#pragma unroll
      for (int t = 0; t < NFT; ++t)
#pragma unroll
        for (int s = 0; s < KC; ++s) ak[t][s] = M::ld_tile(&sKt[(16 * t + col) * LDC], s, g);
#pragma unroll
      for (int t = 0; t < NFT; ++t)
#pragma unroll
        for (int s = 0; s < KC; ++s) S[t] = M::mma(ak[t][s], vfr[s], S[t]);
    }
    __syncthreads();

    // ---- phase C: intra-chunk read-out, normalize, store; next chunk's decay
    if constexpr (FULL) {
      frag bp[NCT][M::steps_upto(NCT - 1)];
#pragma unroll
      for (int bt = 0; bt < NCT; ++bt)
#pragma unroll
        for (int s = 0; s < M::steps_upto(bt); ++s) bp[bt][s] = M::ld_tile(&sP[(16 * bt + col) * LDC], s, g);
#pragma unroll
      for (int bt = 0; bt < NCT; ++bt) {
        const int cc = 16 * bt + col;
#pragma unroll
        for (int s = 0; s < M::steps_upto(bt); ++s) oacc[bt] = M::mma(vfr[s], bp[bt][s], oacc[bt]);
        const int64_t c = tc + cc;
        if (c < t1) {
          float den = sDenInter[cc];
#pragma unroll
          for (int a = 0; a <= bt; ++a) den += sDenPart[a][cc];
          store4(O + c * p.so_t + ncol + 4 * g, oacc[bt] * (1.f / den));
        }
      }
    }
    if (wv == 0 && ci + 1 < nch) decay(tc + C, buf ^ 1);
  }
  __syncthreads();

  // Write the end state.
  float *dst = nullptr;
  if constexpr (FULL) {
    if (seg == p.nseg - 1) dst = p.s_final ? p.s_final + bh * BLK : nullptr;
  } else {
    dst = p.ws_state + ((int64_t)seg * BH + bh) * BLK;
    if (half == 0 && tid == 0) p.ws_lam[(int64_t)seg * BH + bh] = (float)lam;
  }
  if (dst) {
#pragma unroll
    for (int t = 0; t < NFT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(int64_t)(16 * t + 4 * g + r) * p.dv + ncol + col] = S[t][r];
    if (half == 0)
      for (int i = tid; i < F; i += NT) dst[(int64_t)F * p.dv + i] = sZ[i];
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
