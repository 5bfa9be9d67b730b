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
// Work split (all matrix products are 16x16 MFMA tiles): four feature waves and
// NS state waves; feature wave w and state wave w run on the same SIMD, so each SIMD
// interleaves softmax VALU work with MFMA work.
//   * feature wave w featurizes token tile w of the chunk for q and k, stores
//     phiQ, phiK^T (and phiK of tile 0) in LDS, then forms its share of the score
//     tiles and of z; feature waves run one chunk ahead of the state waves;
//   * state wave s owns value columns [32s, 32s + 32) of S in accumulators: the
//     read-out, the output rows and the state update for those columns.
// Layout choices:
//   * q, k and v rows are read from HBM straight into operand fragments; v is
//     turned into the accumulator layout by one MFMA against a 0/1 selector, and
//     phiK into phiK^T the same way;
//   * S is fed back as the A operand of the read-out in tile order (hm_device.hpp);
//   * output rows are staged in LDS and leave as whole rows;
//   * the next chunk's q, k, v, dt are loaded into registers while the current
//     chunk computes.
#pragma once

#include "hm_device.hpp"

namespace hm {

constexpr int CHUNK = 64;
// MODE_TRAIN is the full pass that also saves what the backward pass reads;
// MODE_ROPE, or'ed into any of them, turns phi(q) and phi(k) by their positions
// (rotary encoding, HedgeMamba explainer §5.2 step 3) before they are used.
enum { MODE_FULL = 0, MODE_LOCAL = 1, MODE_TRAIN = 2, MODE_ROPE = 4 };

constexpr int MAX_FUSE = 4;  // most slots the full pass composes into one start state

struct FwdParams {
  const void *q, *k, *v, *wq, *wk;
  const float *dt, *a_log;
  const float *s_start0;  // start state of segment 0 (NULL = zeros)
  float *s_final;         // written by the last segment (NULL = not written)
  void *o;
  float *ws_state;        // [(nseg-1)*lsub][B*H][F*dv+F]: local end states, then start states
  float *ws_lam;          // [(nseg-1)*lsub][B*H]: summed log-decay of each slot's tokens
  int64_t B, H, n, dv;
  int64_t sq_b, sq_h, sq_t, sk_b, sk_h, sk_t, sv_b, sv_h, sv_t, so_b, so_h, so_t;
  int64_t sw_h, sdt_b, sdt_h, sdt_t;
  const void *gate;       // optional gate pre-activation, o's shape (NULL = none)
  int64_t sg_b, sg_h, sg_t;
  // MODE_TRAIN only: checkpoints, the float32 state (S then z, state layout) at the
  // start of every ck_every-th chunk [B*H][ceil(nchunks / ck_every)][F*dv + F], the
  // per-token denominator [B*H][n] (unnormalized phi(q), as used for o) and the
  // output before any gate [B*H][n][dv] in float32
  float *save_ck, *save_den, *save_o;
  int64_t nchunks;
  int64_t ck_every;       // chunks per checkpoint (the backward's chunk ranges)
  int64_t nck;            // checkpoints per (b, h)
  int64_t seg_len;        // tokens per segment, a multiple of CHUNK
  int64_t nitems;         // (b,h,segment) items in this launch
  int nseg;               // segments of the whole sequence
  int nseg_run;           // segments covered by this launch (nseg, or the slots for MODE_LOCAL)
  // The segment pass may cut every segment into lsub pieces (slots of seg_len/lsub
  // tokens, one workgroup each).  The full pass takes the start state of segment
  // s >= 1 from slot s*lsub-1, composing on load the nfuse slots that end there.
  int lsub;
  int nfuse;              // 1 .. MAX_FUSE; 1 for MODE_TRAIN
  int dsplit;             // workgroups per item, each owning dv/dsplit columns
  int rope_dims;          // MODE_ROPE: rotated features (multiple of 32, <= F)
  float rope_base;
  const int64_t *rope_pos0;  // MODE_ROPE: position of token 0 per batch row (NULL = 0)
};

template <typename F> __device__ __forceinline__ F zfrag() { return F{}; }

// One 16-byte piece of output row times SiLU of the matching gate piece: eight
// bf16 or four float values, held as the raw 16 bytes.
__device__ __forceinline__ f32x4 gate_piece(f32x4 o, f32x4 g, bf16) {
  const bf16x8 ov = __builtin_bit_cast(bf16x8, o), gv = __builtin_bit_cast(bf16x8, g);
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)((float)ov[e] * silu_f32((float)gv[e]));
  return __builtin_bit_cast(f32x4, r);
}
__device__ __forceinline__ f32x4 gate_piece(f32x4 o, f32x4 g, float) {
  f32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = o[e] * silu_f32(g[e]);
  return r;
}

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

// CH is the chunk length: 64, or 128 (full pass only).  The waves always work on
// 64-token blocks.  With 128-token chunks the two blocks of a chunk are read out
// against the state at the chunk's start, the second block's intra-chunk part
// also takes its scores against the first block's keys (16 off-diagonal tiles),
// and the state update of both blocks is applied once the chunk has been read out
// (in order: S = e^{L_1}(e^{L_0} S + K0~^T V0) + K1~^T V1, the same sums).
// Decay factors of one 64-token block by one wave (lane = token): the inclusive
// log-decay prefix L, e^{L}, e^{L_last - L} (0 past the sequence's end) and
// e^{L_last}; lam accumulates L_last.  The prefix sums are carried in float64:
// differences L_c - L_c' of large prefix sums would lose ~|L| * 2^-24 in float32,
// and |L| reaches the thousands.
template <bool DECAY>
__device__ __forceinline__ void decay_factors(double *sLb, float *seLb, float *seKb, float &sLastb, bool valid,
                                              float dtn, float expA, double &lam, int lane) {
  if constexpr (DECAY) {
    const double L = wave_inclusive_scan(valid ? (double)(-softplus_f32(dtn) * expA) : 0.0);
    const double Ll = lane63(L);
    sLb[lane] = L;
    seLb[lane] = __expf((float)L);
    seKb[lane] = valid ? __expf((float)(Ll - L)) : 0.f;
    if (lane == 0) sLastb = __expf((float)Ll);
    lam += Ll;
  } else {
    if (lane == 0) sLastb = 1.f;
  }
}

template <typename T, int DK, int FH, int DW, bool DECAY, int MODE, int CH>
__global__ __launch_bounds__(fwd_waves(DW) * 64) void fwd_kernel(const FwdParams p) {
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int C = CHUNK;                 // block length
  constexpr int MB = CH / C;               // blocks per chunk
  static_assert(MB == 1 || (MB == 2 && (MODE & 3) == MODE_FULL), "128-token chunks: full pass without saves");
  constexpr int NKT = MB == 1 ? 2 : 3;     // phi(k)^T block buffers (a chunk's two blocks stay until its update)
  constexpr int NDB = MB == 1 ? 3 : 4;     // decay-factor block buffers
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
  constexpr int LDW = DK + PAD, LDQ = F + PAD, LDC = C + PAD, LDO = DW + 32 / (int)sizeof(T);
  constexpr int LDP = MB * C + PAD;        // score rows: the chunk's keys
  constexpr bool FULL = (MODE & 3) != MODE_LOCAL;
  constexpr bool SAVE = (MODE & 3) == MODE_TRAIN;
  constexpr bool ROPE = (MODE & MODE_ROPE) != 0;
  constexpr int TPF_ = FULL ? 2 : 1;       // featurize tasks per feature wave
  constexpr int KVL = EPL == 8 ? 1 : 4;    // K-steps of the v re-layout per tile
  constexpr float L2E = 1.4426950408889634f;
  static_assert(NCT == 4, "four token tiles per chunk");
  static_assert(NTW >= 1 && NTW <= 2 && NTW * 16 * NS == DW, "value tile split");
  static_assert(DK % M::KS == 0 && F % M::KS == 0, "K multiples");

  __shared__ __align__(16) T sWq[FULL ? FH * LDW : 8];    // W^T: sW[f][d] = W[d][f]
  __shared__ __align__(16) T sKt[NKT][F * LDC];             // decay-weighted phi(k)^T per block, tile order
  // W_k^T is read only before the block loop (into registers): with a third phi(k)^T
  // buffer (first written at block 2) it shares that buffer
  __shared__ __align__(16) T sWk_own[MB == 1 ? FH * LDW : 8];
  static_assert(MB == 1 || FH * LDW <= F * LDC, "W_k^T fits the shared buffer");
  T *const sWk = MB == 1 ? sWk_own : sKt[NKT - 1];
  __shared__ __align__(16) T sQ[FULL ? 2 : 1][FULL ? C * LDQ : 8];  // phi(q) (unnormalized), tile order
  __shared__ __align__(16) T sK0[FULL ? 16 * LDQ : 8];              // phi(k) of token tile 0, tile order
  __shared__ __align__(16) T sP[FULL ? C * LDP : 8];                 // masked decayed scores, keys of the chunk
  __shared__ __align__(16) T sO[FULL ? C * LDO : 8];                 // normalized output rows
  __shared__ __align__(16) T sG[FULL && MB == 1 ? C * DW : 8];       // gate rows, in store-piece order
  __shared__ __align__(16) double sL[NDB][C];               // inclusive log-decay prefix per block, float64
  __shared__ __align__(16) float seL[NDB][C];
  __shared__ __align__(16) float seK[NDB][C];
  __shared__ float sLast[NDB];
  __shared__ __align__(16) float sDenPart[MB * NCT][C];     // score row sums per key tile of the chunk
  __shared__ __align__(16) float sDenInter[2][C];
  __shared__ __align__(16) float sZ[2][F];                  // z after each chunk (by chunk parity)
  __shared__ __align__(16) double sRev[ROPE ? F / 2 : 1];   // rotation rate of each feature pair

  const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, g = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: lets the compiler keep it scalar
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
  double pos_b = 0.0;  // position of token 0 of this sequence
  if constexpr (ROPE) {
    if (tid < p.rope_dims / 2) sRev[tid] = rope_rev(tid, p.rope_dims, p.rope_base);
    pos_b = p.rope_pos0 ? (double)p.rope_pos0[b] : 0.0;
  }

  // W^T into LDS: sW[f][d] = W[d][f].  W is read as 16-byte vectors, all of them
  // issued before the first LDS write.
  {
    constexpr int EP = 16 / (int)sizeof(T);
    constexpr int NV = DK * FH / EP;                 // vectors per matrix
    constexpr int VPT = (NV + NT - 1) / NT;          // vectors per thread
    typedef T tvec __attribute__((ext_vector_type(16 / sizeof(T))));
    const T *wk = (const T *)p.wk + h * p.sw_h;
    const T *wq = (const T *)p.wq + h * p.sw_h;
    tvec vk[VPT], vq[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int v = tid + i * NT;
      if (v < NV) {
        vk[i] = *reinterpret_cast<const tvec *>(wk + v * EP);
        if constexpr (FULL) vq[i] = *reinterpret_cast<const tvec *>(wq + v * EP);
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int v = tid + i * NT;
      if (v < NV) {
        const int d = v * EP / FH, f0 = v * EP % FH;
#pragma unroll
        for (int e = 0; e < EP; ++e) {
          sWk[(f0 + e) * LDW + d] = vk[i][e];
          if constexpr (FULL) sWq[(f0 + e) * LDW + d] = vq[i][e];
        }
      }
    }
  }

  // start state: s_start0 for segment (or slot) 0 in both passes; the segment pass
  // starts later slots from zero.  The full pass reads the start state of a later
  // segment from the workspace: slot seg*lsub-1, or the composition of the nfuse
  // slots ending there, start = e^{lam(u)} start + local(u) ([SSM] §4.2).
  const float *st = nullptr;
  int nst = 1;  // slots composed into the start state
  if (seg == 0) st = p.s_start0 ? p.s_start0 + bh * BLK : nullptr;
  else if constexpr (FULL) {
    nst = p.nfuse;
    st = p.ws_state + ((int64_t)(seg * p.lsub - nst) * BH + bh) * BLK;
  }
  // slot u of the composition: its state and e^{lam(u)} (u = 1 .. nst-1)
  auto slot_state = [&](int u) { return st + (int64_t)u * BH * BLK; };
  auto slot_decay = [&](int u) { return expf(p.ws_lam[(int64_t)(seg * p.lsub - nst + u) * BH + bh]); };
  const int64_t nch = t1 > t0 ? (t1 - t0 + C - 1) / C : 0;
  float *dst = nullptr;  // end state destination
  if constexpr (FULL) {
    if (seg == p.nseg - 1) dst = p.s_final ? p.s_final + bh * BLK : nullptr;
  } else {
    dst = p.ws_state + ((int64_t)seg * BH + bh) * BLK;
  }

  // The two roles run separate loops with the same two barriers per iteration j:
  //   half A: feature waves featurize chunk j (phiQ, phiK, phiK^T, den_inter);
  //           state waves read out chunk j-1 (inter and intra parts), normalize, store;
  //   half B: feature waves form chunk j's score tiles and advance z;
  //           state waves advance S over chunk j-1.
  // Wave w of each role runs on SIMD w % 4, so every SIMD pairs the softmax VALU
  // work of one feature wave with the MFMA work of one state wave.
  if (fwave) {
    // ---------------------------------------------------------------- feature waves
    // Wave w featurizes token tile w of the chunk: q (FULL only) and k.
    constexpr int XQ = 0, XK = TPF_ - 1;  // xf slots of the q and k rows
    uint32_t xoff[TPF_];
#pragma unroll
    for (int i = 0; i < TPF_; ++i)
      xoff[i] = (uint32_t)(((int64_t)(16 * wv + col) * (FULL && i == XQ ? p.sq_t : p.sk_t) + EPL * g) * sizeof(T));

    // z: column 0 of an [F x 16] accumulator block, feature tiles dealt to the
    // feature waves (wave w owns tiles ZT*w .. ZT*w + ZT-1); a copy of each chunk's
    // end value goes to sZ for the inter-chunk denominators.
    constexpr int ZT = (NFT + 3) / 4;
    f32x4 Z[ZT];
    // The intra read-out of token tile b (b even) takes K-steps over tiles b and
    // b+1; score tile (b+1, b) lies above the diagonal and must read as zero.  It is
    // zeroed once where the last block of a chunk keeps its diagonal scores, and, with
    // two blocks per chunk, again at every first block (the second block's
    // off-diagonal scores overwrite those places).
    auto zero_above = [&](int kt0) {
      if constexpr (FULL && EPL == 8) {
#pragma unroll
        for (int b2 = 0; b2 < NCT; b2 += 2)
          store4(&sP[(16 * b2 + col) * LDP + M::tpos(16 * (kt0 + b2 + 1) + 4 * g)], zero4());
      }
    };
    if (wv == 0) zero_above(NCT * (MB - 1));

    frag xf[TPF_][KD];
    auto load_xi = [&](int64_t tc, int i) {
      const bool ok = tc + 16 * wv + col < t1;
      const T *base = FULL && i == XQ ? Q + tc * p.sq_t : K + tc * p.sk_t;
#pragma unroll
      for (int s = 0; s < KD; ++s) xf[i][s] = ok ? M::ld_contig(at(base, xoff[i]) + s * M::KS, 0) : zfrag<frag>();
    };
    auto load_x = [&](int64_t tc) {
#pragma unroll
      for (int i = 0; i < TPF_; ++i) load_xi(tc, i);
    };
    float dtn = 0.f;
    auto load_dt = [&](int64_t tc) {
      if constexpr (DECAY) dtn = tc + lane < t1 ? DT[(tc + lane) * p.sdt_t] : 0.f;
    };
    // Wave 2 (one of the two with two score tiles): decay factors of the chunk starting
    // at tc into buffer `bufi`
    double lam = 0.0;
    auto decay = [&](int64_t tc, int bufi) {
      decay_factors<DECAY>(sL[bufi], seL[bufi], seK[bufi], sLast[bufi], tc + lane < t1, dtn, expA, lam, lane);
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
      if (FULL && wv == 2) {
        load_dt(t0);
        decay(t0, 0);
        if (nch > 1) load_dt(t0 + C);
      }
    }
    // z of the start state into sZ[1], every slot's value requested before any is
    // combined (the feature waves set the pace of the whole workgroup)
    for (int i = tid; i < F; i += 4 * 64) {
      float zs[MAX_FUSE];
#pragma unroll
      for (int u = 0; u < MAX_FUSE; ++u) zs[u] = st && u < nst ? slot_state(u)[(int64_t)F * p.dv + i] : 0.f;
      float x = zs[0];
#pragma unroll
      for (int u = 1; u < MAX_FUSE; ++u)
        if (u < nst) x = slot_decay(u) * x + zs[u];
      sZ[1][i] = x;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ZT; ++i) {
      const int t = ZT * wv + i;
      Z[i] = t < NFT && col == 0 ? *reinterpret_cast<const f32x4 *>(&sZ[1][16 * t + 4 * g]) : zero4();
    }

    // W_k^T fragments stay in registers for the whole segment (A operands); W_q^T
    // is read from LDS per chunk.
    frag wk[NFH][KD];
#pragma unroll
    for (int t = 0; t < NFH; ++t)
#pragma unroll
      for (int s = 0; s < KD; ++s) wk[t][s] = M::ld_contig(sWk + (16 * t + col) * LDW + s * M::KS, g);

    // One token's features into a tile-order LDS row: the bf16 operand fragments
    // are already in that order (one 16-byte write each); f32 rows take the
    // accumulator tiles.
    auto store_frags = [&](T *row, const frag *fr, const f32x4 *ph) {
      if constexpr (EPL == 8) {
#pragma unroll
        for (int s = 0; s < KF; ++s) *reinterpret_cast<frag *>(row + 32 * s + 8 * g) = fr[s];
      } else {
#pragma unroll
        for (int t = 0; t < NFT; ++t) store4(row + M::tpos(16 * t + 4 * g), ph[t]);
      }
    };

    // softmax([u, -u]) of one token per lane column, shifted by max|u|: ph[t] for
    // t < NFH holds e^{u}, ph[NFH + t] holds e^{-u}; returns the row sum.
    auto features = [&](const f32x4 *u, f32x4 *ph) {
      float m = 0.f;
#pragma unroll
      for (int t = 0; t < NFH; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(u[t][r]));
      const float ml = group_max(m) * L2E;
      float sum = 0.f;
#pragma unroll
      for (int t = 0; t < NFH; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = u[t][r];
          const float ep = __builtin_amdgcn_exp2f(__builtin_fmaf(x, L2E, -ml));
          const float em = __builtin_amdgcn_exp2f(__builtin_fmaf(-x, L2E, -ml));
          ph[t][r] = ep;
          ph[NFH + t][r] = em;
          sum += ep + em;
        }
      return group_sum(sum);
    };

    // score tile (a, bt) of the block in buffers bf / df: Pt[c'][c] for c' in tile
    // a (A operand rows), c in tile bt (B operand columns), masked to c' <= c and
    // decay-weighted, into sP (row c, tile order over the chunk's keys, the block's
    // keys from key tile kt0 on); row sums into sDenPart.
    auto score_tile = [&](int a, int bt, const frag *fa, const frag *fb, int df, int kt0) {
      f32x4 acc = zero4();
#pragma unroll
      for (int s = 0; s < KF; ++s) acc = M::mma(fa[s], fb[s], acc);
      const int cc = 16 * bt + col;
      double lc = 0.0;
      if constexpr (DECAY) lc = sL[df][cc];
      f32x4 w;
      if (a == bt) {  // diagonal tile: causal mask
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int cp = 16 * a + 4 * g + r;
          float xv = cp <= cc ? acc[r] : 0.f;
          if constexpr (DECAY) {
            if (cp <= cc) xv *= __expf((float)(lc - sL[df][cp]));
          }
          w[r] = xv;
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float xv = acc[r];
          if constexpr (DECAY) xv *= __expf((float)(lc - sL[df][16 * a + 4 * g + r]));
          w[r] = xv;
        }
      }
      store4(&sP[cc * LDP + M::tpos(16 * (kt0 + a) + 4 * g)], w);
      // row sums of the weights as rounded for the product with V, so that each output
      // is an exact convex combination under one set of weights: o_t - v_t then keeps
      // its relative accuracy when a fast decay makes it small (the backward pass
      // differentiates through it)
      const float dsum = group_sum((float)(T)w[0] + (float)(T)w[1] + (float)(T)w[2] + (float)(T)w[3]);
      if (g == 0) sDenPart[kt0 + a][cc] = dsum;
    };
    // Off-diagonal score tile of a two-block chunk: keys c' in tile a of the chunk's
    // first block (decay buffer dfp), queries c in tile bt of its second block (df),
    // all c' < c: weight e^{L_c - L_c'} with L counted from the chunk's start, i.e.
    // e^{Lb1_c + (Lb0_last - Lb0_c')} with the blocks' own inclusive prefixes.
    auto score_tile_off = [&](int a, int bt, const frag *fa, const frag *fb, int df, int dfp) {
      f32x4 acc = zero4();
#pragma unroll
      for (int s = 0; s < KF; ++s) acc = M::mma(fa[s], fb[s], acc);
      const int cc = 16 * bt + col;
      f32x4 w = acc;
      if constexpr (DECAY) {
        const double lc = sL[df][cc] + sL[dfp][C - 1];
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = acc[r] * __expf((float)(lc - sL[dfp][16 * a + 4 * g + r]));
      }
      store4(&sP[cc * LDP + M::tpos(16 * a + 4 * g)], w);
      const float dsum = group_sum((float)(T)w[0] + (float)(T)w[1] + (float)(T)w[2] + (float)(T)w[3]);
      if (g == 0) sDenPart[a][cc] = dsum;
    };
    frag kf_prev[MB > 1 ? KF : 1];  // phi(k) of this wave's tile of the chunk's first block

    for (int64_t j = 0; j <= nch; ++j) {
      const int64_t tf = t0 + j * C;
      const int bf = (int)(j & 1);
      const int kb = (int)(j % NKT);
      const int df = (int)(j % NDB);
      const int bi = MB == 1 ? 0 : (int)(j % MB);  // block within its chunk (segments start on chunk bounds)
      const int cr = 16 * wv + col;  // this lane's token row in the block
      frag qf[FULL ? KF : 1], kf[KF];  // phiQ, phiK of token tile wv (tile order)
      // ---- half A: featurize token tile wv of chunk j
      if constexpr (SAVE) {
        if (j < nch && wv == 2 && half == 0 && (tf / C) % p.ck_every == 0) {
          const float *zp = sZ[(j + 1) & 1];  // z at the start of chunk j, a checkpoint
          float *zs = p.save_ck + (bh * p.nck + tf / C / p.ck_every) * BLK + (int64_t)F * p.dv;
          for (int i = lane; i < F; i += 64) zs[i] = zp[i];
        }
      }
      if (j < nch) {
        f32x4 uq[NFH], uk[NFH];
#pragma unroll
        for (int t = 0; t < NFH; ++t) {
          uk[t] = zero4();
#pragma unroll
          for (int s = 0; s < KD; ++s) uk[t] = M::mma(wk[t][s], xf[XK][s], uk[t]);
        }
        // the next chunk's rows go out in two groups: k's once its projection has
        // consumed them, q's after the inter-chunk denominators (issuing all eight
        // loads at one point measured 3-5 % slower)
        if (j + 1 < nch && FULL) load_xi(tf + C, XK);
        if constexpr (FULL) {
#pragma unroll
          for (int t = 0; t < NFH; ++t) {
            frag wq[KD];
#pragma unroll
            for (int s = 0; s < KD; ++s) wq[s] = M::ld_contig(sWq + (16 * t + col) * LDW + s * M::KS, g);
            uq[t] = zero4();
#pragma unroll
            for (int s = 0; s < KD; ++s) uq[t] = M::mma(wq[s], xf[XQ][s], uq[t]);
          }
        }
        if (j + 1 < nch && !FULL) load_x(tf + C);
        f32x4 ph[NFT];
        if constexpr (FULL) {
          // phi(q) unnormalized: a positive per-query factor cancels in o's ratio.
          // den_inter = e^{L_c} phiQ_c . z, with z at the end of the previous chunk.
          features(uq, ph);
          if constexpr (ROPE) rope_apply<NFT>(ph, sRev, g, pos_b + (double)(tf + cr), p.rope_dims);
#pragma unroll
          for (int s = 0; s < KF; ++s) qf[s] = M::from_acc(ph, s);
          store_frags(&sQ[bf][cr * LDQ], qf, ph);
          // z at the chunk's start: after the previous block, or (second block of a chunk)
          // after the block before that, whose buffer is rewritten only in this half B
          const float *zp = sZ[bi == 0 ? (j + 1) & 1 : j & 1];
          float dz = 0.f;
#pragma unroll
          for (int t = 0; t < NFT; ++t) {
            const f32x4 z4 = *reinterpret_cast<const f32x4 *>(zp + 16 * t + 4 * g);
#pragma unroll
            for (int r = 0; r < 4; ++r) dz = __builtin_fmaf(ph[t][r], z4[r], dz);
          }
          dz = group_sum(dz);
          if (g == 0) {
            float sc = DECAY ? seL[df][cr] : 1.f;  // e^{L} from the chunk's start
            if (MB > 1 && DECAY && bi == 1) sc *= sLast[(j - 1) % NDB];
            sDenInter[bf][cr] = dz * sc;
          }
          if (j + 1 < nch) load_xi(tf + C, XQ);
        }
        {
          float inv = __builtin_amdgcn_rcpf(features(uk, ph));
          if constexpr (!DECAY) {
            if (tf + cr >= t1) inv = 0.f;  // rows past the end contribute nothing
          }
#pragma unroll
          for (int t = 0; t < NFT; ++t) ph[t] *= inv;
          if constexpr (ROPE) rope_apply<NFT>(ph, sRev, g, pos_b + (double)(tf + cr), p.rope_dims);
#pragma unroll
          for (int s = 0; s < KF; ++s) kf[s] = M::from_acc(ph, s);
          if constexpr (FULL) {
            // phiK rows of token tile 0, for the one score tile formed from phiQ's side
            if (wv == 0) store_frags(&sK0[col * LDQ], kf, ph);
          }
          f32x4 w4;
          if constexpr (DECAY) w4 = *reinterpret_cast<const f32x4 *>(&seK[df][16 * wv + 4 * g]);
          // phiK^T tile uo (decay-weighted): lane (g, col f') gets phiK[16wv+4g+r][16uo+f'],
          // in groups of four tiles
#pragma unroll
          for (int u0 = 0; u0 < NFT; u0 += 4) {
            f32x4 tr[4];
#pragma unroll
            for (int uo = u0; uo < u0 + 4 && uo < NFT; ++uo) {
              tr[uo - u0] = zero4();
              if constexpr (EPL == 8) {
                tr[uo - u0] = M::mma(kf[uo >> 1], ksel[uo & 1], tr[uo - u0]);
              } else {
#pragma unroll
                for (int s = 4 * uo; s < 4 * uo + 4; ++s) tr[uo - u0] = M::mma(kf[s], ksel[s & 3], tr[uo - u0]);
              }
            }
#pragma unroll
            for (int uo = u0; uo < u0 + 4 && uo < NFT; ++uo) {
              if constexpr (DECAY) tr[uo - u0] *= w4;
              store4(&sKt[kb][(16 * uo + col) * LDC + M::tpos(16 * wv + 4 * g)], tr[uo - u0]);
            }
          }
        }
      }
      // The segment pass has one barrier per chunk: its state waves carry z and the
      // decay factors (see there), so the feature waves only featurize.
      if constexpr (FULL) __syncthreads();
      // ---- half B: score tiles and z over chunk j, decay of chunk j+1 (wave 2)
      if (FULL && j < nch) {
        if constexpr (FULL) {
          // Ten causal tiles (a <= b): wave w forms (w, w) from its own phiK and
          // phiQ, wave w < 3 also (w, b) for b = w+1 .. min(w+2, 3) with phiQ of
          // tile b read back, and wave 3 forms (0, 3) with phiK of tile 0 read back.
          if (wv < 3) {
            const int nb = wv < 2 ? 2 : 1;
            frag bq[2][KF];
#pragma unroll
            for (int i = 0; i < 2; ++i)
              if (i < nb) {
#pragma unroll
                for (int s = 0; s < KF; ++s) bq[i][s] = M::ld_tile(&sQ[bf][(16 * (wv + 1 + i) + col) * LDQ], s, g);
              }
            score_tile(wv, wv, kf, qf, df, NCT * bi);
#pragma unroll
            for (int i = 0; i < 2; ++i)
              if (i < nb) score_tile(wv, wv + 1 + i, kf, bq[i], df, NCT * bi);
          } else {
            frag ak[KF];
#pragma unroll
            for (int s = 0; s < KF; ++s) ak[s] = M::ld_tile(&sK0[col * LDQ], s, g);
            score_tile(wv, wv, kf, qf, df, NCT * bi);
            score_tile(0, wv, ak, qf, df, NCT * bi);
          }
          if constexpr (MB > 1) {
            if (bi == 0) {
              // first block of a chunk: keep this tile's phi(k) for the second block's
              // off-diagonal scores, and clear the places those leave above the diagonal
              if (wv == 0) zero_above(0);
#pragma unroll
              for (int s = 0; s < KF; ++s) kf_prev[s] = kf[s];
            } else {
              // second block: the 16 tiles against the first block's keys; wave w owns key
              // tile w and takes each query tile's phi(q), its own from registers
              const int dfp = (int)((j - 1) % NDB);
#pragma unroll
              for (int bt = 0; bt < NCT; ++bt) {
                frag fq[KF];
#pragma unroll
                for (int s = 0; s < KF; ++s)
                  fq[s] = bt == wv ? qf[s] : M::ld_tile(&sQ[bf][(16 * bt + col) * LDQ], s, g);
                score_tile_off(wv, bt, kf_prev, fq, df, dfp);
              }
            }
          }
        }
        // z <- e^{L_last} z + sum_c' phi~(k_c'): phi~(k)^T times a ones column
        const float el = DECAY ? sLast[df] : 1.f;
#pragma unroll
        for (int i = 0; i < ZT; ++i) {
          const int t = ZT * wv + i;
          if (t < NFT) {
            frag ak[KC];
#pragma unroll
            for (int s = 0; s < KC; ++s) ak[s] = M::ld_tile(&sKt[kb][(16 * t + col) * LDC], s, g);
            if constexpr (DECAY) Z[i] *= el;
#pragma unroll
            for (int s = 0; s < KC; ++s) Z[i] = M::mma(ak[s], ones, Z[i]);
            if (col == 0) *reinterpret_cast<f32x4 *>(&sZ[bf][16 * t + 4 * g]) = Z[i];
          }
        }
        if (wv == 2 && j + 1 < nch) {
          decay(tf + C, (int)((j + 1) % NDB));
          if (j + 2 < nch) load_dt(tf + 2 * C);
        }
      }
      __syncthreads();
    }
    if (FULL && dst && col == 0 && half == 0) {
#pragma unroll
      for (int i = 0; i < ZT; ++i) {
        const int t = ZT * wv + i;
        if (t < NFT) {
#pragma unroll
          for (int r = 0; r < 4; ++r) dst[(int64_t)F * p.dv + 16 * t + 4 * g + r] = Z[i][r];
        }
      }
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
    // v rows of the chunk, in registers.  bf16: lane (g, col) holds
    // v[token col][8g .. 8g+7] of the wave's 16*NTW columns (one 16-byte load; lanes
    // g >= 2*NTW idle), turned into each value tile's accumulator layout by a
    // selector product.  f32: lane (g, col) holds v[token col][16jj + g + 4s].
    constexpr int VJ = EPL == 8 ? 1 : NTW;
    uint32_t voff[VJ];
#pragma unroll
    for (int jj = 0; jj < VJ; ++jj)
      voff[jj] = (uint32_t)(((int64_t)col * p.sv_t + ncol + 16 * jj + (EPL == 8 ? 8 * g : g)) * sizeof(T));
    frag vf[VJ][NCT][KVL];
    auto load_v = [&](int64_t tc) {
#pragma unroll
      for (int bt = 0; bt < NCT; ++bt) {
        const T *base = V + (tc + 16 * bt) * p.sv_t;
        const bool ok = tc + 16 * bt + col < t1;
        if constexpr (EPL == 8) {
          vf[0][bt][0] = (ok && g < 2 * NTW) ? M::ld_contig(at(base, voff[0]), 0) : zfrag<frag>();
        } else {
#pragma unroll
          for (int jj = 0; jj < NTW; ++jj)
#pragma unroll
            for (int s = 0; s < KVL; ++s) vf[jj][bt][s] = ok ? at(base, voff[jj])[4 * s] : 0.f;
        }
      }
    };
    frag vsel[NTW][KVL];
#pragma unroll
    for (int jj = 0; jj < NTW; ++jj)
#pragma unroll
      for (int s = 0; s < KVL; ++s) {
        if constexpr (EPL == 8) vsel[jj][s] = M::select([&](int e) { return 8 * g + e == 16 * jj + col; });
        else vsel[jj][s] = M::select([&](int) { return 4 * s + g == col; });
      }

    // the gate rows of the chunk at ts into sG, one 16-byte piece per lane and pass
    // (no registers held while the read-out runs); in half B each lane reads back
    // the pieces it brought in
    auto issue_gate_rows = [&](int64_t ts) {
      if constexpr (FULL && MB == 1) {
        if (p.gate) {
          constexpr int EP = 16 / (int)sizeof(T), PPR = DW / EP, NIT = C * PPR / (NS * 64);
          const T *gb = (const T *)p.gate + b * p.sg_b + h * p.sg_h + ts * p.sg_t + half * DW;
#pragma unroll
          for (int it = 0; it < NIT; ++it) {
            const int i = (it * NS + sw) * 64 + lane, row = i / PPR, pc = i % PPR;
            if (ts + row < t1)
              __builtin_amdgcn_global_load_lds(
                  (const __attribute__((address_space(1))) void *)(gb + (int64_t)row * p.sg_t + pc * EP),
                  (__attribute__((address_space(3))) void *)&sG[(it * NS + sw) * 64 * EP], 16, 0, 0);
          }
        }
      }
    };

    // Segment pass: z of the segment (tiles ZTS*sw ..) lives in the state waves, and
    // one state wave (the second, when there are several) computes the decay factors,
    // one chunk ahead of the featurization
    constexpr int ZTS = (NFT + NS - 1) / NS;
    const int dwave = NS > 1 ? 1 : 0;
    f32x4 Zs[FULL ? 1 : ZTS];
    const frag ones = M::select([&](int) { return col == 0; });
    float dtn = 0.f;
    auto load_dt = [&](int64_t tc) {
      if constexpr (DECAY) dtn = tc + lane < t1 ? DT[(tc + lane) * p.sdt_t] : 0.f;
    };
    double lam = 0.0;
    auto decay = [&](int64_t tc, int bufi) {
      decay_factors<DECAY>(sL[bufi], seL[bufi], seK[bufi], sLast[bufi], tc + lane < t1, dtn, expA, lam, lane);
    };
    if constexpr (!FULL) {
#pragma unroll
      for (int i = 0; i < ZTS; ++i) {
        const int t = ZTS * sw + i;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          Zs[i][r] = st && t < NFT && col == 0 ? st[(int64_t)F * p.dv + 16 * t + 4 * g + r] : 0.f;
      }
      if (nch > 0 && sw == dwave) {
        load_dt(t0);
        decay(t0, 0);
        if (nch > 1) load_dt(t0 + C);
      }
    }
    if (nch > 0) load_v(t0);
    __syncthreads();
    // The other slots of a composed start state.  This waits for the loads, so it
    // comes after the barrier: the feature waves featurize the first chunk meanwhile
    // and S is first read in the next iteration.  (The training pass gets whole start
    // states: its state waves have no registers to spare.)
    for (int u = 1; !SAVE && u < nst; ++u) {
      const float e = slot_decay(u);
      const float *su = slot_state(u);
#pragma unroll
      for (int jj = 0; jj < NTW; ++jj)
#pragma unroll
        for (int t = 0; t < NFT; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            S[jj][t][r] = e * S[jj][t][r] + su[(int64_t)(16 * t + 4 * g + r) * p.dv + ncol + 16 * jj + col];
    }

    frag vfr[NTW][KC];  // v of the block being read out, tile order
    frag vfr_prev[MB > 1 ? NTW : 1][MB > 1 ? KC : 1];  // v of the chunk's first block (two-block chunks)
    // S += phi~(K)^T V over one block (its phi(k)^T buffer, its v fragments), after
    // S *= e^{L_last} of that block
    auto update_state = [&](const T *kt, const frag (*vb)[KC], int dbuf) {
      if constexpr (DECAY) {
        const float el = sLast[dbuf];
#pragma unroll
        for (int jj = 0; jj < NTW; ++jj)
#pragma unroll
          for (int t = 0; t < NFT; ++t) S[jj][t] *= el;
      }
#pragma unroll
      for (int t = 0; t < NFT; ++t) {
        frag ak[KC];
#pragma unroll
        for (int s = 0; s < KC; ++s) ak[s] = M::ld_tile(&kt[(16 * t + col) * LDC], s, g);
#pragma unroll
        for (int jj = 0; jj < NTW; ++jj)
#pragma unroll
          for (int s = 0; s < KC; ++s) S[jj][t] = M::mma(ak[s], vb[jj][s], S[jj][t]);
      }
    };
    for (int64_t j = 0; j <= nch; ++j) {
      const int64_t ts = t0 + (j - 1) * C;  // block handled in this iteration (j >= 1)
      const int bs = (int)((j + 1) & 1);
      const int ks = (int)((j - 1 + NKT) % NKT);
      const int ds = (int)((j - 1 + NDB) % NDB);
      const int bi = MB == 1 ? 0 : (int)((j - 1 + MB) % MB);  // block within its chunk
      // ---- half A: read-out of chunk j-1
      if (j >= 1) {
        if constexpr (SAVE) issue_gate_rows(ts);
        if constexpr (SAVE) {
          if ((ts / C) % p.ck_every == 0) {
            // a checkpoint: the float32 state at the start of chunk j-1 (this
            // iteration's read-out state).  The training pass runs with one workgroup
            // per (b, h), so the row stride is the compile-time DW: one base address per
            // feature tile, the rest instruction offsets
            float *sv = p.save_ck + (bh * p.nck + ts / C / p.ck_every) * BLK + ncol + col;
#pragma unroll
            for (int t = 0; t < NFT; ++t) {
              float *rowp = sv + (16 * t + 4 * g) * DW;
#pragma unroll
              for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int jj = 0; jj < NTW; ++jj) rowp[r * DW + 16 * jj] = S[jj][t][r];
            }
          }
        }
        // v of chunk ts -> accumulator layout: lane (g, col n) holds v[16bt + 4g + r][n]
#pragma unroll
        for (int jj = 0; jj < NTW; ++jj) {
          f32x4 vacc[NCT];
#pragma unroll
          for (int bt = 0; bt < NCT; ++bt) {
            vacc[bt] = zero4();
#pragma unroll
            for (int s = 0; s < KVL; ++s) vacc[bt] = M::mma(vf[EPL == 8 ? 0 : jj][bt][s], vsel[jj][s], vacc[bt]);
          }
#pragma unroll
          for (int s = 0; s < KC; ++s) vfr[jj][s] = M::from_acc(vacc, s);
        }
        // gate rows of chunk j-1 straight to LDS (see issue_gate_rows); without the
        // training saves they go out once the re-layout has consumed this chunk's v
        // rows, so that the wait for those is not also a wait for the gate rows
        // (measured 2-6 % faster on the gated layer).  With the saves they go out
        // first: a pending LDS load makes the barrier ending this half wait for every
        // outstanding global access, which there includes the saved state's stores.
        if constexpr (!SAVE) issue_gate_rows(ts);
        if (j < nch) load_v(ts + C);
        // The segment pass has no read-out: its state waves advance S over chunk j-1
        // here, beside the featurization of chunk j (its phi(k)^T, decay factors and
        // v fragments are complete), instead of after it in half B.
        if constexpr (!FULL) {
          update_state(sKt[ks], vfr, ds);
          // z <- e^{L_last} z + sum_c' phi~(k_c'): phi~(k)^T times a ones column
          const float el = DECAY ? sLast[ds] : 1.f;
#pragma unroll
          for (int i = 0; i < ZTS; ++i) {
            const int t = ZTS * sw + i;
            if (t < NFT) {
              frag ak[KC];
#pragma unroll
              for (int s = 0; s < KC; ++s) ak[s] = M::ld_tile(&sKt[ks][(16 * t + col) * LDC], s, g);
              if constexpr (DECAY) Zs[i] *= el;
#pragma unroll
              for (int s = 0; s < KC; ++s) Zs[i] = M::mma(ak[s], ones, Zs[i]);
            }
          }
        }
        if constexpr (FULL) {
          frag sfr[NTW][KF];
#pragma unroll
          for (int jj = 0; jj < NTW; ++jj)
#pragma unroll
            for (int s = 0; s < KF; ++s) sfr[jj][s] = M::from_acc(S[jj], s);
          float den[NCT];
#pragma unroll
          for (int bt = 0; bt < NCT; ++bt) {
            const int cc = 16 * bt + col;
            den[bt] = sDenInter[bs][cc];
#pragma unroll
            for (int a = 0; a < MB * NCT; ++a)
              if (a <= NCT * bi + bt) den[bt] += sDenPart[a][cc];
          }
          // e^{L} from the chunk's start: the second block of a chunk adds its first's total
          const float cscale = MB > 1 && DECAY && bi == 1 ? sLast[(j - 2 + NDB) % NDB] : 1.f;
          if (SAVE && sw == 0 && g == 0 && half == 0) {
#pragma unroll
            for (int bt = 0; bt < NCT; ++bt)
              if (ts + 16 * bt + col < t1) p.save_den[bh * p.n + ts + 16 * bt + col] = den[bt];
          }
          f32x4 oacc[NTW][NCT];
#pragma unroll
          for (int bt = 0; bt < NCT; ++bt) {
            const int cc = 16 * bt + col;
            frag bq[KF];
#pragma unroll
            for (int s = 0; s < KF; ++s) bq[s] = M::ld_tile(&sQ[bs][cc * LDQ], s, g);
            frag bp[M::steps_upto(MB * NCT - 1)];
#pragma unroll
            for (int s = 0; s < M::steps_upto(MB * NCT - 1); ++s)
              if (s < M::steps_upto(NCT * bi + bt)) bp[s] = M::ld_tile(&sP[cc * LDP], s, g);
#pragma unroll
            for (int jj = 0; jj < NTW; ++jj) {
              // inter: S^T phiQ^T e^{L_c};  intra: V^T Pt
              f32x4 acc = zero4();
#pragma unroll
              for (int s = 0; s < KF; ++s) acc = M::mma(sfr[jj][s], bq[s], acc);
              if constexpr (DECAY) acc *= seL[ds][cc] * cscale;
              if (MB == 1 || bi == 0) {
#pragma unroll
                for (int s = 0; s < M::steps_upto(bt); ++s) acc = M::mma(vfr[jj][s], bp[s], acc);
              } else if constexpr (MB > 1) {
                // keys of the chunk's first block, then of this block
#pragma unroll
                for (int s = 0; s < KC; ++s) acc = M::mma(vfr_prev[jj][s], bp[s], acc);
#pragma unroll
                for (int s = 0; s < M::steps_upto(bt); ++s) acc = M::mma(vfr[jj][s], bp[KC + s], acc);
              }
              oacc[jj][bt] = acc;
            }
          }
#pragma unroll
          for (int bt = 0; bt < NCT; ++bt) {
            const float inv = __builtin_amdgcn_rcpf(den[bt]);
#pragma unroll
            for (int jj = 0; jj < NTW; ++jj) oacc[jj][bt] *= inv;
          }
          if constexpr (SAVE) {
            // float32 output rows for the backward pass: lane (g, col) holds token
            // 16bt + col, columns 16 NTW sw + 16 jj + 4g .. +3
            // (row stride DW: the training pass has one workgroup per (b, h))
            float *os0 = p.save_o + (bh * p.n + ts + col) * DW + 16 * NTW * sw + 4 * g;
#pragma unroll
            for (int bt = 0; bt < NCT; ++bt)
              if (ts + 16 * bt + col < t1) {
#pragma unroll
                for (int jj = 0; jj < NTW; ++jj) *reinterpret_cast<f32x4 *>(os0 + 16 * bt * DW + 16 * jj) = oacc[jj][bt];
              }
          }
          // output rows to LDS; they leave for HBM as whole rows in half B
          T *orow = &sO[col * LDO + 16 * NTW * sw + 4 * g];
#pragma unroll
          for (int bt = 0; bt < NCT; ++bt)
#pragma unroll
            for (int jj = 0; jj < NTW; ++jj) store4(orow + 16 * bt * LDO + 16 * jj, oacc[jj][bt]);
        }
      }
      if constexpr (!FULL) {
        // decay factors of chunk j+1 (read by the feature waves next iteration)
        if (sw == dwave && j + 1 < nch) {
          decay(t0 + (j + 1) * C, (int)((j + 1) % NDB));
          if (j + 2 < nch) load_dt(t0 + (j + 2) * C);
        }
      }
      if constexpr (FULL) __syncthreads();
      // ---- half B: output rows of chunk j-1 to HBM (non-temporal: nothing here reads them
      //      back), state update over chunk j-1
      if (FULL && j >= 1) {
        if constexpr (FULL) {
          constexpr int EP = 16 / (int)sizeof(T);          // elements per 16-byte piece
          constexpr int PPR = DW / EP;                      // pieces per row
          constexpr int NIT = C * PPR / (NS * 64);         // pieces per lane
          static_assert(NIT * NS * 64 == C * PPR, "whole rows per pass");
          T *ob = O + ts * p.so_t + half * DW;
          if (MB == 1 && p.gate) {
            // mixer gate: o * SiLU(g) on the rounded output, the gate rows from LDS;
            // two pieces at a time so that the gate adds few live registers
            constexpr int GB = NIT < 2 ? NIT : 2;
#pragma unroll
            for (int i0 = 0; i0 < NIT; i0 += GB) {
              f32x4 piece[GB];
#pragma unroll
              for (int u = 0; u < GB; ++u) {
                const int i = ((i0 + u) * NS + sw) * 64 + lane, row = i / PPR, pc = i % PPR;
                piece[u] = gate_piece(*reinterpret_cast<const f32x4 *>(&sO[row * LDO + pc * EP]),
                                      *reinterpret_cast<const f32x4 *>(&sG[i * EP]), T{});
              }
#pragma unroll
              for (int u = 0; u < GB; ++u) {
                const int i = ((i0 + u) * NS + sw) * 64 + lane, row = i / PPR, pc = i % PPR;
                if (ts + row < t1)
                  __builtin_nontemporal_store(piece[u], reinterpret_cast<f32x4 *>(ob + (int64_t)row * p.so_t + pc * EP));
              }
              __builtin_amdgcn_sched_barrier(0);
            }
          } else {
            f32x4 piece[NIT];
#pragma unroll
            for (int it = 0; it < NIT; ++it) {
              const int i = (it * NS + sw) * 64 + lane, row = i / PPR, pc = i % PPR;
              piece[it] = *reinterpret_cast<const f32x4 *>(&sO[row * LDO + pc * EP]);
            }
#pragma unroll
            for (int it = 0; it < NIT; ++it) {
              const int i = (it * NS + sw) * 64 + lane, row = i / PPR, pc = i % PPR;
              if (ts + row < t1)
                __builtin_nontemporal_store(piece[it], reinterpret_cast<f32x4 *>(ob + (int64_t)row * p.so_t + pc * EP));
            }
          }
        }
        if constexpr (MB == 1) {
          if constexpr (FULL) update_state(sKt[ks], vfr, ds);
        } else {
          // the chunk's update once both blocks are read out (or at the segment's end)
          if (bi == MB - 1) {
            update_state(sKt[(j - 2 + NKT) % NKT], vfr_prev, (int)((j - 2 + NDB) % NDB));
            update_state(sKt[ks], vfr, ds);
          } else if (j == nch) {
            update_state(sKt[ks], vfr, ds);
          } else {
#pragma unroll
            for (int jj = 0; jj < NTW; ++jj)
#pragma unroll
              for (int s = 0; s < KC; ++s) vfr_prev[jj][s] = vfr[jj][s];
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
    if constexpr (!FULL) {
      if (half == 0) {
        if (dst && col == 0) {
#pragma unroll
          for (int i = 0; i < ZTS; ++i) {
            const int t = ZTS * sw + i;
            if (t < NFT) {
#pragma unroll
              for (int r = 0; r < 4; ++r) dst[(int64_t)F * p.dv + 16 * t + 4 * g + r] = Zs[i][r];
            }
          }
        }
        if (sw == dwave && lane == 0) p.ws_lam[(int64_t)seg * BH + bh] = (float)lam;
      }
    }
  }
}

// Running start states from the segment pass's slots (in place): slot 0 already
// began from s_init and holds the state after it, and for u = 1 .. nslot-1
//   state(u) = e^{lam(u)} state(u-1) + local(u),
// the composition of affine maps of [SSM] §4.2 with a scalar decay; the start
// state of segment s is then slot s*lsub-1, and only those slots are written back
// (the running value stays in a register).  Optionally copies s_init to `init_copy`
// first (used when s_init aliases s_final).
static __global__ __launch_bounds__(256) void combine_kernel(float *ws_state, const float *ws_lam, const float *s_init,
                                                      float *init_copy, int64_t BH, int64_t BLK, int nslot, int lsub) {
  const int64_t bh = blockIdx.y;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= BLK) return;
  if (init_copy) init_copy[bh * BLK + e] = s_init ? s_init[bh * BLK + e] : 0.f;
  if (nslot < 2) return;
  float cur = ws_state[bh * BLK + e];
  for (int u = 1; u < nslot; ++u) {
    const int64_t slot = (int64_t)u * BH + bh;
    cur = expf(ws_lam[slot]) * cur + ws_state[slot * BLK + e];
    if ((u + 1) % lsub == 0) ws_state[slot * BLK + e] = cur;
  }
}

}  // namespace hm
