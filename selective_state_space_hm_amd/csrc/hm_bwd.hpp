// Backward pass of causal, normalized Hedgehog linear attention.
//
// Pages: "线性注意力（Linear Attention）详解" (cnblogs) parts 2-5 (the causal kernel
// form, the recurrent state and its chunk-wise evaluation), "HedgeMamba：融合线性
// 注意力与状态空间模型的高效序列建模" §2.1 (Hedgehog map), §2.3 (numerator and
// denominator), §3 (the model is trained, so the mixer needs gradients), and the
// quant67 SSM lecture §3.2 (softplus step size).
//
// Notation per (b, h) and chunk of C tokens, L_t the chunk-local inclusive sum of
// log a, Lam its value at the chunk's last token, phiq the unnormalized feature
// row exp([u, -u] - max|u|) the forward used (o does not depend on its scale),
// phik the softmax feature row, S_c / z_c the state at the chunk's start:
//   dnum_t = dO_t / den_t,  dden_t = -(dO_t . o_t) / den_t
//   A[t][j] = [j <= t] e^{L_t - L_j} (v_j . dnum_t + dden_t)
//   dphiq_t = sum_j A[t][j] phik_j + e^{L_t} (S_c dnum_t + dden_t z_c)
//   G (gradient of the state at a chunk's end, carried from the last chunk back):
//     G <- e^{Lam} G + sum_t e^{L_t} phiq_t dnum_t^T,   g likewise with dden
//   dphik_j = sum_t A[t][j] phiq_t + e^{Lam - L_j} (G v_j + g)
//   dv_j = sum_t [j <= t] e^{L_t - L_j} (phiq_t . phik_j) dnum_t + e^{Lam - L_j} G^T phik_j
//   d log a_t = sum over the (query s, key j) pairs with j < t <= s of
//     W_sj = [j <= s] e^{L_s - L_j} (phiq_s . phik_j)(dnum_s . v_j + dden_s): per chunk,
//     the in-chunk pairs strictly below the diagonal, Q_s = e^{L_s} phiq_s . (S_c dnum_s
//     + dden_s z_c) for keys before the chunk, K_j = e^{Lam - L_j} phik_j . (G v_j + g)
//     for queries after it, and X_c = e^{Lam} (<G, S_c> + <g, z_c>) for pairs spanning
//     it.  No term is a difference of the diagonal's nearly equal parts (v_t against
//     o_t under a fast decay), so the result keeps its relative accuracy.
//   through the maps: du'_q = phiq * dphiq (the max shift is a scale);
//     du'_k = phik * (dphik - phik . dphik) (softmax); du = du'[:f] - du'[f:];
//     dx = du W^T, dW = sum_t x_t^T du_t.
//   With the rotary encoding every product above runs on the turned features
//   (bwd_prep stores them turned); only the maps' backward needs the unturned
//   phi and dphi, which are the transposed rotation applied to both (the dot
//   product phik . dphik is the same in either frame).
// The training forward keeps the state only at the start of every chunk range of
// the per-chunk kernels (a checkpoint per range; the quant67 SSM lecture §4.3:
// recompute rather than store the intermediate states); bwd_states rebuilds the
// chunk-start states S_c, z_c from them.
// Kernels, launched in this order on one stream:
//   bwd_prep   (per chunk)  features, dnum, dden, L
//   bwd_states (per (b,h), a range of chunks, first to last)  S_c, z_c from the checkpoint
//   bwd_gstate (per (b,h), chunks last to first)  G, g at every chunk end; dS_init
//   bwd_dq     (per (b,h), a range of chunks)  dq, partial dW_q, Q_s
//   bwd_dk     (same)  dk, partial dW_k, K_j
//   bwd_dv     (same)  dv, the in-chunk pair sums, X_c
//   bwd_decay  (per (b,h))  d dt, partial dA_log
//   bwd_reduce (per weight element)  dW_q, dW_k, dA_log
// Every matrix product runs on MFMA from LDS rows that are contiguous along K;
// operands needed the other way round are written to LDS transposed.
#pragma once

#include <hip/hip_runtime.h>

#include "hm_bwd_params.hpp"
#include "hm_device.hpp"

namespace hm {

namespace bw {

constexpr int C = 64;  // chunk length (the forward's)

template <typename T> constexpr int ep() { return 16 / (int)sizeof(T); }

// acc += A[16 rows][K] * B[16 rows][K]^T, both row-major in LDS with K contiguous:
// A row (lane % 16) starts at A + row * la, B row (lane % 16) at B + row * lb.
// acc[r] is element (4g + r, lane % 16) of the 16x16 product.
// The operand registers stay allocated until the chain's result has been read:
// measured on gfx950, a VALU write (here an accumulator read into a VGPR that had
// just been freed) to a source register of an MFMA still waiting on the previous
// MFMA of its chain changed that MFMA's operand.  The empty asm below reads every
// fragment and passes the accumulator through, so the fragments stay live until the
// result is available and later uses of the result come after it.  It is not
// volatile: independent work (the next product's LDS reads) may still move above it.
template <typename T, int K>
__device__ __forceinline__ f32x4 mm(const T *A, int la, const T *B, int lb, f32x4 acc) {
  using M = Mma<T>;
  constexpr int NK = K / M::KS;
  const int lane = threadIdx.x & 63, i = lane & 15, g = lane >> 4;
  typename M::frag a[NK], b[NK];
#pragma unroll
  for (int s = 0; s < NK; ++s) {
    a[s] = M::ld_contig(A + i * la + s * M::KS, g);
    b[s] = M::ld_contig(B + i * lb + s * M::KS, g);
  }
#pragma unroll
  for (int s = 0; s < NK; ++s) acc = M::mma(a[s], b[s], acc);
#pragma unroll
  for (int s = 0; s < NK; ++s) asm("" : "+v"(acc) : "v"(a[s]), "v"(b[s]));
  return acc;
}

// The A-operand fragments of one 16-row band (row lane % 16 at A + row * la, K
// contiguous), loaded once and reused by every product of a phase that shares them.
template <typename T, int K> struct Frags {
  typename Mma<T>::frag f[K / Mma<T>::KS];
  __device__ __forceinline__ void load(const T *A, int la) {
    const int lane = threadIdx.x & 63, i = lane & 15, g = lane >> 4;
#pragma unroll
    for (int s = 0; s < K / Mma<T>::KS; ++s) f[s] = Mma<T>::ld_contig(A + i * la + s * Mma<T>::KS, g);
  }
};
// acc += A * B^T as mm(), with A's fragments preloaded (kept live to the end of the
// chain like mm's own)
template <typename T, int K>
__device__ __forceinline__ f32x4 mm(const Frags<T, K> &a, const T *B, int lb, f32x4 acc) {
  using M = Mma<T>;
  constexpr int NK = K / M::KS;
  const int lane = threadIdx.x & 63, i = lane & 15, g = lane >> 4;
  typename M::frag b[NK];
#pragma unroll
  for (int s = 0; s < NK; ++s) b[s] = M::ld_contig(B + i * lb + s * M::KS, g);
#pragma unroll
  for (int s = 0; s < NK; ++s) acc = M::mma(a.f[s], b[s], acc);
#pragma unroll
  for (int s = 0; s < NK; ++s) asm("" : "+v"(acc) : "v"(a.f[s]), "v"(b[s]));
  return acc;
}

// acc += A * B^T as mm(), with B's fragments preloaded
template <typename T, int K>
__device__ __forceinline__ f32x4 mm(const T *A, int la, const Frags<T, K> &b, f32x4 acc) {
  using M = Mma<T>;
  constexpr int NK = K / M::KS;
  const int lane = threadIdx.x & 63, i = lane & 15, g = lane >> 4;
  typename M::frag a[NK];
#pragma unroll
  for (int s = 0; s < NK; ++s) a[s] = M::ld_contig(A + i * la + s * M::KS, g);
#pragma unroll
  for (int s = 0; s < NK; ++s) acc = M::mma(a[s], b.f[s], acc);
#pragma unroll
  for (int s = 0; s < NK; ++s) asm("" : "+v"(acc) : "v"(a[s]), "v"(b.f[s]));
  return acc;
}

// S[m] = e * S[m] + A_rt B_ct^T over tiles tt = wave + NW m (rt = tt / CT, ct = tt % CT)
// of an [F][CT * 16] accumulator, A and B rows K-contiguous in LDS.  When CT divides
// NW every tile of a wave has the same ct, and B's fragments are read once.
template <typename T, int K, int NTT, int TILES, int CT, int NW = 4>
__device__ __forceinline__ void tiles_mm(f32x4 (&S)[NTT], float e, const T *A, const T *B, int ld) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if constexpr (NW % CT == 0) {
    Frags<T, K> fb;
    fb.load(B + 16 * (w % CT) * ld, ld);
#pragma unroll
    for (int m = 0; m < NTT; ++m) {
      const int tt = w + NW * m;
      if (tt < TILES) S[m] = mm<T, K>(A + 16 * (tt / CT) * ld, ld, fb, S[m] * e);
    }
  } else {
#pragma unroll
    for (int m = 0; m < NTT; ++m) {
      const int tt = w + NW * m;
      if (tt < TILES) S[m] = mm<T, K>(A + 16 * (tt / CT) * ld, ld, B + 16 * (tt % CT) * ld, ld, S[m] * e);
    }
  }
}

template <typename T> struct Vec { typedef T type __attribute__((ext_vector_type(16 / sizeof(T)))); };

// A workgroup's [ROWS][COLS] state tile, rounded to T, from accumulator tiles to
// global rows (stride gs elements) in two steps: tile_to_lds() writes element
// (16 rt + 4g + r, 16 ct + i) of tile tt = wave + NW m into LDS rows (stride lo);
// after a barrier, lds_to_global() sends whole 16-byte pieces.  Four 2-byte stores
// per tile and lane become one 16-byte store per lane and pass: measured in the
// chunk-serial kernels, issuing the scattered stores took a quarter of their time.
template <typename T, int NTT, int TILES, int CT, int NW = 4>
__device__ __forceinline__ void tile_to_lds(T *dst, int lo, const f32x4 (&X)[NTT]) {
  const int lane = threadIdx.x & 63, g = lane >> 4, i = lane & 15, w = threadIdx.x >> 6;
#pragma unroll
  for (int m = 0; m < NTT; ++m) {
    const int tt = w + NW * m;
    if (tt < TILES) {
      const int rt = tt / CT, ct = tt % CT;
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(16 * rt + 4 * g + r) * lo + 16 * ct + i] = (T)X[m][r];
    }
  }
}
// The first `valid` of ROWS rows [COLS] from LDS (stride lo) to global rows (stride
// gs elements) as 16-byte pieces.
template <typename T, int ROWS, int COLS, int NT = 256>
__device__ __forceinline__ void rows_to_global(T *dst, int64_t gs, const T *src, int lo, int valid) {
  constexpr int E = ep<T>(), PPR = COLS / E, N = ROWS * PPR;
  typedef typename Vec<T>::type V;
#pragma unroll
  for (int idx = threadIdx.x; idx < N; idx += NT) {
    const int r = idx / PPR, pc = idx % PPR;
    if (r < valid) *reinterpret_cast<V *>(dst + r * gs + pc * E) = *reinterpret_cast<const V *>(src + r * lo + pc * E);
  }
}
template <typename T, int ROWS, int COLS, int NT = 256>
__device__ __forceinline__ void lds_to_global(T *dst, int64_t gs, const T *src, int lo) {
  constexpr int E = ep<T>(), PPR = COLS / E, N = ROWS * PPR;
  typedef typename Vec<T>::type V;
#pragma unroll
  for (int idx = threadIdx.x; idx < N; idx += NT) {
    const int r = idx / PPR, pc = idx % PPR;
    *reinterpret_cast<V *>(dst + r * gs + pc * E) = *reinterpret_cast<const V *>(src + r * lo + pc * E);
  }
}

// ROWS x COLS from global rows (stride gs elements) into LDS rows (ld), rows at or
// beyond `valid` zeroed; 16-byte pieces, every load of a thread issued before its
// first LDS write (compile-time trip counts, fully unrolled).
template <typename T, int ROWS, int COLS, int NT = 256>
__device__ __forceinline__ void stage(T *dst, int ld, const T *src, int64_t gs, int valid) {
  constexpr int E = ep<T>(), PPR = COLS / E, N = ROWS * PPR, PER = (N + NT - 1) / NT;
  typedef typename Vec<T>::type V;
  V x[PER];
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int idx = threadIdx.x + NT * m, r = idx / PPR, pc = idx % PPR;
    x[m] = (idx < N && r < valid) ? *reinterpret_cast<const V *>(src + r * gs + pc * E) : V{};
  }
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int idx = threadIdx.x + NT * m, r = idx / PPR, pc = idx % PPR;
    if (idx < N) *reinterpret_cast<V *>(dst + r * ld + pc * E) = x[m];
  }
}
// stage() in two halves, for operands whose LDS buffer frees up later: the loads
// go out with an earlier phase's (one memory round trip less per chunk) and the
// LDS writes happen once the buffer is free.
template <typename T, int ROWS, int COLS, int NT = 256> struct Staged {
  static constexpr int E = ep<T>(), PPR = COLS / E, N = ROWS * PPR, PER = (N + NT - 1) / NT;
  typename Vec<T>::type x[PER];
  __device__ __forceinline__ void load(const T *src, int64_t gs, int valid) {
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int idx = threadIdx.x + NT * m, r = idx / PPR, pc = idx % PPR;
      x[m] = (idx < N && r < valid) ? *reinterpret_cast<const typename Vec<T>::type *>(src + r * gs + pc * E)
                                    : typename Vec<T>::type{};
    }
  }
  __device__ __forceinline__ void store(T *dst, int ld) const {
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int idx = threadIdx.x + NT * m, r = idx / PPR, pc = idx % PPR;
      if (idx < N) *reinterpret_cast<typename Vec<T>::type *>(dst + r * ld + pc * E) = x[m];
    }
  }
};

// stage_t() in two halves (no row scale).
template <typename T, int ROWS, int COLS, int NT = 256> struct StagedT {
  static constexpr int E = ep<T>(), PPR = COLS / E;
  static constexpr int NP = sizeof(T) == 2 ? ROWS / 2 : ROWS, N = NP * PPR, PER = (N + NT - 1) / NT;
  typename Vec<T>::type x0[PER], x1[sizeof(T) == 2 ? PER : 1];
  __device__ __forceinline__ void load(const T *src, int64_t gs, int valid) {
    typedef typename Vec<T>::type V;
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int idx = threadIdx.x + NT * m;
      if constexpr (sizeof(T) == 2) {
        const int r = 2 * (idx % NP), pc = idx / NP;
        x0[m] = (idx < N && r < valid) ? *reinterpret_cast<const V *>(src + r * gs + pc * E) : V{};
        x1[m] = (idx < N && r + 1 < valid) ? *reinterpret_cast<const V *>(src + (r + 1) * gs + pc * E) : V{};
      } else {
        const int r = idx % ROWS, pc = idx / ROWS;
        x0[m] = (idx < N && r < valid) ? *reinterpret_cast<const V *>(src + r * gs + pc * E) : V{};
      }
    }
  }
  // rscale (optional): row r is multiplied by rscale[r] and rounded to T once more
  __device__ __forceinline__ void store(T *dst, int ld, const float *rscale = nullptr) const {
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int idx = threadIdx.x + NT * m;
      if (idx >= N) continue;
      if constexpr (sizeof(T) == 2) {
        const int r = 2 * (idx % NP), pc = idx / NP;
        const float s0 = rscale ? rscale[r] : 1.f, s1 = rscale ? rscale[r + 1] : 1.f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          // through named T values: the bit cast of a vector-element expression
          // itself gave wrong bits here
          const T lo = rscale ? (T)((float)x0[m][e] * s0) : x0[m][e];
          const T hi = rscale ? (T)((float)x1[m][e] * s1) : x1[m][e];
          const uint32_t packed =
              (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
          *reinterpret_cast<uint32_t *>(dst + (pc * E + e) * ld + r) = packed;
        }
      } else {
        const int r = idx % ROWS, pc = idx / ROWS;
        const float s0 = rscale ? rscale[r] : 1.f;
#pragma unroll
        for (int e = 0; e < E; ++e) dst[(pc * E + e) * ld + r] = rscale ? (T)((float)x0[m][e] * s0) : x0[m][e];
      }
    }
  }
};

// the same rows written transposed: dst[c * ld + r] = scale_r * src[r][c].
// Consecutive lanes take consecutive source rows (two rows per lane for bf16,
// packed into one 4-byte write), so the LDS writes of a wave are contiguous.
template <typename T, int ROWS, int COLS, bool SCALE = false>
__device__ __forceinline__ void stage_t(T *dst, int ld, const T *src, int64_t gs, int valid,
                                        const float *rscale = nullptr) {
  constexpr int E = ep<T>(), PPR = COLS / E;
  typedef typename Vec<T>::type V;
  if constexpr (sizeof(T) == 2) {
    constexpr int NP = ROWS / 2, N = NP * PPR, PER = (N + 255) / 256;
    V x0[PER], x1[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int idx = threadIdx.x + 256 * m, r = 2 * (idx % NP), pc = idx / NP;
      x0[m] = (idx < N && r < valid) ? *reinterpret_cast<const V *>(src + r * gs + pc * E) : V{};
      x1[m] = (idx < N && r + 1 < valid) ? *reinterpret_cast<const V *>(src + (r + 1) * gs + pc * E) : V{};
    }
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int idx = threadIdx.x + 256 * m, r = 2 * (idx % NP), pc = idx / NP;
      if (idx < N) {
        const float s0 = SCALE ? rscale[r] : 1.f, s1 = SCALE ? rscale[r + 1] : 1.f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const T a = SCALE ? (T)((float)x0[m][e] * s0) : x0[m][e];
          const T b2 = SCALE ? (T)((float)x1[m][e] * s1) : x1[m][e];
          const uint32_t packed =
              (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b2) << 16);
          *reinterpret_cast<uint32_t *>(dst + (pc * E + e) * ld + r) = packed;
        }
      }
    }
  } else {
    constexpr int N = ROWS * PPR, PER = (N + 255) / 256;
    V x[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int idx = threadIdx.x + 256 * m, r = idx % ROWS, pc = idx / ROWS;
      x[m] = (idx < N && r < valid) ? *reinterpret_cast<const V *>(src + r * gs + pc * E) : V{};
    }
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int idx = threadIdx.x + 256 * m, r = idx % ROWS, pc = idx / ROWS;
      if (idx < N) {
        const float s0 = SCALE ? rscale[r] : 1.f;
#pragma unroll
        for (int e = 0; e < E; ++e) dst[(pc * E + e) * ld + r] = SCALE ? (T)((float)x[m][e] * s0) : x[m][e];
      }
    }
  }
}

// accumulator tile -> LDS, row-major (row 4g + r, column lane % 16) or transposed
template <typename T>
__device__ __forceinline__ void put(T *dst, int ld, f32x4 a) {
  const int lane = threadIdx.x & 63, i = lane & 15, g = lane >> 4;
#pragma unroll
  for (int r = 0; r < 4; ++r) dst[(4 * g + r) * ld + i] = (T)a[r];
}
template <typename T>
__device__ __forceinline__ void put_t(T *dst, int ld, f32x4 a) {
  const int lane = threadIdx.x & 63, i = lane & 15, g = lane >> 4;
#pragma unroll
  for (int r = 0; r < 4; ++r) dst[i * ld + 4 * g + r] = (T)a[r];
}

// W [d][f] (head h) into LDS, as stored (ld = f + pad) or transposed (ld = d + pad):
// 16-byte loads, all issued before the first LDS write (NT threads)
template <typename T, int DK, int FH, int NT = 256>
__device__ __forceinline__ void load_w(T *dst, int ld, const T *w, bool transposed) {
  constexpr int E = ep<T>(), NV = DK * FH / E, PER = (NV + NT - 1) / NT;
  typedef typename Vec<T>::type V;
  V x[PER];
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int v = threadIdx.x + NT * m;
    x[m] = v < NV ? *reinterpret_cast<const V *>(w + v * E) : V{};
  }
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int v = threadIdx.x + NT * m;
    if (v >= NV) continue;
    const int i = v * E / FH, f0 = v * E % FH;
    if (transposed) {
#pragma unroll
      for (int e = 0; e < E; ++e) dst[(f0 + e) * ld + i] = x[m][e];
    } else {
      *reinterpret_cast<V *>(dst + i * ld + f0) = x[m];
    }
  }
}

// du'[f] = phi_u[f] * (dphi_u[f] - dot) in place of dph, for the rows t = 4g + r
// of a 16-row band whose features sit as dph[ft][r] (column 16 ft + lane % 16):
// phi is read from the LDS rows ph + (4g + r) * ld in the turned frame, and phi_u,
// dphi_u are phi and dph turned back (RT = dims / 32 feature tiles pair with the
// tiles RT later; RT = 0 means no rotation).  pos is the position of row 4g.
template <int NFT, int RT, typename T>
__device__ __forceinline__ void phi_dphi_rt(f32x4 *dph, const T *ph, int ld, const double *rev, double pos,
                                            const float *dot) {
  const int lane = threadIdx.x & 63, i = lane & 15, g = lane >> 4;
#pragma unroll
  for (int ft = 0; ft < NFT; ++ft) {
    if (ft < RT) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const T *row = ph + (4 * g + r) * ld;
        float c, s, p1 = (float)row[16 * ft + i], p2 = (float)row[16 * (ft + RT) + i];
        float d1 = dph[ft][r], d2 = dph[ft + RT][r];
        rope_cs(rev[16 * ft + i], pos + r, c, s);
        rope_turn<true>(p1, p2, c, s);
        rope_turn<true>(d1, d2, c, s);
        dph[ft][r] = p1 * (d1 - dot[r]);
        dph[ft + RT][r] = p2 * (d2 - dot[r]);
      }
    } else if (ft >= 2 * RT) {
#pragma unroll
      for (int r = 0; r < 4; ++r) dph[ft][r] = (float)ph[(4 * g + r) * ld + 16 * ft + i] * (dph[ft][r] - dot[r]);
    }
  }
}
template <int NFT, typename T>
__device__ __forceinline__ void phi_dphi(f32x4 *dph, const T *ph, int ld, const double *rev, double pos,
                                         const float *dot, int dims) {
  switch (dims >> 5) {
    case 0: phi_dphi_rt<NFT, 0>(dph, ph, ld, rev, pos, dot); break;
    case 1: phi_dphi_rt<NFT, 1>(dph, ph, ld, rev, pos, dot); break;
    case 2: if constexpr (NFT >= 4) phi_dphi_rt<NFT, 2>(dph, ph, ld, rev, pos, dot); break;
    case 3: if constexpr (NFT >= 6) phi_dphi_rt<NFT, 3>(dph, ph, ld, rev, pos, dot); break;
    case 4: if constexpr (NFT >= 8) phi_dphi_rt<NFT, 4>(dph, ph, ld, rev, pos, dot); break;
    default: break;
  }
}
// Each thread's share of the rotation rates rope_rev(i) for i < dims/2, into LDS.
__device__ __forceinline__ void fill_rev(double *rev, const BwdParams &p) {
  if ((int)threadIdx.x < p.rope_dims / 2) rev[threadIdx.x] = rope_rev(threadIdx.x, p.rope_dims, p.rope_base);
}
__device__ __forceinline__ double pos_of(const BwdParams &p, int64_t b) {
  return p.rope_pos0 ? (double)p.rope_pos0[b] : 0.0;
}

__device__ __forceinline__ float sum16(float v) {
  v += __shfl_xor(v, 1);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 4);
  v += __shfl_xor(v, 8);
  return v;
}

}  // namespace bw

// The chunk range [c0, c1) of workgroup `grp` of a (b, h) in the per-chunk kernels.
__device__ __forceinline__ void chunk_range(const BwdParams &p, int grp, int64_t &c0, int64_t &c1) {
  const int64_t per = (p.nch + p.ngrp - 1) / p.ngrp;
  c0 = grp * per;
  c1 = c0 + per < p.nch ? c0 + per : p.nch;
}

// Waves of a bwd_states / bwd_gstate workgroup: each wave carries TILES / 8 of the
// share's state tiles through the chunks, two waves per SIMD.
constexpr int kChainWaves = 8;

// Waves of a bwd_dq workgroup: two per SIMD, each 16-row band of the chunk split
// between two waves by column tiles, so that one wave's MFMA chains and LDS waits
// overlap the other's.  The rotary variants keep one wave per band: the rotation pairs
// feature tiles across that split.
constexpr int bwd_waves(bool rope) { return rope ? 4 : 8; }

// ---------------------------------------------------------------- bwd_prep
// One workgroup per (b, h, chunk): phiq (unnormalized, as the forward computed
// it), phik (softmax), dnum, dden and L for the chunk's tokens.
template <typename T, int DK, int FH, int DV, bool ROPE>
__global__ __launch_bounds__(256) void bwd_prep(const BwdParams p) {
  using namespace bw;
  constexpr int F = 2 * FH, PAD = Mma<T>::PAD, LDW = DK + PAD, E = ep<T>();
  constexpr float L2E = 1.4426950408889634f;
  __shared__ __align__(16) T sW[2][FH * LDW];
  __shared__ __align__(16) T sX[C * LDW];
  __shared__ double sRev[ROPE ? FH : 1];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, i = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // one chunk per workgroup: many small workgroups hide the latency best here
  const int64_t bh = blockIdx.x / p.nch, b = bh / p.H, h = bh % p.H;
  const int64_t c0 = blockIdx.x % p.nch, c1 = c0 + 1;
  load_w<T, DK, FH>(sW[0], LDW, (const T *)p.wq + h * p.sw_h, true);
  load_w<T, DK, FH>(sW[1], LDW, (const T *)p.wk + h * p.sw_h, true);
  if constexpr (ROPE) fill_rev(sRev, p);
  for (int64_t c = c0; c < c1; ++c) {
  const int64_t t0 = c * C;
  const int nv = (int)(p.n - t0 < C ? p.n - t0 : C);
  // q and k rows go out together; k is written to LDS once q's projection is done
  Staged<T, C, DK> xq, xk;
  xq.load((const T *)p.q + b * p.sq_b + h * p.sq_h + t0 * p.sq_t, p.sq_t, nv);
  xk.load((const T *)p.k + b * p.sk_b + h * p.sk_h + t0 * p.sk_t, p.sk_t, nv);
  for (int proj = 0; proj < 2; ++proj) {
    if (proj == 0) xq.store(sX, LDW);
    else xk.store(sX, LDW);
    __syncthreads();
    // u^T tiles: rows f, columns the wave's 16 tokens
    f32x4 u[FH / 16];
    float m = 0.f;
#pragma unroll
    for (int rt = 0; rt < FH / 16; ++rt) {
      u[rt] = mm<T, DK>(sW[proj] + 16 * rt * LDW, LDW, sX + 16 * w * LDW, LDW, zero4());
#pragma unroll
      for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(u[rt][r]));
    }
    const float ml = group_max(m) * L2E;
    float sum = 0.f;
    f32x4 ep_[FH / 16], em_[FH / 16];
#pragma unroll
    for (int rt = 0; rt < FH / 16; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ep_[rt][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(u[rt][r], L2E, -ml));
        em_[rt][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(-u[rt][r], L2E, -ml));
        sum += ep_[rt][r] + em_[rt][r];
      }
    const float inv = proj == 1 ? __builtin_amdgcn_rcpf(group_sum(sum)) : 1.f;
    const int t = 16 * w + i;
    // the feature row of token t: tile rt < FH/16 from +u, the rest from -u
    f32x4 ph4[F / 16];
#pragma unroll
    for (int rt = 0; rt < FH / 16; ++rt) {
      ph4[rt] = ep_[rt] * inv;
      ph4[FH / 16 + rt] = em_[rt] * inv;
    }
    if constexpr (ROPE) rope_apply<F / 16>(ph4, sRev, g, pos_of(p, b) + (double)(t0 + t), p.rope_dims);
    if (t < nv) {
      T *ph = (T *)(proj == 0 ? p.phq : p.phk) + (bh * p.n + t0 + t) * F;
#pragma unroll
      for (int ft = 0; ft < F / 16; ++ft) store4(ph + 16 * ft + 4 * g, ph4[ft]);  // four consecutive features per lane
    }
    __syncthreads();
  }
  // chunk-local log-decay prefix, float64 sums as in the forward
  if (p.dt && w == 0) {
    const bool valid = lane < nv;
    const float dtv = valid ? p.dt[b * p.sdt_b + h * p.sdt_h + (t0 + lane) * p.sdt_t] : 0.f;
    const float la = valid ? -softplus_f32(dtv) * expf(p.a_log[h]) : 0.f;
    const double L = wave_inclusive_scan((double)la);
    if (valid) p.Lc[bh * p.n + t0 + lane] = (float)L;
  }
  // dnum = dO / den, dden = -(dO . o) / den with o the float32 output the training
  // forward saved (before any gate); with a gate g, dO here is d_o * SiLU(g) and
  // d_gate = d_o * o * SiLU'(g).  PPR threads per row.
  constexpr int PPR = DV / E, RPP = 256 / PPR;
  typedef typename Vec<T>::type V;
  const T *DO = (const T *)p.d_o + b * p.so_b + h * p.so_h + t0 * p.so_t;
  const float *O = p.so32 + (bh * p.n + t0) * DV;
  constexpr int NIT = C / RPP;
  // every load of the pass goes out before the first store (the compiler cannot
  // move loads above stores to other buffers by itself)
  V xdo[NIT], xg[NIT];
  f32x4 xo[NIT][E / 4 > 0 ? E / 4 : 1];
  float xden[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int r = it * RPP + tid / PPR, pc = tid % PPR;
    const bool valid = r < nv;
    xdo[it] = valid ? *reinterpret_cast<const V *>(DO + r * p.so_t + pc * E) : V{};
#pragma unroll
    for (int q4 = 0; q4 < E / 4; ++q4)
      xo[it][q4] = valid ? *reinterpret_cast<const f32x4 *>(O + r * DV + pc * E + 4 * q4) : zero4();
    xg[it] = (valid && p.gate)
                 ? *reinterpret_cast<const V *>((const T *)p.gate + b * p.sg_b + h * p.sg_h + (t0 + r) * p.sg_t + pc * E)
                 : V{};
    xden[it] = valid ? p.sden[bh * p.n + t0 + r] : 1.f;
  }
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int r0 = it * RPP;
    const int r = r0 + tid / PPR, pc = tid % PPR;
    const bool valid = r < nv;
    float dv_[E], ov[E];
#pragma unroll
    for (int e = 0; e < E; ++e) dv_[e] = ov[e] = 0.f;
    if (valid) {
      const V x = xdo[it];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        dv_[e] = (float)x[e];
        ov[e] = xo[it][e / 4][e % 4];
      }
      if (p.gate) {
        const V gv = xg[it];
        V dg;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float x2 = (float)gv[e], sg = 1.f / (1.f + expf(-x2));
          dg[e] = (T)(dv_[e] * ov[e] * sg * (1.f + x2 * (1.f - sg)));
          dv_[e] *= x2 * sg;
        }
        *reinterpret_cast<V *>((T *)p.d_gate + b * p.sg_b + h * p.sg_h + (t0 + r) * p.sg_t + pc * E) = dg;
      }
    }
    // dden from the same rounded dnum the products use: with a fast decay
    // dnum_t . v_t + dden_t = dnum_t . (v_t - o_t) nearly cancels, and the two
    // terms must carry the same rounding of dnum for the difference to survive
    const float rden = valid ? 1.f / xden[it] : 0.f;
    V nv_;
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      nv_[e] = (T)(dv_[e] * rden);
      part += (float)nv_[e] * ov[e];
    }
    for (int off = 1; off < PPR; off <<= 1) part += __shfl_xor(part, off);
    if (valid) {
      *reinterpret_cast<V *>((T *)p.dnum + (bh * p.n + t0 + r) * DV + pc * E) = nv_;
      if (pc == 0) p.dden[bh * p.n + t0 + r] = -part;
    }
  }
  }
}

// ---------------------------------------------------------------- bwd_states
// The state at the start of every chunk, from the checkpoint the training forward
// kept at the start of each chunk range: one workgroup per (b, h), range (the
// ranges of bwd_dq / bwd_dk / bwd_dv) and share of the value columns (DS shares
// of DV/DS; the columns of S are independent), chunks first to last,
//   S <- e^{Lam} S + sum_j e^{Lam - L_j} phik_j v_j^T,   z likewise with v_j = 1,
// (the forward's state update, on the phik rows bwd_prep wrote), S_c in the dtype
// and z_c in float32 to the workspace before each chunk's update.  S [F][DV/DS]
// lives in accumulators, tile tt = wave + 8m, as G in bwd_gstate; in the first
// share thread 2f owns z[f].  The shares of one (b, h, range) go to one XCD
// (they read the same phik rows through its L2).  The next chunk's operands are
// fetched while the current chunk's products run.
template <typename T, int DK, int FH, int DV, int DS>
__global__ __launch_bounds__(kChainWaves * 64) void bwd_states(const BwdParams p) {
  using namespace bw;
  constexpr int NW = kChainWaves, NT = 64 * NW;
  constexpr int F = 2 * FH, PAD = Mma<T>::PAD, LDC_ = C + PAD, DVW = DV / DS;
  constexpr int CT = DVW / 16, TILES = (F / 16) * CT, NTT = (TILES + NW - 1) / NW;
  static_assert(2 * F <= NT && C == 64, "two threads per feature for z, 32 tokens each");
  static_assert(DVW % 16 == 0, "whole column tiles per share");
  __shared__ __align__(16) T sA[F * LDC_];    // (e^{Lam - L_j} phik_j)^T: [f][j]
  __shared__ __align__(16) T sB[DVW * LDC_];  // v^T of the share's columns: [c][j]
  constexpr int LO = DVW + PAD;
  __shared__ __align__(16) T sOut[F * LO];    // S_c of the share's columns, rounded to T
  __shared__ __align__(16) float sw[C];       // e^{Lam - L_j}, 0 past the sequence's end
  __shared__ float sLam[1];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, i = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int64_t item = blockIdx.x;  // (b, h) * ngrp + range
  int share = 0;
  if constexpr (DS > 1) {
    const int64_t rnd = blockIdx.x >> 3;
    share = (int)(rnd % DS);
    item = (rnd / DS) * 8 + (blockIdx.x & 7);
    if (item >= p.B * p.H * p.ngrp) return;
  }
  const int grp = (int)(item % p.ngrp);
  const int64_t bh = item / p.ngrp, b = bh / p.H, h = bh % p.H;
  const int col0 = share * DVW;
  const bool zshare = share == 0;
  int64_t c0, c1;
  chunk_range(p, grp, c0, c1);
  if (c0 >= c1) return;
  const int64_t BLK = (int64_t)F * DV + F;
  // checkpoint grp of this (b, h): the ranges that hold chunks, ceil(nch / per) of them
  const int64_t per = (p.nch + p.ngrp - 1) / p.ngrp, nck = (p.nch + per - 1) / per;
  const float *ck = p.sck + (bh * nck + grp) * BLK;
  f32x4 S[NTT];
#pragma unroll
  for (int m = 0; m < NTT; ++m) {
    S[m] = zero4();
    const int tt = w + NW * m;
    if (tt < TILES) {
      const int rt = tt / CT, ct = tt % CT;
#pragma unroll
      for (int r = 0; r < 4; ++r) S[m][r] = ck[(16 * rt + 4 * g + r) * DV + col0 + 16 * ct + i];
    }
  }
  const int zf_ = tid >> 1, zh = tid & 1;
  const bool zown = zshare && zh == 0 && zf_ < F;
  float zf = zown ? ck[(int64_t)F * DV + zf_] : 0.f;
  StagedT<T, C, F, NT> pf_k;
  StagedT<T, C, DVW, NT> pf_v;
  float pf_L = 0.f;  // thread t < C: the chunk-local log-decay prefix of token t
  auto load_chunk = [&](int64_t t0, int nv) {
    pf_k.load((const T *)p.phk + (bh * p.n + t0) * F, F, nv);
    pf_v.load((const T *)p.v + b * p.sv_b + h * p.sv_h + t0 * p.sv_t + col0, p.sv_t, nv);
    if (tid < C) pf_L = p.dt ? p.Lc[bh * p.n + t0 + (tid < nv ? tid : nv - 1)] : 0.f;
  };
  load_chunk(c0 * C, (int)(p.n - c0 * C < C ? p.n - c0 * C : C));
  for (int64_t c = c0; c < c1; ++c) {
    const int64_t t0 = c * C;
    const int nv = (int)(p.n - t0 < C ? p.n - t0 : C);
    // the state at the start of chunk c
    tile_to_lds<T, NTT, TILES, CT, NW>(sOut, LO, S);
    if (zown) p.wz[(bh * p.nch + c) * F + zf_] = zf;
    if (tid == nv - 1) sLam[0] = pf_L;
    __syncthreads();
    lds_to_global<T, F, DVW, NT>((T *)p.wS + (bh * p.nch + c) * ((int64_t)F * DV) + col0, DV, sOut, LO);
    if (tid < C) sw[tid] = tid < nv ? (p.dt ? __expf(sLam[0] - pf_L) : 1.f) : 0.f;
    __syncthreads();
    pf_k.store(sA, LDC_, sw);
    pf_v.store(sB, LDC_);
    const float eLam = p.dt ? __expf(sLam[0]) : 1.f;
    if (c + 1 < c1) load_chunk(t0 + C, (int)(p.n - t0 - C < C ? p.n - t0 - C : C));
    __syncthreads();
    tiles_mm<T, C, NTT, TILES, CT, NW>(S, eLam, sA, sB, LDC_);
    if (zshare && zf_ < F) {
      // z[f] += sum_j of the phik row as the products used it (rounded to the dtype):
      // threads 2f and 2f+1 each sum 32 tokens
      typedef T t4 __attribute__((ext_vector_type(4)));
      const T *row = sA + zf_ * LDC_ + 32 * zh;
      float acc = 0.f;
#pragma unroll
      for (int t = 0; t < 32; t += 4) {
        const t4 a4 = *reinterpret_cast<const t4 *>(row + t);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const T x = a4[e];
          acc += (float)x;
        }
      }
      acc += __shfl_xor(acc, 1);
      zf = eLam * zf + acc;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- bwd_gstate
// One workgroup per (b, h) and share of the value columns (DS shares of DV/DS;
// the columns of G are independent), chunks from last to first: G and g at every
// chunk's end go to the workspace; after chunk 0 they are the gradient of the
// initial state.  G [F][DV/DS] lives in accumulators, tile tt = wave + 8m; the
// first share also carries g.  With DS > 1, consecutive workgroups go to
// different XCDs and the shares of one (b, h) share an XCD (and its copy of phi(q)
// in L2).
template <typename T, int DK, int FH, int DV, int DS>
__global__ __launch_bounds__(kChainWaves * 64) void bwd_gstate(const BwdParams p) {
  using namespace bw;
  constexpr int NW = kChainWaves, NT = 64 * NW;
  constexpr int F = 2 * FH, PAD = Mma<T>::PAD, LDC_ = C + PAD, DVW = DV / DS;
  constexpr int CT = DVW / 16, TILES = (F / 16) * CT, NTT = (TILES + NW - 1) / NW;
  static_assert(DVW % 16 == 0, "whole column tiles per share");
  __shared__ __align__(16) T sA[F * LDC_];    // (e^{L_t} phiq_t)^T: [f][t]
  __shared__ __align__(16) T sB[DVW * LDC_];  // dnum^T of the share's columns: [c][t]
  constexpr int LO = DVW + PAD;
  __shared__ __align__(16) T sOut[F * LO];    // G of the share's columns, rounded to T
  __shared__ __align__(16) float sdd[C], seL[C];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, i = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int64_t bh = blockIdx.x;
  int share = 0;
  if constexpr (DS > 1) {
    const int64_t rnd = blockIdx.x >> 3;
    share = (int)(rnd % DS);
    bh = (rnd / DS) * 8 + (blockIdx.x & 7);
    if (bh >= p.B * p.H) return;
  }
  const int col0 = share * DVW;
  const bool zshare = share == 0;  // the share that carries g
  // g[f] = sum_t (e^{L_t} phiq_t)[f] dden_t: threads 2f and 2f+1 each sum half of
  // the chunk's tokens; thread 2f owns g[f]
  const int gf = tid >> 1, gh = tid & 1;
  const bool gown = zshare && gh == 0 && gf < F;
  static_assert(2 * F <= NT && C == 64, "two threads per feature, 32 tokens each");
  const int64_t BLK = (int64_t)F * DV + F;
  f32x4 G[NTT];
  float gz = 0.f;
#pragma unroll
  for (int m = 0; m < NTT; ++m) {
    G[m] = zero4();
    const int tt = w + NW * m;
    if (tt < TILES && p.ds_final) {
      const int rt = tt / CT, ct = tt % CT;
#pragma unroll
      for (int r = 0; r < 4; ++r) G[m][r] = p.ds_final[bh * BLK + (16 * rt + 4 * g + r) * DV + col0 + 16 * ct + i];
    }
  }
  if (gown && p.ds_final) gz = p.ds_final[bh * BLK + (int64_t)F * DV + gf];
  // the (earlier) chunk's phi(q) and dnum are fetched while the current chunk's
  // products run: the chunks are visited one after the other, so each chunk's load
  // latency would otherwise stand alone
  StagedT<T, C, F, NT> pf_q;
  StagedT<T, C, DVW, NT> pf_n;
  // and its per-token log-decay and dden (thread t < C holds token t)
  float pf_L = 0.f, pf_dd = 0.f;
  bool pf_ok = false;
  auto load_tok = [&](int64_t t0, int nv) {
    if (tid < C) {
      pf_ok = tid < nv;
      pf_L = pf_ok && p.dt ? p.Lc[bh * p.n + t0 + tid] : 0.f;
      pf_dd = pf_ok ? p.dden[bh * p.n + t0 + tid] : 0.f;
    }
  };
  if (p.nch > 0) {
    const int64_t t0 = (p.nch - 1) * C;
    const int nv = (int)(p.n - t0 < C ? p.n - t0 : C);
    pf_q.load((const T *)p.phq + (bh * p.n + t0) * F, F, nv);
    pf_n.load((const T *)p.dnum + (bh * p.n + t0) * DV + col0, DV, nv);
    load_tok(t0, nv);
  }
  for (int64_t c = p.nch - 1; c >= 0; --c) {
    const int64_t t0 = c * C;
    const int nv = (int)(p.n - t0 < C ? p.n - t0 : C);
    // G, g at the end of chunk c
    tile_to_lds<T, NTT, TILES, CT, NW>(sOut, LO, G);
    if (gown) p.gz[(bh * p.nch + c) * F + gf] = gz;
    if (tid < C) {
      seL[tid] = pf_ok ? (p.dt ? __expf(pf_L) : 1.f) : 0.f;
      sdd[tid] = pf_dd;
    }
    __syncthreads();
    lds_to_global<T, F, DVW, NT>((T *)p.gS + (bh * p.nch + c) * ((int64_t)F * DV) + col0, DV, sOut, LO);
    pf_q.store(sA, LDC_, seL);
    pf_n.store(sB, LDC_);
    if (c > 0) {
      const int64_t tp = t0 - C;  // the previous chunk is always full
      pf_q.load((const T *)p.phq + (bh * p.n + tp) * F, F, C);
      pf_n.load((const T *)p.dnum + (bh * p.n + tp) * DV + col0, DV, C);
      load_tok(tp, C);
    }
    const float eLam = seL[nv - 1];  // e^{Lambda} of the chunk (1 without decay)
    __syncthreads();
    tiles_mm<T, C, NTT, TILES, CT, NW>(G, eLam, sA, sB, LDC_);
    if (zshare && gf < F) {
      typedef T t4 __attribute__((ext_vector_type(4)));
      const T *row = sA + gf * LDC_ + 32 * gh;
      const float *dd = sdd + 32 * gh;
      float acc = 0.f;
#pragma unroll
      for (int t = 0; t < 32; t += 4) {
        const t4 a4 = *reinterpret_cast<const t4 *>(row + t);
        const f32x4 d4 = *reinterpret_cast<const f32x4 *>(dd + t);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const T x = a4[e];
          acc = __builtin_fmaf((float)x, d4[e], acc);
        }
      }
      acc += __shfl_xor(acc, 1);
      gz = eLam * gz + acc;
    }
    __syncthreads();
  }
  if (p.ds_init) {
#pragma unroll
    for (int m = 0; m < NTT; ++m) {
      const int tt = w + NW * m;
      if (tt < TILES) {
        const int rt = tt / CT, ct = tt % CT;
#pragma unroll
        for (int r = 0; r < 4; ++r) p.ds_init[bh * BLK + (16 * rt + 4 * g + r) * DV + col0 + 16 * ct + i] = G[m][r];
      }
    }
    if (gown) p.ds_init[bh * BLK + (int64_t)F * DV + gf] = gz;
  }
}


// ---------------------------------------------------------------- bwd_dq
// dphiq -> du_q -> dq = du_q W_q^T, and this workgroup's share of dW_q.
template <typename T, int DK, int FH, int DV, bool ROPE>
__global__ __launch_bounds__(bwd_waves(ROPE) * 64) void bwd_dq(const BwdParams p) {
  using namespace bw;
  constexpr int F = 2 * FH, PAD = Mma<T>::PAD;
  constexpr int NW = bwd_waves(ROPE), NT = 64 * NW, NH = NW / 4;  // waves, threads, waves per 16-row band
  constexpr int LW = FH + PAD, LN = DV + PAD, LVQ = (DV > F ? DV : F) + PAD, LC = C + PAD, LS = DV + PAD;
  constexpr int OW = 0, ON = OW + DK * LW, OVQ = ON + C * LN, OA = OVQ + C * LVQ, OKT = OA + C * LC,
                OS = OKT + F * LC, ODU = OS + F * LS, ODUT = ODU + C * LW, OXT = ODUT + FH * LC, TOT = OXT + DK * LC;
  __shared__ __align__(16) T sm[TOT];
  __shared__ float sL[C], sdd[C], sz[F], sQs[NH][C];
  __shared__ double sRev[ROPE ? FH : 1];
  T *sW = sm + OW, *sDN = sm + ON, *sVQ = sm + OVQ, *sA = sm + OA, *sKT = sm + OKT, *sS = sm + OS, *sDu = sm + ODU,
    *sDuT = sm + ODUT, *sXT = sm + OXT;
  constexpr int FT = FH / 16, TW = (DK / 16) * FT, NTW = (TW + NW - 1) / NW;
  constexpr int MJ = (C / 16) / NH, MF = (FT + NH - 1) / NH, MD = (DK / 16 + NH - 1) / NH;  // tiles per wave
  static_assert((C / 16) % NH == 0, "key tiles split evenly");
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, i = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rt = w & 3, hw = w >> 2;  // the wave's row band and its share of the band's column tiles
  const int grp = blockIdx.x % p.ngrp;
  const int64_t bh = blockIdx.x / p.ngrp, b = bh / p.H, h = bh % p.H;
  int64_t c0, c1;
  chunk_range(p, grp, c0, c1);
  load_w<T, DK, FH, NT>(sW, LW, (const T *)p.wq + h * p.sw_h, false);
  if constexpr (ROPE) fill_rev(sRev, p);
  const double pos_b = ROPE ? pos_of(p, b) : 0.0;
  f32x4 dW[NTW];
#pragma unroll
  for (int m = 0; m < NTW; ++m) dW[m] = zero4();
  // A chunk's operands are fetched while the previous chunk's products run (the chunks
  // of a range are visited one after another, so each load latency would otherwise
  // stand alone); all of them go out before the first LDS write.  The four-wave
  // (rotary) variants hold twice the registers per thread for them and fetch at the
  // chunk's top instead.
  constexpr bool PREFETCH = NH > 1;
  Staged<T, C, F, NT> phq_next;  // phi(q) rows, written over v once A is formed
  Staged<T, C, DV, NT> st_dn, st_v;
  StagedT<T, C, DK, NT> st_x;
  StagedT<T, C, F, NT> st_k;
  Staged<T, F, DV, NT> st_s;
  float tl = 0.f, tdd = 0.f, tz = 0.f;  // per-token log-decay and dden, z at the chunk start
  auto fetch = [&](int64_t c) {
    const int64_t t0 = c * C;
    const int nv = (int)(p.n - t0 < C ? p.n - t0 : C);
    st_dn.load((const T *)p.dnum + (bh * p.n + t0) * DV, DV, nv);
    st_v.load((const T *)p.v + b * p.sv_b + h * p.sv_h + t0 * p.sv_t, p.sv_t, nv);
    st_x.load((const T *)p.q + b * p.sq_b + h * p.sq_h + t0 * p.sq_t, p.sq_t, nv);
    st_k.load((const T *)p.phk + (bh * p.n + t0) * F, F, nv);
    st_s.load((const T *)p.wS + (bh * p.nch + c) * ((int64_t)F * DV), DV, F);
    phq_next.load((const T *)p.phq + (bh * p.n + t0) * F, F, nv);
    if (tid < C) {
      tl = p.dt ? p.Lc[bh * p.n + t0 + (tid < nv ? tid : nv - 1)] : 0.f;  // padding rows: log a = 0
      tdd = tid < nv ? p.dden[bh * p.n + t0 + tid] : 0.f;
    }
    if (tid < F) tz = p.wz[(bh * p.nch + c) * F + tid];
  };
  if (PREFETCH && c0 < c1) fetch(c0);
  for (int64_t c = c0; c < c1; ++c) {
    const int64_t t0 = c * C;
    const int nv = (int)(p.n - t0 < C ? p.n - t0 : C);
    if constexpr (!PREFETCH) fetch(c);
    st_dn.store(sDN, LN);
    st_v.store(sVQ, LVQ);
    st_x.store(sXT, LC);
    st_k.store(sKT, LC);
    st_s.store(sS, LS);
    if (tid < C) {
      sL[tid] = tl;
      sdd[tid] = tdd;
    }
    if (tid < F) sz[tid] = tz;
    __syncthreads();
    // A[t][j] = [j <= t] e^{L_t - L_j} (dnum_t . v_j + dden_t); rows t of this wave's
    // band, key tiles jt = hw + NH m
    Frags<T, DV> fdn;  // the band's dnum rows, shared by the wave's tiles
    fdn.load(sDN + 16 * rt * LN, LN);
#pragma unroll
    for (int m = 0; m < MJ; ++m) {
      const int jt = hw + NH * m;
      const f32x4 d1 = mm(fdn, sVQ + 16 * jt * LVQ, LVQ, zero4());
      f32x4 a;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * rt + 4 * g + r, j = 16 * jt + i;
        a[r] = j <= t ? __expf(sL[t] - sL[j]) * (d1[r] + sdd[t]) : 0.f;
      }
      put<T>(sA + 16 * rt * LC + 16 * jt, LC, a);
    }
    __syncthreads();
    phq_next.store(sVQ, LVQ);
    if (PREFETCH && c + 1 < c1) fetch(c + 1);
    __syncthreads();
    // dphiq[t][F] = sum_j A[t][j] phik[j][F] + e^{L_t} (S_c dnum_t + dden_t z_c)[F], for
    // the feature tiles ft = hw + NH m and ft + FT (the pair that du combines)
    f32x4 dph[MF][2];
    float qs[4] = {0.f, 0.f, 0.f, 0.f};  // Q_t partial: phiq_t . (inter part of dphiq_t)
    Frags<T, C> fa;  // the band's rows of A and of dnum, shared by the feature tiles
    Frags<T, DV> fdn2;
    fa.load(sA + 16 * rt * LC, LC);
    fdn2.load(sDN + 16 * rt * LN, LN);
#pragma unroll
    for (int m = 0; m < MF; ++m) {
      const int fb = hw + NH * m;
      if (fb < FT) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int ft = fb + hf * FT;
          const f32x4 a1 = mm(fa, sKT + 16 * ft * LC, LC, zero4());
          const f32x4 a2 = mm(fdn2, sS + 16 * ft * LS, LS, zero4());
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = 16 * rt + 4 * g + r;
            const float eL = t < nv ? (p.dt ? __expf(sL[t]) : 1.f) : 0.f;
            const float inter = eL * (a2[r] + sdd[t] * sz[16 * ft + i]);
            dph[m][hf][r] = a1[r] + inter;
            qs[r] += (float)sVQ[t * LVQ + 16 * ft + i] * inter;
          }
        }
      }
    }
    if (p.a_log) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * rt + 4 * g + r;
        const float q4 = sum16(qs[r]);
        if constexpr (NH == 1) {
          if (i == 0 && t < nv) p.eQ[bh * p.n + t0 + t] = q4;
        } else {
          if (i == 0) sQs[hw][t] = q4;  // the band's waves' partials are added below
        }
      }
    }
    // du_q = phiq * dphiq over [u, -u] (unturned frame): du[f] = du'[f] - du'[f + FH]
    if constexpr (ROPE) {
      static_assert(NH == 1, "the rotation pairs feature tiles across the column split");
      f32x4 d[F / 16];
#pragma unroll
      for (int m = 0; m < MF; ++m) {
        d[m] = dph[m][0];
        d[m + FT] = dph[m][1];
      }
      const float zero[4] = {0.f, 0.f, 0.f, 0.f};
      phi_dphi<F / 16>(d, sVQ + 16 * rt * LVQ, LVQ, sRev, pos_b + (double)(t0 + 16 * rt + 4 * g), zero, p.rope_dims);
#pragma unroll
      for (int m = 0; m < MF; ++m) {
        dph[m][0] = d[m];
        dph[m][1] = d[m + FT];
      }
    }
#pragma unroll
    for (int m = 0; m < MF; ++m) {
      const int ft = hw + NH * m;
      if (ft < FT) {
        f32x4 du;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * rt + 4 * g + r, f = 16 * ft + i;
          du[r] = ROPE ? dph[m][0][r] - dph[m][1][r]
                       : (float)sVQ[t * LVQ + f] * dph[m][0][r] - (float)sVQ[t * LVQ + FH + f] * dph[m][1][r];
        }
        put<T>(sDu + 16 * rt * LW + 16 * ft, LW, du);
        put_t<T>(sDuT + 16 * ft * LC + 16 * rt, LC, du);
      }
    }
    __syncthreads();
    if constexpr (NH > 1) {
      if (p.a_log && tid < nv) {
        float q = 0.f;
#pragma unroll
        for (int u = 0; u < NH; ++u) q += sQs[u][tid];
        p.eQ[bh * p.n + t0 + tid] = q;
      }
    }
    // dq = du_q W_q^T (stored straight from the accumulators: staging the rows
    // through LDS for 16-byte stores measured 6 us slower on the Pythia layer)
    T *DQ = (T *)p.dq + b * p.sq_b + h * p.sq_h + t0 * p.sq_t;
    Frags<T, FH> fdu;  // the band's du rows, shared by the wave's d tiles
    fdu.load(sDu + 16 * rt * LW, LW);
#pragma unroll
    for (int m = 0; m < MD; ++m) {
      const int it = hw + NH * m;
      if (it < DK / 16) {
        const f32x4 a = mm(fdu, sW + 16 * it * LW, LW, zero4());
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * rt + 4 * g + r;
          if (t < nv) DQ[t * p.sq_t + 16 * it + i] = (T)a[r];
        }
      }
    }
    // dW_q += X_q^T du_q
#pragma unroll
    for (int m = 0; m < NTW; ++m) {
      const int tt = w + NW * m;
      if (tt < TW) dW[m] = mm<T, C>(sXT + 16 * (tt / FT) * LC, LC, sDuT + 16 * (tt % FT) * LC, LC, dW[m]);
    }
    __syncthreads();
  }
  float *part = p.dwq_part + (bh * p.ngrp + grp) * (int64_t)(DK * FH);
#pragma unroll
  for (int m = 0; m < NTW; ++m) {
    const int tt = w + NW * m;
    if (tt < TW) {
#pragma unroll
      for (int r = 0; r < 4; ++r) part[(16 * (tt / FT) + 4 * g + r) * FH + 16 * (tt % FT) + i] = dW[m][r];
    }
  }
}

// ---------------------------------------------------------------- bwd_dk
// dphik -> dL_t and du_k (softmax) -> dk = du_k W_k^T, and the share of dW_k.
template <typename T, int DK, int FH, int DV, bool ROPE>
__global__ __launch_bounds__(bwd_waves(ROPE) * 64) void bwd_dk(const BwdParams p) {
  using namespace bw;
  constexpr int F = 2 * FH, PAD = Mma<T>::PAD;
  constexpr int NW = bwd_waves(ROPE), NT = 64 * NW, NH = NW / 4;  // waves, threads, waves per 16-row band
  constexpr int LW = FH + PAD, LV = DV + PAD, LNK = (DV > F ? DV : F) + PAD, LC = C + PAD, LG = DV + PAD;
  constexpr int OW = 0, OV = OW + DK * LW, ONK = OV + C * LV, OA = ONK + C * LNK, OQT = OA + C * LC,
                OG = OQT + F * LC, ODU = OG + F * LG, ODUT = ODU + C * LW, OXT = ODUT + FH * LC, TOT = OXT + DK * LC;
  __shared__ __align__(16) T sm[TOT];
  __shared__ float sL[C], sdd[C], sg[F], sDot[NH][C], sKs[NH][C];
  __shared__ double sRev[ROPE ? FH : 1];
  T *sW = sm + OW, *sV = sm + OV, *sNK = sm + ONK, *sAT = sm + OA, *sQT = sm + OQT, *sG = sm + OG, *sDu = sm + ODU,
    *sDuT = sm + ODUT, *sXT = sm + OXT;
  constexpr int FT = FH / 16, TW = (DK / 16) * FT, NTW = (TW + NW - 1) / NW;
  constexpr int MJ = (C / 16) / NH, MF = (FT + NH - 1) / NH, MD = (DK / 16 + NH - 1) / NH;  // tiles per wave
  static_assert((C / 16) % NH == 0, "query tiles split evenly");
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, i = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rt = w & 3, hw = w >> 2;  // the wave's row band and its share of the band's column tiles
  const int grp = blockIdx.x % p.ngrp;
  const int64_t bh = blockIdx.x / p.ngrp, b = bh / p.H, h = bh % p.H;
  int64_t c0, c1;
  chunk_range(p, grp, c0, c1);
  load_w<T, DK, FH, NT>(sW, LW, (const T *)p.wk + h * p.sw_h, false);
  if constexpr (ROPE) fill_rev(sRev, p);
  const double pos_b = ROPE ? pos_of(p, b) : 0.0;
  f32x4 dW[NTW];
#pragma unroll
  for (int m = 0; m < NTW; ++m) dW[m] = zero4();
  // the next chunk's operands are fetched during this chunk's products, as in bwd_dq
  constexpr bool PREFETCH = NH > 1;
  Staged<T, C, F, NT> phk_next;  // phi(k) rows, written over dnum once A^T is formed
  Staged<T, C, DV, NT> st_dn, st_v;
  StagedT<T, C, DK, NT> st_x;
  StagedT<T, C, F, NT> st_q;
  Staged<T, F, DV, NT> st_g;
  float tl = 0.f, tdd = 0.f, tg = 0.f;  // per-token log-decay and dden, g at the chunk end
  auto fetch = [&](int64_t c) {
    const int64_t t0 = c * C;
    const int nv = (int)(p.n - t0 < C ? p.n - t0 : C);
    st_dn.load((const T *)p.dnum + (bh * p.n + t0) * DV, DV, nv);
    st_v.load((const T *)p.v + b * p.sv_b + h * p.sv_h + t0 * p.sv_t, p.sv_t, nv);
    st_x.load((const T *)p.k + b * p.sk_b + h * p.sk_h + t0 * p.sk_t, p.sk_t, nv);
    st_q.load((const T *)p.phq + (bh * p.n + t0) * F, F, nv);
    st_g.load((const T *)p.gS + (bh * p.nch + c) * ((int64_t)F * DV), DV, F);
    phk_next.load((const T *)p.phk + (bh * p.n + t0) * F, F, nv);
    if (tid < C) {
      tl = p.dt ? p.Lc[bh * p.n + t0 + (tid < nv ? tid : nv - 1)] : 0.f;  // padding rows: log a = 0
      tdd = tid < nv ? p.dden[bh * p.n + t0 + tid] : 0.f;
    }
    if (tid < F) tg = p.gz[(bh * p.nch + c) * F + tid];
  };
  if (PREFETCH && c0 < c1) fetch(c0);
  for (int64_t c = c0; c < c1; ++c) {
    const int64_t t0 = c * C;
    const int nv = (int)(p.n - t0 < C ? p.n - t0 : C);
    if constexpr (!PREFETCH) fetch(c);
    st_dn.store(sNK, LNK);
    st_v.store(sV, LV);
    st_x.store(sXT, LC);
    st_q.store(sQT, LC);
    st_g.store(sG, LG);
    if (tid < C) {
      sL[tid] = tl;
      sdd[tid] = tdd;
    }
    if (tid < F) sg[tid] = tg;
    __syncthreads();
    // A^T[j][t] = [j <= t] e^{L_t - L_j} (v_j . dnum_t + dden_t); rows j of this wave's
    // band, query tiles tt = hw + NH m
    Frags<T, DV> fv;  // the band's v rows, shared by the wave's tiles
    fv.load(sV + 16 * rt * LV, LV);
#pragma unroll
    for (int m = 0; m < MJ; ++m) {
      const int tt = hw + NH * m;
      const f32x4 d1 = mm(fv, sNK + 16 * tt * LNK, LNK, zero4());
      f32x4 a;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * rt + 4 * g + r, t = 16 * tt + i;
        a[r] = j <= t ? __expf(sL[t] - sL[j]) * (d1[r] + sdd[t]) : 0.f;
      }
      put<T>(sAT + 16 * rt * LC + 16 * tt, LC, a);
    }
    __syncthreads();
    phk_next.store(sNK, LNK);
    if (PREFETCH && c + 1 < c1) fetch(c + 1);
    __syncthreads();
    // dphik[j][F] = sum_t A^T[j][t] phiq[t][F] + e^{Lam - L_j} (G v_j + g)[F], for the
    // feature tiles ft = hw + NH m and ft + FT (the pair that du combines)
    const float Lam = sL[nv - 1];
    f32x4 dph[MF][2];
    float ks[4] = {0.f, 0.f, 0.f, 0.f};  // K_j partial: phik_j . (inter part of dphik_j)
    float ds[4] = {0.f, 0.f, 0.f, 0.f};  // phik_j . dphik_j partial
    Frags<T, C> fat;  // the band's rows of A^T and of v, shared by the feature tiles
    Frags<T, DV> fv2;
    fat.load(sAT + 16 * rt * LC, LC);
    fv2.load(sV + 16 * rt * LV, LV);
#pragma unroll
    for (int m = 0; m < MF; ++m) {
      const int fb = hw + NH * m;
      if (fb < FT) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int ft = fb + hf * FT;
          const f32x4 a1 = mm(fat, sQT + 16 * ft * LC, LC, zero4());
          const f32x4 a2 = mm(fv2, sG + 16 * ft * LG, LG, zero4());
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = 16 * rt + 4 * g + r;
            const float e = j < nv ? (p.dt ? __expf(Lam - sL[j]) : 1.f) : 0.f;
            const float inter = e * (a2[r] + sg[16 * ft + i]);
            const float phk = (float)sNK[j * LNK + 16 * ft + i];
            dph[m][hf][r] = a1[r] + inter;
            ks[r] += phk * inter;
            ds[r] += phk * dph[m][hf][r];
          }
        }
      }
    }
    // phik . dphik per token for the softmax backward, and K_j
    float dot[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 16 * rt + 4 * g + r;
      dot[r] = sum16(ds[r]);
      const float k4 = sum16(ks[r]);
      if constexpr (NH == 1) {
        if (p.a_log && i == 0 && j < nv) p.eK[bh * p.n + t0 + j] = k4;
      } else {
        if (i == 0) {
          sDot[hw][j] = dot[r];
          sKs[hw][j] = k4;
        }
      }
    }
    if constexpr (NH > 1) {
      // the band's waves hold halves of each row: add their partials
      __syncthreads();
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * rt + 4 * g + r;
        float d = 0.f;
#pragma unroll
        for (int u = 0; u < NH; ++u) d += sDot[u][j];
        dot[r] = d;
      }
      if (p.a_log && tid < nv) {
        float k = 0.f;
#pragma unroll
        for (int u = 0; u < NH; ++u) k += sKs[u][tid];
        p.eK[bh * p.n + t0 + tid] = k;
      }
    }
    // du_k = phik * (dphik - phik . dphik) over [u, -u] (unturned frame)
    if constexpr (ROPE) {
      static_assert(NH == 1, "the rotation pairs feature tiles across the column split");
      f32x4 d[F / 16];
#pragma unroll
      for (int m = 0; m < MF; ++m) {
        d[m] = dph[m][0];
        d[m + FT] = dph[m][1];
      }
      phi_dphi<F / 16>(d, sNK + 16 * rt * LNK, LNK, sRev, pos_b + (double)(t0 + 16 * rt + 4 * g), dot, p.rope_dims);
#pragma unroll
      for (int m = 0; m < MF; ++m) {
        dph[m][0] = d[m];
        dph[m][1] = d[m + FT];
      }
    }
#pragma unroll
    for (int m = 0; m < MF; ++m) {
      const int ft = hw + NH * m;
      if (ft < FT) {
        f32x4 du;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * rt + 4 * g + r, f = 16 * ft + i;
          du[r] = ROPE ? dph[m][0][r] - dph[m][1][r]
                       : (float)sNK[j * LNK + f] * (dph[m][0][r] - dot[r]) -
                             (float)sNK[j * LNK + FH + f] * (dph[m][1][r] - dot[r]);
        }
        put<T>(sDu + 16 * rt * LW + 16 * ft, LW, du);
        put_t<T>(sDuT + 16 * ft * LC + 16 * rt, LC, du);
      }
    }
    __syncthreads();
    T *DK_ = (T *)p.dk + b * p.sk_b + h * p.sk_h + t0 * p.sk_t;
    Frags<T, FH> fdu;  // the band's du rows, shared by the wave's d tiles
    fdu.load(sDu + 16 * rt * LW, LW);
#pragma unroll
    for (int m = 0; m < MD; ++m) {
      const int it = hw + NH * m;
      if (it < DK / 16) {
        const f32x4 a = mm(fdu, sW + 16 * it * LW, LW, zero4());
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * rt + 4 * g + r;
          if (j < nv) DK_[j * p.sk_t + 16 * it + i] = (T)a[r];
        }
      }
    }
#pragma unroll
    for (int m = 0; m < NTW; ++m) {
      const int tt = w + NW * m;
      if (tt < TW) dW[m] = mm<T, C>(sXT + 16 * (tt / FT) * LC, LC, sDuT + 16 * (tt % FT) * LC, LC, dW[m]);
    }
    __syncthreads();
  }
  float *part = p.dwk_part + (bh * p.ngrp + grp) * (int64_t)(DK * FH);
#pragma unroll
  for (int m = 0; m < NTW; ++m) {
    const int tt = w + NW * m;
    if (tt < TW) {
#pragma unroll
      for (int r = 0; r < 4; ++r) part[(16 * (tt / FT) + 4 * g + r) * FH + 16 * (tt % FT) + i] = dW[m][r];
    }
  }
}

// ---------------------------------------------------------------- bwd_dv
// dv[j] = sum_t [j <= t] e^{L_t - L_j} (phiq_t . phik_j) dnum_t + e^{Lam - L_j} G^T phik_j
template <typename T, int DK, int FH, int DV>
__global__ __launch_bounds__(bwd_waves(false) * 64) void bwd_dv(const BwdParams p) {
  using namespace bw;
  constexpr int F = 2 * FH, PAD = Mma<T>::PAD;
  constexpr int NW = bwd_waves(false), NT = 64 * NW, NH = NW / 4;  // waves, threads, waves per 16-row band
  constexpr int LF = F + PAD, LC = C + PAD, LV = DV + PAD;
  constexpr int OK_ = 0, OQ = OK_ + C * LF, OP = OQ + C * LF, ONT = OP + C * LC, OGT = ONT + DV * LC,
                OV = OGT + DV * LF, ON = OV + C * LV, TOT = ON + C * LV;
  constexpr int MT = (C / 16) / NH, MV = (DV / 16 + NH - 1) / NH;  // tiles per wave
  static_assert((C / 16) % NH == 0, "query tiles split evenly");
  __shared__ __align__(16) T sm[TOT];
  __shared__ float sL[C], sdd[C], sCol[4][C], sRow[NH][C];
  __shared__ double sX[NW];
  T *sK = sm + OK_, *sQ = sm + OQ, *sP = sm + OP, *sNT = sm + ONT, *sGT = sm + OGT, *sV = sm + OV, *sN = sm + ON;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, i = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rt = w & 3, hw = w >> 2;  // the wave's row band and its share of the band's column tiles
  const int grp = blockIdx.x % p.ngrp;
  const int64_t bh = blockIdx.x / p.ngrp, b = bh / p.H, h = bh % p.H;
  int64_t c0, c1;
  chunk_range(p, grp, c0, c1);
  static_assert(LF >= DV + PAD, "dv rows fit the phi(q) buffer");
  // dv rows of a chunk are formed in sQ (dead by then) and leave as 16-byte row
  // pieces at the top of the next iteration, while its operand loads are in flight
  // (155 -> 147 us on the Pythia layer; the same for dq and dk measured slower)
  T *DV_ = nullptr;
  int nv_prev = 0;
  // the next chunk's operands are fetched during this chunk's products, as in bwd_dq
  Staged<T, C, F, NT> st_k, st_q;
  StagedT<T, C, DV, NT> st_nt;
  StagedT<T, F, DV, NT> st_gt;
  float tl = 0.f, tdd = 0.f;  // per-token log-decay and dden
  auto fetch = [&](int64_t c) {
    const int64_t t0 = c * C;
    const int nv = (int)(p.n - t0 < C ? p.n - t0 : C);
    st_k.load((const T *)p.phk + (bh * p.n + t0) * F, F, nv);
    st_q.load((const T *)p.phq + (bh * p.n + t0) * F, F, nv);
    st_nt.load((const T *)p.dnum + (bh * p.n + t0) * DV, DV, nv);
    st_gt.load((const T *)p.gS + (bh * p.nch + c) * ((int64_t)F * DV), DV, F);
    if (tid < C) {
      tl = p.dt ? p.Lc[bh * p.n + t0 + (tid < nv ? tid : nv - 1)] : 0.f;  // padding rows: log a = 0
      tdd = tid < nv ? p.dden[bh * p.n + t0 + tid] : 0.f;
    }
  };
  if (c0 < c1) fetch(c0);
  for (int64_t c = c0; c < c1; ++c) {
    const int64_t t0 = c * C;
    const int nv = (int)(p.n - t0 < C ? p.n - t0 : C);
    {
      if (c > c0) {
        rows_to_global<T, C, DV, NT>(DV_, p.sv_t, sQ, LF, nv_prev);
        __syncthreads();
      }
      st_k.store(sK, LF);
      st_q.store(sQ, LF);
      st_nt.store(sNT, LC);
      st_gt.store(sGT, LF);
      if (tid < C) {
        sL[tid] = tl;
        sdd[tid] = tdd;
      }
    }
    if (p.a_log) {
      stage<T, C, DV, NT>(sV, LV, (const T *)p.v + b * p.sv_b + h * p.sv_h + t0 * p.sv_t, p.sv_t, nv);
      stage<T, C, DV, NT>(sN, LV, (const T *)p.dnum + (bh * p.n + t0) * DV, DV, nv);
    }
    if (c + 1 < c1) fetch(c + 1);
    __syncthreads();
    // Pt[j][t] = [j <= t] e^{L_t - L_j} phik_j . phiq_t, and for the decay gradient the
    // pair weights W^T[j][t] = [j < t] Pt[j][t] (v_j . dnum_t + dden_t): their sums
    // along t (pairs with key j) and along j (pairs with query t); rows j of the wave's
    // band, query tiles tt = hw + NH m
    float rowsum[4] = {0.f, 0.f, 0.f, 0.f};
    Frags<T, F> fk;  // the band's phi(k) rows, shared by every tile below
    fk.load(sK + 16 * rt * LF, LF);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int tt = hw + NH * m;
      const f32x4 s = mm(fk, sQ + 16 * tt * LF, LF, zero4());
      f32x4 a, d1 = zero4();
      if (p.a_log) d1 = mm<T, DV>(sV + 16 * rt * LV, LV, sN + 16 * tt * LV, LV, zero4());
      float colsum = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * rt + 4 * g + r, t = 16 * tt + i;
        a[r] = j <= t ? __expf(sL[t] - sL[j]) * s[r] : 0.f;
        const float wt = j < t ? a[r] * (d1[r] + sdd[t]) : 0.f;
        rowsum[r] += wt;
        colsum += wt;
      }
      if (p.a_log) {
        colsum += __shfl_xor(colsum, 16);
        colsum += __shfl_xor(colsum, 32);
        if (g == 0) sCol[rt][16 * tt + i] = colsum;
      }
      put<T>(sP + 16 * rt * LC + 16 * tt, LC, a);
    }
    if (p.a_log) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float rs = sum16(rowsum[r]);
        if (i == 0) sRow[hw][16 * rt + 4 * g + r] = rs;
      }
      // X_c = e^{Lam} (<G_end, S_c> + <g_end, z_c>): pairs spanning the whole chunk
      const T *Sc = (const T *)p.wS + (bh * p.nch + c) * ((int64_t)F * DV);
      const T *Gc = (const T *)p.gS + (bh * p.nch + c) * ((int64_t)F * DV);
      typedef typename Vec<T>::type V;
      constexpr int EV = ep<T>(), NV = F * DV / EV, PV = (NV + NT - 1) / NT;
      V sv[PV], gv[PV];
#pragma unroll
      for (int m = 0; m < PV; ++m) {
        const bool ok = tid + NT * m < NV;
        sv[m] = ok ? reinterpret_cast<const V *>(Sc)[tid + NT * m] : V{};
        gv[m] = ok ? reinterpret_cast<const V *>(Gc)[tid + NT * m] : V{};
      }
      double x = 0.0;
#pragma unroll
      for (int m = 0; m < PV; ++m) {
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < EV; ++e) part += (float)sv[m][e] * (float)gv[m][e];
        x += (double)part;
      }
      if (tid < F) x += (double)p.wz[(bh * p.nch + c) * F + tid] * p.gz[(bh * p.nch + c) * F + tid];
      for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
      if (lane == 0) sX[w] = x;
    }
    __syncthreads();
    if (p.a_log) {
      // per token: (pairs with key u, query later in the chunk) - (pairs with query u,
      // key earlier in the chunk); the chunk-level constant X_c
      if (tid < nv) {
        float rs = 0.f;
#pragma unroll
        for (int u = 0; u < NH; ++u) rs += sRow[u][tid];
        p.eW[bh * p.n + t0 + tid] = rs - (sCol[0][tid] + sCol[1][tid] + sCol[2][tid] + sCol[3][tid]);
      }
      if (tid == 0) {
        const float eLam = p.dt ? __expf(sL[nv - 1]) : 1.f;
        double xs = 0.0;
#pragma unroll
        for (int u = 0; u < NW; ++u) xs += sX[u];
        p.Xc[bh * p.nch + c] = (float)(xs * eLam);
      }
    }
    const float Lam = sL[nv - 1];
    DV_ = (T *)p.dv + b * p.sv_b + h * p.sv_h + t0 * p.sv_t;
    nv_prev = nv;
    Frags<T, C> fp;  // the band's rows of the masked scores
    fp.load(sP + 16 * rt * LC, LC);
#pragma unroll
    for (int m = 0; m < MV; ++m) {
      const int ct = hw + NH * m;
      if (ct < DV / 16) {
        const f32x4 a1 = mm(fp, sNT + 16 * ct * LC, LC, zero4());
        const f32x4 a2 = mm(fk, sGT + 16 * ct * LF, LF, zero4());
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * rt + 4 * g + r;
          const float e = p.dt ? __expf(Lam - sL[j]) : 1.f;
          sQ[j * LF + 16 * ct + i] = (T)(a1[r] + e * a2[r]);  // rows into sQ
        }
      }
    }
    __syncthreads();
  }
  if (c1 > c0) rows_to_global<T, C, DV, NT>(DV_, p.sv_t, sQ, LF, nv_prev);
}

// ---------------------------------------------------------------- bwd_decay
// Per (b, h): d log a_t = X_c + sum_{s >= t} Q_s + sum_{u < t} (K_u + eW_u), with
// the chunk-local sums taken by one wave per chunk (float64); then d dt_t =
// d log a_t (-sigmoid(dt_t) e^{A_log}) and the (b, h) share of dA_log = sum_t
// d log a_t log a_t.
__global__ __launch_bounds__(256) void bwd_decay(const BwdParams p) {
  __shared__ double sRed[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t bh = blockIdx.x, b = bh / p.H, h = bh % p.H;
  const float expA = expf(p.a_log[h]);
  double da = 0.0;
  for (int64_t c = w; c < p.nch; c += 4) {
    const int64_t t = c * 64 + lane;
    const bool valid = t < p.n;
    const double q = valid ? p.eQ[bh * p.n + t] : 0.0;
    const double e = valid ? (double)p.eK[bh * p.n + t] + p.eW[bh * p.n + t] : 0.0;
    double qsum = q;
    for (int off = 32; off > 0; off >>= 1) qsum += __shfl_xor(qsum, off);
    const double excl = wave_inclusive_scan(e - q) - (e - q);  // sum_{u < t} (e_u - q_u)
    const double dla = (double)p.Xc[bh * p.nch + c] + qsum + excl;
    if (valid) {
      const int64_t off = b * p.sdt_b + h * p.sdt_h + t * p.sdt_t;
      const float x = p.dt[off];
      const float sig = 1.f / (1.f + expf(-x));
      p.ddt[off] = (float)(dla * (double)(-sig * expA));
      da += dla * (double)(-softplus_f32(x) * expA);
    }
  }
  for (int off = 32; off > 0; off >>= 1) da += __shfl_xor(da, off);
  if (lane == 0) sRed[w] = da;
  __syncthreads();
  if (tid == 0) p.da_part[bh] = (float)(sRed[0] + sRed[1] + sRed[2] + sRed[3]);
}

// ---------------------------------------------------------------- bwd_reduce
// dW = sum of the workgroup shares (over every (b, h) for a shared W, over b for
// per-head W): 32 consecutive weight elements per workgroup, the shares split over
// eight thread groups, each walking its shares eight loads at a time; dA_log[h] =
// sum_b of the (b, h) shares.  (64 elements over four groups, one load pair at a
// time: 30 us on the Pythia layer for 17 MB of shares, latency-bound.)
template <int DK, int FH>
__global__ __launch_bounds__(256) void bwd_reduce(const BwdParams p, int per_head) {
  constexpr int EW = 32, NG = 256 / EW;
  __shared__ float sq[NG][EW], sk[NG][EW];
  constexpr int64_t W = (int64_t)DK * FH;
  const int tid = threadIdx.x, el = tid % EW, pg = tid / EW;
  const int64_t e = (int64_t)blockIdx.x * EW + el;  // over nh * W
  const int64_t nh = per_head ? p.H : 1;
  float aq = 0.f, ak = 0.f;
  if (e < nh * W) {
    const int64_t h = e / W, x = e % W;
    // the shares of head h (per-head W) or of every head, slot = (bh * ngrp + grp)
    const int64_t nslot = per_head ? p.B * p.ngrp : p.B * p.H * p.ngrp;
#pragma unroll 8
    for (int64_t k2 = pg; k2 < nslot; k2 += NG) {
      int64_t slot;
      if (per_head) {
        const int64_t bb = k2 / p.ngrp, gI = k2 % p.ngrp;
        slot = (bb * p.H + h) * p.ngrp + gI;
      } else {
        slot = k2;
      }
      aq += p.dwq_part[slot * W + x];
      ak += p.dwk_part[slot * W + x];
    }
  }
  sq[pg][el] = aq;
  sk[pg][el] = ak;
  __syncthreads();
  if (pg == 0 && e < nh * W) {
    float tq = 0.f, tk = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < NG; ++g2) {
      tq += sq[g2][el];
      tk += sk[g2][el];
    }
    p.dwq[e] = tq;
    p.dwk[e] = tk;
  }
  if (p.da_log && blockIdx.x == 0) {
    for (int64_t hh = tid; hh < p.H; hh += 256) {
      float s2 = 0.f;
      for (int64_t bb = 0; bb < p.B; ++bb) s2 += p.da_part[bb * p.H + hh];
      p.da_log[hh] = s2;
    }
  }
}

}  // namespace hm
