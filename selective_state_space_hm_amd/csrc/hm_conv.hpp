// Short causal conv of the mixer, depthwise over the token axis: K taps per
// channel, tap K-1 on the current token, the K-1 rows before token 0 taken from
// `prev` (zeros when absent).  Identity at the stage-1 init (taps 0, ..., 0, 1).
// Pages: "HedgeMamba：融合线性注意力与状态空间模型的高效序列建模" §2.2 (Mamba's
// light conv mixes neighbouring tokens), §2.3 item 4 (HedgeMamba keeps it), §3.1
// (the identity init).
//
// Work split: one thread per (b, h, run of CONV_RUN tokens, 16-byte channel
// group); runs away from the sequence's ends take a path with no bounds checks.  It loads the run's rows and the K-1 rows before it as 16-byte
// vectors, all issued before the first product, and keeps its channels' taps in
// registers.  HBM-bound: one read and one write of each row (the K-1 halo rows
// of a run are the previous run's, mostly cache hits).
#pragma once

#include <hip/hip_runtime.h>

#include "hm_device.hpp"

namespace hm {

constexpr int CONV_RUN = 8;

struct ConvParams {
  const void *x;
  void *y;
  const float *w, *bias;
  const void *prev;
  void *fin;
  int64_t B, H, n, d;
  int64_t sx_b, sx_h, sx_t, sy_b, sy_h, sy_t, sw_h, sb_h;
  int64_t runs, groups;  // token runs per (b, h), 16-byte channel groups per row
};

template <typename T, int K>
__global__ __launch_bounds__(256) void conv_kernel(ConvParams p) {
  constexpr int EP = 16 / (int)sizeof(T);  // channels per 16-byte vector
  constexpr int NR = K - 1 + CONV_RUN;     // rows held: K-1 halo rows, then the run
  typedef T tvec __attribute__((ext_vector_type(EP)));
  // one flat grid over (b, h, run, channel group), channel group fastest; the host
  // keeps the thread count below 2^31 so that 32-bit index math suffices
  const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
  const uint32_t G = (uint32_t)p.groups, R = (uint32_t)p.runs;
  if (gid >= (uint32_t)(p.B * p.H) * R * G) return;
  const uint32_t cg = gid % G, rest = gid / G, run = rest % R, bh = rest / R;
  const uint32_t b = bh / (uint32_t)p.H, h = bh % (uint32_t)p.H;
  const int64_t c0 = (int64_t)cg * EP;
  const T *X = (const T *)p.x + b * p.sx_b + h * p.sx_h + c0;
  const int64_t PB = (int64_t)(K - 1) * p.d;  // prev / final block of one (b, h)
  const T *P = p.prev ? (const T *)p.prev + bh * PB + c0 : nullptr;

  // the stream row of token t: x for t >= 0, prev for -(K-1) <= t < 0
  auto row = [&](int64_t t) -> tvec {
    if (t >= 0) return *reinterpret_cast<const tvec *>(X + t * p.sx_t);
    if (P) return *reinterpret_cast<const tvec *>(P + (K - 1 + t) * p.d);
    return tvec{};
  };

  const int64_t t0 = (int64_t)run * CONV_RUN;
  float wt[EP][K], bs[EP];
  {
    const f32x4 *W = reinterpret_cast<const f32x4 *>(p.w + h * p.sw_h + c0 * K);
#pragma unroll
    for (int i = 0; i < EP * K / 4; ++i) {
      const f32x4 v = W[i];
#pragma unroll
      for (int u = 0; u < 4; ++u) wt[(4 * i + u) / K][(4 * i + u) % K] = v[u];
    }
#pragma unroll
    for (int e = 0; e < EP; ++e) bs[e] = p.bias ? p.bias[h * p.sb_h + c0 + e] : 0.f;
  }
  auto out = [&](const tvec *r, int i) {
    tvec o;
#pragma unroll
    for (int e = 0; e < EP; ++e) {
      float acc = bs[e];
#pragma unroll
      for (int j = 0; j < K; ++j) acc = __builtin_fmaf(wt[e][j], (float)r[i + j][e], acc);
      o[e] = (T)acc;
    }
    return o;
  };
  T *Y = (T *)p.y + b * p.sy_b + h * p.sy_h + c0;
  tvec r[NR];
  if (t0 >= K - 1 && t0 + CONV_RUN <= p.n) {
    // interior run: every row is an x row; addresses advance by one stride per row
    const char *src = (const char *)(X + (t0 - (K - 1)) * p.sx_t);
    const int64_t xs = p.sx_t * (int64_t)sizeof(T), ys = p.sy_t * (int64_t)sizeof(T);
#pragma unroll
    for (int i = 0; i < NR; ++i, src += xs) r[i] = *reinterpret_cast<const tvec *>(src);
    char *dst = (char *)(Y + t0 * p.sy_t);
#pragma unroll
    for (int i = 0; i < CONV_RUN; ++i, dst += ys) *reinterpret_cast<tvec *>(dst) = out(r, i);
  } else {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int64_t t = t0 - (K - 1) + i;
      r[i] = t < p.n ? row(t) : tvec{};
    }
#pragma unroll
    for (int i = 0; i < CONV_RUN; ++i)
      if (t0 + i < p.n) *reinterpret_cast<tvec *>(Y + (t0 + i) * p.sy_t) = out(r, i);
  }
  // The last K-1 stream rows, the prev of a call that continues this sequence.
  // Only run 0 reads prev, and it reads every row before writing: `fin` may be
  // the same buffer as `prev` (a decode step updates its conv state in place).
  if constexpr (K > 1) {
    if (p.fin && run == 0) {
      tvec f[K - 1];
#pragma unroll
      for (int i = 0; i < K - 1; ++i) f[i] = row(p.n - (K - 1) + i);
      T *Fo = (T *)p.fin + bh * PB + c0;
#pragma unroll
      for (int i = 0; i < K - 1; ++i) *reinterpret_cast<tvec *>(Fo + (int64_t)i * p.d) = f[i];
    }
  }
}

}  // namespace hm
