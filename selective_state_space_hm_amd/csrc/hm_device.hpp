// Device-side building blocks for the gfx950 kernels: element types, the two
// 16x16 MFMA shapes used (bf16: 16x16x32, f32: 16x16x4), operand fragment
// loads, and wave reductions.
//
// Fragment conventions for a 16x16 MFMA tile (64 lanes, lane = 16*g + col):
//   A operand: lane holds row (lane % 16) and a K-slice chosen by g;
//   B operand: lane holds column (lane % 16) and the same K-slice for the same g;
//   accumulator: lane holds column col and rows 4g .. 4g+3.
// The MFMA sums A[i][k]*B[k][j] over every (g, slot) pair, so any K ordering works
// as long as the A and B fragments of one product use the same one.  Two orderings
// are used:
//   contiguous:  slot e of group g is k = k0 + 8g + e (bf16) or k0 + g (f32);
//   tile order:  K runs over 16-row tiles as they sit in accumulators, so that
//                accumulator tiles can be fed back as operands with no shuffle:
//                bf16 step s covers tiles 2s and 2s+1, slot e -> 32s + 16(e/4) + 4g + e%4;
//                f32  step s covers tile s/4,            slot 0 -> 16(s/4) + 4g + s%4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hm {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

template <typename T> struct Mma;

template <> struct Mma<bf16> {
  static constexpr int KS = 32;   // K of one instruction
  static constexpr int PAD = 8;   // LDS row padding in elements (16 bytes)
  using frag = bf16x8;

  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // contiguous order, row pointer already offset to k0
  __device__ __forceinline__ static frag ld_contig(const bf16 *p, int g) {
    return *reinterpret_cast<const bf16x8 *>(p + 8 * g);
  }
  // Rows that are read in tile order are stored permuted: logical index
  // k = 32s + 16h + 4g + r sits at 32s + 8g + 4h + r, so the eight values slot e
  // of group g needs in step s are contiguous (one 16-byte read), and four
  // logically consecutive values (one accumulator column) stay contiguous.
  __device__ __forceinline__ static int tpos(int k) {
    return (k & ~31) | (((k >> 2) & 3) << 3) | (((k >> 4) & 1) << 2) | (k & 3);
  }
  // tile order, K-step s, from a permuted row
  __device__ __forceinline__ static frag ld_tile(const bf16 *row, int s, int g) {
    return *reinterpret_cast<const bf16x8 *>(row + 32 * s + 8 * g);
  }
  // tile order, K-step s, from accumulator tiles (one f32x4 per 16-row tile)
  __device__ __forceinline__ static frag from_acc(const f32x4 *t, int s) {
    const f32x4 a = t[2 * s], b = t[2 * s + 1];
    return frag{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3],
                (bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
  }
  // K-steps needed to cover `tiles` 16-row tiles in tile order
  static constexpr int steps(int tiles) { return tiles / 2; }
  // highest K-step (exclusive) whose tiles are all <= tile `b`, rounded up to a step
  static constexpr int steps_upto(int b) { return b / 2 + 1; }
  // the tile and row-in-tile (0..15) that slot e of group g reads in K-step s
  __device__ __forceinline__ static int tile_of(int s, int e) { return 2 * s + (e >> 2); }
  __device__ __forceinline__ static int row_of(int g, int e) { return 4 * g + (e & 3); }
  // selector fragment: slot value 1 where pred(slot) holds
  template <typename P> __device__ __forceinline__ static frag select(P pred) {
    frag r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = pred(e) ? (bf16)1.0f : (bf16)0.0f;
    return r;
  }
  static constexpr int EPL = 8;
};

template <> struct Mma<float> {
  static constexpr int KS = 4;
  static constexpr int PAD = 4;
  using frag = float;

  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag ld_contig(const float *p, int g) { return p[g]; }
  __device__ __forceinline__ static int tpos(int k) { return k; }
  __device__ __forceinline__ static frag ld_tile(const float *row, int s, int g) {
    return row[16 * (s >> 2) + 4 * g + (s & 3)];
  }
  __device__ __forceinline__ static frag from_acc(const f32x4 *t, int s) { return t[s >> 2][s & 3]; }
  static constexpr int steps(int tiles) { return tiles * 4; }
  static constexpr int steps_upto(int b) { return 4 * (b + 1); }
  template <typename P> __device__ __forceinline__ static frag select(P pred) {
    return pred(0) ? 1.0f : 0.0f;
  }
  static constexpr int EPL = 1;
};

// Sum / max across the four 16-lane groups (lanes col, col+16, col+32, col+48),
// with the gfx950 lane-swap instructions: permlane32_swap(v, v) leaves lane l
// holding v[l mod 32] in one result and v[l mod 32 + 32] in the other, and
// permlane16_swap does the same for the two 16-lane rows of each half.
__device__ __forceinline__ float xor32_pair(float v, bool want_max) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return want_max ? fmaxf(a, b) : a + b;
}
__device__ __forceinline__ float xor16_pair(float v, bool want_max) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return want_max ? fmaxf(a, b) : a + b;
}
__device__ __forceinline__ float group_sum(float v) { return xor16_pair(xor32_pair(v, false), false); }
__device__ __forceinline__ float group_max(float v) { return xor16_pair(xor32_pair(v, true), true); }

// Inclusive prefix sum over the 64 lanes of a wave in float64, with DPP row
// shifts inside each 16-lane row and row broadcasts across rows.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ double dpp_f64(double x) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(x), CTRL, ROWMASK, 0xf, true);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(x), CTRL, ROWMASK, 0xf, true);
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double wave_inclusive_scan(double x) {
  x += dpp_f64<0x111, 0xf>(x);  // row_shr:1
  x += dpp_f64<0x112, 0xf>(x);  // row_shr:2
  x += dpp_f64<0x114, 0xf>(x);  // row_shr:4
  x += dpp_f64<0x118, 0xf>(x);  // row_shr:8
  x += dpp_f64<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_f64<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}
__device__ __forceinline__ double lane63(double x) {
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(x), 63),
                          __builtin_amdgcn_readlane(__double2loint(x), 63));
}

// log(1 + e^x) in float32; above x = 20 the correction e^-x is below float32
// resolution relative to x.
__device__ __forceinline__ float softplus_f32(float x) {
  return x > 20.f ? x : log1pf(expf(x));
}

// x * sigmoid(x) in float32 (the reciprocal to ~1 ulp); for x < -88 the exponential
// overflows to +inf and the result is -0, the correct limit.
__device__ __forceinline__ float silu_f32(float x) {
  return x * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}

template <typename T> __device__ __forceinline__ T to_elem(float x) { return (T)x; }

// Rotary position encoding of the features (HedgeMamba explainer §5.2 step 3, in
// the GPT-NeoX rotate-half form): feature i < dims/2 pairs with i + dims/2 and the
// pair turns by pos * base^(-2i/dims).  rope_rev is that rate in revolutions per
// position, in float64; rope_cs reduces pos * rate to [-1/2, 1/2] revolutions in
// float64, so the hardware sine and cosine (which take revolutions; about 1.2e-7
// absolute error on that range, measured) see an argument exact to float32
// rounding at any position.
__device__ inline double rope_rev(int i, int dims, float base) {
  return exp2(-2.0 * (double)i / (double)dims * log2((double)base)) * 0.15915494309189535;  // / (2 pi)
}
__device__ __forceinline__ void rope_cs(double rev, double pos, float &c, float &s) {
  double r = pos * rev;
  r -= __builtin_rint(r);
  const float x = (float)r;
  c = __builtin_amdgcn_cosf(x);
  s = __builtin_amdgcn_sinf(x);
}
// (x1, x2) -> (x1 c - x2 s, x2 c + x1 s) forward (INV = false), the transpose
// (x1 c + x2 s, x2 c - x1 s) for INV = true.
template <bool INV>
__device__ __forceinline__ void rope_turn(float &x1, float &x2, float c, float s) {
  const float a = x1, b = x2;
  if constexpr (INV) {
    x1 = __builtin_fmaf(a, c, b * s);
    x2 = __builtin_fmaf(b, c, -(a * s));
  } else {
    x1 = __builtin_fmaf(a, c, -(b * s));
    x2 = __builtin_fmaf(b, c, a * s);
  }
}
// Features held as 16-feature tiles of one token per lane (tile t, slot r is feature
// 16t + 4g + r): the pair partner of tile t is tile t + RT, RT = dims/32, in the
// same lane and slot.  rev[i] is rope_rev(i, ...) for i < dims/2.
template <int RT, bool INV>
__device__ __forceinline__ void rope_tiles(f32x4 *ph, const double *rev, int g, double pos) {
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float c, s, x1 = ph[t][r], x2 = ph[t + RT][r];
      rope_cs(rev[16 * t + 4 * g + r], pos, c, s);
      rope_turn<INV>(x1, x2, c, s);
      ph[t][r] = x1;
      ph[t + RT][r] = x2;
    }
}
// dims (a multiple of 32, at most 16*NFT) picks the tile pairing at run time; the
// switch is uniform, each arm fully unrolled.
template <int NFT, bool INV = false>
__device__ __forceinline__ void rope_apply(f32x4 *ph, const double *rev, int g, double pos, int dims) {
  switch (dims >> 5) {
    case 1: rope_tiles<1, INV>(ph, rev, g, pos); break;
    case 2: if constexpr (NFT >= 4) rope_tiles<2, INV>(ph, rev, g, pos); break;
    case 3: if constexpr (NFT >= 6) rope_tiles<3, INV>(ph, rev, g, pos); break;
    case 4: if constexpr (NFT >= 8) rope_tiles<4, INV>(ph, rev, g, pos); break;
    default: break;
  }
}

// Four consecutive elements as one vector store / load.
__device__ __forceinline__ void store4(bf16 *p, f32x4 v) {
  *reinterpret_cast<bf16x4 *>(p) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}
__device__ __forceinline__ void store4(float *p, f32x4 v) { *reinterpret_cast<f32x4 *>(p) = v; }
// Store four values already rounded to T (given as floats holding T values).
__device__ __forceinline__ f32x4 round4(f32x4 v, bf16) {
  return f32x4{(float)(bf16)v[0], (float)(bf16)v[1], (float)(bf16)v[2], (float)(bf16)v[3]};
}
__device__ __forceinline__ f32x4 round4(f32x4 v, float) { return v; }

}  // namespace hm
