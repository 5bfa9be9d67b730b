// Host side of the C ABI declared in include/hm.h: argument validation (before
// any HIP call), plan selection, launch-table lookup and launches.
#include <hip/hip_runtime.h>

#include <utility>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "hm.h"
#include "hm_bwd_params.hpp"
#include "hm_kernels.hpp"
#include "hm_pc.hpp"
#include "hm_cp.hpp"

namespace {

thread_local std::string g_err;

hm_status fail(hm_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

hm_status ok() {
  g_err.clear();
  return HM_OK;
}

size_t esize(int dt) { return dt == HM_BF16 ? 2 : 4; }
bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }
bool stride_ok(int64_t s, int dt) { return s >= 0 && ((size_t)s * esize(dt)) % 16 == 0; }

struct Tables {
  hm::Table parts[12];
  Tables() {
    parts[0] = hm::table_fwd_bf16();
    parts[1] = hm::table_fwd_bf16_decay();
    parts[2] = hm::table_fwd_f32();
    parts[3] = hm::table_step_feat();
    parts[4] = hm::table_train();
    parts[5] = hm::table_fwd_rope_bf16();
    parts[6] = hm::table_fwd_rope_bf16_decay();
    parts[7] = hm::table_fwd_rope_f32();
    parts[8] = hm::table_fwd_c128();
    parts[9] = hm::table_fwd_f32_d64();
    parts[10] = hm::table_step_bf16();
    parts[11] = hm::table_step_f32();
  }
};
const Tables &tables() {
  static Tables t;
  return t;
}

const hm::FwdEntry *find_fwd(int dt, int64_t dk, int64_t fh, int64_t dw, int decay, int mode, int chunk = hm::CHUNK) {
  for (const auto &part : tables().parts)
    for (int i = 0; i < part.nfwd; ++i) {
      const auto &e = part.fwd[i];
      if (e.dtype == dt && e.dk == dk && e.fh == fh && e.dw == dw && e.decay == decay && e.mode == mode &&
          e.chunk == chunk)
        return &e;
    }
  return nullptr;
}
const hm::StepEntry *find_step(int dt, int64_t dk, int64_t fh, int64_t dv, int decay) {
  for (const auto &part : tables().parts)
    for (int i = 0; i < part.nstep; ++i) {
      const auto &e = part.step[i];
      if (e.dtype == dt && e.dk == dk && e.fh == fh && e.dv == dv && e.decay == decay) return &e;
    }
  return nullptr;
}
const hm::FeatEntry *find_feat(int dt, int pdt, int64_t dk, int64_t fh) {
  for (const auto &part : tables().parts)
    for (int i = 0; i < part.nfeat; ++i) {
      const auto &e = part.feat[i];
      if (e.dtype == dt && e.phi_dtype == pdt && e.dk == dk && e.fh == fh) return &e;
    }
  return nullptr;
}

// The chunk-parallel prefill (any d in {16, 32, 64, 128}; its kernels take d at run time)
const hm::CpEntry *find_cp(int dt, int64_t d, int64_t fh, int64_t dv) {
  if (d != 16 && d != 32 && d != 64 && d != 128) return nullptr;
  const hm::CpTable parts[] = {hm::table_cp_bf16(), hm::table_cp_f32()};
  for (const auto &part : parts)
    for (int i = 0; i < part.ncp; ++i) {
      const auto &e = part.cp[i];
      if (e.dtype == dt && e.fh == fh && e.dv == dv) return &e;
    }
  return nullptr;
}

// MODE_ROPE when the rotary encoding is on
template <typename A> int rmode(const A *a) { return a->rope_dims ? hm::MODE_ROPE : 0; }

// The rotary fields shared by the entry points (see hm.h).
hm_status validate_rope(int32_t dims, float base, const int64_t *pos, int64_t f, bool pos_required) {
  if (dims == 0) return ok();
  if (dims < 0 || dims > 2 * f || dims % 2)
    return fail(HM_ERR_SHAPE, "rope_dims %d: 0 or an even number of at most 2f = %lld", dims, (long long)(2 * f));
  if (dims % 32) return fail(HM_ERR_UNSUPPORTED, "rope_dims %d: multiples of 32 are built", dims);
  if (!(base > 0.f) || !std::isfinite(base)) return fail(HM_ERR_SHAPE, "rope_base must be positive and finite");
  if (pos_required && !pos) return fail(HM_ERR_NULL, "rope_pos is required when rope_dims > 0");
  if ((uintptr_t)pos % 8) return fail(HM_ERR_ALIGN, "rope positions must be 8-byte aligned");
  return ok();
}

hm_status check_launch(const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(HM_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

// ------------------------------------------------------------------ prefill
struct Plan {
  bool cp;              // the chunk-parallel path (chunk 256, or sizes without a fused kernel)
  int64_t nc;           // cp: chunks per sequence
  int chunk, segments, dsplit;
  int lsub;             // segment-pass slots per segment (pieces of seg_len / lsub tokens)
  int64_t seg_len;
  bool alias;           // s_init and s_final overlap
  bool init_copy;       // s_init is copied into the workspace first
  size_t ws_state_floats, ws_lam_floats, ws_init_floats;
  size_t bytes() const { return 4 * (ws_state_floats + ws_lam_floats + ws_init_floats); }
};

hm_status validate_cp(const hm_linattn_fwd_args *a);
hm_status validate_fused(const hm_linattn_fwd_args *a);

hm_status validate_fwd(const hm_linattn_fwd_args *a) {
  if (!a) return fail(HM_ERR_NULL, "args is NULL");
  if (a->dtype != HM_F32 && a->dtype != HM_BF16) return fail(HM_ERR_DTYPE, "dtype %d is not HM_F32 or HM_BF16", a->dtype);
  if (a->B < 0 || a->H < 0 || a->n < 0 || a->d <= 0 || a->f <= 0 || a->dv <= 0)
    return fail(HM_ERR_SHAPE, "sizes must be B, H, n >= 0 and d, f, dv >= 1");
  // with no token to process, q, k, v, w and o are never touched and may be NULL
  if (a->B * a->H * a->n > 0 && (!a->q || !a->k || !a->v || !a->w_q || !a->w_k || !a->o))
    return fail(HM_ERR_NULL, "q, k, v, w_q, w_k and o must be non-NULL");
  if (a->B * a->H * a->n > 0 && (a->dt == nullptr) != (a->a_log == nullptr))
    return fail(HM_ERR_NULL, "dt and a_log must be given together");
  const int64_t strides[] = {a->sq_b, a->sq_h, a->sq_t, a->sk_b, a->sk_h, a->sk_t, a->sv_b,
                             a->sv_h, a->sv_t, a->so_b, a->so_h, a->so_t, a->sw_h};
  for (int64_t s : strides)
    if (s < 0) return fail(HM_ERR_SHAPE, "strides must be non-negative");
  if (a->sdt_b < 0 || a->sdt_h < 0 || a->sdt_t < 0) return fail(HM_ERR_SHAPE, "dt strides must be non-negative");
  if (a->n > 1 && (a->so_t < a->dv || a->sq_t < a->d || a->sk_t < a->d || a->sv_t < a->dv))
    return fail(HM_ERR_SHAPE, "token stride smaller than the row length (rows overlap)");
  const void *ptrs[] = {a->q, a->k, a->v, a->w_q, a->w_k, a->o};
  for (const void *p : ptrs)
    if (!aligned16(p)) return fail(HM_ERR_ALIGN, "q, k, v, w_q, w_k, o must be 16-byte aligned");
  if (a->gate) {
    if (a->sg_b < 0 || a->sg_h < 0 || a->sg_t < 0) return fail(HM_ERR_SHAPE, "gate strides must be non-negative");
    if (!aligned16(a->gate)) return fail(HM_ERR_ALIGN, "gate must be 16-byte aligned");
    if (!stride_ok(a->sg_b, a->dtype) || !stride_ok(a->sg_h, a->dtype) || !stride_ok(a->sg_t, a->dtype))
      return fail(HM_ERR_ALIGN, "every stride times the element size must be a multiple of 16 bytes");
  }
  if ((a->s_init && !aligned16(a->s_init)) || (a->s_final && !aligned16(a->s_final)))
    return fail(HM_ERR_ALIGN, "state buffers must be 16-byte aligned");
  for (int64_t s : strides)
    if (!stride_ok(s, a->dtype)) return fail(HM_ERR_ALIGN, "every stride times the element size must be a multiple of 16 bytes");
  if (a->chunk != 0 && a->chunk != 64 && a->chunk != 128 && a->chunk != 256)
    return fail(HM_ERR_UNSUPPORTED, "chunk %d: built are 0 (auto), 64, 128 and 256", a->chunk);
  if (a->segments < 0) return fail(HM_ERR_SHAPE, "segments must be >= 0");
  if (a->dsplit < 0 || a->dsplit > 2) return fail(HM_ERR_UNSUPPORTED, "dsplit must be 0, 1 or 2");
  {
    const hm_status rs = validate_rope(a->rope_dims, a->rope_base, a->rope_pos0, a->f, false);
    if (rs != HM_OK) return rs;
  }
  if (a->chunk == 256) return validate_cp(a);
  const hm_status fs = validate_fused(a);
  // sizes without a fused kernel run the chunk-parallel path when nothing else asks for one
  if (fs == HM_ERR_UNSUPPORTED && !a->dsplit && !a->segments && !a->gate && !a->rope_dims && !a->save &&
      find_cp(a->dtype, a->d, a->f, a->dv))
    return validate_cp(a);
  return fs;
}

// The plain prefill on the chunk-parallel path: no gate, rotary encoding or
// training saves, one workgroup per (b, h, chunk) and no segments.
hm_status validate_cp(const hm_linattn_fwd_args *a) {
  if (!find_cp(a->dtype, a->d, a->f, a->dv))
    return fail(HM_ERR_UNSUPPORTED, "no chunk-parallel kernel for dtype=%d d=%lld f=%lld dv=%lld", a->dtype,
                (long long)a->d, (long long)a->f, (long long)a->dv);
  if (a->gate || a->rope_dims || a->save)
    return fail(HM_ERR_UNSUPPORTED, "chunk 256 and the sizes without a fused kernel run the chunk-parallel "
                                    "path, which is built for the plain prefill: no gate, rotary encoding or "
                                    "training saves");
  if (a->segments) return fail(HM_ERR_UNSUPPORTED, "the chunk-parallel path takes segments = 0 (every chunk is one)");
  if (a->dsplit > 1) return fail(HM_ERR_UNSUPPORTED, "the chunk-parallel path takes dsplit 0 or 1");
  return ok();
}

// The fused kernels (chunk 64 or 128): whether one is built for the request.
hm_status validate_fused(const hm_linattn_fwd_args *a) {
  if (a->chunk == 128 && (a->save || a->gate || a->rope_dims))
    return fail(HM_ERR_UNSUPPORTED, "chunk 128 is built for the plain prefill: no training saves, gate or rotary "
                                    "encoding (use chunk 64 for those)");
  const int decay = a->dt != nullptr && a->a_log != nullptr;
  const int ch = a->chunk ? a->chunk : hm::CHUNK;
  // the full-pass kernel for dsplit 1 must exist for the size to count as supported
  if (!find_fwd(a->dtype, a->d, a->f, a->dv, decay, hm::MODE_FULL | rmode(a), ch) &&
      !find_fwd(a->dtype, a->d, a->f, a->dv / 2, decay, hm::MODE_FULL | rmode(a), ch))
    return fail(HM_ERR_UNSUPPORTED, "no kernel built for dtype=%d d=%lld f=%lld dv=%lld chunk=%d", a->dtype,
                (long long)a->d, (long long)a->f, (long long)a->dv, ch);
  if (a->dsplit == 2 && (a->dv % 2 || !find_fwd(a->dtype, a->d, a->f, a->dv / 2, decay, hm::MODE_FULL | rmode(a), ch)))
    return fail(HM_ERR_UNSUPPORTED, "dsplit=2 is not built for dv=%lld", (long long)a->dv);
  if (a->dsplit == 1 && !find_fwd(a->dtype, a->d, a->f, a->dv, decay, hm::MODE_FULL | rmode(a), ch))
    return fail(HM_ERR_UNSUPPORTED, "dsplit=1 is not built for dv=%lld", (long long)a->dv);
  if (a->save) {
    if (a->dsplit > 1) return fail(HM_ERR_UNSUPPORTED, "saving for the backward pass runs with dsplit 1");
    if (!find_fwd(a->dtype, a->d, a->f, a->dv, decay, hm::MODE_TRAIN | rmode(a)))
      return fail(HM_ERR_UNSUPPORTED, "no training kernel for dtype=%d d=%lld f=%lld dv=%lld", a->dtype,
                  (long long)a->d, (long long)a->f, (long long)a->dv);
    if (!aligned16(a->save)) return fail(HM_ERR_ALIGN, "save must be 16-byte aligned");
  }
  return ok();
}

// The backward's per-chunk kernels split each (b, h) into ngrp ranges of `per`
// chunks, enough (b, h, range) workgroups to fill the 256 compute units.
struct BwdGroups {
  int64_t ngrp, per, nck;  // ranges, chunks per range, ranges that hold chunks
};
BwdGroups bwd_groups(int64_t BH, int64_t n) {
  const int64_t nch = (n + hm::CHUNK - 1) / hm::CHUNK;
  int64_t ng = BH > 0 ? (256 + BH - 1) / BH : 1;
  if (ng > nch) ng = nch;
  if (ng < 1) ng = 1;
  BwdGroups gr{};
  gr.ngrp = ng;
  gr.per = nch > 0 ? (nch + ng - 1) / ng : 1;
  gr.nck = nch > 0 ? (nch + gr.per - 1) / gr.per : 0;
  return gr;
}
// What the training forward saves, per (b, h): the float32 state at the start of
// each of the backward's chunk ranges [nck][F*dv + F] (the checkpoints from which
// the backward recomputes every chunk-start state), the per-token denominator in
// float32 [n] and the float32 output before the gate [n][dv]; regions 256-byte
// aligned.
struct SaveLayout {
  size_t off_ck, off_den, off_o, bytes;
};
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
SaveLayout save_layout(int dtype, int64_t BH, int64_t n, int64_t f, int64_t dv) {
  (void)dtype;
  const int64_t F = 2 * f;
  const BwdGroups gr = bwd_groups(BH, n);
  SaveLayout l{};
  l.off_ck = 0;
  l.off_den = align256((size_t)(BH * gr.nck * (F * dv + F)) * 4);
  l.off_o = l.off_den + align256((size_t)(BH * n) * 4);
  l.bytes = l.off_o + align256((size_t)(BH * n * dv) * 4);
  return l;
}

// Whether a validated request runs on the chunk-parallel path.
bool is_cp(const hm_linattn_fwd_args *a) {
  if (a->chunk == 256) return true;
  const int decay = a->dt != nullptr && a->a_log != nullptr;
  const int ch = a->chunk ? a->chunk : hm::CHUNK;
  return !find_fwd(a->dtype, a->d, a->f, a->dv, decay, hm::MODE_FULL | rmode(a), ch) &&
         !find_fwd(a->dtype, a->d, a->f, a->dv / 2, decay, hm::MODE_FULL | rmode(a), ch);
}

Plan make_plan(const hm_linattn_fwd_args *a) {
  Plan p{};
  const int decay = a->dt != nullptr && a->a_log != nullptr;
  const int64_t BH = a->B * a->H;
  const int64_t F = 2 * a->f;
  const int64_t BLK = F * a->dv + F;
  if (is_cp(a)) {
    // chunk-parallel: every chunk's local state, then its start state, in the workspace
    p.cp = true;
    p.chunk = a->chunk ? a->chunk : hm::CHUNK;
    p.nc = (a->n + p.chunk - 1) / p.chunk;
    p.segments = p.nc > 0 ? (int)p.nc : 1;
    p.dsplit = 1;
    p.lsub = 1;
    p.seg_len = p.chunk;
    p.ws_state_floats = (size_t)(BH * p.nc) * BLK;
    p.ws_lam_floats = ((size_t)(BH * p.nc) + 3) / 4 * 4;
    return p;
  }
  // chunk: 64 unless asked (128-token chunks add intra-chunk work for fewer state passes)
  const int C = a->chunk ? a->chunk : hm::CHUNK;
  p.chunk = C;
  // dsplit: one workgroup owns all value columns of a (b, h) whenever that
  // kernel is built (splitting duplicates the featurization and measured slower)
  if (a->save) {
    p.dsplit = 1;
  } else if (a->dsplit) {
    p.dsplit = a->dsplit;
  } else {
    const bool can1 = find_fwd(a->dtype, a->d, a->f, a->dv, decay, hm::MODE_FULL | rmode(a), C) != nullptr;
    p.dsplit = can1 ? 1 : 2;
  }
  const int64_t nchunks = (a->n + C - 1) / C;
  int64_t segs;
  if (a->segments) {
    segs = a->segments;
  } else {
    // one workgroup per compute unit (256 on MI355X): split each sequence into
    // enough segments, each at least 4 chunks long
    const int64_t wg = BH * p.dsplit;
    segs = wg >= 256 || wg == 0 ? 1 : (256 + wg - 1) / wg;
    const int64_t cap = nchunks / 4 > 1 ? nchunks / 4 : 1;
    if (segs > cap) segs = cap;
  }
  if (segs > nchunks) segs = nchunks > 0 ? nchunks : 1;
  if (segs < 1) segs = 1;
  const int64_t per = nchunks > 0 ? (nchunks + segs - 1) / segs : 1;
  p.seg_len = per * C;
  p.segments = nchunks > 0 ? (int)((nchunks + per - 1) / per) : 1;
  // aliasing of s_init and s_final: several workgroups per (b, h) would race
  p.alias = false;
  if (a->s_init && a->s_final) {
    const char *i0 = (const char *)a->s_init, *f0 = (const char *)a->s_final;
    const size_t len = (size_t)BH * BLK * 4;
    p.alias = i0 < f0 + len && f0 < i0 + len;
  }
  // The segment pass runs one workgroup per slot.  When its (b, h, segment) items
  // fill less than half the chip, it cuts every segment into lsub equal pieces
  // (no work is duplicated; the full pass composes the pieces' maps), as long as
  // that stays within one workgroup per compute unit.
  p.lsub = 1;
  if (p.segments > 1) {
    const int64_t items = BH * (p.segments - 1) * p.dsplit;
    for (int cand = 4; cand > 1; cand /= 2) {
      if (per % cand == 0 && items * cand <= 256) {
        p.lsub = cand;
        break;
      }
    }
  }
  p.init_copy = p.alias && (p.segments > 1 || p.dsplit > 1);
  const int64_t slots = p.segments > 1 ? (int64_t)(p.segments - 1) * p.lsub : 0;
  p.ws_state_floats = (size_t)slots * BH * BLK;
  p.ws_lam_floats = (size_t)slots * BH;
  p.ws_lam_floats = (p.ws_lam_floats + 3) / 4 * 4;
  p.ws_init_floats = p.init_copy ? (size_t)BH * BLK : 0;
  return p;
}

}  // namespace

extern "C" {

hm_status hm_linattn_fwd_workspace_size(const hm_linattn_fwd_args *a, size_t *bytes) {
  if (!bytes) return fail(HM_ERR_NULL, "bytes is NULL");
  hm_status st = validate_fwd(a);
  if (st != HM_OK) return st;
  *bytes = make_plan(a).bytes();
  return ok();
}

hm_status hm_linattn_fwd_plan(const hm_linattn_fwd_args *a, int32_t *chunk, int32_t *segments, int32_t *dsplit) {
  hm_status st = validate_fwd(a);
  if (st != HM_OK) return st;
  Plan p = make_plan(a);
  if (chunk) *chunk = p.chunk;
  if (segments) *segments = p.segments;
  if (dsplit) *dsplit = p.dsplit;
  return ok();
}

}  // extern "C"

namespace {
// The prefill after validation and planning, with the workspace `wsp` (at least
// pl.bytes() bytes, 16-byte aligned; NULL when that is 0).
// The chunk-parallel path: local states, their scan over the chunks, outputs.
hm_status run_cp(const hm_linattn_fwd_args *a, const Plan &pl, void *wsp, hipStream_t s) {
  hm_status st = HM_OK;
  const int64_t BH = a->B * a->H, F = 2 * a->f, BLK = F * a->dv + F;
  const hm::CpEntry *e = find_cp(a->dtype, a->d, a->f, a->dv);
  if (!e) return fail(HM_ERR_UNSUPPORTED, "no chunk-parallel kernel");
  hm::CpParams p{};
  p.q = a->q; p.k = a->k; p.v = a->v; p.wq = a->w_q; p.wk = a->w_k;
  p.dt = a->dt; p.a_log = a->a_log;
  p.s_init = a->s_init; p.s_final = a->s_final;
  p.o = a->o;
  p.ws_state = (float *)wsp;
  p.ws_lam = wsp ? (float *)wsp + pl.ws_state_floats : nullptr;
  p.B = a->B; p.H = a->H; p.n = a->n; p.nc = pl.nc;
  p.d = (int)a->d; p.chunk = pl.chunk;
  p.sq_b = a->sq_b; p.sq_h = a->sq_h; p.sq_t = a->sq_t;
  p.sk_b = a->sk_b; p.sk_h = a->sk_h; p.sk_t = a->sk_t;
  p.sv_b = a->sv_b; p.sv_h = a->sv_h; p.sv_t = a->sv_t;
  p.so_b = a->so_b; p.so_h = a->so_h; p.so_t = a->so_t;
  p.sw_h = a->sw_h; p.sdt_b = a->sdt_b; p.sdt_h = a->sdt_h; p.sdt_t = a->sdt_t;
  if (pl.nc > 0) {
    e->local(p, (unsigned)(BH * pl.nc), s);
    if ((st = check_launch("chunk-parallel local states")) != HM_OK) return st;
  }
  hipLaunchKernelGGL(hm::cp_scan_kernel, dim3((unsigned)((BLK + 255) / 256), (unsigned)BH), dim3(256), 0, s, p, BLK,
                     (int)F, (int)a->dv);
  if ((st = check_launch("chunk-parallel state scan")) != HM_OK) return st;
  if (pl.nc > 0) {
    // chunks padded to a multiple of 8: the kernel maps a chunk's query blocks onto one XCD
    e->out(p, (unsigned)((BH * pl.nc + 7) / 8 * 8 * (pl.chunk / hm::CP_BLK)), s);
    if ((st = check_launch("chunk-parallel outputs")) != HM_OK) return st;
  }
  return ok();
}

hm_status run_fwd(const hm_linattn_fwd_args *a, const Plan &pl, void *wsp, void *stream) {
  hm_status st = HM_OK;
  const int64_t BH = a->B * a->H;
  if (BH == 0) return ok();
  if (a->n == 0 && !a->s_final) return ok();
  if (pl.cp) return run_cp(a, pl, wsp, (hipStream_t)stream);
  const int decay = a->dt != nullptr && a->a_log != nullptr;
  const int64_t dw = a->dv / pl.dsplit;
  // the full pass at the plan's chunk length; the segment pass works in 64-token
  // chunks at any chunk length (the end state is the same sum)
  const hm::FwdEntry *full =
      find_fwd(a->dtype, a->d, a->f, dw, decay, (a->save ? hm::MODE_TRAIN : hm::MODE_FULL) | rmode(a), pl.chunk);
  const hm::FwdEntry *local = find_fwd(a->dtype, a->d, a->f, dw, decay, hm::MODE_LOCAL | rmode(a));
  if (!full || !local) return fail(HM_ERR_UNSUPPORTED, "no kernel for dv/dsplit=%lld", (long long)dw);
  hipStream_t s = (hipStream_t)stream;

  float *ws = (float *)wsp;
  float *ws_state = ws;
  float *ws_lam = ws ? ws + pl.ws_state_floats : nullptr;
  float *ws_init = ws ? ws + pl.ws_state_floats + pl.ws_lam_floats : nullptr;
  const int64_t F = 2 * a->f;
  const int64_t BLK = F * a->dv + F;

  hm::FwdParams p{};
  p.q = a->q; p.k = a->k; p.v = a->v; p.wq = a->w_q; p.wk = a->w_k;
  p.dt = a->dt; p.a_log = a->a_log;
  p.s_start0 = pl.init_copy ? ws_init : a->s_init;
  p.s_final = a->s_final;
  p.o = a->o;
  p.ws_state = ws_state; p.ws_lam = ws_lam;
  p.B = a->B; p.H = a->H; p.n = a->n; p.dv = a->dv;
  p.sq_b = a->sq_b; p.sq_h = a->sq_h; p.sq_t = a->sq_t;
  p.sk_b = a->sk_b; p.sk_h = a->sk_h; p.sk_t = a->sk_t;
  p.sv_b = a->sv_b; p.sv_h = a->sv_h; p.sv_t = a->sv_t;
  p.so_b = a->so_b; p.so_h = a->so_h; p.so_t = a->so_t;
  p.sw_h = a->sw_h; p.sdt_b = a->sdt_b; p.sdt_h = a->sdt_h; p.sdt_t = a->sdt_t;
  p.gate = a->gate; p.sg_b = a->sg_b; p.sg_h = a->sg_h; p.sg_t = a->sg_t;
  p.rope_dims = a->rope_dims; p.rope_base = a->rope_base; p.rope_pos0 = a->rope_pos0;
  p.seg_len = pl.seg_len;
  p.nseg = pl.segments;
  p.dsplit = pl.dsplit;
  p.nchunks = (a->n + hm::CHUNK - 1) / hm::CHUNK;
  if (a->save) {
    const SaveLayout sl = save_layout(a->dtype, BH, a->n, a->f, a->dv);
    if (a->save_bytes < sl.bytes)
      return fail(HM_ERR_WORKSPACE, "save buffer of %zu bytes required, got %zu", sl.bytes, a->save_bytes);
    const BwdGroups gr = bwd_groups(BH, a->n);
    p.save_ck = (float *)((char *)a->save + sl.off_ck);
    p.save_den = (float *)((char *)a->save + sl.off_den);
    p.save_o = (float *)((char *)a->save + sl.off_o);
    p.ck_every = gr.per;
    p.nck = gr.nck;
  }

  auto grid_for = [&](int64_t items, int ds) { return (unsigned)(((items + 7) / 8) * 8 * ds); };
  const int nslot = pl.segments > 1 ? (pl.segments - 1) * pl.lsub : 0;
  if (pl.segments > 1) {
    // Segment pass: end state of every slot (piece of a segment) before the last
    // segment, slot 0 starting from s_init (read before anything writes s_final)
    // and the others from zero.  With whole segments as slots it owns fewer value
    // columns per workgroup when that fills more of the chip.
    const hm::FwdEntry *loc = local;
    int lds = pl.dsplit;
    for (int cand = 4; pl.lsub == 1 && cand > pl.dsplit; cand /= 2) {
      const hm::FwdEntry *e = a->dv % cand ? nullptr : find_fwd(a->dtype, a->d, a->f, a->dv / cand, decay, hm::MODE_LOCAL | rmode(a));
      if (e && BH * (pl.segments - 1) * cand <= 256) {
        loc = e;
        lds = cand;
        break;
      }
    }
    hm::FwdParams pp = p;
    pp.s_start0 = a->s_init;
    pp.dsplit = lds;
    pp.seg_len = pl.seg_len / pl.lsub;
    pp.nseg_run = nslot;
    pp.nitems = BH * nslot;
    loc->launch(pp, grid_for(pp.nitems, lds), s);
    if ((st = check_launch("segment pass")) != HM_OK) return st;
  }
  // With two segments the full pass composes the slots of segment 0 as it loads
  // its start state (the training pass excepted); otherwise the running start
  // states are composed here in place.  Also the copy of s_init when it aliases
  // s_final.
  const bool fuse = pl.segments == 2 && !a->save;
  const bool compose = nslot > 1 && !fuse;
  p.lsub = pl.lsub;
  p.nfuse = fuse ? pl.lsub : 1;
  if (compose || pl.init_copy) {
    dim3 grid((unsigned)((BLK + 255) / 256), (unsigned)BH);
    hipLaunchKernelGGL(hm::combine_kernel, grid, dim3(256), 0, s, ws_state, ws_lam, a->s_init,
                       pl.init_copy ? ws_init : nullptr, BH, BLK, compose ? nslot : 0, pl.lsub);
    if ((st = check_launch("segment combine")) != HM_OK) return st;
  }
  p.nseg_run = pl.segments;
  p.nitems = BH * pl.segments;
  full->launch(p, grid_for(p.nitems, pl.dsplit), s);
  return check_launch("prefill");
}

// Scratch of hm_linattn_fwd_noalloc: one copy per GPU, held until the process ends.
// In host code `scratch` names a host-side stand-in, never the device memory: its
// device address comes from hipGetSymbolAddress, once per device, and only that
// address is passed on.
static __device__ __align__(256) unsigned char scratch[HM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch`, looked up on the first call made with
// that device current.
hm_status scratch_for_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(HM_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(HM_ERR_UNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(HM_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return ok();
}
}  // namespace

extern "C" {

hm_status hm_linattn_fwd(const hm_linattn_fwd_args *a, void *stream) {
  hm_status st = validate_fwd(a);
  if (st != HM_OK) return st;
  const Plan pl = make_plan(a);
  if (pl.bytes() > 0) {
    if (!a->workspace) return fail(HM_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", pl.bytes());
    if (a->workspace_bytes < pl.bytes())
      return fail(HM_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", pl.bytes(), a->workspace_bytes);
    if (!aligned16(a->workspace)) return fail(HM_ERR_ALIGN, "workspace must be 16-byte aligned");
  }
  return run_fwd(a, pl, a->workspace, stream);
}

hm_status hm_linattn_fwd_noalloc(const hm_linattn_fwd_args *a, void *stream) {
  hm_status st = validate_fwd(a);
  if (st != HM_OK) return st;
  const Plan pl = make_plan(a);
  if (pl.bytes() > (size_t)HM_NOALLOC_SCRATCH_BYTES)
    return fail(HM_ERR_WORKSPACE,
                "this plan needs %zu bytes of scratch, above the %d bytes hm_linattn_fwd_noalloc holds per device "
                "(fewer segments, or hm_linattn_fwd with a workspace)",
                pl.bytes(), HM_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  if (pl.bytes() > 0 && (st = scratch_for_current_device(&ws)) != HM_OK) return st;
  return run_fwd(a, pl, ws, stream);
}

hm_status hm_linattn_save_size(const hm_linattn_fwd_args *a, size_t *bytes) {
  if (!bytes) return fail(HM_ERR_NULL, "bytes is NULL");
  if (!a) return fail(HM_ERR_NULL, "args is NULL");
  if (a->dtype != HM_F32 && a->dtype != HM_BF16) return fail(HM_ERR_DTYPE, "dtype %d is not HM_F32 or HM_BF16", a->dtype);
  if (a->B < 0 || a->H < 0 || a->n < 0 || a->f <= 0 || a->dv <= 0)
    return fail(HM_ERR_SHAPE, "sizes must be B, H, n >= 0 and f, dv >= 1");
  *bytes = save_layout(a->dtype, a->B * a->H, a->n, a->f, a->dv).bytes;
  return ok();
}

// ------------------------------------------------------------------ backward
namespace {
struct BwdLayout {
  size_t phq, phk, dnum, dden, Lc, eQ, eK, eW, Xc, gS, gz, wS, wz, dwq, dwk, da, bytes;
  int ngrp;
};
BwdLayout bwd_layout(const hm_linattn_bwd_args *a) {
  BwdLayout l{};
  const int64_t BH = a->B * a->H, n = a->n, F = 2 * a->f, nch = (n + hm::CHUNK - 1) / hm::CHUNK;
  const size_t es = esize(a->dtype);
  // enough (b, h, chunk range) workgroups to fill the 256 compute units
  const int64_t ng = bwd_groups(BH, n).ngrp;
  l.ngrp = (int)ng;
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += align256(bytes); return at; };
  l.phq = take((size_t)(BH * n * F) * es);
  l.phk = take((size_t)(BH * n * F) * es);
  l.dnum = take((size_t)(BH * n * a->dv) * es);
  l.dden = take((size_t)(BH * n) * 4);
  l.Lc = take((size_t)(BH * n) * 4);
  l.eQ = take((size_t)(BH * n) * 4);
  l.eK = take((size_t)(BH * n) * 4);
  l.eW = take((size_t)(BH * n) * 4);
  l.Xc = take((size_t)(BH * nch) * 4);
  l.gS = take((size_t)(BH * nch * F * a->dv) * es);
  l.gz = take((size_t)(BH * nch * F) * 4);
  l.wS = take((size_t)(BH * nch * F * a->dv) * es);
  l.wz = take((size_t)(BH * nch * F) * 4);
  l.dwq = take((size_t)(BH * ng * a->d * a->f) * 4);
  l.dwk = take((size_t)(BH * ng * a->d * a->f) * 4);
  l.da = take((size_t)BH * 4);
  l.bytes = o;
  return l;
}
const hm::BwdEntry *find_bwd(int dt, int64_t dk, int64_t fh, int64_t dv, int rope) {
  const hm::BwdTable t = hm::table_bwd();
  for (int i = 0; i < t.nbwd; ++i)
    if (t.bwd[i].dtype == dt && t.bwd[i].dk == dk && t.bwd[i].fh == fh && t.bwd[i].dv == dv && t.bwd[i].rope == rope)
      return &t.bwd[i];
  return nullptr;
}
hm_status validate_bwd(const hm_linattn_bwd_args *a) {
  if (!a) return fail(HM_ERR_NULL, "args is NULL");
  if (a->dtype != HM_F32 && a->dtype != HM_BF16) return fail(HM_ERR_DTYPE, "dtype %d is not HM_F32 or HM_BF16", a->dtype);
  if (a->B < 0 || a->H < 0 || a->n < 0 || a->d <= 0 || a->f <= 0 || a->dv <= 0)
    return fail(HM_ERR_SHAPE, "sizes must be B, H, n >= 0 and d, f, dv >= 1");
  if (a->B * a->H > 0) {
    if (!a->w_q || !a->w_k || !a->d_wq || !a->d_wk)
      return fail(HM_ERR_NULL, "w_q, w_k, d_wq and d_wk must be non-NULL");
    if (a->n > 0 && (!a->q || !a->k || !a->v || !a->d_o || !a->d_q || !a->d_k || !a->d_v || !a->save))
      return fail(HM_ERR_NULL, "q, k, v, d_o, save, d_q, d_k and d_v must be non-NULL");
    if (a->gate && a->n > 0 && !a->d_gate) return fail(HM_ERR_NULL, "d_gate is required with a gate");
  }
  // with no token dt may be NULL beside A_log (an empty tensor); d_a_log is then zero
  if (a->n > 0 && (a->dt == nullptr) != (a->a_log == nullptr)) return fail(HM_ERR_NULL, "dt and a_log must be given together");
  if (a->a_log && a->B * a->H > 0 && (!a->d_a_log || (a->n > 0 && !a->d_dt)))
    return fail(HM_ERR_NULL, "d_dt and d_a_log are required with dt");
  const int64_t strides[] = {a->sq_b, a->sq_h, a->sq_t, a->sk_b, a->sk_h, a->sk_t, a->sv_b, a->sv_h,
                             a->sv_t, a->so_b, a->so_h, a->so_t, a->sg_b, a->sg_h, a->sg_t, a->sw_h};
  for (int64_t s : strides)
    if (s < 0) return fail(HM_ERR_SHAPE, "strides must be non-negative");
  if (a->sdt_b < 0 || a->sdt_h < 0 || a->sdt_t < 0) return fail(HM_ERR_SHAPE, "dt strides must be non-negative");
  if (a->n > 1 && (a->so_t < a->dv || a->sq_t < a->d || a->sk_t < a->d || a->sv_t < a->dv ||
                   (a->gate && a->sg_t < a->dv)))
    return fail(HM_ERR_SHAPE, "token stride smaller than the row length (rows overlap)");
  if (a->sw_h != 0 && a->sw_h != a->d * a->f)
    return fail(HM_ERR_SHAPE, "sw_h must be 0 (one W) or d*f (contiguous per-head W)");
  const void *ptrs[] = {a->q, a->k, a->v, a->w_q, a->w_k, a->d_o, a->gate, a->d_gate, a->d_q, a->d_k, a->d_v,
                        a->save, a->workspace, a->d_s_final, a->d_s_init};
  for (const void *p : ptrs)
    if (!aligned16(p)) return fail(HM_ERR_ALIGN, "tensors, save and workspace must be 16-byte aligned");
  for (int64_t s : strides)
    if (!stride_ok(s, a->dtype)) return fail(HM_ERR_ALIGN, "every stride times the element size must be a multiple of 16 bytes");
  {
    const hm_status rs = validate_rope(a->rope_dims, a->rope_base, a->rope_pos0, a->f, false);
    if (rs != HM_OK) return rs;
  }
  if (!find_bwd(a->dtype, a->d, a->f, a->dv, a->rope_dims != 0))
    return fail(HM_ERR_UNSUPPORTED, "no backward kernels for dtype=%d d=%lld f=%lld dv=%lld", a->dtype,
                (long long)a->d, (long long)a->f, (long long)a->dv);
  return ok();
}
}  // namespace

hm_status hm_linattn_bwd_workspace_size(const hm_linattn_bwd_args *a, size_t *bytes) {
  if (!bytes) return fail(HM_ERR_NULL, "bytes is NULL");
  hm_status st = validate_bwd(a);
  if (st != HM_OK) return st;
  *bytes = bwd_layout(a).bytes;
  return ok();
}

hm_status hm_linattn_bwd(const hm_linattn_bwd_args *a, void *stream) {
  hm_status st = validate_bwd(a);
  if (st != HM_OK) return st;
  const int64_t BH = a->B * a->H;
  if (BH == 0) return ok();
  const SaveLayout sl = save_layout(a->dtype, BH, a->n, a->f, a->dv);
  if (a->save_bytes < sl.bytes) return fail(HM_ERR_WORKSPACE, "save buffer of %zu bytes expected, got %zu", sl.bytes, a->save_bytes);
  const BwdLayout wl = bwd_layout(a);
  if (!a->workspace || a->workspace_bytes < wl.bytes)
    return fail(HM_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", wl.bytes, a->workspace ? a->workspace_bytes : 0);
  char *ws = (char *)a->workspace;
  const char *sv = (const char *)a->save;
  hm::BwdParams p{};
  p.q = a->q; p.k = a->k; p.v = a->v; p.wq = a->w_q; p.wk = a->w_k;
  p.dt = a->n > 0 ? a->dt : nullptr; p.a_log = a->a_log; p.d_o = a->d_o; p.ds_final = a->d_s_final;
  p.gate = a->gate; p.d_gate = a->d_gate; p.sg_b = a->sg_b; p.sg_h = a->sg_h; p.sg_t = a->sg_t;
  p.sck = (const float *)(sv + sl.off_ck); p.sden = (const float *)(sv + sl.off_den);
  p.wS = ws + wl.wS; p.wz = (float *)(ws + wl.wz);
  p.so32 = (const float *)(sv + sl.off_o);
  p.phq = ws + wl.phq; p.phk = ws + wl.phk; p.dnum = ws + wl.dnum;
  p.dden = (float *)(ws + wl.dden); p.Lc = (float *)(ws + wl.Lc);
  p.eQ = (float *)(ws + wl.eQ); p.eK = (float *)(ws + wl.eK); p.eW = (float *)(ws + wl.eW);
  p.Xc = (float *)(ws + wl.Xc);
  p.gS = ws + wl.gS; p.gz = (float *)(ws + wl.gz);
  p.dwq_part = (float *)(ws + wl.dwq); p.dwk_part = (float *)(ws + wl.dwk); p.da_part = (float *)(ws + wl.da);
  p.dq = a->d_q; p.dk = a->d_k; p.dv = a->d_v;
  p.dwq = a->d_wq; p.dwk = a->d_wk; p.ddt = a->d_dt; p.da_log = a->a_log ? a->d_a_log : nullptr; p.ds_init = a->d_s_init;
  p.B = a->B; p.H = a->H; p.n = a->n; p.nch = (a->n + hm::CHUNK - 1) / hm::CHUNK;
  p.sq_b = a->sq_b; p.sq_h = a->sq_h; p.sq_t = a->sq_t; p.sk_b = a->sk_b; p.sk_h = a->sk_h; p.sk_t = a->sk_t;
  p.sv_b = a->sv_b; p.sv_h = a->sv_h; p.sv_t = a->sv_t; p.so_b = a->so_b; p.so_h = a->so_h; p.so_t = a->so_t;
  p.sw_h = a->sw_h; p.sdt_b = a->sdt_b; p.sdt_h = a->sdt_h; p.sdt_t = a->sdt_t;
  p.ngrp = wl.ngrp;
  p.rope_dims = a->rope_dims; p.rope_base = a->rope_base; p.rope_pos0 = a->rope_pos0;
  find_bwd(a->dtype, a->d, a->f, a->dv, a->rope_dims != 0)->launch(p, (hipStream_t)stream);
  return check_launch("backward");
}

// ------------------------------------------------------------------ decode
}  // extern "C"

namespace {
// Checks shared by the decode steps (hm_linattn_step, hm_linattn_pc_step).
hm_status validate_step(const hm_linattn_step_args *a) {
  if (!a) return fail(HM_ERR_NULL, "args is NULL");
  if (a->dtype != HM_F32 && a->dtype != HM_BF16) return fail(HM_ERR_DTYPE, "dtype %d is not HM_F32 or HM_BF16", a->dtype);
  if (a->B < 0 || a->H < 0 || a->d <= 0 || a->f <= 0 || a->dv <= 0)
    return fail(HM_ERR_SHAPE, "sizes must be B, H >= 0 and d, f, dv >= 1");
  if (a->B * a->H > 0 && (!a->q || !a->k || !a->v || !a->w_q || !a->w_k || !a->o || !a->state))
    return fail(HM_ERR_NULL, "q, k, v, w_q, w_k, state and o must be non-NULL");
  if ((a->dt == nullptr) != (a->a_log == nullptr)) return fail(HM_ERR_NULL, "dt and a_log must be given together");
  const int64_t strides[] = {a->sq_b, a->sq_h, a->sk_b, a->sk_h, a->sv_b, a->sv_h, a->so_b, a->so_h, a->sw_h};
  for (int64_t s : strides)
    if (s < 0) return fail(HM_ERR_SHAPE, "strides must be non-negative");
  if (a->sdt_b < 0 || a->sdt_h < 0) return fail(HM_ERR_SHAPE, "dt strides must be non-negative");
  const void *ptrs[] = {a->q, a->k, a->v, a->w_q, a->w_k, a->o, a->state};
  for (const void *p : ptrs)
    if (!aligned16(p)) return fail(HM_ERR_ALIGN, "q, k, v, w_q, w_k, o and state must be 16-byte aligned");
  if (a->gate) {
    if (a->sg_b < 0 || a->sg_h < 0) return fail(HM_ERR_SHAPE, "gate strides must be non-negative");
    if (!aligned16(a->gate)) return fail(HM_ERR_ALIGN, "gate must be 16-byte aligned");
    if (!stride_ok(a->sg_b, a->dtype) || !stride_ok(a->sg_h, a->dtype))
      return fail(HM_ERR_ALIGN, "every stride times the element size must be a multiple of 16 bytes");
  }
  for (int64_t s : strides)
    if (!stride_ok(s, a->dtype)) return fail(HM_ERR_ALIGN, "every stride times the element size must be a multiple of 16 bytes");
  if (a->conv_width < 0) return fail(HM_ERR_SHAPE, "conv_width must be >= 0");
  if (a->conv_width > 4) return fail(HM_ERR_UNSUPPORTED, "conv_width %d: 1 to 4 taps are built", a->conv_width);
  if (a->conv_width > 0) {
    if (a->B * a->H > 0 && (!a->conv_wq || !a->conv_wk || (a->conv_width > 1 && (!a->conv_sq || !a->conv_sk))))
      return fail(HM_ERR_NULL, "conv taps and conv states must be non-NULL when conv_width > 0");
    if (a->scw_h < 0 || a->scb_h < 0) return fail(HM_ERR_SHAPE, "conv strides must be non-negative");
    const uintptr_t ea = (uintptr_t)esize(a->dtype) - 1;
    if (((uintptr_t)a->conv_wq | (uintptr_t)a->conv_wk | (uintptr_t)a->conv_bq | (uintptr_t)a->conv_bk) & 3 ||
        ((uintptr_t)a->conv_sq | (uintptr_t)a->conv_sk) & ea)
      return fail(HM_ERR_ALIGN, "conv taps, bias and states must be aligned to their element size");
  }
  {
    const hm_status rs = validate_rope(a->rope_dims, a->rope_base, a->rope_pos, a->f, a->B * a->H > 0);
    if (rs != HM_OK) return rs;
  }
  return ok();
}

hm::StepParams step_params(const hm_linattn_step_args *a) {
  hm::StepParams p{};
  p.q = a->q; p.k = a->k; p.v = a->v; p.wq = a->w_q; p.wk = a->w_k;
  p.dt = a->dt; p.a_log = a->a_log; p.state = a->state; p.o = a->o;
  p.B = a->B; p.H = a->H;
  p.sq_b = a->sq_b; p.sq_h = a->sq_h; p.sk_b = a->sk_b; p.sk_h = a->sk_h;
  p.sv_b = a->sv_b; p.sv_h = a->sv_h; p.so_b = a->so_b; p.so_h = a->so_h;
  p.sw_h = a->sw_h; p.sdt_b = a->sdt_b; p.sdt_h = a->sdt_h;
  p.gate = a->gate; p.sg_b = a->sg_b; p.sg_h = a->sg_h;
  p.cwidth = a->conv_width;
  p.cwq = a->conv_wq; p.cwk = a->conv_wk; p.cbq = a->conv_bq; p.cbk = a->conv_bk;
  p.csq = a->conv_sq; p.csk = a->conv_sk; p.scw_h = a->scw_h; p.scb_h = a->scb_h;
  p.rope_dims = a->rope_dims; p.rope_base = a->rope_base; p.rope_pos = a->rope_pos;
  return p;
}
}  // namespace

extern "C" {

hm_status hm_linattn_step(const hm_linattn_step_args *a, void *stream) {
  hm_status st = validate_step(a);
  if (st != HM_OK) return st;
  const int decay = a->dt != nullptr;
  const hm::StepEntry *e = find_step(a->dtype, a->d, a->f, a->dv, decay);
  if (!e)
    return fail(HM_ERR_UNSUPPORTED, "no decode kernel for dtype=%d d=%lld f=%lld dv=%lld", a->dtype, (long long)a->d,
                (long long)a->f, (long long)a->dv);
  const int64_t BH = a->B * a->H;
  if (BH == 0) return ok();
  const hm::StepParams p = step_params(a);
  e->launch(p, (unsigned)BH, (hipStream_t)stream);
  return check_launch("decode step");
}

// ------------------------------------------------------------------ per-channel decay
}  // extern "C"

namespace {
const hm::PcEntry *find_pc(int dt, int64_t dk, int64_t fh, int64_t dv) {
  const hm::PcTable t = hm::table_pc();
  for (int i = 0; i < t.npc; ++i)
    if (t.pc[i].dtype == dt && t.pc[i].dk == dk && t.pc[i].fh == fh && t.pc[i].dv == dv) return &t.pc[i];
  return nullptr;
}
// A_log: [dv][F] rows per head, shared (sa_h = 0) or one block per head.
hm_status validate_a_log_pc(const float *a_log, int64_t sa_h, int64_t dv, int64_t F) {
  if (sa_h != 0 && sa_h != dv * F) return fail(HM_ERR_SHAPE, "sa_h must be 0 (shared A_log) or dv*2f (one per head)");
  if (!aligned16(a_log)) return fail(HM_ERR_ALIGN, "a_log must be 16-byte aligned");
  return ok();
}
}  // namespace

extern "C" {

// Segments of the per-channel prefill: automatic when fewer than 65 workgroups
// (one per (b, h) and cpw channels) would run, up to 256 / workgroups segments of
// at least four chunks; workspace = one state block per segment and (b, h) plus dv
// floats per segment boundary.
struct PcPlan {
  int nseg;
  int64_t seg_len;
  size_t off_dsum, bytes;
};
PcPlan pc_plan(const hm_linattn_pc_args *a, int cpw) {
  const int64_t BH = a->B * a->H, nch = (a->n + hm::CHUNK - 1) / hm::CHUNK, F = 2 * a->f;
  int64_t ns = a->segments;
  if (ns <= 0) {
    const int64_t wgs = BH * (a->dv / cpw);
    ns = 1;
    if (wgs > 0 && wgs <= 64) {
      ns = 256 / wgs;
      if (ns > nch / 4) ns = nch / 4;
    }
  }
  if (ns > nch) ns = nch;
  if (ns < 1) ns = 1;
  PcPlan pl{};
  pl.seg_len = ((nch + ns - 1) / ns) * hm::CHUNK;
  pl.nseg = a->n > 0 ? (int)((a->n + pl.seg_len - 1) / pl.seg_len) : 1;
  if (pl.nseg <= 1) {
    pl.nseg = 1;
    pl.seg_len = a->n;
    return pl;
  }
  pl.off_dsum = align256((size_t)(BH * pl.nseg * 2 * a->dv * F) * 4);
  pl.bytes = pl.off_dsum + (size_t)(BH * (pl.nseg - 1) * a->dv) * 4;
  return pl;
}
hm_status pc_plan_checked(const hm_linattn_pc_args *a, PcPlan *pl) {
  if (!a) return fail(HM_ERR_NULL, "args is NULL");
  if (a->dtype != HM_F32 && a->dtype != HM_BF16) return fail(HM_ERR_DTYPE, "dtype %d is not HM_F32 or HM_BF16", a->dtype);
  if (a->B < 0 || a->H < 0 || a->n < 0 || a->d <= 0 || a->f <= 0 || a->dv <= 0)
    return fail(HM_ERR_SHAPE, "sizes must be B, H, n >= 0 and d, f, dv >= 1");
  if (a->segments < 0) return fail(HM_ERR_SHAPE, "segments must be >= 0 (0 = automatic)");
  const hm::PcEntry *e = find_pc(a->dtype, a->d, a->f, a->dv);
  if (!e)
    return fail(HM_ERR_UNSUPPORTED, "no per-channel kernel for dtype=%d d=%lld f=%lld dv=%lld", a->dtype,
                (long long)a->d, (long long)a->f, (long long)a->dv);
  *pl = pc_plan(a, e->cpw);
  return ok();
}

hm_status hm_linattn_pc_fwd_plan(const hm_linattn_pc_args *a, int32_t *segments) {
  if (!segments) return fail(HM_ERR_NULL, "segments is NULL");
  PcPlan pl{};
  const hm_status st = pc_plan_checked(a, &pl);
  if (st != HM_OK) return st;
  *segments = pl.nseg;
  return ok();
}

hm_status hm_linattn_pc_fwd_workspace_size(const hm_linattn_pc_args *a, size_t *bytes) {
  if (!bytes) return fail(HM_ERR_NULL, "bytes is NULL");
  PcPlan pl{};
  const hm_status st = pc_plan_checked(a, &pl);
  if (st != HM_OK) return st;
  *bytes = pl.bytes;
  return ok();
}

hm_status hm_linattn_pc_fwd(const hm_linattn_pc_args *a, void *stream) {
  if (!a) return fail(HM_ERR_NULL, "args is NULL");
  if (a->segments < 0) return fail(HM_ERR_SHAPE, "segments must be >= 0 (0 = automatic)");
  if (a->dtype != HM_F32 && a->dtype != HM_BF16) return fail(HM_ERR_DTYPE, "dtype %d is not HM_F32 or HM_BF16", a->dtype);
  if (a->B < 0 || a->H < 0 || a->n < 0 || a->d <= 0 || a->f <= 0 || a->dv <= 0)
    return fail(HM_ERR_SHAPE, "sizes must be B, H, n >= 0 and d, f, dv >= 1");
  const int64_t BH = a->B * a->H, F = 2 * a->f;
  if (BH * a->n > 0 && (!a->q || !a->k || !a->v || !a->w_q || !a->w_k || !a->o || !a->dt || !a->a_log))
    return fail(HM_ERR_NULL, "q, k, v, w_q, w_k, o, dt and a_log must be non-NULL");
  const int64_t strides[] = {a->sq_b, a->sq_h, a->sq_t, a->sk_b, a->sk_h, a->sk_t, a->sv_b,
                             a->sv_h, a->sv_t, a->so_b, a->so_h, a->so_t, a->sw_h};
  for (int64_t s : strides)
    if (s < 0) return fail(HM_ERR_SHAPE, "strides must be non-negative");
  if (a->sdt_b < 0 || a->sdt_h < 0 || a->sdt_t < 0 || a->sg_b < 0 || a->sg_h < 0 || a->sg_t < 0 || a->sa_h < 0)
    return fail(HM_ERR_SHAPE, "strides must be non-negative");
  if (a->n > 1 && (a->so_t < a->dv || a->sq_t < a->d || a->sk_t < a->d || a->sv_t < a->dv || a->sdt_t < a->dv ||
                   (a->gate && a->sg_t < a->dv)))
    return fail(HM_ERR_SHAPE, "token stride smaller than the row length (rows overlap)");
  const void *ptrs[] = {a->q, a->k, a->v, a->w_q, a->w_k, a->o, a->gate, a->s_init, a->s_final};
  for (const void *p : ptrs)
    if (!aligned16(p)) return fail(HM_ERR_ALIGN, "q, k, v, w_q, w_k, o, gate and the states must be 16-byte aligned");
  if ((uintptr_t)a->dt & 3) return fail(HM_ERR_ALIGN, "dt must be 4-byte aligned");
  for (int64_t s : strides)
    if (!stride_ok(s, a->dtype)) return fail(HM_ERR_ALIGN, "every stride times the element size must be a multiple of 16 bytes");
  if (a->gate && (!stride_ok(a->sg_b, a->dtype) || !stride_ok(a->sg_h, a->dtype) || !stride_ok(a->sg_t, a->dtype)))
    return fail(HM_ERR_ALIGN, "every stride times the element size must be a multiple of 16 bytes");
  hm_status st = validate_a_log_pc(a->a_log, a->sa_h, a->dv, F);
  if (st != HM_OK) return st;
  if ((st = validate_rope(a->rope_dims, a->rope_base, a->rope_pos0, a->f, false)) != HM_OK) return st;
  if (a->s_init && a->s_final && a->s_init != a->s_final) {
    // each thread reads its own state elements first and writes the same ones last, so
    // the same buffer is safe; a partial overlap would let workgroups race
    const char *i0 = (const char *)a->s_init, *f0 = (const char *)a->s_final;
    const size_t len = (size_t)BH * 2 * a->dv * F * 4;
    if (i0 < f0 + len && f0 < i0 + len) return fail(HM_ERR_SHAPE, "s_init and s_final overlap without being the same buffer");
  }
  const hm::PcEntry *e = find_pc(a->dtype, a->d, a->f, a->dv);
  if (!e)
    return fail(HM_ERR_UNSUPPORTED, "no per-channel kernel for dtype=%d d=%lld f=%lld dv=%lld", a->dtype,
                (long long)a->d, (long long)a->f, (long long)a->dv);
  const PcPlan pl = pc_plan(a, e->cpw);
  if (pl.bytes > 0) {
    if (!a->workspace || a->workspace_bytes < pl.bytes)
      return fail(HM_ERR_WORKSPACE, "workspace of %zu bytes needed for %d segments (got %zu)", pl.bytes, pl.nseg,
                  a->workspace ? a->workspace_bytes : (size_t)0);
    if (!aligned16(a->workspace)) return fail(HM_ERR_ALIGN, "workspace must be 16-byte aligned");
  }
  if (BH == 0 || (a->n == 0 && !a->s_final)) return ok();
  hm::PcParams p{};
  p.nseg = pl.nseg;
  p.seg_len = pl.seg_len;
  if (pl.nseg > 1) {
    p.slots = (float *)a->workspace;
    p.dsum = (float *)((char *)a->workspace + pl.off_dsum);
  }
  p.q = a->q; p.k = a->k; p.v = a->v; p.wq = a->w_q; p.wk = a->w_k;
  p.dt = a->dt; p.a_log = a->a_log; p.s_init = a->s_init; p.s_final = a->s_final; p.o = a->o; p.gate = a->gate;
  p.B = a->B; p.H = a->H; p.n = a->n;
  p.sq_b = a->sq_b; p.sq_h = a->sq_h; p.sq_t = a->sq_t; p.sk_b = a->sk_b; p.sk_h = a->sk_h; p.sk_t = a->sk_t;
  p.sv_b = a->sv_b; p.sv_h = a->sv_h; p.sv_t = a->sv_t; p.so_b = a->so_b; p.so_h = a->so_h; p.so_t = a->so_t;
  p.sg_b = a->sg_b; p.sg_h = a->sg_h; p.sg_t = a->sg_t;
  p.sw_h = a->sw_h; p.sdt_b = a->sdt_b; p.sdt_h = a->sdt_h; p.sdt_t = a->sdt_t; p.sa_h = a->sa_h;
  p.rope_dims = a->rope_dims; p.rope_base = a->rope_base; p.rope_pos0 = a->rope_pos0;
  e->fwd(p, (hipStream_t)stream);
  return check_launch("per-channel prefill");
}

hm_status hm_linattn_pc_step(const hm_linattn_pc_step_args *a, void *stream) {
  if (!a) return fail(HM_ERR_NULL, "args is NULL");
  // the fields shared with hm_linattn_step pass through its checks
  hm_linattn_step_args sa{};
  sa.q = a->q; sa.k = a->k; sa.v = a->v; sa.w_q = a->w_q; sa.w_k = a->w_k;
  sa.dt = a->dt; sa.a_log = a->a_log; sa.state = a->state; sa.o = a->o;
  sa.dtype = a->dtype; sa.conv_width = a->conv_width;
  sa.B = a->B; sa.H = a->H; sa.d = a->d; sa.f = a->f; sa.dv = a->dv;
  sa.sq_b = a->sq_b; sa.sq_h = a->sq_h; sa.sk_b = a->sk_b; sa.sk_h = a->sk_h; sa.sv_b = a->sv_b; sa.sv_h = a->sv_h;
  sa.so_b = a->so_b; sa.so_h = a->so_h; sa.sw_h = a->sw_h; sa.sdt_b = a->sdt_b; sa.sdt_h = a->sdt_h;
  sa.gate = a->gate; sa.sg_b = a->sg_b; sa.sg_h = a->sg_h;
  sa.conv_wq = a->conv_wq; sa.conv_wk = a->conv_wk; sa.conv_bq = a->conv_bq; sa.conv_bk = a->conv_bk;
  sa.conv_sq = a->conv_sq; sa.conv_sk = a->conv_sk; sa.scw_h = a->scw_h; sa.scb_h = a->scb_h;
  sa.rope_dims = a->rope_dims; sa.rope_base = a->rope_base; sa.rope_pos = a->rope_pos;
  hm_status st = validate_step(&sa);
  if (st != HM_OK) return st;
  const int64_t BH = a->B * a->H;
  if (BH > 0 && (!a->dt || !a->a_log)) return fail(HM_ERR_NULL, "dt and a_log are required");
  if (a->sa_h < 0) return fail(HM_ERR_SHAPE, "strides must be non-negative");
  if ((uintptr_t)a->dt & 3) return fail(HM_ERR_ALIGN, "dt must be 4-byte aligned");
  if ((st = validate_a_log_pc(a->a_log, a->sa_h, a->dv, 2 * a->f)) != HM_OK) return st;
  const hm::PcEntry *e = find_pc(a->dtype, a->d, a->f, a->dv);
  if (!e)
    return fail(HM_ERR_UNSUPPORTED, "no per-channel kernel for dtype=%d d=%lld f=%lld dv=%lld", a->dtype,
                (long long)a->d, (long long)a->f, (long long)a->dv);
  if (BH == 0) return ok();
  hm::PcStepParams p{};
  p.s = step_params(&sa);
  p.dt = a->dt; p.a_log = a->a_log; p.state = a->state;
  p.sdt_b = a->sdt_b; p.sdt_h = a->sdt_h; p.sa_h = a->sa_h;
  e->step(p, (hipStream_t)stream);
  return check_launch("per-channel decode step");
}

// ------------------------------------------------------------------ short conv
hm_status hm_causal_conv(const hm_causal_conv_args *a, void *stream) {
  if (!a) return fail(HM_ERR_NULL, "args is NULL");
  if (a->dtype != HM_F32 && a->dtype != HM_BF16) return fail(HM_ERR_DTYPE, "dtype %d is not HM_F32 or HM_BF16", a->dtype);
  if (a->B < 0 || a->H < 0 || a->n < 0 || a->d <= 0 || a->width <= 0)
    return fail(HM_ERR_SHAPE, "sizes must be B, H, n >= 0 and d, width >= 1");
  if (a->width > 4) return fail(HM_ERR_UNSUPPORTED, "width %d: 1 to 4 taps are built", a->width);
  const int64_t BH = a->B * a->H;
  const size_t es = esize(a->dtype);
  if (BH > 0 && a->n > 0 && (!a->x || !a->y || !a->w)) return fail(HM_ERR_NULL, "x, y and w must be non-NULL");
  const int64_t strides[] = {a->sx_b, a->sx_h, a->sx_t, a->sy_b, a->sy_h, a->sy_t, a->sw_h, a->sb_h};
  for (int64_t s : strides)
    if (s < 0) return fail(HM_ERR_SHAPE, "strides must be non-negative");
  if (a->n > 1 && a->sy_t < a->d) return fail(HM_ERR_SHAPE, "token stride of y smaller than the row length (rows overlap)");
  if (((size_t)a->d * es) % 16) return fail(HM_ERR_UNSUPPORTED, "d times the element size must be a multiple of 16 bytes");
  if (!aligned16(a->x) || !aligned16(a->y) || !aligned16(a->w) || !aligned16(a->prev) || !aligned16(a->final_rows))
    return fail(HM_ERR_ALIGN, "x, y, w, prev and final_rows must be 16-byte aligned");
  if (((uintptr_t)a->bias & 3) != 0) return fail(HM_ERR_ALIGN, "bias must be 4-byte aligned");
  if (!stride_ok(a->sx_b, a->dtype) || !stride_ok(a->sx_h, a->dtype) || !stride_ok(a->sx_t, a->dtype) ||
      !stride_ok(a->sy_b, a->dtype) || !stride_ok(a->sy_h, a->dtype) || !stride_ok(a->sy_t, a->dtype) ||
      ((size_t)a->sw_h * 4) % 16)
    return fail(HM_ERR_ALIGN, "every stride times the element size must be a multiple of 16 bytes");
  if (BH == 0) return ok();
  // byte ranges: y must not overlap an input; final_rows is prev itself or apart from it
  auto span = [&](const void *p, int64_t sb, int64_t sh, int64_t st, int64_t rows) {
    const char *lo = (const char *)p;
    const int64_t last = (a->B - 1) * sb + (a->H - 1) * sh + (rows - 1) * st + a->d;
    return std::make_pair(lo, lo + (size_t)last * es);
  };
  auto apart = [](std::pair<const char *, const char *> u, std::pair<const char *, const char *> v) {
    return u.second <= v.first || v.second <= u.first;
  };
  const int64_t R = a->width - 1, blk = R * a->d;
  if (a->n > 0) {
    const auto ys = span(a->y, a->sy_b, a->sy_h, a->sy_t, a->n);
    if (!apart(ys, span(a->x, a->sx_b, a->sx_h, a->sx_t, a->n))) return fail(HM_ERR_SHAPE, "y overlaps x");
    if (R > 0 && a->prev && !apart(ys, span(a->prev, a->H * blk, blk, a->d, R))) return fail(HM_ERR_SHAPE, "y overlaps prev");
    if (R > 0 && a->final_rows && !apart(ys, span(a->final_rows, a->H * blk, blk, a->d, R)))
      return fail(HM_ERR_SHAPE, "y overlaps final_rows");
  }
  if (R > 0 && a->prev && a->final_rows && a->prev != a->final_rows &&
      !apart(span(a->prev, a->H * blk, blk, a->d, R), span(a->final_rows, a->H * blk, blk, a->d, R)))
    return fail(HM_ERR_SHAPE, "final_rows overlaps prev without being the same buffer");
  const hm::ConvTable ct = hm::table_conv();
  const hm::ConvEntry *e = nullptr;
  for (int i = 0; i < ct.nconv; ++i)
    if (ct.conv[i].dtype == a->dtype && ct.conv[i].width == a->width) e = &ct.conv[i];
  if (!e) return fail(HM_ERR_UNSUPPORTED, "no conv kernel for dtype=%d width=%d", a->dtype, a->width);
  if (a->n == 0 && (R == 0 || !a->final_rows)) return ok();
  hm::ConvParams p{};
  p.x = a->x; p.y = a->y; p.w = a->w; p.bias = a->bias; p.prev = R > 0 ? a->prev : nullptr;
  p.fin = R > 0 ? a->final_rows : nullptr;
  p.B = a->B; p.H = a->H; p.n = a->n; p.d = a->d;
  p.sx_b = a->sx_b; p.sx_h = a->sx_h; p.sx_t = a->sx_t;
  p.sy_b = a->sy_b; p.sy_h = a->sy_h; p.sy_t = a->sy_t; p.sw_h = a->sw_h; p.sb_h = a->sb_h;
  p.runs = a->n > 0 ? (a->n + hm::CONV_RUN - 1) / hm::CONV_RUN : 1;
  p.groups = (int64_t)((size_t)a->d * es / 16);
  const int64_t threads = BH * p.runs * p.groups;
  if (threads >= (int64_t)1 << 31) return fail(HM_ERR_UNSUPPORTED, "B*H*n*d too large: more than 2^31 conv threads");
  e->launch(p, dim3((unsigned)((threads + 255) / 256)), (hipStream_t)stream);
  return check_launch("causal conv");
}

// ------------------------------------------------------------------ featurize
hm_status hm_featurize(const hm_featurize_args *a, void *stream) {
  if (!a) return fail(HM_ERR_NULL, "args is NULL");
  if ((a->dtype != HM_F32 && a->dtype != HM_BF16) || (a->phi_dtype != HM_F32 && a->phi_dtype != HM_BF16))
    return fail(HM_ERR_DTYPE, "dtype %d / phi_dtype %d must be HM_F32 or HM_BF16", a->dtype, a->phi_dtype);
  if (a->B < 0 || a->H < 0 || a->n < 0 || a->d <= 0 || a->f <= 0)
    return fail(HM_ERR_SHAPE, "sizes must be B, H, n >= 0 and d, f >= 1");
  if (a->B * a->H * a->n > 0 && (!a->x || !a->w || !a->phi)) return fail(HM_ERR_NULL, "x, w and phi must be non-NULL");
  if (a->sx_b < 0 || a->sx_h < 0 || a->sx_t < 0 || a->sw_h < 0 || a->sp_b < 0 || a->sp_h < 0 || a->sp_t < 0)
    return fail(HM_ERR_SHAPE, "strides must be non-negative");
  if (a->n > 1 && (a->sx_t < a->d || a->sp_t < 2 * a->f))
    return fail(HM_ERR_SHAPE, "token stride smaller than the row length (rows overlap)");
  if (!aligned16(a->x) || !aligned16(a->w) || !aligned16(a->phi))
    return fail(HM_ERR_ALIGN, "x, w and phi must be 16-byte aligned");
  if (!stride_ok(a->sx_b, a->dtype) || !stride_ok(a->sx_h, a->dtype) || !stride_ok(a->sx_t, a->dtype) ||
      !stride_ok(a->sw_h, a->dtype) || !stride_ok(a->sp_b, a->phi_dtype) || !stride_ok(a->sp_h, a->phi_dtype) ||
      !stride_ok(a->sp_t, a->phi_dtype))
    return fail(HM_ERR_ALIGN, "every stride times the element size must be a multiple of 16 bytes");
  {
    const hm_status rs = validate_rope(a->rope_dims, a->rope_base, a->rope_pos0, a->f, false);
    if (rs != HM_OK) return rs;
  }
  if (a->conv_width < 0 || a->conv_width > 4)
    return fail(HM_ERR_UNSUPPORTED, "conv_width %d: built are 0 (none) to 4", a->conv_width);
  if (a->conv_width > 0 && a->B * a->H * a->n > 0 && !a->conv_w) return fail(HM_ERR_NULL, "conv_width > 0 needs conv_w");
  if (a->scw_h < 0 || a->scb_h < 0) return fail(HM_ERR_SHAPE, "conv strides must be non-negative");
  if (a->conv_prev && !aligned16(a->conv_prev)) return fail(HM_ERR_ALIGN, "conv_prev must be 16-byte aligned");
  const hm::FeatEntry *e = find_feat(a->dtype, a->phi_dtype, a->d, a->f);
  if (!e)
    return fail(HM_ERR_UNSUPPORTED, "no featurize kernel for dtype=%d phi_dtype=%d d=%lld f=%lld", a->dtype,
                a->phi_dtype, (long long)a->d, (long long)a->f);
  const int64_t BH = a->B * a->H;
  if (BH == 0 || a->n == 0) return ok();
  hm::FeatParams p{};
  p.x = a->x; p.w = a->w; p.phi = a->phi;
  p.B = a->B; p.H = a->H; p.n = a->n;
  p.sx_b = a->sx_b; p.sx_h = a->sx_h; p.sx_t = a->sx_t; p.sw_h = a->sw_h;
  p.sp_b = a->sp_b; p.sp_h = a->sp_h; p.sp_t = a->sp_t;
  p.rope_dims = a->rope_dims; p.rope_base = a->rope_base; p.rope_pos0 = a->rope_pos0;
  p.cwidth = a->conv_width; p.cw = a->conv_w; p.cb = a->conv_b; p.cprev = a->conv_prev;
  p.scw_h = a->scw_h; p.scb_h = a->scb_h;
  const int64_t per = 64 * hm::kFeatBlocks;  // tokens per workgroup
  e->launch(p, dim3((unsigned)((a->n + per - 1) / per), (unsigned)BH), (hipStream_t)stream);
  return check_launch("featurize");
}

const char *hm_status_string(int s) {
  switch (s) {
    case HM_OK: return "HM_OK";
    case HM_ERR_NULL: return "HM_ERR_NULL";
    case HM_ERR_SHAPE: return "HM_ERR_SHAPE";
    case HM_ERR_DTYPE: return "HM_ERR_DTYPE";
    case HM_ERR_ALIGN: return "HM_ERR_ALIGN";
    case HM_ERR_UNSUPPORTED: return "HM_ERR_UNSUPPORTED";
    case HM_ERR_WORKSPACE: return "HM_ERR_WORKSPACE";
    case HM_ERR_HIP: return "HM_ERR_HIP";
    default: return "HM_ERR_UNKNOWN";
  }
}

const char *hm_last_error_message(void) { return g_err.c_str(); }

int hm_abi_version(void) { return HM_ABI_VERSION; }

size_t hm_args_size(int which) {
  switch (which) {
    case 0: return sizeof(hm_featurize_args);
    case 1: return sizeof(hm_linattn_fwd_args);
    case 2: return sizeof(hm_linattn_step_args);
    case 3: return sizeof(hm_causal_conv_args);
    case 4: return sizeof(hm_linattn_bwd_args);
    case 5: return sizeof(hm_linattn_pc_args);
    case 6: return sizeof(hm_linattn_pc_step_args);
    default: return 0;
  }
}

}  // extern "C"
