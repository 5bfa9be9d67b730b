// Arguments of the backward-pass kernels (filled by the C ABI layer).
#pragma once

#include <stdint.h>

namespace hm {

struct BwdParams {
  const void *q, *k, *v, *wq, *wk;
  const float *dt, *a_log;
  const void *d_o;
  const void *gate;          // the forward's gate (NULL = none); d_gate gets its gradient
  void *d_gate;
  int64_t sg_b, sg_h, sg_t;
  const float *ds_final;     // dloss/ds_final (NULL = 0)
  const float *so32;         // saved float32 output before the gate [BH][n][dv]
  const float *sck;          // saved checkpoints: the float32 state at the start of every chunk range
                             // of the per-chunk kernels, [BH][ngrp][F*dv + F] (state layout)
  const float *sden;         // saved denominators [BH][n]
  void *wS;                  // workspace [BH][nch][F][dv] (dtype): chunk-start states, recomputed
  float *wz;                 // workspace [BH][nch][F]: z at every chunk start
  void *phq, *phk, *dnum;    // workspace [BH][n][F], [BH][n][F], [BH][n][dv] (dtype)
  float *dden, *Lc;          // workspace [BH][n]
  float *eQ, *eK, *eW;       // workspace [BH][n]: per-token pieces of d log a (see bwd_decay)
  float *Xc;                 // workspace [BH][nch]: pairs spanning a whole chunk
  void *gS;                  // workspace [BH][nch][F][dv] (dtype)
  float *gz;                 // workspace [BH][nch][F]
  float *dwq_part, *dwk_part;  // workspace [BH * ngrp][d][f]
  float *da_part;            // workspace [BH]
  void *dq, *dk, *dv;
  float *dwq, *dwk, *ddt, *da_log, *ds_init;
  int64_t B, H, n, nch;
  int64_t sq_b, sq_h, sq_t, sk_b, sk_h, sk_t, sv_b, sv_h, sv_t, so_b, so_h, so_t;
  int64_t sw_h, sdt_b, sdt_h, sdt_t;
  int ngrp;                  // chunk ranges per (b, h) in bwd_dq / bwd_dk / bwd_dv
  int rope_dims;             // the forward's rotary encoding (0 = off)
  float rope_base;
  const int64_t *rope_pos0;  // position of token 0 per batch row (NULL = 0)
};

}  // namespace hm
