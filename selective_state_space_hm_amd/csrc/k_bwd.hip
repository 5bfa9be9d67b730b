// Training-mode prefill (with and without the rotary encoding) and backward-pass
// instantiations: bf16 (d, f, dv) = (64, 32, 64) and (128, 64, 128); float32
// (16, 16, 16) and (32, 16, 32).
#include "hm_bwd.hpp"
#include "hm_kernels.hpp"

namespace hm {

template <typename T, int DK, int FH, int DV, bool ROPE>
void launch_bwd(const BwdParams &p, hipStream_t s) {
  const unsigned BH = (unsigned)(p.B * p.H);
  if (p.nch > 0) hipLaunchKernelGGL((bwd_prep<T, DK, FH, DV, ROPE>), dim3(BH * (unsigned)p.nch), dim3(256), 0, s, p);
  // the chunk-start states, recomputed from the forward's checkpoints; each range is
  // a chain of chunks, so the value columns are split in two to put two workgroups
  // on every compute unit (measured on the Pythia layer: 75 us unsplit, 66 us in
  // two, 89 us in four, where the redundant phi(k) reads take over)
  if (p.nch > 0) {
    const unsigned items = BH * (unsigned)p.ngrp;
    if constexpr (DV % 32 == 0) {
      hipLaunchKernelGGL((bwd_states<T, DK, FH, DV, 2>), dim3((items + 7) / 8 * 16), dim3(kChainWaves * 64), 0, s, p);
    } else {
      hipLaunchKernelGGL((bwd_states<T, DK, FH, DV, 1>), dim3(items), dim3(kChainWaves * 64), 0, s, p);
    }
  }
  // the gradient-state pass visits the chunks one after another, so with fewer
  // (b, h) than compute units it splits the value columns in two
  // (a four-way split measured slower on the Pythia layer: 105 vs 91 us)
  if constexpr (DV % 32 == 0) {
    if (BH < 256) {
      hipLaunchKernelGGL((bwd_gstate<T, DK, FH, DV, 2>), dim3((BH + 7) / 8 * 16), dim3(kChainWaves * 64), 0, s, p);
    } else {
      hipLaunchKernelGGL((bwd_gstate<T, DK, FH, DV, 1>), dim3(BH), dim3(kChainWaves * 64), 0, s, p);
    }
  } else {
    hipLaunchKernelGGL((bwd_gstate<T, DK, FH, DV, 1>), dim3(BH), dim3(kChainWaves * 64), 0, s, p);
  }
  hipLaunchKernelGGL((bwd_dq<T, DK, FH, DV, ROPE>), dim3(BH * (unsigned)p.ngrp), dim3(bwd_waves(ROPE) * 64), 0, s, p);
  hipLaunchKernelGGL((bwd_dk<T, DK, FH, DV, ROPE>), dim3(BH * (unsigned)p.ngrp), dim3(bwd_waves(ROPE) * 64), 0, s, p);
  if (p.nch > 0) hipLaunchKernelGGL((bwd_dv<T, DK, FH, DV>), dim3(BH * (unsigned)p.ngrp), dim3(bwd_waves(false) * 64), 0, s, p);
  if (p.a_log) hipLaunchKernelGGL(bwd_decay, dim3(BH), dim3(256), 0, s, p);  // dt may be NULL only when n = 0
  const int per_head = p.sw_h != 0;
  const int64_t nw = (per_head ? p.H : 1) * (int64_t)DK * FH;
  hipLaunchKernelGGL((bwd_reduce<DK, FH>), dim3((unsigned)((nw + 31) / 32)), dim3(256), 0, s, p, per_head);
}

#define HM_TRAIN(T, TC, DK, FH, DV)                                                   \
  HM_FWD_ENTRY(T, TC, DK, FH, DV, 0, 2), HM_FWD_ENTRY(T, TC, DK, FH, DV, 1, 2),      \
      HM_FWD_ENTRY(T, TC, DK, FH, DV, 0, 6), HM_FWD_ENTRY(T, TC, DK, FH, DV, 1, 6)
static const FwdEntry kTrain[] = {
    HM_TRAIN(bf16, HM_DT_BF16, 64, 32, 64), HM_TRAIN(bf16, HM_DT_BF16, 128, 64, 128),
    HM_TRAIN(float, HM_DT_F32, 16, 16, 16), HM_TRAIN(float, HM_DT_F32, 32, 16, 32),
};
#define HM_BWD(T, TC, DK, FH, DV) \
  {TC, DK, FH, DV, 0, &launch_bwd<T, DK, FH, DV, false>}, {TC, DK, FH, DV, 1, &launch_bwd<T, DK, FH, DV, true>}
static const BwdEntry kBwd[] = {
    HM_BWD(bf16, HM_DT_BF16, 64, 32, 64), HM_BWD(bf16, HM_DT_BF16, 128, 64, 128),
    HM_BWD(float, HM_DT_F32, 16, 16, 16), HM_BWD(float, HM_DT_F32, 32, 16, 32),
};
Table table_train() { return Table{kTrain, (int)(sizeof(kTrain) / sizeof(kTrain[0])), nullptr, 0, nullptr, 0}; }
BwdTable table_bwd() { return BwdTable{kBwd, (int)(sizeof(kBwd) / sizeof(kBwd[0]))}; }

}  // namespace hm
