// Decode-step and featurizer instantiations.
#include "hm_kernels.hpp"

namespace hm {
#define HM_STEP(T, TC, DK, FH, DV) \
  {TC, DK, FH, DV, 0, &launch_step<T, DK, FH, DV, false>}, {TC, DK, FH, DV, 1, &launch_step<T, DK, FH, DV, true>}
static const StepEntry kStep[] = {
    HM_STEP(bf16, HM_DT_BF16, 64, 32, 64),   HM_STEP(bf16, HM_DT_BF16, 64, 32, 128),
    HM_STEP(bf16, HM_DT_BF16, 64, 64, 64),   HM_STEP(bf16, HM_DT_BF16, 64, 64, 128),
    HM_STEP(bf16, HM_DT_BF16, 128, 32, 64),  HM_STEP(bf16, HM_DT_BF16, 128, 32, 128),
    HM_STEP(bf16, HM_DT_BF16, 128, 64, 64),  HM_STEP(bf16, HM_DT_BF16, 128, 64, 128),
    HM_STEP(bf16, HM_DT_BF16, 32, 16, 32),   HM_STEP(bf16, HM_DT_BF16, 64, 32, 32),
    HM_STEP(bf16, HM_DT_BF16, 128, 64, 32),  HM_STEP(float, HM_DT_F32, 16, 16, 16),   HM_STEP(float, HM_DT_F32, 16, 16, 32),
    HM_STEP(float, HM_DT_F32, 32, 16, 16),   HM_STEP(float, HM_DT_F32, 32, 16, 32),
};
#define HM_FEAT(T, TC, TO, TOC, DK, FH) {TC, TOC, DK, FH, &launch_feat<T, TO, DK, FH>}
#define HM_FEAT_F(T, TC, TO, TOC, DK) \
  HM_FEAT(T, TC, TO, TOC, DK, 16), HM_FEAT(T, TC, TO, TOC, DK, 32), HM_FEAT(T, TC, TO, TOC, DK, 64)
static const FeatEntry kFeat[] = {
    HM_FEAT_F(bf16, HM_DT_BF16, bf16, HM_DT_BF16, 32),  HM_FEAT_F(bf16, HM_DT_BF16, bf16, HM_DT_BF16, 64),
    HM_FEAT_F(bf16, HM_DT_BF16, bf16, HM_DT_BF16, 128), HM_FEAT_F(bf16, HM_DT_BF16, float, HM_DT_F32, 32),
    HM_FEAT_F(bf16, HM_DT_BF16, float, HM_DT_F32, 64),  HM_FEAT_F(bf16, HM_DT_BF16, float, HM_DT_F32, 128),
    HM_FEAT_F(float, HM_DT_F32, float, HM_DT_F32, 16),  HM_FEAT_F(float, HM_DT_F32, float, HM_DT_F32, 32),
    HM_FEAT_F(float, HM_DT_F32, float, HM_DT_F32, 64),  HM_FEAT_F(float, HM_DT_F32, float, HM_DT_F32, 128),
};
Table table_step_feat() {
  return Table{nullptr, 0, kStep, (int)(sizeof(kStep) / sizeof(kStep[0])), kFeat, (int)(sizeof(kFeat) / sizeof(kFeat[0]))};
}
}  // namespace hm
