// Featurizer instantiations (the decode steps are in k_step_bf16.hip and k_step_f32.hip).
#include "hm_kernels.hpp"

namespace hm {
#define HM_FEAT(T, TC, TO, TOC, DK, FH) {TC, TOC, DK, FH, &launch_feat<T, TO, DK, FH>}
#define HM_FEAT_F(T, TC, TO, TOC, DK) \
  HM_FEAT(T, TC, TO, TOC, DK, 16), HM_FEAT(T, TC, TO, TOC, DK, 32), HM_FEAT(T, TC, TO, TOC, DK, 64)
static const FeatEntry kFeat[] = {
    HM_FEAT_F(bf16, HM_DT_BF16, bf16, HM_DT_BF16, 16),  HM_FEAT_F(bf16, HM_DT_BF16, float, HM_DT_F32, 16),
    HM_FEAT_F(bf16, HM_DT_BF16, bf16, HM_DT_BF16, 32),  HM_FEAT_F(bf16, HM_DT_BF16, bf16, HM_DT_BF16, 64),
    HM_FEAT_F(bf16, HM_DT_BF16, bf16, HM_DT_BF16, 128), HM_FEAT_F(bf16, HM_DT_BF16, float, HM_DT_F32, 32),
    HM_FEAT_F(bf16, HM_DT_BF16, float, HM_DT_F32, 64),  HM_FEAT_F(bf16, HM_DT_BF16, float, HM_DT_F32, 128),
    HM_FEAT_F(float, HM_DT_F32, float, HM_DT_F32, 16),  HM_FEAT_F(float, HM_DT_F32, float, HM_DT_F32, 32),
    HM_FEAT_F(float, HM_DT_F32, float, HM_DT_F32, 64),  HM_FEAT_F(float, HM_DT_F32, float, HM_DT_F32, 128),
};
Table table_step_feat() {
  return Table{nullptr, 0, nullptr, 0, kFeat, (int)(sizeof(kFeat) / sizeof(kFeat[0]))};
}
}  // namespace hm
