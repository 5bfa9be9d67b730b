// Decode-step instantiations, f32: d in {16, 32, 64, 128} x f in {16, 32, 64} x
// dv in {16, 32, 64, 128}, with and without decay.
#include "hm_kernels.hpp"

namespace hm {
#define HM_STEP(DK, FH, DV) \
  {HM_DT_F32, DK, FH, DV, 0, &launch_step<float, DK, FH, DV, false>}, {HM_DT_F32, DK, FH, DV, 1, &launch_step<float, DK, FH, DV, true>}
#define HM_STEP_V(DK, FH) HM_STEP(DK, FH, 16), HM_STEP(DK, FH, 32), HM_STEP(DK, FH, 64), HM_STEP(DK, FH, 128)
#define HM_STEP_F(DK) HM_STEP_V(DK, 16), HM_STEP_V(DK, 32), HM_STEP_V(DK, 64)
static const StepEntry kStep[] = {HM_STEP_F(16), HM_STEP_F(32), HM_STEP_F(64), HM_STEP_F(128)};
Table table_step_f32() { return Table{nullptr, 0, kStep, (int)(sizeof(kStep) / sizeof(kStep[0])), nullptr, 0}; }
}  // namespace hm
