// Prefill and decode-step instantiations for float32 at d = 64: (f, dv) in
// {(16, 16), (16, 32), (32, 32), (32, 64)}, both decay variants.  These hold more
// float32 operand fragments than the register file leaves a wave and spill a few
// registers; they serve the float32 precision path, not the measured bf16 one.
#include "hm_kernels.hpp"

namespace hm {
#define HM_STEP_F(DK, FH, DV) \
  {HM_DT_F32, DK, FH, DV, 0, &launch_step<float, DK, FH, DV, false>}, {HM_DT_F32, DK, FH, DV, 1, &launch_step<float, DK, FH, DV, true>}
#define HM_SET64(DEC)                                                                                          \
  HM_FWD_PAIR(float, HM_DT_F32, 64, 16, 16, DEC), HM_FWD_PAIR(float, HM_DT_F32, 64, 16, 32, DEC),              \
      HM_FWD_PAIR(float, HM_DT_F32, 64, 32, 32, DEC), HM_FWD_PAIR(float, HM_DT_F32, 64, 32, 64, DEC)
static const FwdEntry kFwd[] = {HM_SET64(0), HM_SET64(1)};
static const StepEntry kStep[] = {HM_STEP_F(64, 16, 16), HM_STEP_F(64, 16, 32), HM_STEP_F(64, 32, 32),
                                  HM_STEP_F(64, 32, 64)};
Table table_fwd_f32_d64() {
  return Table{kFwd, (int)(sizeof(kFwd) / sizeof(kFwd[0])), kStep, (int)(sizeof(kStep) / sizeof(kStep[0])), nullptr, 0};
}
}  // namespace hm
