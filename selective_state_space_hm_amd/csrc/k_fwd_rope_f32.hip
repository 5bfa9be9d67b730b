// Prefill instantiations with rotary encoding of the features: float32, both decay
// variants, (d, f) = (16, 16) and (32, 16).
#include "hm_kernels.hpp"

namespace hm {
#define HM_SET(DK, DEC) \
  HM_ROPE_PAIR(float, HM_DT_F32, DK, 16, 16, DEC), HM_ROPE_PAIR(float, HM_DT_F32, DK, 16, 32, DEC)
static const FwdEntry kFwd[] = {HM_SET(16, 0), HM_SET(16, 1), HM_SET(32, 0), HM_SET(32, 1)};
Table table_fwd_rope_f32() { return Table{kFwd, (int)(sizeof(kFwd) / sizeof(kFwd[0])), nullptr, 0, nullptr, 0}; }
}  // namespace hm
