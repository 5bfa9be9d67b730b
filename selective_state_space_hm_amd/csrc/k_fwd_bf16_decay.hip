// Prefill instantiations: bf16, per-head Mamba-style decay.
#include "hm_kernels.hpp"

namespace hm {
#define HM_DEC 1
#define HM_SET(DK, FH)                                                                       \
  HM_FWD_PAIR(bf16, HM_DT_BF16, DK, FH, 32, HM_DEC), HM_FWD_PAIR(bf16, HM_DT_BF16, DK, FH, 64, HM_DEC), \
      HM_FWD_PAIR(bf16, HM_DT_BF16, DK, FH, 128, HM_DEC)
static const FwdEntry kFwd[] = {HM_SET(64, 32), HM_SET(64, 64), HM_SET(128, 32), HM_SET(128, 64)};
Table table_fwd_bf16_decay() { return Table{kFwd, (int)(sizeof(kFwd) / sizeof(kFwd[0])), nullptr, 0, nullptr, 0}; }
}  // namespace hm
