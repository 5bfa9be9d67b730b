// Prefill instantiations: bf16, identity decay (a_t = 1).  dv = 32 (one 32-column
// workgroup) also serves the dsplit = 2 halves of dv = 64.
#include "hm_kernels.hpp"

namespace hm {
#define HM_DEC 0
#define HM_SET(DK, FH)                                                                       \
  HM_FWD_PAIR(bf16, HM_DT_BF16, DK, FH, 32, HM_DEC), HM_FWD_PAIR(bf16, HM_DT_BF16, DK, FH, 64, HM_DEC), \
      HM_FWD_PAIR(bf16, HM_DT_BF16, DK, FH, 128, HM_DEC)
static const FwdEntry kFwd[] = {HM_SET(64, 32), HM_SET(64, 64), HM_SET(128, 32), HM_SET(128, 64),
                                HM_FWD_PAIR(bf16, HM_DT_BF16, 32, 16, 32, HM_DEC)};
Table table_fwd_bf16() { return Table{kFwd, (int)(sizeof(kFwd) / sizeof(kFwd[0])), nullptr, 0, nullptr, 0}; }
}  // namespace hm
