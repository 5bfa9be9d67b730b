// Prefill instantiations with 128-token chunks (full pass; the segment pass is
// the 64-token one, whose end states do not depend on the chunk length):
// bf16 (d, f) = (128, 64), (64, 32) with 32, 64 or 128 value columns per workgroup,
// float32 (d, f) = (16, 16), (32, 16) with 16 or 32; identity and per-head decay.
#include "hm_kernels.hpp"

namespace hm {
#define HM_SET_B(DK, FH, DEC)                                                                     \
  HM_FWD_C128(bf16, HM_DT_BF16, DK, FH, 32, DEC), HM_FWD_C128(bf16, HM_DT_BF16, DK, FH, 64, DEC), \
      HM_FWD_C128(bf16, HM_DT_BF16, DK, FH, 128, DEC)
#define HM_SET_F(DK, DEC) HM_FWD_C128(float, HM_DT_F32, DK, 16, 16, DEC), HM_FWD_C128(float, HM_DT_F32, DK, 16, 32, DEC)
static const FwdEntry kFwd[] = {HM_SET_B(128, 64, 0), HM_SET_B(128, 64, 1), HM_SET_B(64, 32, 0), HM_SET_B(64, 32, 1),
                                HM_SET_F(16, 0),      HM_SET_F(16, 1),      HM_SET_F(32, 0),     HM_SET_F(32, 1)};
Table table_fwd_c128() { return Table{kFwd, (int)(sizeof(kFwd) / sizeof(kFwd[0])), nullptr, 0, nullptr, 0}; }
}  // namespace hm
