// Prefill instantiations with rotary encoding of the features: bf16, Mamba-style decay,
// (d, f) = (128, 64) and (64, 32).
#include "hm_kernels.hpp"

namespace hm {
#define HM_DEC 1
static const FwdEntry kFwd[] = {
    HM_ROPE_PAIR(bf16, HM_DT_BF16, 128, 64, 32, HM_DEC), HM_ROPE_PAIR(bf16, HM_DT_BF16, 128, 64, 64, HM_DEC),
    HM_ROPE_PAIR(bf16, HM_DT_BF16, 128, 64, 128, HM_DEC), HM_ROPE_PAIR(bf16, HM_DT_BF16, 64, 32, 32, HM_DEC),
    HM_ROPE_PAIR(bf16, HM_DT_BF16, 64, 32, 64, HM_DEC),
};
Table table_fwd_rope_bf16_decay() { return Table{kFwd, (int)(sizeof(kFwd) / sizeof(kFwd[0])), nullptr, 0, nullptr, 0}; }
}  // namespace hm
