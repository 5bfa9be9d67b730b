// Short causal conv instantiations: f32 and bf16, K = 1..4 taps.
#include "hm_kernels.hpp"

namespace hm {
#define HM_CONV(T, TC, K) {TC, K, &launch_conv<T, K>}
static const ConvEntry kConv[] = {
    HM_CONV(float, HM_DT_F32, 1),  HM_CONV(float, HM_DT_F32, 2),  HM_CONV(float, HM_DT_F32, 3),
    HM_CONV(float, HM_DT_F32, 4),  HM_CONV(bf16, HM_DT_BF16, 1),  HM_CONV(bf16, HM_DT_BF16, 2),
    HM_CONV(bf16, HM_DT_BF16, 3),  HM_CONV(bf16, HM_DT_BF16, 4),
};
ConvTable table_conv() { return ConvTable{kConv, (int)(sizeof(kConv) / sizeof(kConv[0]))}; }
}  // namespace hm
