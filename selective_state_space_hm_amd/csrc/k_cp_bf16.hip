// Chunk-parallel prefill instantiations, bf16: f in {16, 32, 64} x dv in
// {16, 32, 64, 128} (d is a run-time size up to 128).
#include "hm_kernels.hpp"
#include "hm_cp.hpp"

namespace hm {

template <typename T, int FH, int DV>
void launch_cp_local(const CpParams &p, unsigned grid, hipStream_t s) {
  hipLaunchKernelGGL((cp_local_kernel<T, FH, DV>), dim3(grid), dim3(256), 0, s, p);
}
template <typename T, int FH, int DV>
void launch_cp_out(const CpParams &p, unsigned grid, hipStream_t s) {
  hipLaunchKernelGGL((cp_out_kernel<T, FH, DV>), dim3(grid), dim3(256), 0, s, p);
}

#define HM_CP(FH, DV) {HM_DT_BF16, FH, DV, &launch_cp_local<bf16, FH, DV>, &launch_cp_out<bf16, FH, DV>}
#define HM_CP_F(FH) HM_CP(FH, 16), HM_CP(FH, 32), HM_CP(FH, 64), HM_CP(FH, 128)
static const CpEntry kCp[] = {HM_CP_F(16), HM_CP_F(32), HM_CP_F(64)};
CpTable table_cp_bf16() { return CpTable{kCp, (int)(sizeof(kCp) / sizeof(kCp[0]))}; }

}  // namespace hm
