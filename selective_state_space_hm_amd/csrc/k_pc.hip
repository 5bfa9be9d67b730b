// Per-channel-decay instantiations: prefill scan and decode step, bf16 (d, f, dv)
// = (128, 64, 128) and (64, 32, 64), float32 (16, 16, 16) and (32, 16, 32).
#include "hm_kernels.hpp"
#include "hm_pc.hpp"

namespace hm {

// channels per workgroup and lanes per channel of the prefill scan
template <int FH, int DV> constexpr int pc_cpw() { return DV >= 64 ? 64 : DV; }
constexpr int PC_LPC = 8;

template <typename T, int DK, int FH, int DV>
void launch_pc_fwd(const PcParams &p, hipStream_t s) {
  constexpr int CPW = pc_cpw<FH, DV>(), NG = DV / CPW, F = 2 * FH;
  const unsigned BH = (unsigned)(p.B * p.H);
  if (p.nseg > 1) {
    // segment pass, then the start states of the segments
    hipLaunchKernelGGL((pc_fwd_kernel<T, DK, FH, DV, CPW, PC_LPC, true>), dim3(BH * (unsigned)(p.nseg - 1) * NG),
                       dim3(CPW * PC_LPC), 0, s, p);
    const int64_t nel = (int64_t)BH * 2 * DV * F;
    hipLaunchKernelGGL((pc_combine_kernel<DV, F>), dim3((unsigned)((nel + 255) / 256)), dim3(256), 0, s, p);
  }
  hipLaunchKernelGGL((pc_fwd_kernel<T, DK, FH, DV, CPW, PC_LPC, false>), dim3(BH * (unsigned)p.nseg * NG),
                     dim3(CPW * PC_LPC), 0, s, p);
}
// channels per decode workgroup: 1024 (channel, 4-state) items, at most DV
template <int FH, int DV> constexpr int pc_step_cps() { return 2048 / FH < DV ? 2048 / FH : DV; }

template <typename T, int DK, int FH, int DV>
void launch_pc_step(const PcStepParams &p, hipStream_t s) {
  constexpr int CPS = pc_step_cps<FH, DV>();
  const unsigned grid = (unsigned)(p.s.B * p.s.H * (DV / CPS));
  hipLaunchKernelGGL((pc_step_kernel<T, DK, FH, DV, CPS>), dim3(grid), dim3(256), 0, s, p);
}

#define HM_PC(T, TC, DK, FH, DV) \
  {TC, DK, FH, DV, pc_cpw<FH, DV>(), &launch_pc_fwd<T, DK, FH, DV>, &launch_pc_step<T, DK, FH, DV>}
static const PcEntry kPc[] = {
    HM_PC(bf16, HM_DT_BF16, 128, 64, 128), HM_PC(bf16, HM_DT_BF16, 64, 32, 64),
    HM_PC(float, HM_DT_F32, 16, 16, 16),   HM_PC(float, HM_DT_F32, 32, 16, 32),
};
PcTable table_pc() { return PcTable{kPc, (int)(sizeof(kPc) / sizeof(kPc[0]))}; }

}  // namespace hm
