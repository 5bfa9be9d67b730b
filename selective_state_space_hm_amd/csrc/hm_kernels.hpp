// Launch tables: each kernel translation unit exports the instantiations it
// builds; the ABI layer looks a configuration up and launches it.
#pragma once

#include <hip/hip_runtime.h>

#include "hm_conv.hpp"
#include "hm_prefill.hpp"
#include "hm_step.hpp"

namespace hm {

struct FwdEntry {
  int dtype, dk, fh, dw, decay, mode, chunk;
  void (*launch)(const FwdParams &, unsigned grid, hipStream_t);
};
struct StepEntry {
  int dtype, dk, fh, dv, decay;
  void (*launch)(const StepParams &, unsigned grid, hipStream_t);
};
struct FeatEntry {
  int dtype, phi_dtype, dk, fh;
  void (*launch)(const FeatParams &, dim3 grid, hipStream_t);
};
struct Table {
  const FwdEntry *fwd;
  int nfwd;
  const StepEntry *step;
  int nstep;
  const FeatEntry *feat;
  int nfeat;
};

struct ConvEntry {
  int dtype, width;
  void (*launch)(const ConvParams &, dim3 grid, hipStream_t);
};
struct ConvTable {
  const ConvEntry *conv;
  int nconv;
};

struct BwdParams;
struct BwdEntry {
  int dtype, dk, fh, dv, rope;
  void (*launch)(const BwdParams &, hipStream_t);
};
struct BwdTable {
  const BwdEntry *bwd;
  int nbwd;
};

struct PcParams;
struct PcStepParams;
struct PcEntry {
  int dtype, dk, fh, dv;
  int cpw;  // value channels per prefill workgroup
  void (*fwd)(const PcParams &, hipStream_t);
  void (*step)(const PcStepParams &, hipStream_t);
};
struct PcTable {
  const PcEntry *pc;
  int npc;
};

struct CpParams;
struct CpEntry {
  int dtype, fh, dv;
  void (*local)(const CpParams &, unsigned grid, hipStream_t);
  void (*out)(const CpParams &, unsigned grid, hipStream_t);
};
struct CpTable {
  const CpEntry *cp;
  int ncp;
};

// one per kernel translation unit
CpTable table_cp_bf16();
CpTable table_cp_f32();
PcTable table_pc();
ConvTable table_conv();
BwdTable table_bwd();
Table table_train();
Table table_fwd_bf16();
Table table_fwd_bf16_decay();
Table table_fwd_f32();
Table table_fwd_f32_d64();
Table table_fwd_rope_bf16();
Table table_fwd_rope_bf16_decay();
Table table_fwd_rope_f32();
Table table_fwd_c128();
Table table_step_feat();
Table table_step_bf16();
Table table_step_f32();

template <typename T, int DK, int FH, int DW, bool DECAY, int MODE, int CH>
void launch_fwd(const FwdParams &p, unsigned grid, hipStream_t s) {
  hipLaunchKernelGGL((fwd_kernel<T, DK, FH, DW, DECAY, MODE, CH>), dim3(grid), dim3(fwd_waves(DW) * 64), 0, s, p);
}
template <typename T, int DK, int FH, int DV, bool DECAY>
void launch_step(const StepParams &p, unsigned grid, hipStream_t s) {
  hipLaunchKernelGGL((step_kernel<T, DK, FH, DV, DECAY>), dim3(grid), dim3(256), 0, s, p);
}
template <typename T, int K>
void launch_conv(const ConvParams &p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((conv_kernel<T, K>), grid, dim3(256), 0, s, p);
}
template <typename T, typename TO, int DK, int FH>
void launch_feat(const FeatParams &p, dim3 grid, hipStream_t s) {
  if (p.cwidth > 0) hipLaunchKernelGGL((featurize_kernel<T, TO, DK, FH, true>), grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL((featurize_kernel<T, TO, DK, FH, false>), grid, dim3(256), 0, s, p);
}

}  // namespace hm

// dtype codes as in hm.h
#define HM_DT_F32 0
#define HM_DT_BF16 1

#define HM_FWD_ENTRY(T, TC, DK, FH, DW, DEC, MODE) \
  {TC, DK, FH, DW, DEC, MODE, 64, &hm::launch_fwd<T, DK, FH, DW, (DEC != 0), MODE, 64>}
// the full pass with 128-token chunks
#define HM_FWD_C128(T, TC, DK, FH, DW, DEC) \
  {TC, DK, FH, DW, DEC, 0, 128, &hm::launch_fwd<T, DK, FH, DW, (DEC != 0), 0, 128>}
// both modes of one configuration
#define HM_FWD_PAIR(T, TC, DK, FH, DW, DEC) \
  HM_FWD_ENTRY(T, TC, DK, FH, DW, DEC, 0), HM_FWD_ENTRY(T, TC, DK, FH, DW, DEC, 1)
// both modes with the rotary encoding (MODE_ROPE = 4)
#define HM_ROPE_PAIR(T, TC, DK, FH, DW, DEC) \
  HM_FWD_ENTRY(T, TC, DK, FH, DW, DEC, 4), HM_FWD_ENTRY(T, TC, DK, FH, DW, DEC, 5)
