// Compiled attention kernel instances for f32 inputs (generated list;
// edit here and in the host's selection rules together).
#include "fmha_fwd_kernel.h"

namespace fmha {

#define FMHA_INST(DQK, DV, NWM, NWK, BN, ID) \
  {DT_F32, DQK, DV, NWM, NWK, BN, ID, &launch_fwd<FwdCfg<DT_F32, DQK, DV, NWM, NWK, BN>>}

static const FwdKernel kTable[] = {
    FMHA_INST(64, 64, 1, 4, 16, 0),
    FMHA_INST(64, 64, 2, 2, 16, 1),
    FMHA_INST(64, 64, 4, 1, 32, 2),
    FMHA_INST(64, 64, 5, 1, 32, 3),
    FMHA_INST(64, 64, 8, 1, 32, 4),
    FMHA_INST(128, 128, 1, 4, 16, 5),
    FMHA_INST(128, 128, 2, 2, 16, 6),
    FMHA_INST(128, 128, 4, 1, 32, 7),
    FMHA_INST(128, 128, 5, 1, 32, 8),
    FMHA_INST(128, 128, 8, 1, 32, 9),
};

const FwdKernel* registry_f32(int* n) {
  *n = (int)(sizeof(kTable) / sizeof(kTable[0]));
  return kTable;
}

// No decode instances for fp32 inputs (the LDS transpose reads are 8/16-bit).
const FwdKernel* registry_f32_decode(int* n) {
  *n = 0;
  return nullptr;
}

// No 32x32-tile prefill instances for f32 inputs (the 16-row kernel serves them).
const FwdKernel* registry_f32_prefill(int* n) {
  *n = 0;
  return nullptr;
}

}  // namespace fmha
