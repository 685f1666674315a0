// Compiled attention kernel instances for bf16 inputs (generated list;
// edit here and in the host's selection rules together).
#include "fmha_fwd_kernel.h"

namespace fmha {

#define FMHA_INST(DQK, DV, NWM, NWK, BN, ID) \
  {DT_BF16, DQK, DV, NWM, NWK, BN, ID, &launch_fwd<FwdCfg<DT_BF16, DQK, DV, NWM, NWK, BN>>}

static const FwdKernel kTable[] = {
    FMHA_INST(64, 64, 1, 4, 32, 0),
    FMHA_INST(64, 64, 2, 2, 32, 1),
    FMHA_INST(64, 64, 4, 1, 64, 2),
    FMHA_INST(64, 64, 5, 1, 64, 3),
    FMHA_INST(64, 64, 8, 1, 64, 4),
    FMHA_INST(128, 128, 1, 4, 32, 5),
    FMHA_INST(128, 128, 2, 2, 32, 6),
    FMHA_INST(128, 128, 4, 1, 64, 7),
    FMHA_INST(128, 128, 5, 1, 64, 8),
    FMHA_INST(128, 128, 8, 1, 64, 9),
    FMHA_INST(256, 256, 1, 4, 32, 10),
    FMHA_INST(256, 256, 2, 2, 32, 11),
    FMHA_INST(256, 256, 4, 1, 64, 12),
    FMHA_INST(256, 256, 5, 1, 64, 13),
};

const FwdKernel* registry_bf16(int* n) {
  *n = (int)(sizeof(kTable) / sizeof(kTable[0]));
  return kTable;
}

}  // namespace fmha
