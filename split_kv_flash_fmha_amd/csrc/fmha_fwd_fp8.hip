// Compiled attention kernel instances for fp8 inputs (generated list;
// edit here and in the host's selection rules together).
#include "fmha_decode_kernel.h"
#include "fmha_prefill8_kernel.h"
#include "fmha_fwd_kernel.h"

namespace fmha {

#define FMHA_INST(DQK, DV, NWM, NWK, BN, ID) \
  {DT_FP8, DQK, DV, NWM, NWK, BN, ID, &launch_fwd<FwdCfg<DT_FP8, DQK, DV, NWM, NWK, BN>>}

static const FwdKernel kTable[] = {
    FMHA_INST(128, 128, 1, 4, 64, 0),
    FMHA_INST(128, 128, 2, 2, 64, 1),
    FMHA_INST(128, 128, 4, 1, 64, 2),
    FMHA_INST(128, 128, 5, 1, 64, 3),
    FMHA_INST(128, 128, 8, 1, 64, 4),
    FMHA_INST(192, 128, 1, 4, 64, 5),
    FMHA_INST(192, 128, 2, 2, 64, 6),
    FMHA_INST(192, 128, 4, 1, 64, 7),
    FMHA_INST(192, 128, 5, 1, 64, 8),
    FMHA_INST(192, 128, 8, 1, 64, 9),
};

const FwdKernel* registry_fp8(int* n) {
  *n = (int)(sizeof(kTable) / sizeof(kTable[0]));
  return kTable;
}

// Decode instances (<= 16 query rows per (sequence, kv head)): bn = 0 marks them.
#define FMHA_DEC(DQK, DV, NW, ID) \
  {DT_FP8, DQK, DV, 1, NW, 0, ID, &launch_decode<DecCfg<DT_FP8, DQK, DV, NW>>}

static const FwdKernel kDecTable[] = {
    FMHA_DEC(128, 128, 4, 100),
    FMHA_DEC(192, 128, 4, 101),
};

const FwdKernel* registry_fp8_decode(int* n) {
  *n = (int)(sizeof(kDecTable) / sizeof(kDecTable[0]));
  return kDecTable;
}

// 32x32-tile fp8 instances (32 rows per wave, 64-key blocks); nwm picked by
// rows per (sequence, kv head).
#define FMHA_PF8(DQK, DV, NWM, ID) \
  {DT_FP8, DQK, DV, NWM, 1, 64, ID, &launch_prefill8<Pf8Cfg<DQK, DV, NWM, 1>>}

static const FwdKernel kPf8Table[] = {
    FMHA_PF8(192, 128, 3, 210),
    FMHA_PF8(192, 128, 4, 211),
    FMHA_PF8(128, 128, 3, 212),
    FMHA_PF8(128, 128, 4, 213),
};

const FwdKernel* registry_fp8_prefill(int* n) {
  *n = (int)(sizeof(kPf8Table) / sizeof(kPf8Table[0]));
  return kPf8Table;
}

}  // namespace fmha
