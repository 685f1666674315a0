// Compiled attention kernel instances for fp8 inputs (generated list;
// edit here and in the host's selection rules together).
#include "fmha_decode_kernel.h"
#include "fmha_prefill8_kernel.h"
#include "fmha_fwd_kernel.h"

namespace fmha {

// No 16-row-tile (generic) instances for fp8: every fp8 shape with a compiled
// head-dim pair goes to the decode kernel (<= 16 rows) or the fp8 prefill
// kernel (more), so the host never selects one.
const FwdKernel* registry_fp8(int* n) {
  *n = 0;
  return nullptr;
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
