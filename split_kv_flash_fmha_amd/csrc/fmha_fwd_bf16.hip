// Compiled attention kernel instances for bf16 inputs (generated list;
// edit here and in the host's selection rules together).
#include "fmha_decode_kernel.h"
#include "fmha_prefill_kernel.h"
#include "fmha_fwd_kernel.h"

namespace fmha {

#define FMHA_INST(DQK, DV, NWM, NWK, BN, ID) \
  {DT_BF16, DQK, DV, NWM, NWK, BN, ID, &launch_fwd<FwdCfg<DT_BF16, DQK, DV, NWM, NWK, BN>>}

static const FwdKernel kTable[] = {
    FMHA_INST(64, 64, 2, 2, 32, 1),
    FMHA_INST(64, 64, 4, 1, 64, 2),
    FMHA_INST(64, 64, 5, 1, 64, 3),
    FMHA_INST(128, 128, 2, 2, 32, 6),
    FMHA_INST(128, 128, 4, 1, 64, 7),
    FMHA_INST(128, 128, 5, 1, 64, 8),
    FMHA_INST(256, 256, 1, 4, 32, 10),
    FMHA_INST(256, 256, 2, 2, 32, 11),
    FMHA_INST(256, 256, 4, 1, 64, 12),
    FMHA_INST(256, 256, 5, 1, 64, 13),
};

const FwdKernel* registry_bf16(int* n) {
  *n = (int)(sizeof(kTable) / sizeof(kTable[0]));
  return kTable;
}

// Decode instances (<= 16 query rows per (sequence, kv head)): bn = 0 marks them.
#define FMHA_DEC(DQK, DV, NW, ID) \
  {DT_BF16, DQK, DV, 1, NW, 0, ID, &launch_decode<DecCfg<DT_BF16, DQK, DV, NW>>}

static const FwdKernel kDecTable[] = {
    FMHA_DEC(64, 64, 4, 100),
    FMHA_DEC(128, 128, 4, 101),
};

const FwdKernel* registry_bf16_decode(int* n) {
  *n = (int)(sizeof(kDecTable) / sizeof(kDecTable[0]));
  return kDecTable;
}

// Prefill instances (32x32 MFMA tiles, 4 waves x 32 rows; key blocks of 32
// keys for D = 128 and 256 and 64 keys for D = 64: 8 KiB of K or V per block,
// 16 KiB for D = 256).  D = 64 and 128 run three workgroups per CU on
// three-stage rings (the simple loop form: three waves per SIMD from different workgroups, QK,
// softmax and PV of a block in turn); D = 256 runs one workgroup per CU (its
// four-stage rings take 128 KiB) with the cross-block software pipeline.
#define FMHA_PF(D, NWM, BN, ID) \
  {DT_BF16, D, D, NWM, 1, BN, ID, &launch_prefill<PfCfg<DT_BF16, D, NWM, BN, 1>>}
#define FMHA_PF3(D, BN, ID) \
  {DT_BF16, D, D, 4, 1, BN, ID, &launch_prefill<PfCfg<DT_BF16, D, 4, BN, 1, false, 3>>}

static const FwdKernel kPfTable[] = {
    FMHA_PF3(64, 64, 200),
    FMHA_PF3(128, 32, 201),
    FMHA_PF(256, 4, 32, 202),
};

const FwdKernel* registry_bf16_prefill(int* n) {
  *n = (int)(sizeof(kPfTable) / sizeof(kPfTable[0]));
  return kPfTable;
}

}  // namespace fmha
