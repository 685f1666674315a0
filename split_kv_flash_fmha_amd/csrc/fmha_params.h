// Parameters handed from the host library to the kernels (internal).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fmha {

enum DType : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_FP8 = 3 };

struct FwdParams {
  const char* q;
  const char* k;
  const char* v;
  char* o;
  float* lse;        // may be null
  float* o_part;     // split partials [S, total_q, Hq, Dv] (split mode)
  float* lse_part;   // [S, Hq, total_q]
  const int32_t* cu_q;  // null: fixed-length Q
  const int32_t* cu_k;  // null: fixed-length K
  const float* q_descale;  // fp8 only, may be null
  const float* k_descale;
  const float* v_descale;
  int32_t batch;
  int32_t seqlen_q;  // fixed-length Q
  int32_t seqlen_k;  // fixed-length K
  int32_t total_q;   // rows of the partial layout
  int32_t hq;
  int32_t hkv;
  int32_t group;     // hq / hkv
  // strides in BYTES for q/k/v/o
  int64_t q_sb, q_st, q_sh;
  int64_t k_sb, k_st, k_sh;
  int64_t v_sb, v_st, v_sh;
  int64_t o_sb, o_st, o_sh;
  // lse strides in elements
  int64_t lse_sb, lse_sh;
  float scale_log2;  // softmax scale * log2(e)
  int32_t wl, wr;    // resolved window (-1 = unbounded), causal folded into wr
  int32_t num_splits;  // 1: write final O/LSE; >1: write partials
  int32_t chunk;       // keys per split
  int32_t num_q_tiles;
  int32_t out_dtype;
  int32_t tile_order;    // kTileOrder*
  int32_t max_seqlen_k;  // bound on any sequence's key count
  int32_t* counters;     // split mode: 2 per (sequence, kv head, query tile), zero between launches
  int32_t* sched;        // kTileOrderTable: the tile table written by the schedule kernel
  int32_t persistent;    // kTileOrderTable: workgroups claim table positions until none is left
  int32_t fused_combine; // split mode: the split workgroups combine the partials themselves
};

// Block -> tile orders of the attention launch.
constexpr int32_t kTileOrderGrouped = 0;       // by (sequence, kv head), XCD-grouped
constexpr int32_t kTileOrderLongestFirst = 1;  // all tiles by cost, longest first
constexpr int32_t kTileOrderFullFirst = 2;     // decode splits: full ones, then partial ones by length
constexpr int32_t kTileOrderHeadsTogether = 3; // one query tile, splits: the kv heads of a split on one XCD
constexpr int32_t kTileOrderTable = 4;         // groups dealt to XCDs longest first by a schedule kernel
constexpr int kScheduleMaxBatch = 1024;        // one sequence per thread of the schedule kernel
constexpr int kXcds = 8;                       // block i runs on XCD i % 8
constexpr int kSchedHead = 16;                 // int32 header of the tile table
constexpr int kLongestFirstMaxBatch = 64;      // one sequence per lane of a wave

struct CombineParams {
  const float* o_part;
  const float* lse_part;
  char* o;
  float* lse;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t batch, seqlen_q, seqlen_k, max_seqlen_q, total_q;
  int32_t hq, dv;
  int32_t num_splits, chunk;
  int32_t chunks_per_wg;     // combine_chunks_per_wg()
  int64_t o_sb, o_st, o_sh;  // bytes
  int64_t lse_sb, lse_sh;    // elements
  int32_t out_dtype;
};

typedef hipError_t (*FwdLaunchFn)(const FwdParams&, int64_t grid, hipStream_t);

// One compiled attention kernel instance.
struct FwdKernel {
  int dtype;
  int dqk;
  int dv;
  int nwm;   // waves along query rows (16 rows each)
  int nwk;   // waves splitting the key block
  int bn;    // keys per wave per iteration (0: decode kernel, 32 keys per wave)
  int id;
  FwdLaunchFn launch;
};

// Registries, one per input dtype (defined in fmha_fwd_<dtype>.hip).
const FwdKernel* registry_f32(int* n);
const FwdKernel* registry_f16(int* n);
const FwdKernel* registry_bf16(int* n);
const FwdKernel* registry_fp8(int* n);
// Decode kernels (one 16-row tile, waves stream disjoint key ranges).
const FwdKernel* registry_f32_decode(int* n);
const FwdKernel* registry_f16_decode(int* n);
const FwdKernel* registry_bf16_decode(int* n);
const FwdKernel* registry_fp8_decode(int* n);
// Prefill kernels (32x32 MFMA tiles, 32 rows per wave).
const FwdKernel* registry_f32_prefill(int* n);
const FwdKernel* registry_f16_prefill(int* n);
const FwdKernel* registry_bf16_prefill(int* n);
const FwdKernel* registry_fp8_prefill(int* n);

// Shape of the combine grid: a workgroup (256 threads) takes cw of a row's
// Dv / 4 16-byte column chunks (cw a power of two) and 256 / cw split groups.
// Few rows get narrow column groups (more workgroups in flight); cw is also
// kept small enough that no thread owns more than 16 partial rows.
constexpr int kCombineMaxChunks = 32;   // widest column group (chunks)
constexpr int64_t kCombineMinWgs = 128; // narrower groups until the grid has this many
inline int combine_chunks_per_wg(int dv, int num_splits, int64_t rows) {
  const int nchunk = dv / 4;
  int cw = 1;
  while (cw < nchunk && cw < kCombineMaxChunks) cw *= 2;
  while (cw > 4 && rows * ((nchunk + cw - 1) / cw) < kCombineMinWgs) cw /= 2;
  while (cw > 1 && (num_splits + 256 / cw - 1) / (256 / cw) > 16) cw /= 2;
  return cw;
}
inline int64_t combine_grid(int dv, int num_splits, int64_t rows) {
  const int nchunk = dv / 4, cw = combine_chunks_per_wg(dv, num_splits, rows);
  return rows * ((nchunk + cw - 1) / cw);
}

hipError_t launch_combine(const CombineParams& p, hipStream_t stream);
hipError_t launch_schedule(const FwdParams& p, int rows_per_tile, int key_block, int positions, int32_t* table,
                           hipStream_t stream);
hipError_t launch_check_seqlens(const int32_t* cu, int32_t batch, int32_t total, int32_t max_seqlen,
                                int32_t* result, hipStream_t stream);

}  // namespace fmha
