// Host side of the C ABI: argument checks, default resolution, the automatic
// split choice, workspace sizing, kernel selection and launches.
//
// Everything up to the launch is plain host code that makes no HIP call, so
// fmha_fwd_check / fmha_num_splits / fmha_fwd_workspace_size run (and are
// tested) without a GPU.  Checks follow the pages' rule that an unsupported
// or invalid configuration is refused before any work instead of silently
// dropping rows ("Adds variable sequence lengths to the Hopper CuTe DSL FMHA
// example", section Implementation; "[FlyDSL] Enable FP8 FMHA split-K ...",
// review: an invalid combination raises an error).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "../../include/fmha.h"
#include "fmha_params.h"
#include "fmha_fused_combine.h"

// Split workspace of fmha_fwd_no_alloc: one copy per GPU the library runs on,
// held until the process ends.  In host code `scratch` is only a handle for
// hipGetSymbolAddress; its device address (per device) is what kernels get.
static __device__ __align__(256) char scratch[FMHA_NO_ALLOC_SCRATCH_BYTES];

namespace fmha {
namespace {

constexpr int64_t kMaxGrid = (int64_t)1 << 31;

int elem_bytes(int dt) {
  switch (dt) {
    case FMHA_DTYPE_F32: return 4;
    case FMHA_DTYPE_F16: return 2;
    case FMHA_DTYPE_BF16: return 2;
    case FMHA_DTYPE_FP8_E4M3: return 1;
    default: return 0;
  }
}

const FwdKernel* registry(int dt, int* n) {
  switch (dt) {
    case FMHA_DTYPE_F32: return registry_f32(n);
    case FMHA_DTYPE_F16: return registry_f16(n);
    case FMHA_DTYPE_BF16: return registry_bf16(n);
    case FMHA_DTYPE_FP8_E4M3: return registry_fp8(n);
    default: *n = 0; return nullptr;
  }
}

// Waves per workgroup along rows / keys for a given number of query rows per
// (sequence, kv head): single-token decode (<= 16 rows, incl. GQA packing)
// splits each key block over 4 waves; larger row counts stack 16-row waves.
void pick_shape(int64_t rows, int* nwm, int* nwk) {
  if (rows <= 16) {
    *nwm = 1; *nwk = 4;
  } else if (rows <= 32) {
    *nwm = 2; *nwk = 2;
  } else if (rows <= 64) {
    *nwm = 4; *nwk = 1;
  } else if (rows <= 80) {
    *nwm = 5; *nwk = 1;
  } else {
    *nwm = 8; *nwk = 1;
  }
}

const FwdKernel* decode_registry(int dt, int* n) {
  switch (dt) {
    case FMHA_DTYPE_F32: return registry_f32_decode(n);
    case FMHA_DTYPE_F16: return registry_f16_decode(n);
    case FMHA_DTYPE_BF16: return registry_bf16_decode(n);
    case FMHA_DTYPE_FP8_E4M3: return registry_fp8_decode(n);
    default: *n = 0; return nullptr;
  }
}

const FwdKernel* prefill_registry(int dt, int* n) {
  switch (dt) {
    case FMHA_DTYPE_F32: return registry_f32_prefill(n);
    case FMHA_DTYPE_F16: return registry_f16_prefill(n);
    case FMHA_DTYPE_BF16: return registry_bf16_prefill(n);
    case FMHA_DTYPE_FP8_E4M3: return registry_fp8_prefill(n);
    default: *n = 0; return nullptr;
  }
}

// Smallest 32-row-wave instance whose tile covers `rows`, else the largest.
const FwdKernel* find_prefill(int dt, int dqk, int dv, int64_t rows) {
  int n = 0;
  const FwdKernel* t = prefill_registry(dt, &n);
  const FwdKernel* fit = nullptr;
  const FwdKernel* big = nullptr;
  for (int i = 0; i < n; ++i) {
    if (t[i].dqk != dqk || t[i].dv != dv) continue;
    if (!big || t[i].nwm > big->nwm) big = &t[i];
    if (32 * t[i].nwm >= rows && (!fit || t[i].nwm < fit->nwm)) fit = &t[i];
  }
  return fit ? fit : big;
}

const FwdKernel* find_decode(int dt, int dqk, int dv) {
  int n = 0;
  const FwdKernel* t = decode_registry(dt, &n);
  for (int i = 0; i < n; ++i)
    if (t[i].dqk == dqk && t[i].dv == dv) return &t[i];
  return nullptr;
}

const FwdKernel* find_exact(int dt, int dqk, int dv, int nwm, int nwk) {
  int n = 0;
  const FwdKernel* t = registry(dt, &n);
  for (int i = 0; i < n; ++i)
    if (t[i].dqk == dqk && t[i].dv == dv && t[i].nwm == nwm && t[i].nwk == nwk) return &t[i];
  return nullptr;
}

// Preferred shape first; wide head dims lack the largest row tiles (register
// budget), so fall back to narrower workgroups that cover fewer rows each.
const FwdKernel* find_kernel(int dt, int dqk, int dv, int nwm, int nwk) {
  if (const FwdKernel* k = find_exact(dt, dqk, dv, nwm, nwk)) return k;
  static const int fallback[][2] = {{5, 1}, {4, 1}, {2, 2}, {1, 4}};
  for (const auto& f : fallback)
    if (f[0] < nwm)
      if (const FwdKernel* k = find_exact(dt, dqk, dv, f[0], f[1])) return k;
  return nullptr;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }
bool stride_ok(int64_t s, int eb) { return s >= 0 && (s * eb) % 16 == 0; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Resolved {
  fmha_fwd_plan plan;
  const FwdKernel* kernel;
  int64_t sq_max, sk_max, total_q, total_k;
  bool empty;  // nothing to compute
};

// Automatic split count.  Parallel units of the non-split grid are
// (sequence, kv head, query tile); when they cannot fill the device the key
// range is cut into splits of at least kMinChunk keys.  The split sweeps on
// the pages show time falling steeply until the grid covers the machine and
// flattening or rising past that point.  On MI355X:
//  * the streaming kernels (2 resident workgroups per CU, one 16-row tile)
//    keep improving until each CU has seen ~16 workgroups, which also evens
//    out sequences of different lengths.  The decode kernel, whose splits are
//    ordered full ones first, takes as few as 8 per CU where that gives
//    splits of kDecodeChunk keys: each workgroup spends ~4.5 us on its
//    prologue and merge, and with 544-key splits that was a quarter of its
//    life (GQA decode, 16 x 8 kv heads, keys ~ U[1024, 32768]: 31 splits of
//    1056 keys ran 4 % faster than 60 of 544 on three length draws; long
//    decode, already at 1056 keys, is unchanged);
//  * the multi-row (prefill-family) kernels hold a large LDS ring per
//    workgroup and run fastest with exactly one wave of workgroups: splits
//    are chosen so that units x splits just fits the CU count, since a
//    second round of workgroups on a few CUs doubles the time.
int auto_splits(int64_t units, int64_t key_work, int64_t sk_max, int sb, int num_cus, bool one_round,
                bool decode) {
  constexpr int kTargetPerCu = 16;
  constexpr int64_t kMinChunk = 256;
  constexpr int64_t kDecodeChunk = 1024;
  if (sk_max <= 0) return 1;
  int64_t chunk;
  if (one_round) {
    const int64_t s = num_cus / (units > 0 ? units : 1);
    if (s <= 1) return 1;
    chunk = (sk_max + s - 1) / s;
  } else {
    const int64_t target = (int64_t)kTargetPerCu * num_cus;
    if (units >= target / 2) return 1;
    chunk = (key_work + target - 1) / target;
    if (decode) {
      const int64_t half = target / 2;
      chunk = std::max(chunk, std::min(kDecodeChunk, (key_work + half - 1) / half));
    }
  }
  if (chunk < kMinChunk) chunk = kMinChunk;
  chunk = (chunk + sb - 1) / sb * sb;
  int64_t s = (sk_max + chunk - 1) / chunk;
  if (s < 1) s = 1;
  if (s > FMHA_MAX_SPLITS) s = FMHA_MAX_SPLITS;
  // Keys per split of s splits, as the launch cuts them.  A power-of-two
  // number of key blocks per split starts every split's stream at the same
  // offset modulo a large power of two of bytes (long decode: 1024 keys x
  // 8 KiB rows, so the ~2048 concurrent wave streams are congruent mod
  // 2 MiB); measured on MI355X, such chunks ran 6 % (long decode, 1024 keys)
  // and 14 % (GQA decode, 512 keys) slower than the neighbouring sizes, so
  // take fewer splits until the chunk is not one.
  auto chunk_of = [&](int64_t n) {
    const int64_t c = (sk_max + n - 1) / n;
    return (c + sb - 1) / sb * sb;
  };
  auto pow2_blocks = [&](int64_t c) {
    const int64_t nb = c / sb;
    return nb >= 4 && (nb & (nb - 1)) == 0;
  };
  while (s > 1 && pow2_blocks(chunk_of(s))) --s;
  return (int)s;
}

// What a caller is about to do with the arguments: a pure shape query checks
// no pointer, the partials launch needs q/k/v and the workspace, the full
// forward also needs out.
enum Mode { kQuery, kPartials, kFull };

int resolve(const fmha_fwd_args* a, Mode mode, Resolved* r) {
  if (!a || !r) return FMHA_ERR_INVALID_ARG;
  memset(r, 0, sizeof(*r));
  const int eb = elem_bytes(a->in_dtype);
  if (eb == 0) return FMHA_ERR_INVALID_ARG;
  const int ob = elem_bytes(a->out_dtype);
  if (ob == 0 || a->out_dtype == FMHA_DTYPE_FP8_E4M3) return FMHA_ERR_INVALID_ARG;
  if (a->in_dtype == FMHA_DTYPE_FP8_E4M3) {
    if (a->out_dtype != FMHA_DTYPE_BF16) return FMHA_ERR_UNSUPPORTED;
  } else if (a->out_dtype != a->in_dtype) {
    return FMHA_ERR_UNSUPPORTED;
  }
  if (a->batch < 0 || a->num_heads_q <= 0 || a->num_heads_kv <= 0) return FMHA_ERR_INVALID_ARG;
  if (a->num_heads_q % a->num_heads_kv != 0) return FMHA_ERR_INVALID_ARG;
  if (a->head_dim_qk <= 0 || a->head_dim_v <= 0) return FMHA_ERR_INVALID_ARG;
  if (a->window_left < -1 || a->window_right < -1) return FMHA_ERR_INVALID_ARG;
  if (!(a->softmax_scale >= 0.f) || isinf(a->softmax_scale)) return FMHA_ERR_INVALID_ARG;
  if (a->num_kv_splits < 0 || a->num_kv_splits > FMHA_MAX_SPLITS) return FMHA_ERR_INVALID_ARG;
  if (a->num_cus < 0) return FMHA_ERR_INVALID_ARG;
  if (a->combine_mode < 0 || a->combine_mode > 1) return FMHA_ERR_INVALID_ARG;
  if (a->persistent < 0 || a->persistent > 1) return FMHA_ERR_INVALID_ARG;

  const bool vq = a->cu_seqlens_q != nullptr, vk = a->cu_seqlens_k != nullptr;
  if (vq) {
    if (a->total_q < 0 || a->max_seqlen_q < 0) return FMHA_ERR_INVALID_ARG;
    if (a->max_seqlen_q > a->total_q) return FMHA_ERR_INVALID_ARG;
  } else if (a->seqlen_q < 0) {
    return FMHA_ERR_INVALID_ARG;
  }
  if (vk) {
    if (a->total_k < 0 || a->max_seqlen_k < 0) return FMHA_ERR_INVALID_ARG;
    if (a->max_seqlen_k > a->total_k) return FMHA_ERR_INVALID_ARG;
  } else if (a->seqlen_k < 0) {
    return FMHA_ERR_INVALID_ARG;
  }
  r->sq_max = vq ? a->max_seqlen_q : a->seqlen_q;
  r->sk_max = vk ? a->max_seqlen_k : a->seqlen_k;
  r->total_q = vq ? a->total_q : (int64_t)a->batch * a->seqlen_q;
  r->total_k = vk ? a->total_k : (int64_t)a->batch * a->seqlen_k;
  if (r->total_q >= ((int64_t)1 << 31) || r->total_k >= ((int64_t)1 << 31)) return FMHA_ERR_INVALID_ARG;

  fmha_fwd_plan& pl = r->plan;
  pl.softmax_scale = a->softmax_scale == 0.f ? (float)(1.0 / sqrt((double)a->head_dim_qk)) : a->softmax_scale;
  pl.window_left = a->window_left;
  pl.window_right = a->causal ? 0 : a->window_right;

  const int G = a->num_heads_q / a->num_heads_kv;
  int nwm = 1, nwk = 4;
  pick_shape(r->sq_max * G, &nwm, &nwk);
  // kernel family by query rows per (sequence, kv head): decode (<= 16),
  // 16-row tiles (<= 80), 32x32-tile prefill (more), with fallbacks
  const FwdKernel* kern = nullptr;
  bool prefill = false;
  if (r->sq_max * G <= 16) kern = find_decode(a->in_dtype, a->head_dim_qk, a->head_dim_v);
  // fp8 takes the 32x32-tile kernel from 17 rows (its 16-row kernel stages V
  // byte by byte); f16/bf16 from 81 rows
  const int64_t pf_from = a->in_dtype == FMHA_DTYPE_FP8_E4M3 ? 16 : 80;
  if (!kern && r->sq_max * G > pf_from) {
    kern = find_prefill(a->in_dtype, a->head_dim_qk, a->head_dim_v, r->sq_max * G);
    prefill = kern != nullptr;
  }
  if (!kern) kern = find_kernel(a->in_dtype, a->head_dim_qk, a->head_dim_v, nwm, nwk);
  if (!kern) return FMHA_ERR_UNSUPPORTED;
  r->kernel = kern;
  pl.kernel_id = a->in_dtype * 1000 + kern->id;
  pl.rows_per_tile = (prefill ? 32 : 16) * kern->nwm;
  // decode kernels stream 32-key blocks per wave; splits are cut in multiples of that
  pl.key_block = kern->bn > 0 ? kern->nwk * kern->bn : 32;
  const int64_t rows = r->sq_max * G;
  pl.num_q_tiles = (int32_t)((rows + pl.rows_per_tile - 1) / pl.rows_per_tile);

  // nothing to compute (and nothing written): no query rows, or no key anywhere
  r->empty = a->batch == 0 || r->total_q == 0 || r->sq_max == 0 || r->total_k == 0 || r->sk_max == 0;
  if (!r->empty && mode != kQuery) {
    if (!a->q || !a->k || !a->v || (mode == kFull && !a->out)) return FMHA_ERR_INVALID_ARG;
    if (!aligned(a->q, 16) || !aligned(a->k, 16) || !aligned(a->v, 16) || !aligned(a->out, 16))
      return FMHA_ERR_INVALID_ARG;
    if (a->lse && !aligned(a->lse, 4)) return FMHA_ERR_INVALID_ARG;
    if (!stride_ok(a->q_stride_tok, eb) || !stride_ok(a->q_stride_head, eb) ||
        !stride_ok(a->k_stride_tok, eb) || !stride_ok(a->k_stride_head, eb) ||
        !stride_ok(a->v_stride_tok, eb) || !stride_ok(a->v_stride_head, eb) ||
        !stride_ok(a->o_stride_tok, ob) || !stride_ok(a->o_stride_head, ob))
      return FMHA_ERR_INVALID_ARG;
    if (!vq && (!stride_ok(a->q_stride_batch, eb) || !stride_ok(a->o_stride_batch, ob)))
      return FMHA_ERR_INVALID_ARG;
    if (!vk && (!stride_ok(a->k_stride_batch, eb) || !stride_ok(a->v_stride_batch, eb)))
      return FMHA_ERR_INVALID_ARG;
    if (a->lse && (a->lse_stride_head < 0 || (!vq && a->lse_stride_batch < 0))) return FMHA_ERR_INVALID_ARG;
    // the prefill kernels address the rows of one key block with 32-bit
    // buffer offsets (row * token stride): refuse strides that would wrap
    if (prefill) {
      const int64_t st = std::max(a->k_stride_tok * eb, a->v_stride_tok * eb);
      if ((int64_t)kern->bn * st + 4096 >= ((int64_t)1 << 31)) return FMHA_ERR_UNSUPPORTED;
    }
  }

  // splits
  const int num_cus = a->num_cus > 0 ? a->num_cus : 256;
  const int64_t units = (int64_t)a->batch * a->num_heads_kv * pl.num_q_tiles;
  int S;
  if (a->num_kv_splits > 0) {
    S = a->num_kv_splits;
  } else {
    const int64_t key_work = (int64_t)a->num_heads_kv * pl.num_q_tiles * r->total_k;
    S = auto_splits(units, key_work, r->sk_max, pl.key_block, num_cus, prefill, kern->bn == 0);
  }
  pl.num_splits = S;
  if (S > 1) {
    int64_t chunk = r->sk_max > 0 ? (r->sk_max + S - 1) / S : 1;
    chunk = (chunk + pl.key_block - 1) / pl.key_block * pl.key_block;
    pl.split_chunk = (int32_t)chunk;
    const size_t o_bytes = (size_t)S * (size_t)r->total_q * a->num_heads_q * a->head_dim_v * sizeof(float);
    const size_t l_bytes = (size_t)S * (size_t)a->num_heads_q * (size_t)r->total_q * sizeof(float);
    pl.o_part_offset = 0;
    pl.lse_part_offset = align256(o_bytes);
    // two arrival counters per (sequence, kv head, query tile) for the
    // combine inside the attention launch
    pl.counter_offset = pl.lse_part_offset + align256(l_bytes);
    pl.counter_bytes = align256((size_t)a->batch * a->num_heads_kv * pl.num_q_tiles * kCounterStride * sizeof(int32_t));
    pl.workspace_bytes = pl.counter_offset + pl.counter_bytes;
  } else {
    pl.split_chunk = (int32_t)(r->sk_max > 0 ? r->sk_max : 1);
    pl.workspace_bytes = 0;
  }
  pl.grid_main = r->empty ? 0 : (int64_t)S * units;
  // longest-first tile order where the tiles of a sequence differ in cost (a
  // right-bounded mask: causal) and the kernel's per-workgroup search applies
  // (one split, no left window, at most 64 sequences).  Its grid covers every
  // tile that exists, a bound from the packed query count (sequence b has
  // ceil(rows_b / tile) tiles).
  pl.tile_order = kTileOrderGrouped;
  if (prefill && S == 1 && !r->empty && (pl.window_right >= 0 || pl.window_left >= 0)) {
    const int64_t tiles = (r->total_q * G + (int64_t)a->batch * (pl.rows_per_tile - 1)) / pl.rows_per_tile;
    const int64_t slots = (int64_t)a->batch * pl.num_q_tiles;
    const int64_t cap = tiles < slots ? tiles : slots;
    if (pl.window_left < 0 && a->batch <= kLongestFirstMaxBatch) {
      pl.tile_order = kTileOrderLongestFirst;
      pl.grid_main = (int64_t)a->num_heads_kv * cap;
    } else if (a->batch <= kScheduleMaxBatch && a->num_heads_kv < 2048 && pl.num_q_tiles < (1 << 20) &&
               (int64_t)a->num_heads_kv * cap < ((int64_t)1 << 28) && (mode == kQuery || a->workspace)) {
      // more sequences than lanes, or a left window: (sequence, kv head)
      // groups dealt to XCDs longest first by a schedule kernel into a table
      // in the workspace (without a workspace the grouped order stays).  Each
      // XCD's list gets room for a 1/8 share of the tiles plus one
      // sequence's tiles; the schedule kernel moves what a list holds past
      // its room to the lists with room left, and the rooms together hold
      // every tile (kv heads x cap bounds the tiles)
      const int64_t per_xcd = ((int64_t)a->num_heads_kv * cap + 7) / 8 + pl.num_q_tiles;
      const int64_t positions = 8 * per_xcd;  // < 2^30 (table entries pack the tile in 20 bits)
      pl.tile_order = kTileOrderTable;
      pl.grid_main = positions;
      // persistent: one round of workgroups (three per CU, one at head dim 256)
      // takes the positions from the table (f16/bf16 prefill kernel)
      if (a->persistent && a->in_dtype != FMHA_DTYPE_FP8_E4M3) {
        pl.persistent = 1;
        const int64_t round = (int64_t)num_cus * (kern->dqk >= 256 ? 1 : 3);
        pl.grid_main = positions < round ? positions : round;
      }
      pl.sched_offset = 0;
      pl.sched_items = (int32_t)positions;
      pl.workspace_bytes = align256((size_t)(kSchedHead + 2 * positions) * sizeof(int32_t));
    }
  }
  // multi-row kernels with one query tile per sequence and several splits
  // (the short cached-prefix shape): the kv heads of one split together, so
  // neighbouring heads' rows that share 128-byte lines are fetched once per
  // XCD
  if (prefill && S > 1 && pl.num_q_tiles == 1 && !r->empty) pl.tile_order = kTileOrderHeadsTogether;
  // the decode kernel's splits: full ones first, then the partial ones longest
  // first (the grid keeps its (sequence, kv head, split) size; positions past
  // the last split return at once)
  if (kern->bn == 0 && S > 1 && a->batch <= kLongestFirstMaxBatch && !r->empty)
    pl.tile_order = kTileOrderFullFirst;
  if (pl.grid_main >= kMaxGrid) return FMHA_ERR_INVALID_ARG;
  // the split workgroups combine their partials themselves when the whole
  // grid is resident at once (one workgroup per compute unit at most): the
  // multi-row kernels with one round of splits, e.g. the short cached prefix
  pl.combine_in_kernel = a->combine_mode == 1 && prefill && S > 1 && S <= kFusedMaxSplits && !r->empty &&
                         mode != kPartials &&
                         pl.grid_main <= num_cus && pl.lse_part_offset < ((size_t)1 << 31);
  pl.grid_combine = (r->empty || S == 1 || pl.combine_in_kernel)
                        ? 0
                        : combine_grid(a->head_dim_v, S, r->sq_max * a->num_heads_q * a->batch);
  if (pl.grid_combine >= kMaxGrid) return FMHA_ERR_INVALID_ARG;
  if (mode != kQuery && (S > 1 || pl.tile_order == kTileOrderTable) && !r->empty) {
    if (!a->workspace || !aligned(a->workspace, 256) || a->workspace_bytes < pl.workspace_bytes)
      return FMHA_ERR_WORKSPACE;
  }
  return FMHA_OK;
}

FwdParams make_params(const fmha_fwd_args* a, const Resolved& r) {
  const int eb = elem_bytes(a->in_dtype), ob = elem_bytes(a->out_dtype);
  FwdParams p;
  memset(&p, 0, sizeof(p));
  p.q = (const char*)a->q;
  p.k = (const char*)a->k;
  p.v = (const char*)a->v;
  p.o = (char*)a->out;
  p.lse = a->lse;
  if (r.plan.num_splits > 1) {
    p.o_part = (float*)((char*)a->workspace + r.plan.o_part_offset);
    p.lse_part = (float*)((char*)a->workspace + r.plan.lse_part_offset);
    p.counters = (int32_t*)((char*)a->workspace + r.plan.counter_offset);
  }
  p.cu_q = a->cu_seqlens_q;
  p.cu_k = a->cu_seqlens_k;
  if (a->in_dtype == FMHA_DTYPE_FP8_E4M3) {
    p.q_descale = a->q_descale;
    p.k_descale = a->k_descale;
    p.v_descale = a->v_descale;
  }
  p.batch = a->batch;
  p.seqlen_q = a->seqlen_q;
  p.seqlen_k = a->seqlen_k;
  p.total_q = (int32_t)r.total_q;
  p.hq = a->num_heads_q;
  p.hkv = a->num_heads_kv;
  p.group = a->num_heads_q / a->num_heads_kv;
  p.q_sb = a->q_stride_batch * eb;
  p.q_st = a->q_stride_tok * eb;
  p.q_sh = a->q_stride_head * eb;
  p.k_sb = a->k_stride_batch * eb;
  p.k_st = a->k_stride_tok * eb;
  p.k_sh = a->k_stride_head * eb;
  p.v_sb = a->v_stride_batch * eb;
  p.v_st = a->v_stride_tok * eb;
  p.v_sh = a->v_stride_head * eb;
  p.o_sb = a->o_stride_batch * ob;
  p.o_st = a->o_stride_tok * ob;
  p.o_sh = a->o_stride_head * ob;
  p.lse_sb = a->lse_stride_batch;
  p.lse_sh = a->lse_stride_head;
  p.scale_log2 = (float)((double)r.plan.softmax_scale * 1.4426950408889634);
  p.wl = r.plan.window_left;
  p.wr = r.plan.window_right;
  p.num_splits = r.plan.num_splits;
  p.chunk = r.plan.split_chunk;
  p.num_q_tiles = r.plan.num_q_tiles;
  p.out_dtype = a->out_dtype;
  p.tile_order = r.plan.tile_order;
  if (r.plan.tile_order == kTileOrderTable) {
    p.sched = (int32_t*)((char*)a->workspace + r.plan.sched_offset);
    p.persistent = r.plan.persistent;
  }
  p.max_seqlen_k = (int32_t)r.sk_max;
  return p;
}

CombineParams make_combine(const fmha_fwd_args* a, const Resolved& r) {
  const int ob = elem_bytes(a->out_dtype);
  CombineParams c;
  memset(&c, 0, sizeof(c));
  c.o_part = (const float*)((const char*)a->workspace + r.plan.o_part_offset);
  c.lse_part = (const float*)((const char*)a->workspace + r.plan.lse_part_offset);
  c.o = (char*)a->out;
  c.lse = a->lse;
  c.cu_q = a->cu_seqlens_q;
  c.cu_k = a->cu_seqlens_k;
  c.batch = a->batch;
  c.seqlen_q = a->seqlen_q;
  c.seqlen_k = a->seqlen_k;
  c.max_seqlen_q = (int32_t)r.sq_max;
  c.total_q = (int32_t)r.total_q;
  c.hq = a->num_heads_q;
  c.dv = a->head_dim_v;
  c.num_splits = r.plan.num_splits;
  c.chunk = r.plan.split_chunk;
  c.chunks_per_wg = combine_chunks_per_wg(a->head_dim_v, c.num_splits, r.sq_max * a->num_heads_q * a->batch);
  c.o_sb = a->o_stride_batch * ob;
  c.o_st = a->o_stride_tok * ob;
  c.o_sh = a->o_stride_head * ob;
  c.lse_sb = a->lse_stride_batch;
  c.lse_sh = a->lse_stride_head;
  c.out_dtype = a->out_dtype;
  return c;
}

}  // namespace
}  // namespace fmha

namespace fmha {
namespace {

// Compute units of the current device (cached per device).
constexpr int kMaxCuDevices = 64;
std::atomic<int> g_device_cus[kMaxCuDevices];

int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxCuDevices) return 0;
  n = g_device_cus[dev].load(std::memory_order_relaxed);
  if (n == 0 && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
    g_device_cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

int launch_fwd(const fmha_fwd_args* args, void* stream) {
  Resolved r;
  int st = resolve(args, kFull, &r);
  if (st != FMHA_OK) return st;
  if (r.empty || r.plan.grid_main == 0) return FMHA_OK;
  hipStream_t s = (hipStream_t)stream;
  FwdParams p = make_params(args, r);
  // the in-kernel combine waits for the tile's other split workgroups: only
  // when this device runs the whole grid at once (one workgroup per CU)
  p.fused_combine = r.plan.combine_in_kernel && r.plan.grid_main <= device_cus();
  if (r.plan.tile_order == kTileOrderTable &&
      launch_schedule(p, r.plan.rows_per_tile, r.plan.key_block, r.plan.sched_items, p.sched, s) !=
          hipSuccess)
    return FMHA_ERR_HIP;
  if (r.kernel->launch(p, r.plan.grid_main, s) != hipSuccess) return FMHA_ERR_HIP;
  if (r.plan.num_splits > 1 && !p.fused_combine) {
    const CombineParams c = make_combine(args, r);
    if (launch_combine(c, s) != hipSuccess) return FMHA_ERR_HIP;
  }
  return FMHA_OK;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept for the process.
constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch[kMaxScratchDevices];
std::mutex g_scratch_mu;

int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FMHA_ERR_HIP;
  if (dev < 0 || dev >= kMaxScratchDevices) return FMHA_ERR_HIP;
  void* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return FMHA_ERR_HIP;
      g_scratch[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return FMHA_OK;
}

}  // namespace
}  // namespace fmha

using namespace fmha;

extern "C" {

const char* fmha_status_str(int status) {
  switch (status) {
    case FMHA_OK: return "ok";
    case FMHA_ERR_INVALID_ARG: return "invalid argument";
    case FMHA_ERR_UNSUPPORTED: return "unsupported configuration (no compiled kernel)";
    case FMHA_ERR_WORKSPACE: return "split workspace missing, misaligned or too small";
    case FMHA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

int fmha_fwd_check(const fmha_fwd_args* args, fmha_fwd_plan* plan) {
  Resolved r;
  // with out == NULL the arguments are checked for a partials-only launch
  const int st = resolve(args, (args && args->out) ? kFull : kPartials, &r);
  if (st == FMHA_OK && plan) *plan = r.plan;
  return st;
}

int fmha_num_splits(const fmha_fwd_args* args, int32_t* splits_out) {
  if (!splits_out) return FMHA_ERR_INVALID_ARG;
  Resolved r;
  const int st = resolve(args, kQuery, &r);
  if (st == FMHA_OK) *splits_out = r.plan.num_splits;
  return st;
}

int fmha_fwd_workspace_size(const fmha_fwd_args* args, size_t* bytes_out) {
  if (!bytes_out) return FMHA_ERR_INVALID_ARG;
  Resolved r;
  const int st = resolve(args, kQuery, &r);
  if (st == FMHA_OK) *bytes_out = r.plan.workspace_bytes;
  return st;
}

int fmha_fwd(const fmha_fwd_args* args, void* stream) { return launch_fwd(args, stream); }

int fmha_fwd_no_alloc(const fmha_fwd_args* args, void* stream) {
  if (!args) return FMHA_ERR_INVALID_ARG;
  fmha_fwd_args a = *args;
  void* ws = nullptr;
  const int st = scratch_address(&ws);
  if (st != FMHA_OK) return st;
  // the split partials go to this device's scratch; resolve refuses a plan
  // whose workspace exceeds it (FMHA_ERR_WORKSPACE) before any launch
  a.workspace = ws;
  a.workspace_bytes = FMHA_NO_ALLOC_SCRATCH_BYTES;
  // the combine inside the attention launch counts arrivals in a block that
  // must start at zero; the scratch holds whatever the previous call left, so
  // this entry point always combines with the second launch
  a.combine_mode = 0;
  return launch_fwd(&a, stream);
}

int fmha_fwd_splitkv_partials(const fmha_fwd_args* args, void* stream) {
  Resolved r;
  int st = resolve(args, kPartials, &r);
  if (st != FMHA_OK) return st;
  if (r.plan.num_splits <= 1) return FMHA_ERR_INVALID_ARG;
  if (r.empty || r.plan.grid_main == 0) return FMHA_OK;
  const FwdParams p = make_params(args, r);
  if (r.kernel->launch(p, r.plan.grid_main, (hipStream_t)stream) != hipSuccess) return FMHA_ERR_HIP;
  return FMHA_OK;
}

int fmha_splitkv_combine(const fmha_combine_args* a, void* stream) {
  if (!a) return FMHA_ERR_INVALID_ARG;
  const int ob = elem_bytes(a->out_dtype);
  if (ob == 0 || a->out_dtype == FMHA_DTYPE_FP8_E4M3) return FMHA_ERR_INVALID_ARG;
  // the combine moves 4 consecutive Dv elements per thread
  if (a->batch < 0 || a->num_heads_q <= 0 || a->head_dim_v <= 0 || a->head_dim_v % 4 ||
      a->head_dim_v > 1024)
    return FMHA_ERR_INVALID_ARG;
  if (a->num_splits < 1 || a->num_splits > FMHA_MAX_SPLITS || a->split_chunk < 1) return FMHA_ERR_INVALID_ARG;
  const bool vq = a->cu_seqlens_q != nullptr;
  const int64_t sq_max = vq ? a->max_seqlen_q : a->seqlen_q;
  const int64_t total_q = vq ? a->total_q : (int64_t)a->batch * a->seqlen_q;
  if (sq_max < 0 || total_q < 0 || (!a->cu_seqlens_k && a->seqlen_k < 0)) return FMHA_ERR_INVALID_ARG;
  if (total_q >= ((int64_t)1 << 31)) return FMHA_ERR_INVALID_ARG;  // partial rows are indexed in 32 bits
  if (vq && a->max_seqlen_q > a->total_q) return FMHA_ERR_INVALID_ARG;
  if (a->batch == 0 || total_q == 0 || sq_max == 0) return FMHA_OK;
  if (!a->o_part || !a->lse_part || !a->out) return FMHA_ERR_INVALID_ARG;
  if (!aligned(a->o_part, 16) || !aligned(a->lse_part, 4) || !aligned(a->out, 4 * ob)) return FMHA_ERR_INVALID_ARG;
  if (a->lse && !aligned(a->lse, 4)) return FMHA_ERR_INVALID_ARG;
  if (a->o_stride_tok < 0 || a->o_stride_head < 0 || a->o_stride_tok % 4 || a->o_stride_head % 4 ||
      (!vq && (a->o_stride_batch < 0 || a->o_stride_batch % 4)))
    return FMHA_ERR_INVALID_ARG;
  if (combine_grid(a->head_dim_v, a->num_splits, sq_max * a->num_heads_q * a->batch) >= kMaxGrid) return FMHA_ERR_INVALID_ARG;
  CombineParams c;
  memset(&c, 0, sizeof(c));
  c.o_part = a->o_part;
  c.lse_part = a->lse_part;
  c.o = (char*)a->out;
  c.lse = a->lse;
  c.cu_q = a->cu_seqlens_q;
  c.cu_k = a->cu_seqlens_k;
  c.batch = a->batch;
  c.seqlen_q = a->seqlen_q;
  c.seqlen_k = a->seqlen_k;
  c.max_seqlen_q = (int32_t)sq_max;
  c.total_q = (int32_t)total_q;
  c.hq = a->num_heads_q;
  c.dv = a->head_dim_v;
  c.num_splits = a->num_splits;
  c.chunk = a->split_chunk;
  c.chunks_per_wg = combine_chunks_per_wg(a->head_dim_v, a->num_splits, sq_max * a->num_heads_q * a->batch);
  c.o_sb = a->o_stride_batch * ob;
  c.o_st = a->o_stride_tok * ob;
  c.o_sh = a->o_stride_head * ob;
  c.lse_sb = a->lse_stride_batch;
  c.lse_sh = a->lse_stride_head;
  c.out_dtype = a->out_dtype;
  if (launch_combine(c, (hipStream_t)stream) != hipSuccess) return FMHA_ERR_HIP;
  return FMHA_OK;
}

int fmha_check_seqlens(const int32_t* cu_seqlens, int32_t batch, int32_t total, int32_t max_seqlen,
                       int32_t* result, void* stream) {
  // (the check's index loop steps by 256 and must not pass INT32_MAX)
  if (!cu_seqlens || !result || batch < 0 || batch > INT32_MAX - 256 || total < 0 || max_seqlen < 0)
    return FMHA_ERR_INVALID_ARG;
  if (fmha::launch_check_seqlens(cu_seqlens, batch, total, max_seqlen, result, (hipStream_t)stream) != hipSuccess)
    return FMHA_ERR_HIP;
  return FMHA_OK;
}

int fmha_device_num_cus(int32_t* num_cus_out) {
  if (!num_cus_out) return FMHA_ERR_INVALID_ARG;
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FMHA_ERR_HIP;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return FMHA_ERR_HIP;
  *num_cus_out = n;
  return FMHA_OK;
}

}  // extern "C"
