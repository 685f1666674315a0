// Attention forward kernel for gfx950 (CDNA4): split-KV partials or final
// output, packed variable-length sequences, GQA row packing, bottom-right
// causal / sliding-window / residual masks.
//
// Method (web pages on split-KV flash attention): the online-softmax forward
// of flash attention with exp2, split KV across workgroups for short queries
// ("[Cute,Fwd,Sm100] Support q_stage=1 for inference", description;
// "[FlyDSL] Enable FP8 FMHA split-K ...", description), packed varlen with
// per-sequence offsets, tiles past a sequence's end skipped and tail rows not
// stored ("Adds variable sequence lengths to the Hopper CuTe DSL FMHA
// example", sections Interface and Implementation).
//
// Workgroup = NWM x NWK wavefronts.  The NWM waves own 16 query rows each
// (rows = (query position, query head of the kv group) pairs, so the heads of
// one GQA group fill the MFMA M dimension); the NWK waves split every key
// block between them and are merged through LDS at the end.  Per iteration the
// workgroup stages NWK*BN keys of K (row-major) and V (transposed) in LDS,
// with the next block's global loads in flight in registers.
//
// MFMA formulation (16x16 tiles, fp32 accumulate):
//   S^T[key, row] = K[key, :] . Q[row, :]     A = K tile, B = Q^T
//   O^T[dv, row] += V^T[dv, key] P^T[key, row] A = V^T tile, B = P^T
// With S^T's lane-major layout (lane%16 = row, lane/16 = key group) each lane
// owns one query row, so the softmax row statistics never leave the lane
// group, P^T feeds the second MFMA straight from registers, and the
// per-row rescale of O^T is lane-local.  Contraction indices are assigned to
// (lane group, register slot) consistently between the two operands of each
// MFMA, which is all the instruction requires.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fmha_params.h"

namespace fmha {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// fp8 probabilities are stored as p * 2^8 (exact power of two) to keep small
// probabilities in e4m3's normal range; divided out in the epilogue.
constexpr float kFp8PScale = 256.0f;

template <int DT>
struct Elem;
template <>
struct Elem<DT_F32> {
  static constexpr int bytes = 4;
};
template <>
struct Elem<DT_F16> {
  static constexpr int bytes = 2;
};
template <>
struct Elem<DT_BF16> {
  static constexpr int bytes = 2;
};
template <>
struct Elem<DT_FP8> {
  static constexpr int bytes = 1;
};

// acc += A_chunk * B_chunk over the contraction slots one 16-byte chunk per
// lane holds (4 fp32, 8 f16/bf16, 16 fp8 values -> 4, 1, 2 MFMAs).
template <int DT>
__device__ __forceinline__ f32x4 mfma_chunk(f32x4 acc, u32x4 a, u32x4 b) {
  if constexpr (DT == DT_F32) {
    // one fp32 contraction slot per lane per instruction; components are
    // converted by value (bit-casting a vector component reads element 0)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  } else if constexpr (DT == DT_F16) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
  } else if constexpr (DT == DT_BF16) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  } else {
    u32x2 a0 = {a.x, a.y}, a1 = {a.z, a.w}, b0 = {b.x, b.y}, b1 = {b.z, b.w};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(__builtin_bit_cast(long, a0),
                                                     __builtin_bit_cast(long, b0), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(__builtin_bit_cast(long, a1),
                                                     __builtin_bit_cast(long, b1), acc, 0, 0, 0);
  }
  return acc;
}

// Two fp32 values rounded to nearest even and packed (low half = a): one
// v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32 on gfx950.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Probabilities of S^T tiles [4c', 4c'+VPL/4) of one lane, packed as the
// 16-byte B-operand chunk of the P^T x V^T MFMA in the input element type.
template <int DT>
__device__ __forceinline__ u32x4 pack_p(const f32x4* p) {
  u32x4 r;
  if constexpr (DT == DT_F32) {
    r.x = __float_as_uint(p[0].x);
    r.y = __float_as_uint(p[0].y);
    r.z = __float_as_uint(p[0].z);
    r.w = __float_as_uint(p[0].w);
  } else if constexpr (DT == DT_F16) {
    r.x = pack_f16x2(p[0].x, p[0].y);
    r.y = pack_f16x2(p[0].z, p[0].w);
    r.z = pack_f16x2(p[1].x, p[1].y);
    r.w = pack_f16x2(p[1].z, p[1].w);
  } else if constexpr (DT == DT_BF16) {
    r.x = pack_bf16x2(p[0].x, p[0].y);
    r.y = pack_bf16x2(p[0].z, p[0].w);
    r.z = pack_bf16x2(p[1].x, p[1].y);
    r.w = pack_bf16x2(p[1].z, p[1].w);
  } else {
    const float s = kFp8PScale;
    r.x = pack_fp8x4(p[0].x * s, p[0].y * s, p[0].z * s, p[0].w * s);
    r.y = pack_fp8x4(p[1].x * s, p[1].y * s, p[1].z * s, p[1].w * s);
    r.z = pack_fp8x4(p[2].x * s, p[2].y * s, p[2].z * s, p[2].w * s);
    r.w = pack_fp8x4(p[3].x * s, p[3].y * s, p[3].z * s, p[3].w * s);
  }
  return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Buffer descriptor of nbytes (< 2^31) at base: raw (untyped) 32-bit offsets,
// accesses past nbytes read zero and write nothing.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char* base, int64_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)nbytes, 0x00020000);
}

// Work item of this workgroup: (split, kv head, sequence, query tile) and the
// sequence's query / key offsets and lengths.
struct WorkItem {
  int split, hkv, b, qtile;
  int q_off, sq, k_off, sk;
};

__device__ __forceinline__ void seq_span(const FwdParams& p, int b, WorkItem& w) {
  int q0 = b * p.seqlen_q, q1 = q0 + p.seqlen_q, k0 = b * p.seqlen_k, k1 = k0 + p.seqlen_k;
  if (p.cu_q || p.cu_k) {
    // the four loads are issued together (one round trip)
    const int32_t* cq = p.cu_q ? p.cu_q : p.cu_k;
    const int32_t* ck = p.cu_k ? p.cu_k : p.cu_q;
    const int a0 = cq[b], a1 = cq[b + 1], c0 = ck[b], c1 = ck[b + 1];
    if (p.cu_q) q0 = a0, q1 = a1;
    if (p.cu_k) k0 = c0, k1 = c1;
  }
  w.q_off = q0;
  w.sq = q1 - q0;
  w.k_off = k0;
  w.sk = k1 - k0;
}

// Grouped order (kTileOrderGrouped).  Items are ordered so that the query
// tiles and splits of one (sequence, kv head) -- the workgroups that stream the
// same K and V -- form one group of consecutive items, query tiles in
// descending order.  Workgroups go to the 8 XCDs round-robin (block i on XCD
// i % 8) and each XCD has its own L2: groups are dealt to XCDs in rounds of 8,
// a whole group to one XCD, so the workgroups sharing K and V run on one XCD
// at about the same time.  A last round of fewer than 8 groups is dealt block
// by block.
__device__ __forceinline__ WorkItem grouped_item(const FwdParams& p) {
  constexpr uint32_t kXcds = 8;
  const uint32_t bid = blockIdx.x;
  const uint32_t gsz = (uint32_t)p.num_q_tiles * (uint32_t)p.num_splits;  // items per group
  const uint32_t ngroups = (uint32_t)p.batch * (uint32_t)p.hkv;
  const uint32_t round_items = kXcds * gsz;
  const uint32_t full = (ngroups / kXcds) * round_items;
  uint32_t item = bid;
  if (bid < full) {
    const uint32_t r = bid / round_items, local = bid % round_items;
    item = (r * kXcds + local % kXcds) * gsz + local / kXcds;
  }
  WorkItem w;
  w.qtile = p.num_q_tiles - 1 - (int)(item % (uint32_t)p.num_q_tiles);
  item /= (uint32_t)p.num_q_tiles;
  w.split = (int)(item % (uint32_t)p.num_splits);
  item /= (uint32_t)p.num_splits;
  w.hkv = (int)(item % (uint32_t)p.hkv);
  w.b = (int)(item / (uint32_t)p.hkv);
  seq_span(p, w.b, w);
  return w;
}

// Heads-together order (kTileOrderHeadsTogether; one query tile per
// sequence, several splits).  The splits of one kv head read disjoint key
// ranges, so keeping them on one XCD shares nothing; the kv heads of one
// (sequence, split) read the same tokens, whose rows are adjacent in memory
// and share 128-byte lines when a head's row is not a multiple of 128 bytes
// (192-byte fp8 K rows: heads 2p and 2p + 1 share one line).  Groups are
// (sequence, split) with one item per kv head, dealt whole to XCDs in rounds
// of 8; in the last partial round consecutive items go in pairs to one XCD
// (blocks 8j + x and 8(j + 1) + x, j even), a remainder of fewer than 16
// blocks block by block.
__device__ __forceinline__ WorkItem heads_together_item(const FwdParams& p) {
  constexpr uint32_t kXcds = 8;
  const uint32_t bid = blockIdx.x;
  const uint32_t gsz = (uint32_t)p.hkv;
  const uint32_t ngroups = (uint32_t)p.batch * (uint32_t)p.num_splits;
  const uint32_t round_items = kXcds * gsz;
  const uint32_t full = (ngroups / kXcds) * round_items;
  uint32_t item = bid;
  if (bid < full) {
    const uint32_t r = bid / round_items, local = bid % round_items;
    item = (r * kXcds + local % kXcds) * gsz + local / kXcds;
  } else {
    const uint32_t k = bid - full, rest = ngroups * gsz - full;
    if (k < rest / (2 * kXcds) * (2 * kXcds))
      item = full + ((k / (2 * kXcds)) * kXcds + k % kXcds) * 2 + (k / kXcds) % 2;
  }
  WorkItem w;
  w.qtile = 0;
  w.hkv = (int)(item % gsz);
  item /= gsz;
  w.split = (int)(item % (uint32_t)p.num_splits);
  w.b = (int)(item / (uint32_t)p.num_splits);
  seq_span(p, w.b, w);
  return w;
}

// Inclusive prefix sum of v over the lanes of the wave: a scan within each
// row of 16 lanes (DPP row shifts by 1, 2, 4, 8); then row_bcast:15 adds the
// last lane of rows 0 and 2 to rows 1 and 3, and row_bcast:31 adds lane 31
// (the total of rows 0 and 1) to rows 2 and 3.
__device__ __forceinline__ int wave_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

__device__ __forceinline__ int wave_sum(int v) { return __builtin_amdgcn_readlane(wave_scan(v), 63); }

// Longest-first order (kTileOrderLongestFirst): one split, no left window, at
// most 64 sequences (lane b of every wave holds sequence b).
//
// The hardware hands block i to XCD i % 8 and, within it, to shader engine
// (i / 8) % 4, each with a fixed number of workgroup slots; every such lane
// starts its blocks in order as slots free up.  Sorting all tiles by cost,
// longest first, gives the 32 lanes near-identical cost sequences (consecutive
// blocks cost about the same) and makes each lane's in-order start a
// longest-processing-time-first schedule.  Under a causal mask the tiles of one
// sequence differ in cost; with skewed lengths whole sequences do, and a fixed
// (sequence, tile) -> lane pattern leaves some lanes with far more work.
//
// The cost class of a tile is 1 + ceil(keys / 64), keys = the keys its last
// row attends (0 for a row before the first key: the tile still writes its
// rows); the tiles of one sequence with class >= c form a suffix of its query
// tiles, so the number of items in class >= c has a closed form per sequence.
// Position blockIdx.x is found by a binary search over the class, then by a
// prefix sum over sequences.  Within a class the order is sequence, query tile
// (descending), kv head: with a multiple of 8 kv heads every tile of a
// (sequence, kv head) lands on the same XCD.  Positions past the last tile
// return false.
template <int ROWS>
__device__ __forceinline__ bool longest_first_item(const FwdParams& p, WorkItem& w) {
  constexpr int kUnit = 64;  // keys per cost unit
  const int lane = threadIdx.x & 63;
  const bool real = lane < p.batch;
  WorkItem sp;
  seq_span(p, real ? lane : p.batch - 1, sp);  // clamped: every lane loads in bounds
  const int q0 = sp.q_off, k0 = sp.k_off;
  const int sq = real ? sp.sq : 0, sk = real ? sp.sk : 0;
  const int G = p.group;
  const int nt = (sq > 0 && sk > 0) ? (sq * G + ROWS - 1) / ROWS : 0;  // query tiles
  const int diag = sk - sq + p.wr;  // a row i attends keys <= i + diag (wr >= 0)
  const bool bounded = p.wr >= 0;
  // number of this sequence's tiles with cost class >= c (branch-free; class
  // 1 (need <= 0) holds every tile; a product that wraps is discarded by the
  // last select)
  auto count = [&](int c) -> int {
    const int need = (c - 2) * kUnit + 1;             // keys the last row must attend
    const int t = max(need - 1 - diag, 0);            // first query row attending them
    const unsigned f = (unsigned)t * (unsigned)G / (unsigned)ROWS;
    const int first = (bounded && need > 0) ? (int)min(f, (unsigned)nt) : 0;
    return need > sk ? 0 : nt - first;
  };
  const int H = p.hkv;
  const int pos = blockIdx.x;
  if (pos >= H * wave_sum(nt)) return false;
  int lo = 1, hi = 2 + (p.max_seqlen_k + kUnit - 1) / kUnit;  // items(lo) > pos >= items(hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (H * wave_sum(count(mid)) > pos)
      lo = mid;
    else
      hi = mid;
  }
  const int above = count(lo + 1);
  const int j = pos - H * wave_sum(above);  // index within class lo
  const int kc = count(lo) - above;         // this sequence's tiles in class lo
  const int excl = wave_scan(kc) - kc;      // tiles of class lo in lower sequences
  const uint64_t sel = __ballot(kc > 0 && H * excl <= j && j < H * (excl + kc));
  if (sel == 0) return false;  // not reached: the ranges partition the class
  // (whatever excl holds, the selected lane's test bounds jj to [0, H * kc),
  // so the tile and head below are in range)
  const int b = (int)__builtin_ctzll(sel);
  const int jj = j - H * __builtin_amdgcn_readlane(excl, b);
  w.split = 0;
  w.b = b;
  w.hkv = jj % H;
  w.qtile = __builtin_amdgcn_readlane(nt - above, b) - 1 - jj / H;
  w.q_off = __builtin_amdgcn_readlane(q0, b);
  w.sq = __builtin_amdgcn_readlane(sq, b);
  w.k_off = __builtin_amdgcn_readlane(k0, b);
  w.sk = __builtin_amdgcn_readlane(sk, b);
  return true;
}

// Full-first order (kTileOrderFullFirst): the decode kernel with more than one
// split, at most 64 sequences (lane b of every wave holds sequence b).  With
// splits of `chunk` keys, sequence b has nf_b = sk_b / chunk full splits and,
// when sk_b is not a multiple of chunk, one partial split of the remaining
// keys.  Positions [0, H * sum nf) hold the full splits in (sequence, kv head,
// split) order -- the splits of one (sequence, kv head) on consecutive blocks,
// which the hardware deals to different XCDs -- and the positions after them
// the partial splits, longest first (ties: lower sequence first), the kv heads
// of one sequence consecutive.  The 32 in-order dispatch lanes then end on the
// shortest items instead of a mix of full and partial ones.  Positions past
// the last split return false.
__device__ __forceinline__ bool full_first_item(const FwdParams& p, WorkItem& w) {
  const int lane = threadIdx.x & 63;
  const bool real = lane < p.batch;
  WorkItem sp;
  seq_span(p, real ? lane : p.batch - 1, sp);  // clamped: every lane loads in bounds
  const bool has = real && sp.sq > 0 && sp.sk > 0;
  const int S = p.num_splits, chunk = p.chunk;
  const int nf = has ? min(sp.sk / chunk, S) : 0;         // full splits
  const int rem = has && nf < S ? sp.sk - nf * chunk : 0;  // keys of the partial split
  const int H = p.hkv;
  const int pos = blockIdx.x;
  const int incl = wave_scan(nf);
  const int nfull = H * __builtin_amdgcn_readlane(incl, 63);
  int b, split;
  if (pos < nfull) {
    const int excl = incl - nf;
    const uint64_t sel = __ballot(nf > 0 && H * excl <= pos && pos < H * incl);
    if (sel == 0) return false;  // not reached: the ranges partition [0, nfull)
    b = (int)__builtin_ctzll(sel);
    const int j = pos - H * __builtin_amdgcn_readlane(excl, b);
    const int f = __builtin_amdgcn_readlane(nf, b);
    w.hkv = j / f;
    split = j % f;
  } else {
    const int j = pos - nfull;
    // rank of this sequence's partial split among all partial splits
    int rank = 0;
    for (int i = 0; i < p.batch; ++i) {
      const int ri = __builtin_amdgcn_readlane(rem, i);
      rank += (ri > rem || (ri == rem && i < lane)) ? 1 : 0;
    }
    const uint64_t sel = __ballot(rem > 0 && rank == j / H);
    if (sel == 0) return false;  // past the last partial split
    b = (int)__builtin_ctzll(sel);
    w.hkv = j % H;
    split = __builtin_amdgcn_readlane(nf, b);
  }
  w.split = split;
  w.b = b;
  w.qtile = 0;
  w.q_off = __builtin_amdgcn_readlane(sp.q_off, b);
  w.sq = __builtin_amdgcn_readlane(sp.sq, b);
  w.k_off = __builtin_amdgcn_readlane(sp.k_off, b);
  w.sk = __builtin_amdgcn_readlane(sp.sk, b);
  return true;
}

// Table order (kTileOrderTable): the tile the schedule kernel put at grid
// position pos (fmha_schedule.hip), or none.
__device__ __forceinline__ bool table_item(const FwdParams& p, int pos, WorkItem& w) {
  const int b = p.sched[kSchedHead + 2 * pos];
  if (b < 0) return false;
  const int e = p.sched[kSchedHead + 1 + 2 * pos];
  w.split = 0;
  w.b = b;
  w.hkv = e >> 20;
  w.qtile = e & 0xfffff;
  seq_span(p, b, w);
  return true;
}

// This workgroup's item; false: nothing to do.
template <int ROWS>
__device__ __forceinline__ bool work_item(const FwdParams& p, WorkItem& w) {
  if (p.tile_order == kTileOrderTable) return table_item(p, (int)blockIdx.x, w);
  if (p.tile_order == kTileOrderLongestFirst) return longest_first_item<ROWS>(p, w);
  w = p.tile_order == kTileOrderHeadsTogether ? heads_together_item(p) : grouped_item(p);
  return true;
}

// Per-tensor fp8 scale: *ptr, or 1 when ptr is null.  The load is made
// unconditionally (from `fallback`, any readable 4-byte-aligned address, when
// ptr is null) so a kernel's scale loads are issued together and waited for
// once, instead of one dependent round trip each behind a branch.
__device__ __forceinline__ float load_scale(const float* ptr, const void* fallback) {
  const float v = *(ptr ? ptr : (const float*)fallback);
  return ptr ? v : 1.0f;
}

__device__ __forceinline__ float wave_xor_max(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask));
}

// Store 4 consecutive outputs (fp32 values) as out_dtype.
__device__ __forceinline__ void store_out4(char* dst, int out_dtype, f32x4 v) {
  if (out_dtype == DT_F32) {
    *(f32x4*)dst = v;
  } else if (out_dtype == DT_BF16) {
    u32x2 w = {pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
    *(u32x2*)dst = w;
  } else {
    u32x2 w = {pack_f16x2(v.x, v.y), pack_f16x2(v.z, v.w)};
    *(u32x2*)dst = w;
  }
}

template <int DT_, int DQK_, int DV_, int NWM_, int NWK_, int BN_>
struct FwdCfg {
  static constexpr int DT = DT_;
  static constexpr int DQK = DQK_;
  static constexpr int DV = DV_;
  static constexpr int NWM = NWM_;
  static constexpr int NWK = NWK_;
  static constexpr int BN = BN_;
  static constexpr int BYTES = Elem<DT>::bytes;
  static constexpr int VPL = 16 / BYTES;          // elements per 16-byte chunk
  static constexpr int NTHR = 64 * NWM * NWK;
  static constexpr int SB = NWK * BN;             // keys per iteration
  static constexpr int NT = BN / 16;              // S^T tiles per wave
  static constexpr int CQK = DQK * BYTES / 64;    // QK chunks per row
  static constexpr int CPV = BN / (4 * VPL);      // PV chunks per wave
  static constexpr int TV = DV / 16;              // O^T tiles
  static constexpr int KPITCH = DQK * BYTES + 16; // LDS bytes per K row
  static constexpr int VPITCH = SB * BYTES + 16;  // LDS bytes per V^T row
  static constexpr int RK = DQK * BYTES / 16;     // 16-byte chunks per K row
  static constexpr int RV = DV * BYTES / 16;      // 16-byte chunks per V row
  static constexpr int KCH = (SB * RK + NTHR - 1) / NTHR;
  static constexpr int VCH = (SB * RV + NTHR - 1) / NTHR;
  static constexpr int LDS_KV = SB * KPITCH + DV * VPITCH;
  static constexpr int LDS_MERGE = NWK > 1 ? NWM * NWK * (TV * 64 * 16 + 16 * 8) : 0;
  static constexpr int LDS = LDS_KV > LDS_MERGE ? LDS_KV : LDS_MERGE;
  static_assert(DQK * BYTES % 64 == 0, "head_dim_qk bytes must be a multiple of 64");
  static_assert(DV % 16 == 0 && DV * BYTES % 16 == 0, "head_dim_v must be a multiple of 16");
  static_assert(BN % (4 * VPL) == 0 && BN % 16 == 0, "key block must cover whole chunks");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

// Position of key `kl` (0..BN) of a wave's key block inside its V^T row:
// lane group g = (kl%16)/4 owns slots [g*BN/4, (g+1)*BN/4) and slot
// sigma = 4*(kl/16) + kl%4, matching the order of its S^T registers.
template <int BN>
__device__ __forceinline__ int vt_pos(int kl) {
  return ((kl & 15) >> 2) * (BN / 4) + 4 * (kl >> 4) + (kl & 3);
}

template <class C>
__global__ __launch_bounds__(C::NTHR) void fmha_fwd_kernel(FwdParams p) {
  constexpr int DT = C::DT;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  char* Ks = smem;
  char* Vt = smem + C::SB * C::KPITCH;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % C::NWM;
  const int wk = wave / C::NWM;
  const int lg = lane >> 4;   // lane group (contraction slots)
  const int lr = lane & 15;   // query row within the wave tile / MFMA column

  // ---- tile decode: split fastest, then kv head, batch, query tile (reversed,
  // so the heaviest tiles of causal / long sequences are dispatched first)
  WorkItem wi;
  if (!work_item<16 * C::NWM>(p, wi)) return;
  const int S = p.num_splits;
  const int split = wi.split, hkv = wi.hkv, b = wi.b, qtile = wi.qtile;
  const int q_off = wi.q_off, sq = wi.sq, k_off = wi.k_off, sk = wi.sk;
  const int G = p.group;
  const int rows = sq * G;
  const int row0 = qtile * 16 * C::NWM;
  if (row0 >= rows || sk <= 0) return;  // past the sequence or no keys: rows untouched
  const int kb = split * p.chunk;
  if (kb >= sk) return;                 // split beyond this sequence: not read by the combine
  const int ke = S > 1 ? min(kb + p.chunk, sk) : sk;

  // ---- pointers
  const char* kbase = p.k + (p.cu_k ? (int64_t)k_off * p.k_st : (int64_t)b * p.k_sb) + (int64_t)hkv * p.k_sh;
  const char* vbase = p.v + (p.cu_k ? (int64_t)k_off * p.v_st : (int64_t)b * p.v_sb) + (int64_t)hkv * p.v_sh;

  // ---- this lane's query row
  const int r = row0 + 16 * wm + lr;
  const bool row_ok = r < rows;
  const int iq = row_ok ? r / G : 0;
  const int hq = hkv * G + (row_ok ? r % G : 0);

  float scale_log2 = p.scale_log2;
  float v_scale = 1.0f;
  if constexpr (DT == DT_FP8) {
    scale_log2 *= load_scale(p.q_descale, p.q) * load_scale(p.k_descale, p.q);
    v_scale = load_scale(p.v_descale, p.q);
    v_scale *= 1.0f / kFp8PScale;
  }

  // Q^T fragment (B operand): chunk c of row r holds elements [(4c+lg)*VPL, +VPL)
  u32x4 qf[C::CQK];
  {
    const char* qrow = p.q + (p.cu_q ? (int64_t)(q_off + iq) * p.q_st : (int64_t)b * p.q_sb + (int64_t)iq * p.q_st) +
                       (int64_t)hq * p.q_sh;
#pragma unroll
    for (int c = 0; c < C::CQK; ++c) {
      u32x4 z = {0u, 0u, 0u, 0u};
      qf[c] = row_ok ? *(const u32x4*)(qrow + (4 * c + lg) * 16) : z;
    }
  }

  // ---- key ranges.  Row i may use keys [lo(i), hi(i)] (bottom-right aligned
  // causal / window), intersected with this split's [kb, ke).
  const int shift = sk - sq;
  auto lo_of = [&](int i) { return p.wl >= 0 ? max(i + shift - p.wl, 0) : 0; };
  auto hi_of = [&](int i) { return p.wr >= 0 ? min(i + shift + p.wr, sk - 1) : sk - 1; };
  const int last_row = min(row0 + 16 * C::NWM, rows) - 1;
  const int iq_lo = row0 / G, iq_hi = last_row / G;
  const int tile_lo = max(kb, lo_of(iq_lo));
  const int tile_hi = min(ke - 1, hi_of(iq_hi));
  const int full_lo = max(kb, lo_of(iq_hi));   // blocks inside [full_lo, full_hi]
  const int full_hi = min(ke - 1, hi_of(iq_lo)); // need no mask for any row
  const int my_lo = max(kb, lo_of(iq));
  const int my_hi = min(ke - 1, hi_of(iq));
  const int j_begin = (tile_lo / C::SB) * C::SB;
  const int j_end = tile_hi + 1;
  const int n_iter = j_end > j_begin ? (j_end - j_begin + C::SB - 1) / C::SB : 0;

  // ---- running state (lane-major: one query row per lane)
  f32x4 acc[C::TV];
#pragma unroll
  for (int t = 0; t < C::TV; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running max of scaled log2 scores of row r
  float l_run = 0.f;        // this lane's partial row sum

  u32x4 kreg[C::KCH], vreg[C::VCH];
  auto load_block = [&](int j0) {
#pragma unroll
    for (int n = 0; n < C::KCH; ++n) {
      const int ch = tid + n * C::NTHR;
      const int key = ch / C::RK, part = ch % C::RK;
      u32x4 z = {0u, 0u, 0u, 0u};
      const bool ok = ch < C::SB * C::RK && j0 + key < ke;
      kreg[n] = ok ? *(const u32x4*)(kbase + (int64_t)(j0 + key) * p.k_st + part * 16) : z;
    }
#pragma unroll
    for (int n = 0; n < C::VCH; ++n) {
      const int ch = tid + n * C::NTHR;
      const int key = ch / C::RV, part = ch % C::RV;
      u32x4 z = {0u, 0u, 0u, 0u};
      const bool ok = ch < C::SB * C::RV && j0 + key < ke;
      vreg[n] = ok ? *(const u32x4*)(vbase + (int64_t)(j0 + key) * p.v_st + part * 16) : z;
    }
  };
  auto store_block = [&]() {
#pragma unroll
    for (int n = 0; n < C::KCH; ++n) {
      const int ch = tid + n * C::NTHR;
      if (ch < C::SB * C::RK) {
        const int key = ch / C::RK, part = ch % C::RK;
        *(u32x4*)(Ks + key * C::KPITCH + part * 16) = kreg[n];
      }
    }
#pragma unroll
    for (int n = 0; n < C::VCH; ++n) {
      const int ch = tid + n * C::NTHR;
      if (ch < C::SB * C::RV) {
        const int key = ch / C::RV, part = ch % C::RV;
        const int kw = key / C::BN, kl = key % C::BN;
        char* dst = Vt + (part * C::VPL) * C::VPITCH + (kw * C::BN + vt_pos<C::BN>(kl)) * C::BYTES;
        const u32x4 w = vreg[n];
        if constexpr (C::BYTES == 4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) *(uint32_t*)(dst + e * C::VPITCH) = w[e];
        } else if constexpr (C::BYTES == 2) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            *(uint16_t*)(dst + e * C::VPITCH) = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e)
            *(uint8_t*)(dst + e * C::VPITCH) = (uint8_t)(w[e >> 2] >> ((e & 3) * 8));
        }
      }
    }
  };

  if (n_iter > 0) load_block(j_begin);
  for (int it = 0; it < n_iter; ++it) {
    const int j0 = j_begin + it * C::SB;
    if (it > 0) __syncthreads();
    store_block();
    __syncthreads();
    if (it + 1 < n_iter) load_block(j0 + C::SB);

    // S^T tiles of this wave's BN keys
    const int kw0 = wk * C::BN;
    f32x4 s[C::NT];
#pragma unroll
    for (int u = 0; u < C::NT; ++u) s[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < C::CQK; ++c) {
#pragma unroll
      for (int u = 0; u < C::NT; ++u) {
        const u32x4 kf = *(const u32x4*)(Ks + (kw0 + 16 * u + lr) * C::KPITCH + (4 * c + lg) * 16);
        s[u] = mfma_chunk<DT>(s[u], kf, qf[c]);
      }
    }
    // scale to log2 units and mask; lane holds keys j0 + kw0 + 16u + 4*lg + e
    const bool full = j0 >= full_lo && j0 + C::SB - 1 <= full_hi;
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < C::NT; ++u) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = s[u][e] * scale_log2;
        if (!full) {
          const int j = j0 + kw0 + 16 * u + 4 * lg + e;
          if (j < my_lo || j > my_hi) x = -INFINITY;
        }
        s[u][e] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = wave_xor_max(mx, 16);
    mx = wave_xor_max(mx, 32);
    const float m_new = fmaxf(m_run, mx);
    const float base = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - base);
    float rs = 0.f;
#pragma unroll
    for (int u = 0; u < C::NT; ++u) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pe = fast_exp2(s[u][e] - base);
        s[u][e] = pe;
        rs += pe;
      }
    }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < C::TV; ++t) acc[t] *= alpha;
    // O^T += V^T P^T
#pragma unroll
    for (int c = 0; c < C::CPV; ++c) {
      const u32x4 pf = pack_p<DT>(&s[c * C::VPL / 4]);
#pragma unroll
      for (int t = 0; t < C::TV; ++t) {
        const u32x4 vf = *(const u32x4*)(Vt + (16 * t + lr) * C::VPITCH +
                                         (kw0 + lg * (C::BN / 4) + c * C::VPL) * C::BYTES);
        acc[t] = mfma_chunk<DT>(acc[t], vf, pf);
      }
    }
  }

  // ---- epilogue: row sums across the 4 lane groups, then merge the NWK waves
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  float M = m_run, L = l_tot;
  // with NWK > 1, wave wk finishes the O^T tiles t with t % NWK == wk
  if constexpr (C::NWK > 1) {
    __syncthreads();  // K/V staging no longer read
    float* accbuf = (float*)smem;
    float* mlbuf = (float*)(smem + C::NWM * C::NWK * C::TV * 64 * 16);
    const int wslot = wm * C::NWK + wk;
#pragma unroll
    for (int t = 0; t < C::TV; ++t) *(f32x4*)(accbuf + ((wslot * C::TV + t) * 64 + lane) * 4) = acc[t];
    if (lg == 0) {
      mlbuf[(wslot * 16 + lr) * 2 + 0] = m_run;
      mlbuf[(wslot * 16 + lr) * 2 + 1] = l_tot;
    }
    __syncthreads();
    float mk[C::NWK], lk[C::NWK];
    M = -INFINITY;
#pragma unroll
    for (int k = 0; k < C::NWK; ++k) {
      mk[k] = mlbuf[((wm * C::NWK + k) * 16 + lr) * 2 + 0];
      lk[k] = mlbuf[((wm * C::NWK + k) * 16 + lr) * 2 + 1];
      M = fmaxf(M, mk[k]);
    }
    const float Mb = M == -INFINITY ? 0.f : M;
    L = 0.f;
    float w[C::NWK];
#pragma unroll
    for (int k = 0; k < C::NWK; ++k) {
      w[k] = fast_exp2(mk[k] - Mb);
      L += w[k] * lk[k];
    }
#pragma unroll
    for (int t = 0; t < C::TV; ++t) {
      if (t % C::NWK != wk) continue;
      f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < C::NWK; ++k)
        o += w[k] * *(const f32x4*)(accbuf + (((wm * C::NWK + k) * C::TV + t) * 64 + lane) * 4);
      acc[t] = o;
    }
  }
  if (!row_ok) return;
  const bool live = L > 0.f;
  const float inv = live ? v_scale / L : 0.f;
  const float lse_v = live ? (M + __log2f(L)) * kLn2 : -INFINITY;
  const int dv_lane = 4 * lg;
  if (S > 1) {
    const int64_t tglob = (int64_t)q_off + iq;
    float* op = p.o_part + (((int64_t)split * p.total_q + tglob) * p.hq + hq) * C::DV + dv_lane;
#pragma unroll
    for (int t = 0; t < C::TV; ++t)
      if (t % C::NWK == wk) *(f32x4*)(op + 16 * t) = acc[t] * inv;
    if (lg == 0 && wk == 0) p.lse_part[((int64_t)split * p.hq + hq) * p.total_q + tglob] = lse_v;
  } else {
    char* op = p.o + (p.cu_q ? (int64_t)(q_off + iq) * p.o_st : (int64_t)b * p.o_sb + (int64_t)iq * p.o_st) +
               (int64_t)hq * p.o_sh;
    const int ob = p.out_dtype == DT_F32 ? 4 : 2;
#pragma unroll
    for (int t = 0; t < C::TV; ++t)
      if (t % C::NWK == wk) store_out4(op + (16 * t + dv_lane) * ob, p.out_dtype, acc[t] * inv);
    if (p.lse && lg == 0 && wk == 0) {
      const int64_t li = p.cu_q ? (int64_t)hq * p.lse_sh + q_off + iq : (int64_t)b * p.lse_sb + (int64_t)hq * p.lse_sh + iq;
      p.lse[li] = lse_v;
    }
  }
}

template <class C>
hipError_t launch_fwd(const FwdParams& p, int64_t grid, hipStream_t stream) {
  hipLaunchKernelGGL(fmha_fwd_kernel<C>, dim3((uint32_t)grid), dim3(C::NTHR), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fmha
