// Prefill kernel for gfx950: many query rows per (sequence, kv head), so the
// work is a dense contraction on MFMA.  One workgroup = NWM waves x 32 query
// rows; per key block of BN keys every wave runs
//   S^T[key, row] = K Q^T       (v_mfma_f32_32x32x16_{f16,bf16}, A = K, B = Q^T)
//   O^T[dv, row] += V^T P^T     (A = V^T via ds_read_b64_tr_b16, B = P^T)
// with the online exp2 softmax in between (flash attention forward; web pages
// on split-KV flash attention: "Adds variable sequence lengths to the Hopper
// CuTe DSL FMHA example", sections Implementation and Performance, for the
// varlen grid, masks and row-predicated stores).
//
// 32x32 tiles halve the LDS bytes read per MFMA flop compared with 16x16
// tiles (each K/V fragment feeds 32 query rows).  In the 32x32 output layout
// lane l owns query row l%32 and 16 of the 32 keys of a tile (the other 16
// sit in lane l^32), so a row reduction is 15 local steps plus one exchange
// with the partner lane, and P^T feeds the second MFMA from registers.
//
// K and V blocks move HBM -> LDS with buffer loads that write LDS directly
// (16 bytes per lane, no register staging), rows unpadded with an XOR chunk
// swizzle that keeps both the 16-byte K reads and the V transpose reads free
// of bank conflicts.  K and V each have a ring of four LDS stages: iteration n
// issues K(n+4) and V(n+2) and uses K(n+1) and V(n-1), so the loads of the
// two previous iterations may still be in flight; one barrier per block.
//
// Two loop forms.  The pipelined one (head dim 256: one workgroup per CU):
// iteration n runs PV(n-1) on the MFMA pipe while the VALU takes the row max
// of block n, then QK(n+1) on the MFMA pipe while the VALU takes the
// exponentials of block n; the MFMAs and the VALU work are interleaved in
// chunks inside each wave, so both pipes stay busy even when the other wave
// on the SIMD is stalled.  The simple one (head dims 64 and 128):
// three workgroups per CU on three-stage rings, so each SIMD holds three
// waves of different workgroups, and each wave runs QK(n), the softmax of
// block n and PV(n) in turn with a single S and P buffer (168 registers or
// fewer): the other waves fill one wave's gaps.  Paired timing: equal on
// unmasked 8 x 2048 at D = 128, 4-10 % faster causal, 10-13 % faster at
// D = 64.
//
// Softmax bookkeeping uses a lazily moved reference max per row: p =
// exp2(scale*s - m_ref), with m_ref set from the first key block and moved
// (O and l rescaled by exp2(m_ref_old - m_ref_new), the block's p recomputed)
// only when a lane's sum of p over a block exceeds 2^12 or a row with keys in
// the block has no reference yet.  O and l are accumulated against the same
// m_ref, so O = acc / l and LSE = m_ref + log2 l are exact; p <= 2^12 keeps
// fp16/bf16 P far inside their range.
#pragma once
#include "fmha_decode_kernel.h"
#include "fmha_fused_combine.h"
#include "fmha_fwd_kernel.h"

namespace fmha {

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int DT>
__device__ __forceinline__ f32x16 mfma32(f32x16 acc, u32x4 a, u32x4 b) {
  if constexpr (DT == DT_F16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), acc,
                                                  0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   acc, 0, 0, 0);
  }
}

template <int DT>
__device__ __forceinline__ uint32_t pack2_in(float a, float b) {
  if constexpr (DT == DT_F16)
    return pack_f16x2(a, b);
  else
    return pack_bf16x2(a, b);
}

// P for the PV MFMA, rounded to nearest even: the row sum adds the unrounded
// fp32 p, so the rounding error of P averages out instead of biasing O (one
// conversion instruction per pair for either type)
template <int DT>
__device__ __forceinline__ uint32_t pack2_p(float a, float b) {
  return pack2_in<DT>(a, b);
}

template <int DT_, int D_, int NWM_, int BN_, int RT_, bool PP_ = false, int WGS_ = 0>
struct PfCfg {
  static constexpr int DT = DT_;
  static constexpr int D = D_;          // Dqk == Dv
  static constexpr int NWM = NWM_;      // waves
  // two wave groups alternating MFMA and softmax phases (NWM = 8; paired
  // timing: 3-33 % slower than two free-running 4-wave workgroups per CU, so
  // no instance uses it)
  static constexpr bool PP = PP_;
  static constexpr int RT = RT_;        // 32-row tiles per wave (each K/V fragment feeds RT MFMAs)
  static constexpr int BN = BN_;        // keys per block
  static constexpr int NTHR = 64 * NWM;
  static constexpr int ROWS = 32 * NWM * RT;
  static constexpr int KS = D / 16;     // k-steps of QK (16 d each)
  static constexpr int NT = BN / 32;    // S^T tiles (32 keys each)
  static constexpr int TV = D / 32;     // O^T tiles (32 dv each)
  static constexpr int NG = 2 * NT;     // PV groups (16 keys each)
  static constexpr int ROWB = D * 2;    // bytes per K / V row (unpadded, swizzled)
  static constexpr int RPL = 1024 / ROWB;          // rows per 1 KiB direct-to-LDS load
  static constexpr int TILE = BN * ROWB;           // one K or V block in LDS
  static constexpr int KL = TILE / 1024 / NWM;     // 1 KiB loads per wave per K (or V) block
  // WGS > 0: the simple loop form with WGS workgroups per CU (WGS waves per
  // SIMD) on NS-stage rings, without the cross-block software pipeline (QK,
  // softmax and PV of one block in turn; the other waves of the SIMD fill
  // the gaps); 0: the pipelined form on four-stage rings
  static constexpr int WGS = WGS_;
  static constexpr bool SIMPLE = WGS > 0;          // the simple loop form
  static constexpr int NS = WGS == 0 ? 4 : (WGS >= 3 ? 3 : 2);  // ring depth, K and V each
  static constexpr int LDS = 2 * NS * TILE;
  // two waves per SIMD (one for RT = 2, or when two rings do not fit the
  // 160 KiB of LDS: D = 256 runs one wave per SIMD with all 512 registers)
  static constexpr int MIN_BLOCKS = SIMPLE ? WGS : 2 * LDS > 160 * 1024 ? 1 : (RT == 1 ? 8 : 4) / NWM;
  static_assert(D % 32 == 0 && BN % 32 == 0, "tile sizes");
  static_assert(1024 % ROWB == 0 && KL >= 1 && KL * NWM * 1024 == TILE, "whole 1 KiB loads per wave");
  static_assert(TILE % 256 == 0, "stage offsets keep the low address bits");
  static_assert(!PP || (NWM % 2 == 0 && ROWB != 512), "two equal groups; loads issued in one burst");
  static_assert(!SIMPLE || (!PP && WGS * LDS <= 160 * 1024), "WGS rings per CU");
};

// 16-byte chunk c of row r sits at chunk slot c ^ swz(r) (an XOR on the low
// bits, so it is its own inverse).  Chosen so that both LDS read patterns are
// free of bank conflicts whether the LDS serves 128 or 256 bytes per pass:
//  * K (16-byte A-operand reads): 16 consecutive rows at one chunk;
//  * V (transpose reads): 4 consecutive rows x 4 adjacent chunks per 32 lanes.
template <int ROWB>
__device__ __forceinline__ int k_slot(int r, int c) {
  if constexpr (ROWB >= 256) return c ^ (r & 15);
  else return c ^ ((r ^ (r >> 3)) & 7);
}
template <int ROWB>
__device__ __forceinline__ int v_slot(int r, int c) {
  const int e = r & 3;
  if constexpr (ROWB >= 256) return c ^ (4 * e + 2 * (e >> 1));
  else return c ^ (2 * e);
}

// One 16-byte-per-lane buffer load that writes LDS at lds + 16 * lane.  The
// descriptors cover one key block (rows past its last valid key read as 0),
// so their 32-bit size never wraps.
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t rsrc, char* lds, int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 16, voffset, 0, 0, 0);
}


// Workgroup barrier without the memory-model fences of __syncthreads(): its
// release fence makes the compiler wait for every buffer->LDS load in flight
// (vmcnt(0)), which would drain the load ring at every key block.  The
// kernels wait for the loads a block needs themselves (vmcnt with a count)
// and complete their LDS reads (lgkmcnt) before each barrier; the empty asm
// statements keep the compiler from moving memory operations across it.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---- LDS reads as inline assembly
// The compiler's wait-counter pass cannot tell an LDS read from one that
// aliases a pending buffer->LDS load, so it puts a full vmcnt(0) in front of
// such reads: the MFMAs would then wait for the loads of the next key blocks.
// These kernels order their direct-to-LDS loads themselves (explicit vmcnt
// waits before each block barrier), so the K and V^T fragment reads are
// issued as asm.  The compiler does not count them, so they are completed with
// lgkm_wait<N>() followed by tie() on every loaded register: tie's "+v"
// operand makes each consumer come after the wait.  Counting stays correct
// whatever else the compiler interleaves: LDS operations retire in order, and
// extra operations only make a count-based wait stricter.  tie() on a
// computed value also pins the computation before that point (volatile asm
// keeps its order), which stops the compiler from sinking VALU work meant to
// overlap the MFMAs into the block that consumes it.
template <int... I>
struct int_seq {};
template <int N, int... I>
struct make_int_seq : make_int_seq<N - 1, N - 1, I...> {};
template <int... I>
struct make_int_seq<0, I...> {
  using type = int_seq<I...>;
};
template <int V>
struct int_c {
  static constexpr int value = V;
};
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, int_seq<I...>) {
  (f(int_c<I>{}), ...);
}
// f(int_c<0>{}), ..., f(int_c<N-1>{}): loop indices usable as constants
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, typename make_int_seq<N>::type{});
}

__device__ __forceinline__ uint32_t lds_addr(const void* ptr) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)ptr;
}
template <int OFF>
__device__ __forceinline__ i32x2 lds_tr16(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  i32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ i32x2 lds_tr8(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  i32x2 r;
  asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
template <int N>
__device__ __forceinline__ void lgkm_wait() {
  static_assert(N >= 0 && N < 16, "lgkmcnt");
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N));
}
template <int OFF>
__device__ __forceinline__ u32x4 lds_b128(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
__device__ __forceinline__ void tie(i32x2& r) { asm volatile("" : "+v"(r)); }
__device__ __forceinline__ void tie(u32x4& r) { asm volatile("" : "+v"(r)); }
__device__ __forceinline__ void tie(float& r) { asm volatile("" : "+v"(r)); }
__device__ __forceinline__ void tie(uint32_t& r) { asm volatile("" : "+v"(r)); }
// max over the two 32-lane halves of the wave (lane i and lane i ^ 32)
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Read schedule of the interleaved PV/QK phase: reads are numbered in the
// order MFMA j = 0, 1, ... (PV n = j / 2 for even j, QK n for odd j) needs
// them, three per fragment pair (two V transpose reads, one K read).
constexpr int kPvqkAhead = 6;  // reads issued beyond the ones the next MFMA needs (3..15 timed: 6 best by ~1 %)
// reads that must have completed before MFMA j
constexpr int pvqk_need(int j) { return 3 * (j / 2) + (j % 2 ? 3 : 2); }
// reads issued before MFMA j
constexpr int pvqk_issued(int j, int nr) { return pvqk_need(j) + kPvqkAhead < nr ? pvqk_need(j) + kPvqkAhead : nr; }

// One tile (work item wi) with the workgroup's LDS at smem.
template <class C>
__device__ __forceinline__ void prefill_tile(const FwdParams& p, const WorkItem& wi, char* smem) {
  constexpr int DT = C::DT;
  constexpr int RT = C::RT;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wm = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int hl = lane >> 5;   // lane half: contraction slots / output row group
  const int lr = lane & 31;   // query row within a 32-row tile / MFMA column

  const int S = p.num_splits;
  const int split = wi.split, hkv = wi.hkv, b = wi.b, qtile = wi.qtile;
  const int q_off = wi.q_off, sq = wi.sq, k_off = wi.k_off, sk = wi.sk;
  const int G = p.group;
  const int rows = sq * G;
  const int row0 = qtile * C::ROWS;
  if (row0 >= rows || sk <= 0) return;  // past the sequence or no keys: rows untouched
  const int kb = split * p.chunk;
  if (kb >= sk) return;                 // split beyond this sequence: not read by the combine
  const int ke = S > 1 ? min(kb + p.chunk, sk) : sk;

  // ---- pointers
  const char* kbase = p.k + (p.cu_k ? (int64_t)k_off * p.k_st : (int64_t)b * p.k_sb) + (int64_t)hkv * p.k_sh;
  const char* vbase = p.v + (p.cu_k ? (int64_t)k_off * p.v_st : (int64_t)b * p.v_sb) + (int64_t)hkv * p.v_sh;

  // ---- this lane's query rows: one per 32-row tile rt of the wave
  int iq[RT], hq[RT];
  bool row_ok[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = row0 + 32 * (RT * wm + rt) + lr;
    row_ok[rt] = r < rows;
    iq[rt] = row_ok[rt] ? r / G : 0;
    hq[rt] = hkv * G + (row_ok[rt] ? r % G : 0);
  }

  // Q^T (B operand): k-step s, lane half h holds d = 16s + 8h .. +8.  A lane
  // past the tile's rows reads row 0's Q: its results are never stored, and
  // leaving its Q unmasked keeps the prologue from waiting on the Q loads.
  u32x4 qf[RT][C::KS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const char* qrow = p.q + (p.cu_q ? (int64_t)(q_off + iq[rt]) * p.q_st : (int64_t)b * p.q_sb + (int64_t)iq[rt] * p.q_st) +
                       (int64_t)hq[rt] * p.q_sh;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) qf[rt][s] = *(const u32x4*)(qrow + (16 * s + 8 * hl) * 2);
  }
  const float scale_log2 = p.scale_log2;

  const int shift = sk - sq;
  auto lo_of = [&](int i) { return p.wl >= 0 ? max(i + shift - p.wl, 0) : 0; };
  auto hi_of = [&](int i) { return p.wr >= 0 ? min(i + shift + p.wr, sk - 1) : sk - 1; };
  const int last_row = min(row0 + C::ROWS, rows) - 1;
  const int iq_lo = row0 / G, iq_hi = last_row / G;
  // the tile's key ranges are uniform; readfirstlane keeps them (and the
  // buffer descriptors built from them) in scalar registers
  const int tile_lo = __builtin_amdgcn_readfirstlane(max(kb, lo_of(iq_lo)));
  const int tile_hi = __builtin_amdgcn_readfirstlane(min(ke - 1, hi_of(iq_hi)));
  const int full_lo = __builtin_amdgcn_readfirstlane(max(kb, lo_of(iq_hi)));
  const int full_hi = __builtin_amdgcn_readfirstlane(min(ke - 1, hi_of(iq_lo)));
  int my_lo[RT], my_hi[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    my_lo[rt] = max(kb, lo_of(iq[rt]));
    my_hi[rt] = min(ke - 1, hi_of(iq[rt]));
  }
  const int j_begin = (tile_lo / C::BN) * C::BN;
  const int j_end = tile_hi + 1;
  const int n_iter = j_end > j_begin ? (j_end - j_begin + C::BN - 1) / C::BN : 0;

  f32x16 acc[RT][C::TV];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int t = 0; t < C::TV; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[rt][t][e] = 0.f;
  float m_run[RT], l_run[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.f;
  }

  // One K (or V) block = NWM * KL buffer->LDS loads of 1 KiB (RPL rows each);
  // wave wm issues loads [wm*KL, (wm+1)*KL).  Lane l of a load writes LDS
  // bytes [16l, 16l+16) of it, i.e. slot l % (ROWB/16) of row l / (ROWB/16),
  // so it fetches the chunk that belongs in that slot.  Its byte offset from
  // the block's first row is a loop constant; the block base goes into the
  // buffer descriptor, whose size ends at the last row the tile needs, so rows
  // past it read as zero, and a block past it gets an empty descriptor
  // (nothing is fetched).  Every wave issues the same number of loads per
  // block, so the loads in flight are a compile-time count.
  constexpr int CPR = C::ROWB / 16;  // chunks per row
  int kld_off[C::KL], vld_off[C::KL];
#pragma unroll
  for (int n = 0; n < C::KL; ++n) {
    const int lrow = (wm * C::KL + n) * C::RPL + lane / CPR;
    kld_off[n] = lrow * (int)p.k_st + k_slot<C::ROWB>(lrow, lane % CPR) * 16;
    vld_off[n] = lrow * (int)p.v_st + v_slot<C::ROWB>(lrow, lane % CPR) * 16;
  }
  const uint32_t lds0 = lds_addr(smem);
  // K fragment read addresses: k-step k of tile u (row 32u + lr) sits at
  // (kaddr[u] ^ 32k) within a stage (the swizzle only touches bits 5..7); the
  // stage offset is an immediate
  // (512-byte rows: the same XORs; the k-step and row fields stay disjoint)
  static_assert(C::ROWB == 512 || C::ROWB == 256 || C::ROWB == 128, "swizzles");
  uint32_t kx[C::NT][C::KS];
#pragma unroll
  for (int u = 0; u < C::NT; ++u) {
    const int kaddr = (32 * u + lr) * C::ROWB + k_slot<C::ROWB>(32 * u + lr, hl) * 16;
#pragma unroll
    for (int k = 0; k < C::KS; ++k) kx[u][k] = lds0 + (uint32_t)(kaddr ^ (32 * k));
  }
  // V^T read address of this lane for O^T tile t (dv 32t..) within a stage is
  // vaddr ^ 64t; stage and row steps are immediates
  const int e4 = (lane >> 2) & 3, jq = lane & 3, grp = (lane >> 4) & 1;
  const int vaddr = (4 * hl + e4) * C::ROWB + v_slot<C::ROWB>(e4, 2 * grp + (jq >> 1)) * 16 + 8 * (jq & 1);
  uint32_t vx[C::TV];
#pragma unroll
  for (int t = 0; t < C::TV; ++t) vx[t] = lds0 + (uint32_t)(C::NS * C::TILE + (vaddr ^ (64 * t)));

  // No LDS initialisation: every K and V slot of a stage is written by the
  // block's loads (rows past the tile's range and blocks past it as zeros)
  // before any wave reads it, so the prologue's loads go out at once.

  // descriptor of key block jb: rows [jb, min(jb + BN, j_end)) of K or V
  // (all uniform: built in scalar registers)
  auto block_rsrc = [&](const char* base, int64_t st, int jb) {
    const int rows_left = min(j_end - jb, C::BN);
    const int nb = rows_left > 0 ? (rows_left - 1) * (int)st + C::ROWB : 0;
    return make_rsrc(base + (int64_t)jb * st, nb);
  };
  auto issue_k = [&](int jb, auto ST_) {
    constexpr int ST = decltype(ST_)::value;
    const __amdgpu_buffer_rsrc_t rk = block_rsrc(kbase, p.k_st, jb);
#pragma unroll
    for (int n = 0; n < C::KL; ++n) buffer_to_lds16(rk, smem + ST * C::TILE + (wm * C::KL + n) * 1024, kld_off[n]);
  };
  auto issue_v = [&](int jb, auto ST_) {
    constexpr int ST = decltype(ST_)::value;
    const __amdgpu_buffer_rsrc_t rv = block_rsrc(vbase, p.v_st, jb);
#pragma unroll
    for (int n = 0; n < C::KL; ++n)
      buffer_to_lds16(rv, smem + (C::NS + ST) * C::TILE + (wm * C::KL + n) * 1024, vld_off[n]);
  };
  // at most `n` of this wave's loads in flight (they retire in order)
  auto wait_loads = [](auto N_) {
    constexpr int n = decltype(N_)::value;
    static_assert(n < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
  };

  // P of a key block, packed for the PV MFMA (group g: keys 16g..16g+15):
  // pbuf[it % 2] holds P(it), so P(it) is produced while PV(it-1) still reads
  // P(it-1)
  u32x4 pbuf[2][RT][C::NG];

  // O^T += V^T P^T for one key block from V stage VST with P from pb.  Lane
  // 4e+jq of 16-lane group (hl, grp) reads row 16g+8q+4hl+e, columns
  // 32t+16grp+4jq..+3, and receives column lr of those 4 rows.  Fragment n =
  // (group g, tile t) takes two reads, issued up to PA fragments ahead (all
  // of them up front when NM <= PA + 1); it feeds one MFMA per row tile, which
  // waits only for its own two reads; `between(n)` is VALU work placed after
  // fragment n's MFMAs.
  auto pv = [&](auto VST_, const u32x4 (&pb)[RT][C::NG], auto&& between) {
    constexpr int VST = decltype(VST_)::value;
    constexpr int NM = C::NG * C::TV;
    constexpr int PA = 7;  // fragments in flight beyond the one consumed: lgkmcnt <= 14
    i32x2 vr[NM][2];
    auto read_v = [&](auto N_) {
      constexpr int n = decltype(N_)::value, g = n / C::TV, t = n % C::TV;
      vr[n][0] = lds_tr16<VST * C::TILE + (16 * g) * C::ROWB>(vx[t]);
      vr[n][1] = lds_tr16<VST * C::TILE + (16 * g + 8) * C::ROWB>(vx[t]);
    };
    static_for<(NM < PA + 1 ? NM : PA + 1)>([&](auto N_) { read_v(N_); });
    static_for<NM>([&](auto N_) {
      constexpr int n = decltype(N_)::value, g = n / C::TV, t = n % C::TV;
      if constexpr (n > 0 && n + PA < NM) read_v(int_c<n + PA>{});
      // fragments issued after n: min(PA, NM - 1 - n), two reads each
      lgkm_wait<2 * (NM - 1 - n < PA ? NM - 1 - n : PA)>();
      tie(vr[n][0]);
      tie(vr[n][1]);
      const u32x4 vf = {(uint32_t)vr[n][0].x, (uint32_t)vr[n][0].y, (uint32_t)vr[n][1].x, (uint32_t)vr[n][1].y};
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt][t] = mfma32<DT>(acc[rt][t], vf, pb[rt][g]);
      between(int_c<n>{});
    });
  };

  // S^T = K Q^T for one key block from K stage KST into sd, tile-major, one
  // K fragment per chunk feeding one MFMA per row tile; fragment n comes from
  // slot n % KR of a ring filled KR - 1 fragments ahead; `between(n)` is VALU
  // work placed after fragment n's MFMAs.
  auto qk = [&](auto KST_, f32x16 (&sd)[RT][C::NT], auto&& between) {
    constexpr int KST = decltype(KST_)::value;
    constexpr int NM = C::NT * C::KS;
    constexpr int KR = 5;
    u32x4 kf[KR];
    auto read_k = [&](auto N_) {
      constexpr int n = decltype(N_)::value, u = n / C::KS, k = n % C::KS;
      kf[n % KR] = lds_b128<KST * C::TILE>(kx[u][k]);
    };
    static_for<KR - 1>([&](auto N_) {
      if constexpr (decltype(N_)::value < NM) read_k(N_);
    });
    static_for<NM>([&](auto N_) {
      constexpr int n = decltype(N_)::value, u = n / C::KS, k = n % C::KS;
      if constexpr (n + KR - 1 < NM) read_k(int_c<n + KR - 1>{});
      // reads issued after fragment n: min(KR - 1, NM - 1 - n)
      lgkm_wait<(NM - 1 - n < KR - 1 ? NM - 1 - n : KR - 1)>();
      tie(kf[n % KR]);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        if constexpr (k == 0) {
          f32x16 z;
#pragma unroll
          for (int e = 0; e < 16; ++e) z[e] = 0.f;
          sd[rt][u] = mfma32<DT>(z, kf[n % KR], qf[rt][k]);
        } else {
          sd[rt][u] = mfma32<DT>(sd[rt][u], kf[n % KR], qf[rt][k]);
        }
      }
      between(int_c<n>{});
    });
  };
  auto nothing = [](auto) {};

  // PV(it-1) and QK(it+1) of one iteration interleaved on the MFMA pipe, in
  // the order PV0 QK0 PV1 QK1 ...: the QK accumulation chain (one S^T tile,
  // KS dependent MFMAs) and the PV chains fill each other's latency, and the
  // LDS reads are issued in the order the MFMAs consume them (PV fragment n =
  // two transpose reads, QK fragment n = one read), kPvqkAhead reads ahead of
  // need, each MFMA waiting only for its own reads.  `between(j)` is VALU
  // work placed after MFMA j.
  auto pvqk = [&](auto VST_, const u32x4 (&pb)[RT][C::NG], auto KST_, f32x16 (&sd)[RT][C::NT], auto&& between) {
    constexpr int VST = decltype(VST_)::value, KST = decltype(KST_)::value;
    constexpr int NM = C::NG * C::TV;
    static_assert(NM == C::NT * C::KS, "as many PV as QK fragments");
    constexpr int NR = 3 * NM;
    i32x2 vr[NM][2];
    u32x4 kf[NM];
    auto issue = [&](auto R_) {
      constexpr int r = decltype(R_)::value, n = r / 3, kind = r % 3;
      if constexpr (kind < 2) {
        constexpr int g = n / C::TV, t = n % C::TV;
        vr[n][kind] = lds_tr16<VST * C::TILE + (16 * g + 8 * kind) * C::ROWB>(vx[t]);
      } else {
        constexpr int u = n / C::KS, k = n % C::KS;
        kf[n] = lds_b128<KST * C::TILE>(kx[u][k]);
      }
    };
    static_for<pvqk_issued(0, NR)>([&](auto R_) { issue(R_); });
    static_for<2 * NM>([&](auto J_) {
      constexpr int j = decltype(J_)::value, n = j / 2;
      if constexpr (j > 0) {
        constexpr int from = pvqk_issued(j - 1, NR);
        static_for<pvqk_issued(j, NR) - from>([&](auto D_) { issue(int_c<from + decltype(D_)::value>{}); });
      }
      lgkm_wait<pvqk_issued(j, NR) - pvqk_need(j)>();
      if constexpr (j % 2 == 0) {
        constexpr int g = n / C::TV, t = n % C::TV;
        tie(vr[n][0]);
        tie(vr[n][1]);
        const u32x4 vf = {(uint32_t)vr[n][0].x, (uint32_t)vr[n][0].y, (uint32_t)vr[n][1].x, (uint32_t)vr[n][1].y};
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt][t] = mfma32<DT>(acc[rt][t], vf, pb[rt][g]);
      } else {
        constexpr int u = n / C::KS, k = n % C::KS;
        tie(kf[n]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          if constexpr (k == 0) {
            f32x16 z;
#pragma unroll
            for (int e = 0; e < 16; ++e) z[e] = 0.f;
            sd[rt][u] = mfma32<DT>(z, kf[n], qf[rt][k]);
          } else {
            sd[rt][u] = mfma32<DT>(sd[rt][u], kf[n], qf[rt][k]);
          }
        }
      }
      between(int_c<j>{});
    });
  };

  // Ring of NS = 4 stages for K and for V: K(b) in K stage b%4, V(b) in V
  // stage b%4.  Iteration it issues K(it+4) and V(it+2) and needs K(it+1)
  // (QK) and V(it-1) (PV), both issued three iterations back: the loads of
  // the two previous iterations may stay in flight.  The prologue issues in
  // the same order as iterations -4..-1 would (with empty loads for V(-2) and
  // V(-1)), so the count is uniform.
  static_assert(C::NS == 4 || C::SIMPLE, "ring schedule");
  f32x16 sbuf[2][RT][C::NT];  // S of block it in sbuf[it % 2]
  const int jlast = j_begin + n_iter * C::BN;  // first block past the tile's range
  if constexpr (!C::SIMPLE) if (n_iter > 0) {
    issue_k(j_begin, int_c<0>{});
    issue_v(jlast, int_c<2>{});  // empty
    issue_k(j_begin + C::BN, int_c<1>{});
    issue_v(jlast, int_c<3>{});  // empty
    issue_k(j_begin + 2 * C::BN, int_c<2>{});
    issue_v(j_begin, int_c<0>{});
    issue_k(j_begin + 3 * C::BN, int_c<3>{});
    issue_v(j_begin + C::BN, int_c<1>{});
    wait_loads(int_c<7 * C::KL>{});  // K(0) landed
    block_barrier();
    qk(int_c<0>{}, sbuf[0], nothing);
  }

  // Softmax with a lazily moved reference: the first block sets each row's
  // reference m_run from its max; later blocks take p = exp2(scale*s - m_run)
  // without a max and check afterwards, from the row sums, that no p exceeded
  // kSumLimit (every p <= the sum) and that no row with keys in the block is
  // still without a reference.  Only then (rare) is the row max taken, O and l
  // rescaled, and the block's exponentials recomputed.  The row sum adds the
  // fp32 p (the LSE needs them unrounded).
  constexpr float kSumLimit = 4096.0f;  // 2^12: P stays far inside fp16 range
  constexpr int NPV = C::NG * C::TV, NQK = C::NT * C::KS;  // fragments per phase
  constexpr int NWD = 8 * C::NT;                           // packed P words per block and row tile
  auto exp_word = [&](const f32x16 (&sd)[C::NT], u32x4 (&pb)[C::NG], float nb, float& rs, auto W_) {
    constexpr int w = decltype(W_)::value, i = 2 * w;  // elements i, i + 1
    float p0 = fast_exp2(__builtin_fmaf(sd[i >> 4][i & 15], scale_log2, nb));
    float p1 = fast_exp2(__builtin_fmaf(sd[(i + 1) >> 4][(i + 1) & 15], scale_log2, nb));
    uint32_t word = pack2_p<DT>(p0, p1);
    tie(word);
    pb[w >> 2][w & 3] = word;
    rs += p0 + p1;
    tie(rs);
  };
  // words of P (all row tiles, RT * NWD) done after VALU slot k of NPV + NQK
  // slots (spread evenly)
  auto words_upto = [](int k) { return (k * RT * NWD) / (NPV + NQK); };

  // two-group variant: group 1 runs one barrier behind group 0
  const bool pp_late = C::PP && wm >= C::NWM / 2;

  // ST = it % 4 at compile time: every LDS stage offset is an immediate.
  // FIRST: it == 0 (no PV of a previous block; the reference is set from the
  // block max).  The last iteration also runs QK of the block after the tile
  // (an empty, zero-filled stage) and drops it.
  auto body = [&](auto ST_, auto FIRST_, int it) {
    constexpr int ST = decltype(ST_)::value;
    constexpr int SB = ST & 1;
    constexpr bool FIRST = decltype(FIRST_)::value != 0;
    const int j0 = j_begin + it * C::BN;
    // K(it+1), V(it-1) landed everywhere; every wave is done with K stage ST
    // (QK(it)) and V stage (it+2)%4 (PV(it-2))
    wait_loads(int_c<4 * C::KL>{});
    block_barrier();
    // this iteration's loads: K(it+4) into stage ST and V(it+2) into stage
    // (ST+2)%4, both freed by the barrier.  With one wave per SIMD (the
    // 512-byte rows) they go out one per few MFMA slots, so their issue
    // overlaps the MFMAs; with two, in one burst here, which starts them
    // earlier while the other workgroup's wave keeps the SIMD busy (paired
    // timing: spreading them was 3 % slower at D = 128, 1.7 % faster at 256)
    constexpr bool kSpread = C::ROWB == 512;
    const __amdgpu_buffer_rsrc_t rk = block_rsrc(kbase, p.k_st, j0 + 4 * C::BN);
    const __amdgpu_buffer_rsrc_t rv = block_rsrc(vbase, p.v_st, j0 + 2 * C::BN);
    if constexpr (!kSpread) {
      issue_k(j0 + 4 * C::BN, int_c<ST>{});
      issue_v(j0 + 2 * C::BN, int_c<(ST + 2) % 4>{});
    }
    auto load_slot = [&](auto K_) {
      constexpr int k = decltype(K_)::value, NL = 2 * C::KL, NSL = NPV + NQK;
      static_for<NL>([&](auto I_) {
        constexpr int i = decltype(I_)::value;
        if constexpr (kSpread && (i * NSL) / NL == k) {
          if constexpr (i < C::KL)
            buffer_to_lds16(rk, smem + ST * C::TILE + (wm * C::KL + i) * 1024, kld_off[i]);
          else
            buffer_to_lds16(rv, smem + (C::NS + (ST + 2) % 4) * C::TILE + (wm * C::KL + i - C::KL) * 1024,
                            vld_off[i - C::KL]);
        }
      });
    };
    f32x16 (&s)[RT][C::NT] = sbuf[SB];
    u32x4 (&pc)[RT][C::NG] = pbuf[SB];

    const bool full = j0 >= full_lo && j0 + C::BN - 1 <= full_hi;
    if (!full) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int u = 0; u < C::NT; ++u)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int j = j0 + 32 * u + 8 * (e >> 2) + 4 * hl + (e & 3);
            if (j < my_lo[rt] || j > my_hi[rt]) s[rt][u][e] = -INFINITY;
          }
    }
    auto row_max = [&](int rt) {
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < C::NT; ++u)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[rt][u][e]);
      return max_halves(mx) * scale_log2;  // scale > 0 commutes with max
    };
    if constexpr (FIRST) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) m_run[rt] = row_max(rt);
    }
    float nbase[RT], rs[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      nbase[rt] = -(m_run[rt] == -INFINITY ? 0.f : m_run[rt]);
      rs[rt] = 0.f;
    }
    // reference check (see above); has_keys: the row sees a key of this block
    auto check_reference = [&]() {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const bool has_keys = my_lo[rt] <= j0 + C::BN - 1 && my_hi[rt] >= j0 && my_lo[rt] <= my_hi[rt];
        if (__any(rs[rt] > kSumLimit || (m_run[rt] == -INFINITY && has_keys))) {
          const float m_new = fmaxf(m_run[rt], row_max(rt));
          const float alpha = fast_exp2(m_run[rt] - (m_new == -INFINITY ? 0.f : m_new));
          l_run[rt] *= alpha;
#pragma unroll
          for (int t = 0; t < C::TV; ++t) acc[rt][t] *= alpha;
          m_run[rt] = m_new;
          const float nb2 = -(m_run[rt] == -INFINITY ? 0.f : m_run[rt]);
          rs[rt] = 0.f;
          static_for<NWD>([&](auto W_) { exp_word(s[rt], pc[rt], nb2, rs[rt], W_); });
        }
        l_run[rt] += rs[rt];
      }
    };

    if constexpr (C::PP) {
      // Two groups of NWM / 2 waves (rows [0, ROWS / 2) and [ROWS / 2, ROWS))
      // run the same code with group 1 one barrier behind group 0: between two
      // barriers one group runs the MFMA phase (PV(it-1), QK(it+1)) while the
      // other runs the softmax phase of its previous block, so the two waves
      // of a SIMD (one of each group) alternate between the MFMA pipe and the
      // VALU.  Group 1 reaches the second barrier of an iteration only once
      // its loads up to iteration it-2 have landed: group 0 passes that
      // barrier into its next MFMA phase, which reads K(it+2) and V(it).
      __builtin_amdgcn_s_setprio(1);
      if constexpr (!FIRST)
        pvqk(int_c<(ST + 3) % 4>{}, pbuf[SB ^ 1], int_c<(ST + 1) % 4>{}, sbuf[SB ^ 1], nothing);
      else
        qk(int_c<(ST + 1) % 4>{}, sbuf[SB ^ 1], nothing);
      __builtin_amdgcn_s_setprio(0);
      if (pp_late) wait_loads(int_c<4 * C::KL>{});
      block_barrier();
      static_for<RT * NWD>([&](auto W_) {
        constexpr int w = decltype(W_)::value, rt = w / NWD;
        exp_word(s[rt], pc[rt], nbase[rt], rs[rt], int_c<w % NWD>{});
      });
      check_reference();
    } else {
      // the exponentials of block it are spread over the VALU slots after the
      // MFMAs of PV(it-1) and QK(it+1); word w of the RT * NWD words belongs to
      // row tile w / NWD
      auto slot = [&](auto K_) {
        constexpr int k = decltype(K_)::value;
        load_slot(K_);
        static_for<words_upto(k + 1) - words_upto(k)>([&](auto W_) {
          constexpr int w = words_upto(k) + decltype(W_)::value, rt = w / NWD;
          exp_word(s[rt], pc[rt], nbase[rt], rs[rt], int_c<w % NWD>{});
        });
      };
      if constexpr (!FIRST) {
        // the MFMA phase issues ahead of the other workgroup's wave on this
        // SIMD when both are ready (paired timing: 1-1.5 % on 8x2048, causal
        // or not)
        __builtin_amdgcn_s_setprio(1);
        pvqk(int_c<(ST + 3) % 4>{}, pbuf[SB ^ 1], int_c<(ST + 1) % 4>{}, sbuf[SB ^ 1], [&](auto N_) { slot(N_); });
        __builtin_amdgcn_s_setprio(0);
      } else {
        static_for<NPV>([&](auto N_) { slot(N_); });
        qk(int_c<(ST + 1) % 4>{}, sbuf[SB ^ 1], [&](auto N_) { slot(int_c<NPV + decltype(N_)::value>{}); });
      }
      check_reference();
    }
  };

  // Simple form on NS-stage rings: iteration it waits for K(it), V(it)
  // (issued NS-1 iterations back), takes the barrier (every wave is done with
  // stage (it+NS-1)%NS = (it-1)%NS), issues K(it+NS-1), V(it+NS-1) there,
  // then runs QK(it), the softmax of block it and PV(it).
  constexpr int NS = C::NS;
  auto body_simple = [&](auto ST_, auto FIRST_, int it) {
    constexpr int ST = decltype(ST_)::value;
    constexpr bool FIRST = decltype(FIRST_)::value != 0;
    const int j0 = j_begin + it * C::BN;
    wait_loads(int_c<(NS - 2) * 2 * C::KL>{});
    block_barrier();
    issue_k(j0 + (NS - 1) * C::BN, int_c<(ST + NS - 1) % NS>{});
    issue_v(j0 + (NS - 1) * C::BN, int_c<(ST + NS - 1) % NS>{});
    f32x16 (&s)[RT][C::NT] = sbuf[0];
    u32x4 (&pc)[RT][C::NG] = pbuf[0];
    qk(int_c<ST>{}, s, nothing);
    const bool full = j0 >= full_lo && j0 + C::BN - 1 <= full_hi;
    if (!full) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int u = 0; u < C::NT; ++u)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int j = j0 + 32 * u + 8 * (e >> 2) + 4 * hl + (e & 3);
            if (j < my_lo[rt] || j > my_hi[rt]) s[rt][u][e] = -INFINITY;
          }
    }
    auto row_max = [&](int rt) {
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < C::NT; ++u)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[rt][u][e]);
      return max_halves(mx) * scale_log2;
    };
    if constexpr (FIRST) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) m_run[rt] = row_max(rt);
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float nb = -(m_run[rt] == -INFINITY ? 0.f : m_run[rt]);
      float rs = 0.f;
      static_for<NWD>([&](auto W_) { exp_word(s[rt], pc[rt], nb, rs, W_); });
      const bool has_keys = my_lo[rt] <= j0 + C::BN - 1 && my_hi[rt] >= j0 && my_lo[rt] <= my_hi[rt];
      if (__any(rs > kSumLimit || (m_run[rt] == -INFINITY && has_keys))) {
        const float m_new = fmaxf(m_run[rt], row_max(rt));
        const float alpha = fast_exp2(m_run[rt] - (m_new == -INFINITY ? 0.f : m_new));
        l_run[rt] *= alpha;
#pragma unroll
        for (int t = 0; t < C::TV; ++t) acc[rt][t] *= alpha;
        m_run[rt] = m_new;
        const float nb2 = -(m_run[rt] == -INFINITY ? 0.f : m_run[rt]);
        rs = 0.f;
        static_for<NWD>([&](auto W_) { exp_word(s[rt], pc[rt], nb2, rs, W_); });
      }
      l_run[rt] += rs;
    }
    pv(int_c<ST>{}, pc, nothing);
  };
  if constexpr (C::SIMPLE) {
    if (n_iter > 0) {
      static_for<NS - 1>([&](auto I_) {
        constexpr int i = decltype(I_)::value;
        issue_k(j_begin + i * C::BN, int_c<i>{});
        issue_v(j_begin + i * C::BN, int_c<i>{});
      });
      body_simple(int_c<0>{}, int_c<1>{}, 0);
      int it = 1;
      for (;;) {
        if (it >= n_iter) break;
        body_simple(int_c<1 % NS>{}, int_c<0>{}, it++);
        if (it >= n_iter) break;
        body_simple(int_c<2 % NS>{}, int_c<0>{}, it++);
        if constexpr (NS == 3) {
          if (it >= n_iter) break;
          body_simple(int_c<0>{}, int_c<0>{}, it++);
        }
      }
      // every load of the ring retires before the workgroup's LDS is reused
      __builtin_amdgcn_s_waitcnt(0);
    }
  }
  if constexpr (!C::SIMPLE) if (n_iter > 0) {
    // group 1 of the two-group variant: one barrier of delay (its loads up to
    // K(1) landed first: group 0's first MFMA phase reads K(1))
    if (pp_late) {
      wait_loads(int_c<4 * C::KL>{});
      block_barrier();
    }
    body(int_c<0>{}, int_c<1>{}, 0);
    int it = 1;
    for (;;) {
      if (it >= n_iter) break;
      body(int_c<1>{}, int_c<0>{}, it++);
      if (it >= n_iter) break;
      body(int_c<2>{}, int_c<0>{}, it++);
      if (it >= n_iter) break;
      body(int_c<3>{}, int_c<0>{}, it++);
      if (it >= n_iter) break;
      body(int_c<0>{}, int_c<0>{}, it++);
    }
    // PV of the last block (V stage and P buffer of block n_iter-1); every
    // load of the ring retires here
    __builtin_amdgcn_s_waitcnt(0);
    block_barrier();
    const int last = n_iter - 1;
    switch (last & 3) {
      case 0: pv(int_c<0>{}, pbuf[0], nothing); break;
      case 1: pv(int_c<1>{}, pbuf[1], nothing); break;
      case 2: pv(int_c<2>{}, pbuf[0], nothing); break;
      default: pv(int_c<3>{}, pbuf[1], nothing); break;
    }
    // group 0 of the two-group variant matches group 1's extra barrier
    if (C::PP && !pp_late) block_barrier();
  }

  // ---- epilogue, per row tile
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const float l_tot = l_run[rt] + __shfl_xor(l_run[rt], 32);
    if (!row_ok[rt]) continue;
    const bool live = l_tot > 0.f;
    const float inv = live ? 1.0f / l_tot : 0.f;
    const float lse_v = live ? (m_run[rt] + __log2f(l_tot)) * kLn2 : -INFINITY;
    if (S > 1) {
      const int64_t tglob = (int64_t)q_off + iq[rt];
      float* op = p.o_part + (((int64_t)split * p.total_q + tglob) * p.hq + hq[rt]) * C::D;
#pragma unroll
      for (int t = 0; t < C::TV; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 o = {acc[rt][t][4 * j] * inv, acc[rt][t][4 * j + 1] * inv, acc[rt][t][4 * j + 2] * inv,
                     acc[rt][t][4 * j + 3] * inv};
          store_partial4(op + 32 * t + 8 * j + 4 * hl, o, p.fused_combine);
        }
      if (hl == 0)
        store_partial_lse(p.lse_part + ((int64_t)split * p.hq + hq[rt]) * p.total_q + tglob, lse_v, p.fused_combine);
    } else {
      char* op = p.o + (p.cu_q ? (int64_t)(q_off + iq[rt]) * p.o_st : (int64_t)b * p.o_sb + (int64_t)iq[rt] * p.o_st) +
                 (int64_t)hq[rt] * p.o_sh;
#pragma unroll
      for (int t = 0; t < C::TV; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u32x2 w = {pack2_in<DT>(acc[rt][t][4 * j] * inv, acc[rt][t][4 * j + 1] * inv),
                     pack2_in<DT>(acc[rt][t][4 * j + 2] * inv, acc[rt][t][4 * j + 3] * inv)};
          *(u32x2*)(op + (32 * t + 8 * j + 4 * hl) * 2) = w;
        }
      if (p.lse && hl == 0) {
        const int64_t li = p.cu_q ? (int64_t)hq[rt] * p.lse_sh + q_off + iq[rt]
                                  : (int64_t)b * p.lse_sb + (int64_t)hq[rt] * p.lse_sh + iq[rt];
        p.lse[li] = lse_v;
      }
    }
  }
  // split plans whose grid is resident at once: combine the tile's partials here
  if (S > 1 && p.fused_combine)
    fused_split_combine<C::NTHR, C::D>(p, b, hkv, qtile, split, q_off, row0, min(row0 + C::ROWS, rows), sk);
}

// Grid position of the next tile a persistent workgroup takes: its own XCD's
// list of the tile table first (the tiles placed there for that XCD's L2),
// then the other lists; -1 when every list is exhausted.  The claim counters
// only grow, so each position is taken once.  Thread 0 only.
__device__ __forceinline__ int claim_position(const FwdParams& p, int xcc, int positions) {
  for (int d = 0; d < kXcds; ++d) {
    const int list = (xcc + d) % kXcds;
    const int j = __hip_atomic_fetch_add(p.sched + 1 + list, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int pos = kXcds * j + list;
    if (pos < positions && p.sched[kSchedHead + 2 * pos] >= 0) return pos;
  }
  return -1;
}

// PERSIST = false: one tile per workgroup (blockIdx.x -> work item).
// PERSIST = true (table order): a grid of about one round of workgroups, each
// taking table positions until none is left; the next position is claimed
// while the current tile runs.
template <class C, bool PERSIST>
__global__ __launch_bounds__(C::NTHR, C::MIN_BLOCKS) void fmha_prefill_kernel(FwdParams p) {
  // 256-byte alignment: stage offsets and the XOR swizzles compose by addition
  __shared__ __attribute__((aligned(256))) char smem[C::LDS];
  if constexpr (!PERSIST) {
    WorkItem wi;
    if (!work_item<C::ROWS>(p, wi)) return;
    prefill_tile<C>(p, wi, smem);
  } else {
    __shared__ int s_pos;
    const int positions = p.sched[0];
    unsigned xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    xcc &= kXcds - 1;
    if (threadIdx.x == 0) s_pos = claim_position(p, (int)xcc, positions);
    __syncthreads();
    int pos = s_pos;
    while (pos >= 0) {
      __syncthreads();  // every thread has read s_pos
      // the next slot of this XCD's list, claimed now and looked at after the
      // tile (the atomic's round trip overlaps the tile)
      int j_next = 0;
      if (threadIdx.x == 0)
        j_next = __hip_atomic_fetch_add(p.sched + 1 + xcc, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      WorkItem wi;
      if (table_item(p, pos, wi)) prefill_tile<C>(p, wi, smem);
      if (threadIdx.x == 0) {
        int np = kXcds * j_next + (int)xcc;
        if (np >= positions || p.sched[kSchedHead + 2 * np] < 0) np = claim_position(p, (int)xcc, positions);
        s_pos = np;
      }
      __syncthreads();  // the tile's LDS reads are done before the next tile's loads
      pos = s_pos;
    }
  }
}

template <class C>
hipError_t launch_prefill(const FwdParams& p, int64_t grid, hipStream_t stream) {
  if (p.persistent)
    hipLaunchKernelGGL((fmha_prefill_kernel<C, true>), dim3((uint32_t)grid), dim3(C::NTHR), 0, stream, p);
  else
    hipLaunchKernelGGL((fmha_prefill_kernel<C, false>), dim3((uint32_t)grid), dim3(C::NTHR), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fmha
