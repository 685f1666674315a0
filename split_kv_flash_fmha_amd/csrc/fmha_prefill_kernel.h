// Prefill kernel for gfx950: many query rows per (sequence, kv head), so the
// work is a dense contraction on MFMA.  One workgroup = NWM waves x 32 query
// rows; per iteration it stages BN keys of K and V in LDS and every wave runs
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
// of bank conflicts.  The LDS holds two key blocks: block n+1 is in flight while
// block n is computed, one barrier per block.
//
// Softmax bookkeeping uses a lazily moved reference max per row: p =
// exp2(scale*s - m_ref) with m_ref moved (and O, l rescaled by
// exp2(m_ref_old - m_ref_new)) only when some row's running max exceeds its
// m_ref by more than kRescaleSlack (log2 units).  O and l are accumulated
// against the same m_ref, so O = acc / l and LSE = m_ref + log2 l are exact;
// p <= 2^kRescaleSlack keeps fp16/bf16 P in range.
#pragma once
#include "fmha_decode_kernel.h"
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

constexpr float kRescaleSlack = 8.0f;

template <int DT>
__device__ __forceinline__ uint32_t pack2_p(float a, float b) {
  if constexpr (DT == DT_F16) {
    // P in [0, 2^8]: round-toward-zero packing costs one instruction per pair
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
  } else {
    return pack_bf16x2(a, b);
  }
}

template <int DT_, int D_, int NWM_, int BN_>
struct PfCfg {
  static constexpr int DT = DT_;
  static constexpr int D = D_;          // Dqk == Dv
  static constexpr int NWM = NWM_;      // waves, 32 rows each
  static constexpr int BN = BN_;        // keys per iteration
  static constexpr int NTHR = 64 * NWM;
  static constexpr int ROWS = 32 * NWM;
  static constexpr int KS = D / 16;     // k-steps of QK (16 d each)
  static constexpr int NT = BN / 32;    // S^T tiles (32 keys each)
  static constexpr int TV = D / 32;     // O^T tiles (32 dv each)
  static constexpr int ROWB = D * 2;    // bytes per K / V row (unpadded, swizzled)
  static constexpr int RPL = 1024 / ROWB;          // rows per 1 KiB direct-to-LDS load
  static constexpr int TILE = BN * ROWB;           // one K or V block
  static constexpr int LOADS = 2 * TILE / 1024;    // 1 KiB loads per K+V block
  static constexpr int LPW = LOADS / NWM;          // per wave
  static constexpr int STAGE = 2 * TILE;
  static constexpr int LDS = 2 * STAGE;            // double buffered
  static_assert(D % 32 == 0 && BN % 32 == 0, "tile sizes");
  static_assert(1024 % ROWB == 0 && LOADS % (2 * NWM) == 0, "whole 1 KiB K and V loads per wave");
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

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char* base, int64_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)nbytes, 0x00020000);
}

// ---- LDS transpose reads as inline assembly
// The compiler's wait-counter pass cannot tell a builtin transpose read from
// an LDS read that aliases a pending buffer->LDS load, so it puts a full
// vmcnt(0) in front of the first one: PV would then wait for the loads of the
// next key blocks.  These kernels order their direct-to-LDS loads themselves
// (explicit vmcnt waits before each block barrier), so the V^T reads are
// issued as asm.  The compiler does not count them, so they are completed with
// lgkm_wait<N>() followed by tie() on every loaded register: tie's "+v"
// operand makes each consumer come after the wait.  Counting stays correct
// whatever else the compiler interleaves: LDS operations retire in order, and
// extra operations only make a count-based wait stricter.
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
__device__ __forceinline__ void tie(i32x2& r) { asm volatile("" : "+v"(r)); }

template <class C>
__global__ __launch_bounds__(C::NTHR, 2) void fmha_prefill_kernel(FwdParams p) {
  constexpr int DT = C::DT;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wm = tid >> 6;
  const int hl = lane >> 5;   // lane half: contraction slots / output row group
  const int lr = lane & 31;   // query row within the wave / MFMA column

  int64_t bid = blockIdx.x;
  const int S = p.num_splits;
  const int split = (int)(bid % S);
  bid /= S;
  const int hkv = (int)(bid % p.hkv);
  bid /= p.hkv;
  const int b = (int)(bid % p.batch);
  bid /= p.batch;
  const int qtile = p.num_q_tiles - 1 - (int)bid;

  int q_off, sq, k_off, sk;
  if (p.cu_q) {
    q_off = p.cu_q[b];
    sq = p.cu_q[b + 1] - q_off;
  } else {
    q_off = b * p.seqlen_q;
    sq = p.seqlen_q;
  }
  if (p.cu_k) {
    k_off = p.cu_k[b];
    sk = p.cu_k[b + 1] - k_off;
  } else {
    k_off = b * p.seqlen_k;
    sk = p.seqlen_k;
  }
  const int G = p.group;
  const int rows = sq * G;
  const int row0 = qtile * C::ROWS;
  if (row0 >= rows || sk <= 0) return;
  const int kb = split * p.chunk;
  if (kb >= sk) return;
  const int ke = S > 1 ? min(kb + p.chunk, sk) : sk;

  const char* kbase = p.k + (p.cu_k ? (int64_t)k_off * p.k_st : (int64_t)b * p.k_sb) + (int64_t)hkv * p.k_sh;
  const char* vbase = p.v + (p.cu_k ? (int64_t)k_off * p.v_st : (int64_t)b * p.v_sb) + (int64_t)hkv * p.v_sh;

  const int r = row0 + 32 * wm + lr;
  const bool row_ok = r < rows;
  const int iq = row_ok ? r / G : 0;
  const int hq = hkv * G + (row_ok ? r % G : 0);

  // Q^T (B operand): k-step s, lane half h holds d = 16s + 8h .. +8
  u32x4 qf[C::KS];
  {
    const char* qrow = p.q + (p.cu_q ? (int64_t)(q_off + iq) * p.q_st : (int64_t)b * p.q_sb + (int64_t)iq * p.q_st) +
                       (int64_t)hq * p.q_sh;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      u32x4 z = {0u, 0u, 0u, 0u};
      qf[s] = row_ok ? *(const u32x4*)(qrow + (16 * s + 8 * hl) * 2) : z;
    }
  }
  const float scale_log2 = p.scale_log2;

  const int shift = sk - sq;
  auto lo_of = [&](int i) { return p.wl >= 0 ? max(i + shift - p.wl, 0) : 0; };
  auto hi_of = [&](int i) { return p.wr >= 0 ? min(i + shift + p.wr, sk - 1) : sk - 1; };
  const int last_row = min(row0 + C::ROWS, rows) - 1;
  const int iq_lo = row0 / G, iq_hi = last_row / G;
  const int tile_lo = max(kb, lo_of(iq_lo));
  const int tile_hi = min(ke - 1, hi_of(iq_hi));
  const int full_lo = max(kb, lo_of(iq_hi));
  const int full_hi = min(ke - 1, hi_of(iq_lo));
  const int my_lo = max(kb, lo_of(iq));
  const int my_hi = min(ke - 1, hi_of(iq));
  const int j_begin = (tile_lo / C::BN) * C::BN;
  const int j_end = tile_hi + 1;
  const int n_iter = j_end > j_begin ? (j_end - j_begin + C::BN - 1) / C::BN : 0;

  f32x16 acc[C::TV];
#pragma unroll
  for (int t = 0; t < C::TV; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  // One key block = LOADS buffer->LDS loads of 1 KiB (RPL rows each): wave wm
  // issues loads [wm*LPW, (wm+1)*LPW), K loads first, then V.  Lane l of a
  // load writes LDS bytes [16l, 16l+16) of it, i.e. slot l % (ROWB/16) of row
  // l / (ROWB/16), so it fetches the chunk that belongs in that slot.  Its
  // byte offset from the block's first row is a loop constant; the block base
  // goes into the buffer descriptor, whose size ends at the last valid key, so
  // rows past the key range read as zero.
  constexpr int CPR = C::ROWB / 16;  // chunks per row
  // wave wm loads rows [wm * LPW/2 * RPL, ...) of the K tile and of the V tile
  int kld_off[C::LPW / 2], vld_off[C::LPW / 2];
#pragma unroll
  for (int n = 0; n < C::LPW / 2; ++n) {
    const int lrow = (wm * C::LPW / 2 + n) * C::RPL + lane / CPR;
    kld_off[n] = lrow * (int)p.k_st + k_slot<C::ROWB>(lrow, lane % CPR) * 16;
    vld_off[n] = lrow * (int)p.v_st + v_slot<C::ROWB>(lrow, lane % CPR) * 16;
  }
  // LDS read offsets (bytes within a stage's K / V tile), loop constants
  int koff[C::NT][C::KS];
#pragma unroll
  for (int u = 0; u < C::NT; ++u)
#pragma unroll
    for (int k = 0; k < C::KS; ++k) {
      const int row = 32 * u + lr;
      koff[u][k] = row * C::ROWB + k_slot<C::ROWB>(row, 2 * k + hl) * 16;
    }
  const int e4 = (lane >> 2) & 3, jq = lane & 3, grp = (lane >> 4) & 1;
  int voff[C::TV];  // + (32u + 16m + 8q) * ROWB per read (row & 3 == e4 throughout)
#pragma unroll
  for (int t = 0; t < C::TV; ++t)
    voff[t] = (4 * hl + e4) * C::ROWB + v_slot<C::ROWB>(e4, 4 * t + 2 * grp + (jq >> 1)) * 16 + 8 * (jq & 1);
  uint32_t va[C::TV];  // LDS addresses of the V^T reads (stage and row offsets are immediates)
#pragma unroll
  for (int t = 0; t < C::TV; ++t) va[t] = lds_addr(smem) + (uint32_t)voff[t];

  // zero both stages once so no slot is ever read uninitialised
#pragma unroll
  for (int i = tid * 16; i < C::LDS; i += C::NTHR * 16) *(u32x4*)(smem + i) = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();

  // K and V of block b live in K stage b%2 / V stage b%2.  K runs one block
  // ahead of V: during iteration it the loads of K(it+2) and V(it+1) are in
  // flight while QK(it+1) and PV(it) are computed.
  auto issue_k = [&](int j0, int stage) {
    const __amdgpu_buffer_rsrc_t rk =
        make_rsrc(kbase + (int64_t)j0 * p.k_st, (int64_t)min(ke - 1 - j0, C::BN) * p.k_st + C::ROWB);
    char* base = smem + stage * C::STAGE;
#pragma unroll
    for (int n = 0; n < C::LPW / 2; ++n) buffer_to_lds16(rk, base + (wm * C::LPW / 2 + n) * 1024, kld_off[n]);
  };
  auto issue_v = [&](int j0, int stage) {
    const __amdgpu_buffer_rsrc_t rv =
        make_rsrc(vbase + (int64_t)j0 * p.v_st, (int64_t)min(ke - 1 - j0, C::BN) * p.v_st + C::ROWB);
    char* base = smem + stage * C::STAGE + C::TILE;
#pragma unroll
    for (int n = 0; n < C::LPW / 2; ++n) buffer_to_lds16(rv, base + (wm * C::LPW / 2 + n) * 1024, vld_off[n]);
  };
  auto qk = [&](f32x16 (&sd)[C::NT], int stage) {
    const char* Ks = smem + stage * C::STAGE;
#pragma unroll
    for (int u = 0; u < C::NT; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) sd[u][e] = 0.f;
#pragma unroll
    for (int k = 0; k < C::KS; ++k) {
      u32x4 kf[C::NT];
#pragma unroll
      for (int u = 0; u < C::NT; ++u) kf[u] = *(const u32x4*)(Ks + koff[u][k]);
#pragma unroll
      for (int u = 0; u < C::NT; ++u) sd[u] = mfma32<DT>(sd[u], kf[u], qf[k]);
    }
  };

  f32x16 s_cur[C::NT], s_nxt[C::NT];
  if (n_iter > 0) {
    issue_k(j_begin, 0);
    issue_v(j_begin, 0);
    if (n_iter > 1) issue_k(j_begin + C::BN, 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    qk(s_cur, 0);
  }

  // ST = it % 2 as a compile-time constant, so the stage offsets fold into
  // the LDS instructions' immediate offsets
  auto body = [&](auto ST_, int it) {
    constexpr int ST = decltype(ST_)::value;
    const int j0 = j_begin + it * C::BN;
    // loads of K(it+1) and V(it) have landed everywhere, and every wave is done
    // with K stage ST (QK(it)) and V stage ST^1 (PV(it-1))
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (it + 2 < n_iter) issue_k(j0 + 2 * C::BN, ST);
    if (it + 1 < n_iter) issue_v(j0 + C::BN, ST ^ 1);
    // QK of the next block goes to the MFMA pipe while this block's softmax
    // runs on the VALU
    if (it + 1 < n_iter) qk(s_nxt, ST ^ 1);
    f32x16 (&s)[C::NT] = s_cur;

    const bool full = j0 >= full_lo && j0 + C::BN - 1 <= full_hi;
    if (!full) {
#pragma unroll
      for (int u = 0; u < C::NT; ++u)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int j = j0 + 32 * u + 8 * (e >> 2) + 4 * hl + (e & 3);
          if (j < my_lo || j > my_hi) s[u][e] = -INFINITY;
        }
    }
    // raw row max (scale > 0 commutes with max), one exchange with lane ^ 32
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < C::NT; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[u][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_blk = mx * scale_log2;
    // move the reference max only when some row ran ahead of it by > slack
    if (__any(m_blk > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, m_blk);
      const float alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.f : m_new));
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < C::TV; ++t) acc[t] *= alpha;
      m_run = m_new;
    }
    const float nbase = -(m_run == -INFINITY ? 0.f : m_run);
    float rs = 0.f;
#pragma unroll
    for (int u = 0; u < C::NT; ++u) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pe = fast_exp2(__builtin_fmaf(s[u][e], scale_log2, nbase));
        s[u][e] = pe;
        rs += pe;
      }
    }
    l_run += rs;
    // O^T += V^T P^T, 16 keys per MFMA: group g = (u, m) covers keys
    // 32u+16m+{0..15}.  Lane 4e+jq of 16-lane group (hl, grp) reads row
    // 32u+16m+8q+4hl+e, columns 32t+16grp+4jq..+3, and receives column lr of
    // those 4 rows.  The reads of group g+1 are in flight during group g's MFMAs.
    i32x2 vr[2][C::TV][2];
    auto read_group = [&](auto G_) {
      constexpr int g = decltype(G_)::value, u = g >> 1, m = g & 1;
      static_for<C::TV>([&](auto T_) {
        constexpr int t = decltype(T_)::value;
        vr[g & 1][t][0] = lds_tr16<ST * C::STAGE + C::TILE + (32 * u + 16 * m) * C::ROWB>(va[t]);
        vr[g & 1][t][1] = lds_tr16<ST * C::STAGE + C::TILE + (32 * u + 16 * m + 8) * C::ROWB>(va[t]);
      });
    };
    read_group(int_c<0>{});
    static_for<2 * C::NT>([&](auto G_) {
      constexpr int g = decltype(G_)::value, u = g >> 1, m = g & 1;
      u32x4 pf;
      pf.x = pack2_p<DT>(s[u][8 * m + 0], s[u][8 * m + 1]);
      pf.y = pack2_p<DT>(s[u][8 * m + 2], s[u][8 * m + 3]);
      pf.z = pack2_p<DT>(s[u][8 * m + 4], s[u][8 * m + 5]);
      pf.w = pack2_p<DT>(s[u][8 * m + 6], s[u][8 * m + 7]);
      if constexpr (g + 1 < 2 * C::NT) {
        read_group(int_c<g + 1>{});
        lgkm_wait<2 * C::TV>();
      } else {
        lgkm_wait<0>();
      }
      static_for<C::TV>([&](auto T_) {
        constexpr int t = decltype(T_)::value;
        tie(vr[g & 1][t][0]);
        tie(vr[g & 1][t][1]);
        const u32x4 vf = {(uint32_t)vr[g & 1][t][0].x, (uint32_t)vr[g & 1][t][0].y, (uint32_t)vr[g & 1][t][1].x,
                          (uint32_t)vr[g & 1][t][1].y};
        acc[t] = mfma32<DT>(acc[t], vf, pf);
      });
    });
#pragma unroll
    for (int u = 0; u < C::NT; ++u) s_cur[u] = s_nxt[u];
  };

  for (int it = 0; it < n_iter; it += 2) {
    body(int_c<0>{}, it);
    if (it + 1 < n_iter) body(int_c<1>{}, it + 1);
  }

  // ---- epilogue
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!row_ok) return;
  const bool live = l_tot > 0.f;
  const float inv = live ? 1.0f / l_tot : 0.f;
  const float lse_v = live ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  if (S > 1) {
    const int64_t tglob = (int64_t)q_off + iq;
    float* op = p.o_part + (((int64_t)split * p.total_q + tglob) * p.hq + hq) * C::D;
#pragma unroll
    for (int t = 0; t < C::TV; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 o = {acc[t][4 * j] * inv, acc[t][4 * j + 1] * inv, acc[t][4 * j + 2] * inv, acc[t][4 * j + 3] * inv};
        *(f32x4*)(op + 32 * t + 8 * j + 4 * hl) = o;
      }
    if (hl == 0) p.lse_part[((int64_t)split * p.hq + hq) * p.total_q + tglob] = lse_v;
  } else {
    char* op = p.o + (p.cu_q ? (int64_t)(q_off + iq) * p.o_st : (int64_t)b * p.o_sb + (int64_t)iq * p.o_st) +
               (int64_t)hq * p.o_sh;
#pragma unroll
    for (int t = 0; t < C::TV; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 w = {pack2_in<DT>(acc[t][4 * j] * inv, acc[t][4 * j + 1] * inv),
                   pack2_in<DT>(acc[t][4 * j + 2] * inv, acc[t][4 * j + 3] * inv)};
        *(u32x2*)(op + (32 * t + 8 * j + 4 * hl) * 2) = w;
      }
    if (p.lse && hl == 0) {
      const int64_t li = p.cu_q ? (int64_t)hq * p.lse_sh + q_off + iq : (int64_t)b * p.lse_sb + (int64_t)hq * p.lse_sh + iq;
      p.lse[li] = lse_v;
    }
  }
}

template <class C>
hipError_t launch_prefill(const FwdParams& p, int64_t grid, hipStream_t stream) {
  hipLaunchKernelGGL(fmha_prefill_kernel<C>, dim3((uint32_t)grid), dim3(C::NTHR), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fmha
