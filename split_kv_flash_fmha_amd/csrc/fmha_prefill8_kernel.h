// FP8 (OCP e4m3fn) attention forward for more than 16 query rows per
// (sequence, kv head): the short cached-prefix shape of "[FlyDSL] Enable FP8
// FMHA split-K for short cached-prefix queries" (description and measurement:
// Q=70, Dq=Dk=192, Dv=128, per-tensor scales, split-K + combine) and fp8
// prefill generally.  Same algorithm and pipeline as fmha_prefill_kernel.h
// (32 query rows per wave, K one block ahead of V, QK of block n+1 issued
// before the softmax of block n, lazy reference max), with fp8 operands:
//
//  * S^T = K Q^T on v_mfma_f32_32x32x16_fp8_fp8.  A lane's 16-byte K read
//    covers two k-steps: bytes 0-7 feed one MFMA, bytes 8-15 the next, and Q
//    is loaded with the same byte mapping.
//  * K and V blocks sit in LDS "chunk-major": 16-byte column c of all BN rows
//    is contiguous (BN rows x 16 bytes), which suits any row length (192-byte
//    K rows) and makes each 1 KiB buffer->LDS load one column of 64 rows.  The
//    16-byte K reads of 16 consecutive rows are contiguous; V columns are
//    padded by 64 bytes so the two columns of one transpose-read pass fall in
//    different banks.
//  * O^T += V^T P^T with V^T from ds_read_b64_tr_b8 (8 keys x 16 dv per
//    16-lane group) and P^T stored as e4m3 of p * 2^4.
//  * Three LDS stages for K and for V: loads run two key blocks ahead of use,
//    and each wave waits only for the loads it issued two iterations back.  With the reference max
//    allowed to trail the running max by at most 2^4, p * 2^4 <= 2^8 stays
//    inside e4m3's range; the factor is divided out with the V descale.
#pragma once
#include "fmha_prefill_kernel.h"

namespace fmha {

constexpr float kRescaleSlack8 = 4.0f;
constexpr float kPScale8 = 16.0f;

__device__ __forceinline__ f32x16 mfma32_fp8(f32x16 acc, uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1) {
  const u32x2 a = {a0, a1}, b = {b0, b1};
  return __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(__builtin_bit_cast(long, a), __builtin_bit_cast(long, b), acc, 0,
                                                    0, 0);
}

template <int DQK_, int DV_, int NWM_>
struct Pf8Cfg {
  static constexpr int DQK = DQK_;
  static constexpr int DV = DV_;
  static constexpr int NWM = NWM_;
  static constexpr int BN = 64;          // keys per block: one 1 KiB load per 16-byte column
  static constexpr int NTHR = 64 * NWM;
  static constexpr int ROWS = 32 * NWM;
  static constexpr int KP2 = DQK / 32;   // 16-byte Q/K chunks per lane half (2 k-steps each)
  static constexpr int NT = BN / 32;
  static constexpr int TV = DV / 32;
  static constexpr int KCOLS = DQK / 16;
  static constexpr int VCOLS = DV / 16;
  static constexpr int KCP = BN * 16;        // K column pitch
  static constexpr int VCP = BN * 16 + 64;   // V column pitch
  static constexpr int KTILE = KCOLS * KCP;
  static constexpr int VTILE = VCOLS * VCP;
  static constexpr int NS = 3;                          // LDS ring depth (K and V)
  static constexpr int KL = (KCOLS + NWM - 1) / NWM;    // K column loads per wave per block
  static constexpr int VL = (VCOLS + NWM - 1) / NWM;    // V column loads per wave per block
  static constexpr int LDS = NS * (KTILE + VTILE);
  static_assert(DQK % 32 == 0 && DV % 32 == 0, "head dims");
};

template <class C>
__global__ __launch_bounds__(C::NTHR, 2) void fmha_prefill8_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wm = tid >> 6;
  const int hl = lane >> 5;
  const int lr = lane & 31;

  const WorkItem wi = work_item(p);
  const int S = p.num_splits;
  const int split = wi.split, hkv = wi.hkv, b = wi.b, qtile = wi.qtile;

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

  float scale_log2 = p.scale_log2;
  if (p.q_descale) scale_log2 *= *p.q_descale;
  if (p.k_descale) scale_log2 *= *p.k_descale;
  const float v_scale = (p.v_descale ? *p.v_descale : 1.0f) * (1.0f / kPScale8);

  // Q^T: chunk pair s, lane half h holds Q bytes [32s + 16h, +16): bytes 0-7
  // are the k-slots of MFMA 2s, bytes 8-15 those of MFMA 2s+1
  u32x4 qf[C::KP2];
  {
    const char* qrow = p.q + (p.cu_q ? (int64_t)(q_off + iq) * p.q_st : (int64_t)b * p.q_sb + (int64_t)iq * p.q_st) +
                       (int64_t)hq * p.q_sh;
#pragma unroll
    for (int s = 0; s < C::KP2; ++s) {
      u32x4 z = {0u, 0u, 0u, 0u};
      qf[s] = row_ok ? *(const u32x4*)(qrow + 32 * s + 16 * hl) : z;
    }
  }

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

  // per-lane constant parts of the LDS addresses
  const int k_rd = hl * C::KCP + lr * 16;  // + (2s)*KCP + 32u*16
  const int gq = (lane >> 4) & 1, i16 = lane & 15, e8 = i16 >> 1, jh = i16 & 1;
  const int v_rd = gq * C::VCP + (8 * (e8 >> 2) + 4 * hl + (e8 & 3)) * 16 + 8 * jh;  // + 2t*VCP + (32u+16m)*16

  // zero the LDS once so no slot is read uninitialised
  for (int i = tid * 16; i < C::LDS; i += C::NTHR * 16) *(u32x4*)(smem + i) = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();

  // one 1 KiB load = 16-byte column c of the 64 rows of a block (lane = row);
  // rows past the key range read as zero (descriptor ends at the last key),
  // and a block that starts past it gets an empty descriptor (nothing is
  // fetched).  Every wave issues exactly KL K and VL V loads per block (the
  // last column repeated where the columns do not divide evenly; identical
  // bytes), so the loads a wave has in flight are a compile-time count.
  auto issue_k = [&](int j0, int st) {
    const int64_t nb = j0 < j_end ? (int64_t)min(ke - 1 - j0, C::BN) * p.k_st + C::DQK : 0;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + (int64_t)j0 * p.k_st, nb);
    char* dst = smem + st * C::KTILE;
#pragma unroll
    for (int i = 0; i < C::KL; ++i) {
      const int c = min(wm + i * C::NWM, C::KCOLS - 1);
      buffer_to_lds16(rk, dst + c * C::KCP, lane * (int)p.k_st + c * 16);
    }
  };
  auto issue_v = [&](int j0, int st) {
    const int64_t nb = j0 < j_end ? (int64_t)min(ke - 1 - j0, C::BN) * p.v_st + C::DV : 0;
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + (int64_t)j0 * p.v_st, nb);
    char* dst = smem + C::NS * C::KTILE + st * C::VTILE;
#pragma unroll
    for (int i = 0; i < C::VL; ++i) {
      const int c = min(wm + i * C::NWM, C::VCOLS - 1);
      buffer_to_lds16(rv, dst + c * C::VCP, lane * (int)p.v_st + c * 16);
    }
  };
  auto qk = [&](f32x16 (&sd)[C::NT], int st) {
    const char* Ks = smem + st * C::KTILE + k_rd;
#pragma unroll
    for (int u = 0; u < C::NT; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) sd[u][e] = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < C::KP2; ++s2) {
      u32x4 kf[C::NT];
#pragma unroll
      for (int u = 0; u < C::NT; ++u) kf[u] = *(const u32x4*)(Ks + 2 * s2 * C::KCP + 32 * u * 16);
#pragma unroll
      for (int u = 0; u < C::NT; ++u) {
        sd[u] = mfma32_fp8(sd[u], kf[u].x, kf[u].y, qf[s2].x, qf[s2].y);
        sd[u] = mfma32_fp8(sd[u], kf[u].z, kf[u].w, qf[s2].z, qf[s2].w);
      }
    }
  };
  // at most KL + VL of this wave's loads (one block's K and V) in flight;
  // loads retire in order, so everything issued before them has landed
  constexpr int kInFlight = C::KL + C::VL;
  static_assert(kInFlight < 64, "vmcnt");
  auto wait_older_loads = [] {
    __builtin_amdgcn_s_waitcnt((kInFlight & 15) | ((kInFlight >> 4) << 14) | (7 << 4) | (15 << 8));
  };
  const uint32_t va0 = lds_addr(smem) + (uint32_t)v_rd;

  // Ring of three stages: K(b) in K stage b%3, V(b) in V stage b%3.
  // Iteration it waits for K(it+1) and V(it), issues K(it+3) and V(it+2) and
  // computes QK(it+1) and PV(it): loads run two blocks ahead of their use.
  f32x16 s_cur[C::NT], s_nxt[C::NT];
  if (n_iter > 0) {
    issue_k(j_begin, 0);
    issue_v(j_begin, 0);
    issue_k(j_begin + C::BN, 1);
    issue_k(j_begin + 2 * C::BN, 2);
    issue_v(j_begin + C::BN, 1);
    wait_older_loads();  // K(0), V(0), K(1) landed
    block_barrier();
    qk(s_cur, 0);
  }

  int st = 0;  // it % 3
  for (int it = 0; it < n_iter; ++it) {
    const int j0 = j_begin + it * C::BN;
    const int st1 = st == 2 ? 0 : st + 1;
    const int st2 = st1 == 2 ? 0 : st1 + 1;
    wait_older_loads();
    block_barrier();  // K(it+1), V(it) in LDS everywhere; stages of K(it), V(it-1) free
    issue_k(j0 + 3 * C::BN, st);
    issue_v(j0 + 2 * C::BN, st2);
    if (it + 1 < n_iter) qk(s_nxt, st1);
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
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < C::NT; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[u][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_blk = mx * scale_log2;
    if (__any(m_blk > m_run + kRescaleSlack8)) {
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
    // O^T += V^T P^T: group g = (u, m) covers keys 32u+16m+{0..15}.  Lane
    // 2e+jh of 16-lane group (hl, gq) reads key row 32u+16m+8(e/4)+4hl+e%4,
    // dv bytes 32t+16gq+8jh..+7, and receives dv column lr of those 8 keys.
    // The reads of group g+1 are in flight during group g's MFMAs.
    const uint32_t va = va0 + (uint32_t)(st * C::VTILE);
    i32x2 vr[2][C::TV];
    auto read_group = [&](auto G_) {
      constexpr int g = decltype(G_)::value, u = g >> 1, m = g & 1;
      static_for<C::TV>([&](auto T_) {
        constexpr int t = decltype(T_)::value;
        vr[g & 1][t] = lds_tr8<C::NS * C::KTILE + 2 * t * C::VCP + (32 * u + 16 * m) * 16>(va);
      });
    };
    read_group(int_c<0>{});
    static_for<2 * C::NT>([&](auto G_) {
      constexpr int g = decltype(G_)::value, u = g >> 1, m = g & 1;
      const float ps = kPScale8;
      const uint32_t p0 =
          pack_fp8x4(s[u][8 * m + 0] * ps, s[u][8 * m + 1] * ps, s[u][8 * m + 2] * ps, s[u][8 * m + 3] * ps);
      const uint32_t p1 =
          pack_fp8x4(s[u][8 * m + 4] * ps, s[u][8 * m + 5] * ps, s[u][8 * m + 6] * ps, s[u][8 * m + 7] * ps);
      if constexpr (g + 1 < 2 * C::NT) {
        read_group(int_c<g + 1>{});
        lgkm_wait<C::TV>();
      } else {
        lgkm_wait<0>();
      }
      static_for<C::TV>([&](auto T_) {
        constexpr int t = decltype(T_)::value;
        tie(vr[g & 1][t]);
        acc[t] = mfma32_fp8(acc[t], (uint32_t)vr[g & 1][t].x, (uint32_t)vr[g & 1][t].y, p0, p1);
      });
    });
#pragma unroll
    for (int u = 0; u < C::NT; ++u) s_cur[u] = s_nxt[u];
    st = st1;
  }
  // the ring's last loads (empty descriptors) must retire before the
  // workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(0);

  // ---- epilogue
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!row_ok) return;
  const bool live = l_tot > 0.f;
  const float inv = live ? v_scale / l_tot : 0.f;
  const float lse_v = live ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  if (S > 1) {
    const int64_t tglob = (int64_t)q_off + iq;
    float* op = p.o_part + (((int64_t)split * p.total_q + tglob) * p.hq + hq) * C::DV;
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
        u32x2 w = {pack_bf16x2(acc[t][4 * j] * inv, acc[t][4 * j + 1] * inv),
                   pack_bf16x2(acc[t][4 * j + 2] * inv, acc[t][4 * j + 3] * inv)};
        *(u32x2*)(op + (32 * t + 8 * j + 4 * hl) * 2) = w;
      }
    if (p.lse && hl == 0) {
      const int64_t li = p.cu_q ? (int64_t)hq * p.lse_sh + q_off + iq : (int64_t)b * p.lse_sb + (int64_t)hq * p.lse_sh + iq;
      p.lse[li] = lse_v;
    }
  }
}

template <class C>
hipError_t launch_prefill8(const FwdParams& p, int64_t grid, hipStream_t stream) {
  hipLaunchKernelGGL(fmha_prefill8_kernel<C>, dim3((uint32_t)grid), dim3(C::NTHR), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fmha
