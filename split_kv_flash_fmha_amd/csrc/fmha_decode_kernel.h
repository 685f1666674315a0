// Split-KV decode kernel for gfx950: at most 16 query rows per (sequence, kv
// head) -- single-token decode, the q heads of one GQA group packed into the
// MFMA M dimension ("[Cute,Fwd,Sm100] Support q_stage=1 for inference",
// description: inference never fills a large query tile, so none is
// computed).  The work is HBM streaming of K and V, so the kernel is built as
// a streaming loop:
//
//  * A workgroup of NW waves owns one (batch, kv head, split); its key range is
//    cut into NW contiguous sub-ranges, one per wave, and every wave streams
//    its own keys with no workgroup barrier until the final merge.
//  * K is loaded straight from HBM into the MFMA A-operand registers of
//    S^T = K Q^T (lane%16 = key, 16 contiguous bytes of the key row per lane).
//  * V rows are loaded with 16-byte row-contiguous loads, written row-major to
//    a wave-private LDS tile and read back transposed with gfx950's LDS
//    transpose reads (ds_read_b64_tr_b16 / _b8) as the A operand of
//    O^T += V^T P^T.
//  * The next 32-key block's K and V are in flight (registers) while the
//    current block is computed.  Every K and V byte is read exactly once, so
//    the loads are non-temporal (streamed past the caches instead of
//    displacing other lines).  The rows are whole and contiguous per load,
//    so no line is fetched twice.
//  * The NW waves' (m, l, O) are merged through LDS; the result is written as
//    the final row (no split) or as this split's fp32 partial.
//
// Same MFMA formulation, lane ownership and masking rules as
// fmha_fwd_kernel.h (one query row per lane, row statistics lane-local).
#pragma once
#include "fmha_fwd_kernel.h"

namespace fmha {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

template <int DT_, int DQK_, int DV_, int NW_>
struct DecCfg {
  static constexpr int DT = DT_;
  static constexpr int DQK = DQK_;
  static constexpr int DV = DV_;
  static constexpr int NW = NW_;
  static constexpr int BYTES = Elem<DT>::bytes;
  static constexpr int NTHR = 64 * NW;
  static constexpr int BN = 32;                    // keys per wave per iteration
  static constexpr int NT = BN / 16;               // S^T tiles per block
  static constexpr int CQK = DQK * BYTES / 64;     // 16-byte chunks per lane per key tile
  static constexpr int TV = DV / 16;               // O^T tiles
  static constexpr int VROW = DV * BYTES;          // bytes per V row
  // LDS pitch of a V row: +32 bytes makes both the 16-byte row writes and the
  // 8-byte transpose reads of 2-byte types free of bank conflicts (+16 left
  // the reads two-way conflicted); 1-byte rows have no conflict-free pitch
  static constexpr int VP = VROW + (BYTES == 2 ? 32 : 16);
  static constexpr int VCH = BN * VROW / (64 * 16);  // 16-byte V loads per lane per block
  static constexpr int VROWS_PER_LOAD = 64 * 16 / VROW;
  static constexpr int LDS_V = NW * BN * VP;
  static constexpr int LDS_MERGE = NW * (TV * 64 * 16 + 16 * 8);
  static constexpr int LDS = LDS_V > LDS_MERGE ? LDS_V : LDS_MERGE;
  static_assert(DT == DT_BF16 || DT == DT_F16 || DT == DT_FP8, "decode kernel: 1- or 2-byte inputs");
  static_assert(DQK * BYTES % 64 == 0 && VROW % 16 == 0 && (64 * 16) % VROW == 0, "row sizes");
  static_assert(VCH >= 1, "V load split");
};

template <class C>
__global__ __launch_bounds__(C::NTHR, 2) void fmha_decode_kernel(FwdParams p) {
  constexpr int DT = C::DT;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wk = tid >> 6;
  const int lg = lane >> 4;
  const int lr = lane & 15;
  char* Vs = smem + wk * C::BN * C::VP;  // this wave's V tile

  const int S = p.num_splits;
  WorkItem wi;
  if (p.tile_order == kTileOrderFullFirst) {
    if (!full_first_item(p, wi)) return;
  } else {
    // split fastest: the splits of one (sequence, kv head) on consecutive blocks
    int64_t bid = blockIdx.x;
    wi.split = (int)(bid % S);
    bid /= S;
    wi.hkv = (int)(bid % p.hkv);
    wi.b = (int)(bid / p.hkv);
    seq_span(p, wi.b, wi);
  }
  const int split = wi.split, hkv = wi.hkv, b = wi.b;
  const int q_off = wi.q_off, sq = wi.sq, k_off = wi.k_off, sk = wi.sk;
  const int G = p.group;
  const int rows = sq * G;
  if (rows <= 0 || sk <= 0) return;
  const int kb = split * p.chunk;
  if (kb >= sk) return;
  const int ke = S > 1 ? min(kb + p.chunk, sk) : sk;

  const char* kbase = p.k + (p.cu_k ? (int64_t)k_off * p.k_st : (int64_t)b * p.k_sb) + (int64_t)hkv * p.k_sh;
  const char* vbase = p.v + (p.cu_k ? (int64_t)k_off * p.v_st : (int64_t)b * p.v_sb) + (int64_t)hkv * p.v_sh;

  const int r = lr;
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

  // key ranges (bottom-right causal / window / split), as in fmha_fwd_kernel
  const int shift = sk - sq;
  auto lo_of = [&](int i) { return p.wl >= 0 ? max(i + shift - p.wl, 0) : 0; };
  auto hi_of = [&](int i) { return p.wr >= 0 ? min(i + shift + p.wr, sk - 1) : sk - 1; };
  const int iq_hi = (rows - 1) / G;  // rows <= 16: one tile holds every row
  const int r0 = max(kb, lo_of(0));
  const int r1 = min(ke - 1, hi_of(iq_hi)) + 1;
  const int full_lo = max(kb, lo_of(iq_hi));
  const int full_hi = min(ke - 1, hi_of(0));
  // this wave's contiguous share, in whole 32-key blocks
  const int span = r1 > r0 ? r1 - r0 : 0;
  const int sub = ((span + C::NW - 1) / C::NW + C::BN - 1) / C::BN * C::BN;
  const int w_lo = r0 + wk * sub;
  const int w_hi = min(w_lo + sub, r1);
  const int my_lo = max(max(kb, lo_of(iq)), w_lo);
  const int my_hi = min(min(ke - 1, hi_of(iq)), w_hi - 1);
  const int n_iter = w_hi > w_lo ? (w_hi - w_lo + C::BN - 1) / C::BN : 0;

  f32x4 acc[C::TV];
#pragma unroll
  for (int t = 0; t < C::TV; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;

  // Loads of one 32-key block: K in A-operand layout, V as whole rows.
  auto load = [&](u32x4 (&kr)[C::NT][C::CQK], u32x4 (&vr)[C::VCH], int j0) {
#pragma unroll
    for (int u = 0; u < C::NT; ++u) {
      const int j = j0 + 16 * u + lr;
      const bool ok = j < w_hi;
      const char* src = kbase + (int64_t)j * p.k_st;
#pragma unroll
      for (int c = 0; c < C::CQK; ++c) {
        u32x4 z = {0u, 0u, 0u, 0u};
        kr[u][c] = ok ? __builtin_nontemporal_load((const u32x4*)(src + (4 * c + lg) * 16)) : z;
      }
    }
#pragma unroll
    for (int n = 0; n < C::VCH; ++n) {
      const int flat = n * 64 + lane;
      const int key = flat / (C::VROW / 16), part = flat % (C::VROW / 16);
      const int j = j0 + key;
      u32x4 z = {0u, 0u, 0u, 0u};
      vr[n] = j < w_hi ? __builtin_nontemporal_load((const u32x4*)(vbase + (int64_t)j * p.v_st + part * 16)) : z;
    }
  };

  auto process = [&](const u32x4 (&kr)[C::NT][C::CQK], const u32x4 (&vr)[C::VCH], int j0) {
    // V rows -> wave-private LDS tile (row-major)
#pragma unroll
    for (int n = 0; n < C::VCH; ++n) {
      const int flat = n * 64 + lane;
      const int key = flat / (C::VROW / 16), part = flat % (C::VROW / 16);
      *(u32x4*)(Vs + key * C::VP + part * 16) = vr[n];
    }
    // S^T = K Q^T
    f32x4 s[C::NT];
#pragma unroll
    for (int u = 0; u < C::NT; ++u) {
      s[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < C::CQK; ++c) s[u] = mfma_chunk<DT>(s[u], kr[u][c], qf[c]);
    }
    const bool full = j0 >= full_lo && j0 + C::BN - 1 <= full_hi && j0 + C::BN <= w_hi;
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < C::NT; ++u) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = s[u][e] * scale_log2;
        if (!full) {
          const int j = j0 + 16 * u + 4 * lg + e;
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
    // P^T B operand for one 32-key MFMA: slots 0..3 = tile 0, 4..7 = tile 1
    u32x4 pf;
    if constexpr (C::BYTES == 2) {
      pf = pack_p<DT>(&s[0]);
    } else {
      const float ps = kFp8PScale;
      pf.x = pack_fp8x4(s[0].x * ps, s[0].y * ps, s[0].z * ps, s[0].w * ps);
      pf.y = pack_fp8x4(s[1].x * ps, s[1].y * ps, s[1].z * ps, s[1].w * ps);
      pf.z = 0u;
      pf.w = 0u;
    }
    // O^T += V^T P^T; V^T fragment of lane (g, dv) = keys {16h + 4g + e} at
    // column dv, read transposed from the row-major tile
#pragma unroll
    for (int t = 0; t < C::TV; ++t) {
      u32x4 vf;
      if constexpr (C::BYTES == 2) {
        // 4x16 b16 block per read: lane 4e+j of group g reads row 16h+4g+e, cols 16t+4j..+3
        const int e = (lane >> 2) & 3, jq = lane & 3;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const char* a = Vs + (16 * h + 4 * lg + e) * C::VP + (16 * t + 4 * jq) * 2;
          const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a));
          const i32x2 xi = __builtin_bit_cast(i32x2, x);
          if (h == 0) {
            vf.x = (uint32_t)xi.x;
            vf.y = (uint32_t)xi.y;
          } else {
            vf.z = (uint32_t)xi.x;
            vf.w = (uint32_t)xi.y;
          }
        }
      } else {
        // 8x16 byte block: lane 2e+j of group g reads row key(e), cols 16t+8j..+7,
        // key(e) = 16*(e/4) + 4g + e%4 (slots 0..7 of this lane group)
        const int e = (lane >> 1) & 7, jh = lane & 1;
        const char* a = Vs + (16 * (e >> 2) + 4 * lg + (e & 3)) * C::VP + 16 * t + 8 * jh;
        const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(a));
        vf.x = (uint32_t)x.x;
        vf.y = (uint32_t)x.y;
        vf.z = 0u;
        vf.w = 0u;
      }
      acc[t] *= alpha;
      if constexpr (C::BYTES == 2) {
        acc[t] = mfma_chunk<DT>(acc[t], vf, pf);
      } else {
        const u32x2 a0 = {vf.x, vf.y}, b0 = {pf.x, pf.y};
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(__builtin_bit_cast(long, a0),
                                                           __builtin_bit_cast(long, b0), acc[t], 0, 0, 0);
      }
    }
  };

  u32x4 ka[C::NT][C::CQK], va[C::VCH], kb2[C::NT][C::CQK], vb[C::VCH];
  if (n_iter > 0) load(ka, va, w_lo);
  for (int it = 0; it < n_iter; it += 2) {
    const int j0 = w_lo + it * C::BN;
    if (it + 1 < n_iter) load(kb2, vb, j0 + C::BN);
    process(ka, va, j0);
    if (it + 2 < n_iter) load(ka, va, j0 + 2 * C::BN);
    if (it + 1 < n_iter) process(kb2, vb, j0 + C::BN);
  }

  // ---- merge the NW waves' (m, l, O^T) through LDS
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  __syncthreads();
  float* accbuf = (float*)smem;
  float* mlbuf = (float*)(smem + C::NW * C::TV * 64 * 16);
#pragma unroll
  for (int t = 0; t < C::TV; ++t) *(f32x4*)(accbuf + ((wk * C::TV + t) * 64 + lane) * 4) = acc[t];
  if (lg == 0) {
    mlbuf[(wk * 16 + lr) * 2 + 0] = m_run;
    mlbuf[(wk * 16 + lr) * 2 + 1] = l_tot;
  }
  __syncthreads();
  float mk[C::NW], lk[C::NW];
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < C::NW; ++k) {
    mk[k] = mlbuf[(k * 16 + lr) * 2 + 0];
    lk[k] = mlbuf[(k * 16 + lr) * 2 + 1];
    M = fmaxf(M, mk[k]);
  }
  const float Mb = M == -INFINITY ? 0.f : M;
  float L = 0.f, w[C::NW];
#pragma unroll
  for (int k = 0; k < C::NW; ++k) {
    w[k] = fast_exp2(mk[k] - Mb);
    L += w[k] * lk[k];
  }
  if (!row_ok) return;
  const bool live = L > 0.f;
  const float inv = live ? v_scale / L : 0.f;
  const float lse_v = live ? (M + __log2f(L)) * kLn2 : -INFINITY;
  const int dv_lane = 4 * lg;
  const int64_t tglob = (int64_t)q_off + iq;
  char* op_final = p.o + (p.cu_q ? (int64_t)(q_off + iq) * p.o_st : (int64_t)b * p.o_sb + (int64_t)iq * p.o_st) +
                   (int64_t)hq * p.o_sh;
  float* op_part = S > 1 ? p.o_part + (((int64_t)split * p.total_q + tglob) * p.hq + hq) * C::DV + dv_lane : nullptr;
  const int ob = p.out_dtype == DT_F32 ? 4 : 2;
#pragma unroll
  for (int t = 0; t < C::TV; ++t) {
    if (t % C::NW != wk) continue;
    f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < C::NW; ++k) o += w[k] * *(const f32x4*)(accbuf + ((k * C::TV + t) * 64 + lane) * 4);
    o *= inv;
    if (S > 1)
      *(f32x4*)(op_part + 16 * t) = o;
    else
      store_out4(op_final + (16 * t + dv_lane) * ob, p.out_dtype, o);
  }
  if (lg == 0 && wk == 0) {
    if (S > 1) {
      p.lse_part[((int64_t)split * p.hq + hq) * p.total_q + tglob] = lse_v;
    } else if (p.lse) {
      const int64_t li = p.cu_q ? (int64_t)hq * p.lse_sh + q_off + iq : (int64_t)b * p.lse_sb + (int64_t)hq * p.lse_sh + iq;
      p.lse[li] = lse_v;
    }
  }
}

template <class C>
hipError_t launch_decode(const FwdParams& p, int64_t grid, hipStream_t stream) {
  hipLaunchKernelGGL(fmha_decode_kernel<C>, dim3((uint32_t)grid), dim3(C::NTHR), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fmha
