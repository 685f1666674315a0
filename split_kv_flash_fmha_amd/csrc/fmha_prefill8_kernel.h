// FP8 (OCP e4m3fn) attention forward for more than 16 query rows per
// (sequence, kv head): the short cached-prefix shape of "[FlyDSL] Enable FP8
// FMHA split-K for short cached-prefix queries" (description and measurement:
// Q=70, Dq=Dk=192, Dv=128, per-tensor scales, split-K + combine) and fp8
// prefill generally.  Same algorithm and software pipeline as
// fmha_prefill_kernel.h (32 query rows per wave; iteration n runs PV(n-1) and
// QK(n+1) on the MFMA pipe around the exponentials of block n; reference max
// checked from the row sums), with fp8 operands:
//
//  * S^T = K Q^T on v_mfma_f32_32x32x64_f8f6f4 (64 d per MFMA): lane half h
//    of d chunk c carries d = 64c + 32h + b in byte b, for K (two 16-byte LDS
//    reads) and for Q (held in registers) alike.
//  * K and V blocks sit in LDS row-major, filled by 1 KiB buffer->LDS loads
//    whose 64 lanes fetch whole rows from HBM: K rows with one 16-byte pad
//    slot per row (pitch Dqk + 16), V rows unpadded with their 16-byte chunks
//    XOR-swizzled, both free of bank conflicts for the MFMA-operand and
//    transpose reads.
//  * O^T += V^T P^T on the same MFMA (64 keys per MFMA): byte 16u+4j+i of
//    lane half h carries key 32u+8j+4h+i, which is where the S^T output puts
//    that key, so P^T is packed straight from it; V^T comes from four
//    ds_read_b64_tr_b8 (8 keys x 16 dv per 16-lane group) in the same key
//    order.  P^T is stored as e4m3 of 8p.  The
//    factor 8 is carried by l as well (it cancels in O and is taken out of the
//    LSE); a row's 32 stored values sum to at most 448 unless the check sends
//    the block to the slow path, so each stays inside e4m3's range.
//  * Two row sums: l of the fp32 p (for the LSE) and lq of the e4m3 P that
//    the PV MFMA actually multiplies (for O = acc / lq).  With 3 mantissa
//    bits a single P can be off by 6 %; normalising by the rounded weights
//    keeps O a convex combination of V rows, so a row dominated by a few keys
//    does not carry their rounding times |v|.  lq comes from the MFMA pipe:
//    one 16x16x128 MFMA per block whose B operand is the block's P^T.
//  * Rings of LA + 2 K and V stages in LDS: the loads of LA key blocks are in
//    flight while a block is computed.
#pragma once
#include "fmha_fused_combine.h"
#include "fmha_prefill_kernel.h"

namespace fmha {

constexpr float kPScale8Log2 = 3.0f;  // P stored as e4m3 of 2^3 p
constexpr float kSumLimit8 = 448.0f;  // e4m3's largest finite value

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

// v_mfma_f32_32x32x64_f8f6f4 with e4m3 A and B (format code 0, no scaling).
// Operand lane l: row (A) / column (B) l % 32; its 32 bytes are the k-slots
// of lane half l / 32, byte b of A pairing with byte b of B (the kernel picks
// which key or d each byte carries, the same on both sides).
__device__ __forceinline__ f32x16 mfma64_fp8(f32x16 acc, u32x8 a, u32x8 b) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8, a), __builtin_bit_cast(i32x8, b),
                                                         acc, 0, 0, 0, 0, 0, 0);
}

// v_mfma_f32_16x16x128_f8f6f4 with e4m3 A and B.  Operand lane l: row (A) /
// column (B) l % 16, k-group l / 16 (its 32 bytes, byte b of A pairing with
// byte b of B); output lane l: column l % 16, rows 4 (l / 16) + i in
// register i.
__device__ __forceinline__ f32x4 mfma128_fp8(f32x4 acc, u32x8 a, u32x8 b) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(__builtin_bit_cast(i32x8, a), __builtin_bit_cast(i32x8, b),
                                                          acc, 0, 0, 0, 0, 0, 0);
}

template <int DQK_, int DV_, int NWM_, int LA_>
struct Pf8Cfg {
  static constexpr int DQK = DQK_;
  static constexpr int DV = DV_;
  static constexpr int NWM = NWM_;
  static constexpr int BN = 64;          // keys per block (one PV MFMA deep)
  static constexpr int NTHR = 64 * NWM;
  static constexpr int ROWS = 32 * NWM;
  static constexpr int KC = DQK / 64;    // 64-deep d chunks of QK (one MFMA each)
  static constexpr int NT = BN / 32;
  static constexpr int TV = DV / 32;
  static constexpr int NG = 2 * NT;      // PV groups of 16 keys
  static constexpr int KPITCH = DQK + 16;   // K row pitch in LDS: one 16-byte pad slot per row
  static constexpr int KSLOTS = KPITCH / 16;
  static constexpr int KTILE = BN * KPITCH;
  static constexpr int VTILE = BN * DV;      // V rows unpadded, 16-byte chunks XOR-swizzled
  static constexpr int KLD = KTILE / 1024;   // 1 KiB buffer->LDS loads per K block
  static constexpr int VLD = VTILE / 1024;
  static constexpr int LA = LA_;                        // key blocks of loads in flight
  static constexpr int NSK = LA + 2;                    // K ring stages
  static constexpr int NSV = LA + 2;                    // V ring stages
  static constexpr int KL = (KLD + NWM - 1) / NWM;      // K loads per wave per block
  static constexpr int VL = (VLD + NWM - 1) / NWM;      // V loads per wave per block
  static constexpr int LDS = NSK * KTILE + NSV * VTILE;
  static_assert(DQK % 64 == 0 && DV == 128, "head dims (the V swizzle assumes 8 chunks per row)");
  static_assert(KTILE % 1024 == 0 && VTILE % 1024 == 0, "whole 1 KiB loads per tile");
};

template <class C>
__global__ __launch_bounds__(C::NTHR, 2) void fmha_prefill8_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(256))) char smem[C::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wm = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5;
  const int lr = lane & 31;

  WorkItem wi;
  if (!work_item<C::ROWS>(p, wi)) return;
  const int S = p.num_splits;
  const int split = wi.split, hkv = wi.hkv, b = wi.b, qtile = wi.qtile;
  const int q_off = wi.q_off, sq = wi.sq, k_off = wi.k_off, sk = wi.sk;
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
  scale_log2 *= load_scale(p.q_descale, p.q) * load_scale(p.k_descale, p.q);
  const float v_scale = load_scale(p.v_descale, p.q);

  // Q^T (B operand): d chunk c, lane half h holds Q bytes [64c + 32h, +32)
  // (a lane past the tile's rows reads row 0's Q: its results are never stored,
  // and leaving its Q unmasked keeps the prologue from waiting on the Q loads)
  u32x8 qf[C::KC];
  {
    const char* qrow = p.q + (p.cu_q ? (int64_t)(q_off + iq) * p.q_st : (int64_t)b * p.q_sb + (int64_t)iq * p.q_st) +
                       (int64_t)hq * p.q_sh;
#pragma unroll
    for (int c = 0; c < C::KC; ++c) {
      const u32x4 lo = *(const u32x4*)(qrow + 64 * c + 32 * hl);
      const u32x4 hi = *(const u32x4*)(qrow + 64 * c + 32 * hl + 16);
      qf[c] = u32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
  }

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
  // Row sums of the e4m3 P (see the header): the P^T operand's lane group
  // g = l / 16 holds the 32 P bytes of row 16 (g % 2) + l % 16 over key half
  // g / 2.  A row 0 is e4m3 1.0 (0x38) on groups 0 and 2, A row 1 on groups 1
  // and 3, other rows 0, so output (0, n) accumulates row n's sum and output
  // (1, n) row n + 16's: lanes 0..15 hold them in lq[0] and lq[1].
  const bool one_here = (lane & 15) == ((lane >> 4) & 1) && (lane & 15) < 2;
  const uint32_t ones_w = one_here ? 0x38383838u : 0u;
  const u32x8 ones = {ones_w, ones_w, ones_w, ones_w, ones_w, ones_w, ones_w, ones_w};
  f32x4 lq = {0.f, 0.f, 0.f, 0.f};

  // LDS layout of a key block (64 rows):
  //  * K row r at r * KPITCH, chunk c at 16c (slot KSLOTS-1 is padding): the
  //    16-byte reads of 16 consecutive rows at one chunk hit distinct banks.
  //  * V row r at r * 128, chunk c at slot c ^ vswz(r), vswz(r) =
  //    2 * bit1(r) + 4 * bit3(r): the eight 32-byte row pieces a 32-lane
  //    transpose-read pass touches (rows {0..3, 8..11} + 4h) hit distinct banks.
  // Per-lane parts of the read addresses (stage offsets added per block).
  const uint32_t lds0 = lds_addr(smem);
  const uint32_t k_rd = lds0 + (uint32_t)(lr * C::KPITCH + 32 * hl);  // + 32u*KPITCH + 64c (+16)
  const int gq = (lane >> 4) & 1, i16 = lane & 15, e8 = i16 >> 1, jh = i16 & 1;
  const int vswz_e = 2 * ((e8 >> 1) & 1) + 4 * ((e8 >> 2) & 1);  // vswz of this lane's rows
  uint32_t v_rd[C::TV];  // dv tile t: + (32u+16m)*128
#pragma unroll
  for (int t = 0; t < C::TV; ++t)
    v_rd[t] = lds0 + (uint32_t)(C::NSK * C::KTILE + (8 * (e8 >> 2) + 4 * hl + (e8 & 3)) * C::DV +
                                16 * ((2 * t + gq) ^ vswz_e) + 8 * jh);

  // No LDS initialisation: every slot a read touches is written by a load
  // first (rows past a block's end and empty blocks are loaded as zeros; K pad
  // slots are never read), so the prologue's K/V loads go out at once.

  // One 1 KiB load fills LDS bytes [1024 i, 1024 i + 1024) of a tile; lane l
  // writes 16-byte slot 64 i + l and fetches the row chunk the layout puts
  // there, so the 64 lanes read whole rows (5.3 K rows or 8 V rows) from
  // HBM.  K pad slots take an offset past the descriptor (read as zero, no
  // fetch).  The descriptor covers the rows of the block the tile needs (rows
  // past them read as zero; a block past them gets an empty descriptor and
  // fetches nothing).  Every wave issues exactly KL K and VL V loads per block
  // (the last load repeated where the loads do not divide evenly; identical
  // bytes), so the loads a wave has in flight are a compile-time count.
  auto block_rsrc = [&](const char* base, int64_t st, int jb, int rowb) {
    const int rows_left = min(j_end - jb, C::BN);
    const int nb = rows_left > 0 ? (rows_left - 1) * (int)st + rowb : 0;
    return make_rsrc(base + (int64_t)jb * st, nb);
  };
  int k_src[C::KL], k_dst[C::KL], v_src[C::VL], v_dst[C::VL];
#pragma unroll
  for (int n = 0; n < C::KL; ++n) {
    const int i = min(wm + n * C::NWM, C::KLD - 1);
    const int slot = 64 * i + lane, r = slot / C::KSLOTS, c = slot % C::KSLOTS;
    k_src[n] = c < C::DQK / 16 ? r * (int)p.k_st + 16 * c : 0x7ffffff0;
    k_dst[n] = 1024 * i;
  }
#pragma unroll
  for (int n = 0; n < C::VL; ++n) {
    const int i = min(wm + n * C::NWM, C::VLD - 1);
    const int r = 8 * i + (lane >> 3), c = (lane & 7) ^ (2 * ((r >> 1) & 1) + 4 * ((r >> 3) & 1));
    v_src[n] = r * (int)p.v_st + 16 * c;
    v_dst[n] = 1024 * i;
  }
  auto issue_k = [&](int jb, int st) {
    const __amdgpu_buffer_rsrc_t rk = block_rsrc(kbase, p.k_st, jb, C::DQK);
    char* dst = smem + st * C::KTILE;
#pragma unroll
    for (int n = 0; n < C::KL; ++n) buffer_to_lds16(rk, dst + k_dst[n], k_src[n]);
  };
  auto issue_v = [&](int jb, int st) {
    const __amdgpu_buffer_rsrc_t rv = block_rsrc(vbase, p.v_st, jb, C::DV);
    char* dst = smem + C::NSK * C::KTILE + st * C::VTILE;
#pragma unroll
    for (int n = 0; n < C::VL; ++n) buffer_to_lds16(rv, dst + v_dst[n], v_src[n]);
  };
  auto wait_loads = [](auto N_) {
    constexpr int n = decltype(N_)::value;
    static_assert(n < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
  };

  // P^T of a key block as e4m3 of 8p: the 32-byte B operand of the PV MFMA
  static_assert(C::BN == 64, "one PV MFMA per block and dv tile");
  u32x8 pbuf[2];

  // O^T += V^T P^T from V stage vst: MFMA t (dv tile t) takes V^T from four
  // transpose reads, read (t, g) for key group g = (u, m): lane 2e+jh of
  // 16-lane group (hl, gq) reads key row 32u+16m+8(e/4)+4hl+e%4, dv bytes
  // 32t+16gq+8jh..+7 (at the row's swizzled chunk slot), and receives dv
  // column lr of those 8 keys (bytes 8g..8g+7 of its operand).  Reads run two MFMAs ahead; `between(t)` is VALU work
  // after MFMA t.
  auto pv = [&](int vst, const u32x8& pb, auto&& between) {
    constexpr int NM = C::TV;
    const uint32_t vso = (uint32_t)(vst * C::VTILE);
    i32x2 vr[3][4];
    auto read_frag = [&](auto T_) {
      constexpr int t = decltype(T_)::value;
      static_for<4>([&](auto G_) {
        constexpr int g = decltype(G_)::value, u = g >> 1, m = g & 1;
        vr[t % 3][g] = lds_tr8<(32 * u + 16 * m) * C::DV>(v_rd[t] + vso);
      });
    };
    read_frag(int_c<0>{});
    if constexpr (NM > 1) read_frag(int_c<1>{});
    static_for<NM>([&](auto T_) {
      constexpr int t = decltype(T_)::value;
      if constexpr (t + 2 < NM) {
        read_frag(int_c<t + 2>{});
        lgkm_wait<8>();
      } else if constexpr (t + 1 < NM) {
        lgkm_wait<4>();
      } else {
        lgkm_wait<0>();
      }
      static_for<4>([&](auto G_) { tie(vr[t % 3][decltype(G_)::value]); });
      const u32x8 va = {(uint32_t)vr[t % 3][0].x, (uint32_t)vr[t % 3][0].y, (uint32_t)vr[t % 3][1].x,
                        (uint32_t)vr[t % 3][1].y, (uint32_t)vr[t % 3][2].x, (uint32_t)vr[t % 3][2].y,
                        (uint32_t)vr[t % 3][3].x, (uint32_t)vr[t % 3][3].y};
      acc[t] = mfma64_fp8(acc[t], va, pb);
      between(int_c<t>{});
    });
  };

  // S^T = K Q^T from K stage kst into sd: MFMA n = (tile u, d chunk c) takes
  // K columns 4c+2h and 4c+2h+1 (32 bytes) of rows 32u + lr; reads run two
  // MFMAs ahead; `between(n)` is VALU work after MFMA n.
  auto qk = [&](int kst, f32x16 (&sd)[C::NT], auto&& between) {
    constexpr int NM = C::NT * C::KC;
    const uint32_t kbs = k_rd + (uint32_t)(kst * C::KTILE);
    u32x4 kf[3][2];
    auto read_k = [&](auto N_) {
      constexpr int n = decltype(N_)::value, u = n / C::KC, c = n % C::KC;
      kf[n % 3][0] = lds_b128<32 * u * C::KPITCH + 64 * c>(kbs);
      kf[n % 3][1] = lds_b128<32 * u * C::KPITCH + 64 * c + 16>(kbs);
    };
    read_k(int_c<0>{});
    if constexpr (NM > 1) read_k(int_c<1>{});
    static_for<NM>([&](auto N_) {
      constexpr int n = decltype(N_)::value, u = n / C::KC, c = n % C::KC;
      if constexpr (n + 2 < NM) {
        read_k(int_c<n + 2>{});
        lgkm_wait<4>();
      } else if constexpr (n + 1 < NM) {
        lgkm_wait<2>();
      } else {
        lgkm_wait<0>();
      }
      tie(kf[n % 3][0]);
      tie(kf[n % 3][1]);
      const u32x8 ka = {kf[n % 3][0].x, kf[n % 3][0].y, kf[n % 3][0].z, kf[n % 3][0].w,
                        kf[n % 3][1].x, kf[n % 3][1].y, kf[n % 3][1].z, kf[n % 3][1].w};
      if constexpr (c == 0) {
        f32x16 z;
#pragma unroll
        for (int e = 0; e < 16; ++e) z[e] = 0.f;
        sd[u] = mfma64_fp8(z, ka, qf[c]);
      } else {
        sd[u] = mfma64_fp8(sd[u], ka, qf[c]);
      }
      between(int_c<n>{});
    });
  };
  auto nothing = [](auto) {};

  // exponentials of a block: word w = elements 4(w % 4).. of the lane's S tile
  // w / 4 (keys 32u+8j+4h+i, i < 4, for u = w / 4, j = w % 4), stored as e4m3
  // of 8p in bytes 4w..4w+3 of the PV B operand; rs sums the 8p
  constexpr int NPV = C::TV, NQK = C::NT * C::KC;  // MFMAs per phase
  constexpr int NWD = 4 * C::NT;                   // words per block
  auto exp_word = [&](const f32x16 (&sd)[C::NT], u32x8& pb, float nb, float& rs, auto W_) {
    constexpr int w = decltype(W_)::value, u = w >> 2, e0 = 4 * (w & 3);
    float q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = fast_exp2(__builtin_fmaf(sd[u][e0 + i], scale_log2, nb));
    uint32_t word = pack_fp8x4(q[0], q[1], q[2], q[3]);
    tie(word);
    pb[w] = word;
    rs += (q[0] + q[1]) + (q[2] + q[3]);
    tie(rs);
  };
  auto words_upto = [](int k) { return (k * NWD) / (NPV + NQK); };

  // Rings of NS = LA + 2 stages: K(b) in K stage b % NS, V(b) in V stage
  // b % NS.  Iteration it issues K(it+NS) and V(it+LA) and needs K(it+1) (QK)
  // and V(it-1) (PV), issued NS-1 and LA+1 iterations earlier: the loads of
  // the last LA iterations may still be in flight.  The prologue issues in
  // the order iterations -NS..-1 would (empty loads for V(<0); they land
  // before any real load of the same stage, loads completing in order).
  constexpr int NS = C::NSK;
  static_assert(C::NSV == NS, "one ring depth");
  f32x16 sbuf[2][C::NT];
  const int jlast = j_begin + n_iter * C::BN;
  if (n_iter > 0) {
    static_for<NS>([&](auto I_) {
      constexpr int i = decltype(I_)::value;  // iteration i - NS
      issue_k(j_begin + i * C::BN, i);
      constexpr int vb = i - NS + C::LA;      // V block of that iteration
      if constexpr (vb >= 0)
        issue_v(j_begin + vb * C::BN, vb);
      else
        issue_v(jlast, NS - 1);  // empty
    });
    wait_loads(int_c<(NS - 1) * (C::KL + C::VL) + C::VL>{});  // K(0) landed
    block_barrier();
    qk(0, sbuf[0], nothing);
  }

  int kst = 1;       // (it + 1) % NS: K stage of QK(it+1)
  int vst = NS - 1;  // (it - 1) % NS: V stage of PV(it-1)
  // SB = it % 2 at compile time (S and P buffers stay in registers)
  auto body = [&](auto SB_, auto FIRST_, int it) {
    constexpr int SB = decltype(SB_)::value;
    constexpr bool FIRST = decltype(FIRST_)::value != 0;
    const int j0 = j_begin + it * C::BN;
    wait_loads(int_c<C::LA * (C::KL + C::VL)>{});
    block_barrier();  // K(it+1), V(it-1) in LDS everywhere; K stage it%NS, V stage (it-2)%NS free
    const int kst_free = kst == 0 ? NS - 1 : kst - 1;  // it % NS
    const int vst_free = vst == 0 ? NS - 1 : vst - 1;  // (it + LA) % NS == (it - 2) % NS
    issue_k(j0 + NS * C::BN, kst_free);
    issue_v(j0 + C::LA * C::BN, vst_free);
    f32x16 (&s)[C::NT] = sbuf[SB];
    u32x8& pc = pbuf[SB];

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
    auto row_max = [&]() {
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < C::NT; ++u)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[u][e]);
      return max_halves(mx) * scale_log2;
    };
    if constexpr (FIRST) m_run = row_max();
    const float nbase = kPScale8Log2 - (m_run == -INFINITY ? 0.f : m_run);
    float rs = 0.f;
    auto slot = [&](auto K_) {
      constexpr int k = decltype(K_)::value;
      static_for<words_upto(k + 1) - words_upto(k)>([&](auto W_) {
        exp_word(s, pc, nbase, rs, int_c<words_upto(k) + decltype(W_)::value>{});
      });
    };
    if constexpr (!FIRST) {
      pv(vst, pbuf[SB ^ 1], [&](auto N_) { slot(N_); });
      lq = mfma128_fp8(lq, ones, pbuf[SB ^ 1]);
    } else {
      static_for<NPV>([&](auto N_) { slot(N_); });
    }
    qk(kst, sbuf[SB ^ 1], [&](auto N_) { slot(int_c<NPV + decltype(N_)::value>{}); });
    // reference check: a stored 8p above e4m3's range, or a row with keys in
    // this block and no reference yet, sends the block to the slow path
    const bool has_keys = my_lo <= j0 + C::BN - 1 && my_hi >= j0 && my_lo <= my_hi;
    if (__any(rs > kSumLimit8 || (m_run == -INFINITY && has_keys))) {
      const float m_new = fmaxf(m_run, row_max());
      const float alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.f : m_new));
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < C::TV; ++t) acc[t] *= alpha;
      // lq holds P up to block it - 1, like acc: lanes 0..15 scale row n's
      // sum by their own alpha and row n + 16's by that row's
      lq[0] *= alpha;
      lq[1] *= __shfl(alpha, (lane & 15) + 16);
      m_run = m_new;
      const float nb2 = kPScale8Log2 - (m_run == -INFINITY ? 0.f : m_run);
      rs = 0.f;
      static_for<NWD>([&](auto W_) { exp_word(s, pc, nb2, rs, W_); });
    }
    l_run += rs;
    kst = kst == NS - 1 ? 0 : kst + 1;
    vst = vst == NS - 1 ? 0 : vst + 1;
  };

  if (n_iter > 0) {
    body(int_c<0>{}, int_c<1>{}, 0);
    for (int it = 1; it < n_iter; ++it) {
      body(int_c<1>{}, int_c<0>{}, it);
      if (++it >= n_iter) break;
      body(int_c<0>{}, int_c<0>{}, it);
    }
    // PV of the last block (V stage (n_iter-1) % NS == vst, P of block n_iter-1)
    __builtin_amdgcn_s_waitcnt(0);
    block_barrier();
    if ((n_iter - 1) & 1) {
      pv(vst, pbuf[1], nothing);
      lq = mfma128_fp8(lq, ones, pbuf[1]);
    } else {
      pv(vst, pbuf[0], nothing);
      lq = mfma128_fp8(lq, ones, pbuf[0]);
    }
  }

  // ---- epilogue
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float lq_lo = __shfl(lq[0], lr & 15), lq_hi = __shfl(lq[1], lr & 15);
  const float l_q = lr < 16 ? lq_lo : lq_hi;
  if (row_ok) {
    const bool live = l_tot > 0.f;
    // O by the sum of the rounded weights, the LSE by the exact sum
    const float inv = live && l_q > 0.f ? v_scale / l_q : 0.f;
    // l_run and acc both count 2^kPScale8Log2 * p: the factor cancels in O
    const float lse_v = live ? (m_run + __log2f(l_tot) - kPScale8Log2) * kLn2 : -INFINITY;
    if (S > 1) {
      const int64_t tglob = (int64_t)q_off + iq;
      float* op = p.o_part + (((int64_t)split * p.total_q + tglob) * p.hq + hq) * C::DV;
#pragma unroll
      for (int t = 0; t < C::TV; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 o = {acc[t][4 * j] * inv, acc[t][4 * j + 1] * inv, acc[t][4 * j + 2] * inv, acc[t][4 * j + 3] * inv};
          store_partial4(op + 32 * t + 8 * j + 4 * hl, o, p.fused_combine);
        }
      if (hl == 0) store_partial_lse(p.lse_part + ((int64_t)split * p.hq + hq) * p.total_q + tglob, lse_v, p.fused_combine);
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
  // split plans whose grid is resident at once: combine the tile's partials here
  if (S > 1 && p.fused_combine)
    fused_split_combine<C::NTHR, C::DV>(p, b, hkv, qtile, split, q_off, row0, min(row0 + C::ROWS, rows), sk);
}

template <class C>
hipError_t launch_prefill8(const FwdParams& p, int64_t grid, hipStream_t stream) {
  hipLaunchKernelGGL(fmha_prefill8_kernel<C>, dim3((uint32_t)grid), dim3(C::NTHR), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fmha
