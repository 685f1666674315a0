// Split combine inside the attention launch, for plans whose whole grid is
// resident at once (one round of workgroups: the short cached-prefix shape of
// "[FlyDSL] Enable FP8 FMHA split-K for short cached-prefix queries", whose
// measured call includes attention and split combine).  Same arithmetic as
// fmha_combine.hip: for row (t, h) with partials (O_s, lse_s), s < S_b,
//   L = max_s lse_s;  L = -inf -> O = 0, LSE = -inf;
//   LSE = L + ln sum_s exp(lse_s - L);  O = sum_s exp(lse_s - LSE) O_s.
//
// The S_b split workgroups of one (sequence, kv head, query tile) write their
// partials with device-coherent stores (sc1: written through to the device's
// point of coherence, as the compiler writes an agent-scope atomic store),
// wait until those stores have completed, and count themselves on an arrival
// counter in the workspace (a device-scope atomic); once all S_b have
// arrived, split s combines rows [s R / S_b, (s + 1) R / S_b) of the tile's R
// rows, reading the partials with device-coherent loads (sc1).  Publishing
// this way needs no L2 write-back: the compiler's device-scope release fence
// writes back the whole L2 of the XCD (buffer_wbl2), which made this path
// 2.4x slower than the separate combine launch when every wave issued one.
// A second counter counts departures; the last workgroup to leave resets both
// to zero, so the block of counters is zero before and after every launch (it
// must be zero before the first one).
//
// The wait is bounded: a workgroup that has not seen every split arrive after
// kFusedSpinLimit polls (far beyond any launch whose workgroups are resident
// together), or that draws an arrival ticket outside [0, S_b) (counters not
// zeroed), writes NaN rows for its slice instead of waiting on.  Every wave
// therefore ends.
#pragma once
#include "fmha_fwd_kernel.h"

namespace fmha {

constexpr int kFusedSpinLimit = 1 << 18;  // polls of ~0.5-1 us each
constexpr int kFusedMaxSplits = 64;       // host enables the fused combine up to this many splits

// 16 bytes stored coherently at device scope (global_store_dwordx4 ... sc1);
// completion is waited for with vmcnt before the arrival is counted.
__device__ __forceinline__ void store_coherent4(float* dst, f32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(dst), "v"(v) : "memory");
}
__device__ __forceinline__ float load_coherent(const float* src) {
  return __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A partial of the fused path (coherent) or of the two-launch path (plain).
__device__ __forceinline__ void store_partial4(float* dst, f32x4 v, bool coherent) {
  if (coherent)
    store_coherent4(dst, v);
  else
    *(f32x4*)dst = v;
}
__device__ __forceinline__ void store_partial_lse(float* dst, float v, bool coherent) {
  if (coherent)
    __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *dst = v;
}

// Device-coherent loads (sc1) through a buffer descriptor of the workspace:
// the compiler issues them as independent loads and waits once.
__device__ __forceinline__ float load_coherent_b32(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 16));
}
__device__ __forceinline__ f32x4 load_coherent_b128(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16));
}

constexpr int kCounterStride = 32;  // int32 counters per tile: one 128-byte line each
constexpr int kPastEnd = 0x7ffffff0;  // a buffer offset past any descriptor used here

// Called by every thread of a split workgroup after its partial stores.
// rows_end: one past the tile's last row (rows of the (sequence, kv head)).
// The host enables this path only while the workspace's partial regions stay
// below 2^31 bytes (32-bit buffer offsets).
template <int NTHR, int DV>
__device__ void fused_split_combine(const FwdParams& p, int b, int hkv, int qtile, int split, int q_off,
                                    int row0, int rows_end, int sk) {
  const int tid = threadIdx.x;
  const int G = p.group;
  const int nsb = min((sk + p.chunk - 1) / p.chunk, p.num_splits);
  int* cnt = p.counters + kCounterStride * (((int64_t)b * p.hkv + hkv) * p.num_q_tiles + qtile);
  int* dep = cnt + 1;
  __shared__ int s_ok;

  // publish: every wave's coherent partial stores have completed, then one
  // arrival
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  asm volatile("" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const int ticket = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool ok = ticket >= 0 && ticket < nsb;
    int polls = 0;
    while (ok && __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < nsb) {
      if (++polls >= kFusedSpinLimit) ok = false;
      __builtin_amdgcn_s_sleep(4);
    }
    s_ok = ok;
  }
  __syncthreads();
  const bool ok = s_ok != 0;

  // CH threads per row (one 16-byte column chunk each; a power of two <= 64,
  // so a row's threads are aligned lanes of one wave); thread c of a row loads
  // the lse of splits c, c + CH, ... and the row reduces them with lane
  // shuffles
  constexpr int CH = DV / 4;
  constexpr int RPI = NTHR / CH;
  constexpr int NL = (kFusedMaxSplits + CH - 1) / CH;  // lse values per thread
  static_assert(NTHR % CH == 0 && (CH & (CH - 1)) == 0 && CH <= 64, "rows on aligned lanes");
  const int nrows = rows_end - row0;
  const int lo = row0 + (int)((int64_t)split * nrows / nsb);
  const int hi = row0 + (int)((int64_t)(split + 1) * nrows / nsb);
  const int c = tid % CH;
  const int lane_base = (tid & 63) - c;
  const __amdgpu_buffer_rsrc_t rl =
      make_rsrc((const char*)p.lse_part, (int64_t)p.num_splits * p.hq * p.total_q * 4);
  const __amdgpu_buffer_rsrc_t ro =
      make_rsrc((const char*)p.o_part, (int64_t)p.num_splits * p.total_q * p.hq * DV * 4);
  const int ob = p.out_dtype == DT_F32 ? 4 : 2;
  // all of a wave's threads take the same number of passes (the shuffles
  // need every lane); rows past hi are computed on row lo and not stored
  const int passes = (hi - lo + RPI - 1) / RPI;
  for (int pass = 0; pass < passes; ++pass) {
    const int r = lo + pass * RPI + tid / CH;
    const bool row_live = r < hi;
    const int rr = row_live ? r : lo;
    const int iq = rr / G, h = hkv * G + rr % G;
    const int t = q_off + iq;
    // every load of the row at once: the lse of splits c, c + CH, ... and
    // the O partials of splits [0, CH) (the next CH after the weights, for
    // more than CH splits); splits past nsb use offsets past the descriptor
    // (read as 0, not fetched) and get weight 0
    const int obase = (t * p.hq + h) * DV * 4 + 16 * c;
    const int ostride = p.total_q * p.hq * DV * 4;
    float lv[NL];
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const int sidx = c + k * CH;
      lv[k] = load_coherent_b32(rl, sidx < nsb ? ((sidx * p.hq + h) * p.total_q + t) * 4 : kPastEnd);
    }
    constexpr int NB = CH < 32 ? CH : 32;  // O partial loads in flight per thread
    f32x4 v[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) v[j] = load_coherent_b128(ro, j < nsb ? obase + j * ostride : kPastEnd);
#pragma unroll
    for (int k = 0; k < NL; ++k) lv[k] = c + k * CH < nsb ? lv[k] : -INFINITY;
    float L = lv[0];
#pragma unroll
    for (int k = 1; k < NL; ++k) L = fmaxf(L, lv[k]);
#pragma unroll
    for (int m = 1; m < CH; m <<= 1) L = fmaxf(L, __shfl_xor(L, m));
    float e = 0.f;
#pragma unroll
    for (int k = 0; k < NL; ++k) e += L == -INFINITY ? 0.f : exp2f((lv[k] - L) * kLog2e);
#pragma unroll
    for (int m = 1; m < CH; m <<= 1) e += __shfl_xor(e, m);
    float total = L == -INFINITY ? -INFINITY : L + log2f(e) * kLn2;
    float wk[NL];
#pragma unroll
    for (int k = 0; k < NL; ++k) wk[k] = total == -INFINITY ? 0.f : exp2f((lv[k] - total) * kLog2e);
    // O = sum_s w_s O_s in batches of NB splits (weight of split k CH + j
    // from lane j of the row); the first batch is already in flight
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < NL; ++k) {
#pragma unroll
      for (int jb = 0; jb < CH; jb += NB) {
        if (k * CH + jb >= nsb) break;
        if (k > 0 || jb > 0) {
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            const int sidx = k * CH + jb + j;
            v[j] = load_coherent_b128(ro, sidx < nsb ? obase + sidx * ostride : kPastEnd);
          }
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) o += __shfl(wk[k], lane_base + jb + j) * v[j];
      }
    }
    if (!ok) {
      o = f32x4{NAN, NAN, NAN, NAN};
      total = NAN;
    }
    if (row_live) {
      char* orow = p.o + (p.cu_q ? (int64_t)(q_off + iq) * p.o_st : (int64_t)b * p.o_sb + (int64_t)iq * p.o_st) +
                   (int64_t)h * p.o_sh;
      store_out4(orow + (int64_t)c * 4 * ob, p.out_dtype, o);
      if (p.lse && c == 0) {
        const int64_t li =
            p.cu_q ? (int64_t)h * p.lse_sh + q_off + iq : (int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + iq;
        p.lse[li] = total;
      }
    }
  }

  // leave; the last of the tile's splits to leave resets both counters
  __syncthreads();
  if (tid == 0) {
    if (__hip_atomic_fetch_add(dep, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nsb - 1) {
      __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(dep, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace fmha
