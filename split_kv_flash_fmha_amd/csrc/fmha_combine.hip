// LSE-weighted combine of split-KV partials (second launch of a split
// forward).  Definition ("[FlyDSL] Enable FP8 FMHA split-K for short
// cached-prefix queries", description: attention followed by a split
// combine): for row (t, h) with partials (O_s, lse_s), s < S_b,
//   L = max_s lse_s;  L = -inf -> O = 0, LSE = -inf;
//   LSE = L + ln sum_s exp(lse_s - L);  O = sum_s exp(lse_s - LSE) O_s.
// One wavefront per (query row, head); lanes run along Dv so partial rows
// are read with contiguous 8-byte loads.  Memory-bound and small next to the
// attention launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fmha_params.h"

namespace fmha {

namespace {

constexpr float kLog2eC = 1.4426950408889634f;
constexpr float kLn2C = 0.6931471805599453f;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

__device__ __forceinline__ uint32_t pack2(float a, float b, int out_dtype) {
  if (out_dtype == DT_BF16) {
    __bf16 x = static_cast<__bf16>(a), y = static_cast<__bf16>(b);
    return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
  }
  _Float16 x = static_cast<_Float16>(a), y = static_cast<_Float16>(b);
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

constexpr int kWaves = 4;

__global__ __launch_bounds__(64 * kWaves) void fmha_combine_kernel(CombineParams p) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t per_b = ((int64_t)p.max_seqlen_q * p.hq + kWaves - 1) / kWaves;
  const int b = (int)(blockIdx.x / per_b);
  const int64_t item = (int64_t)(blockIdx.x % per_b) * kWaves + wave;
  const int h = (int)(item % p.hq);
  const int i = (int)(item / p.hq);

  int q_off, sq, sk;
  if (p.cu_q) {
    q_off = p.cu_q[b];
    sq = p.cu_q[b + 1] - q_off;
  } else {
    q_off = b * p.seqlen_q;
    sq = p.seqlen_q;
  }
  sk = p.cu_k ? p.cu_k[b + 1] - p.cu_k[b] : p.seqlen_k;
  if (i >= sq || sk <= 0) return;  // rows of sequences without keys: untouched
  const int nsb = min((sk + p.chunk - 1) / p.chunk, p.num_splits);
  const int64_t t = (int64_t)q_off + i;
  const float* lp = p.lse_part + (int64_t)h * p.total_q + t;
  const int64_t lse_split_stride = (int64_t)p.hq * p.total_q;

  float L = -INFINITY;
  for (int s = lane; s < nsb; s += 64) L = fmaxf(L, lp[s * lse_split_stride]);
  L = wave_max(L);

  float total = -INFINITY;
  if (L != -INFINITY) {
    float sum = 0.f;
    for (int s = lane; s < nsb; s += 64) sum += exp2f((lp[s * lse_split_stride] - L) * kLog2eC);
    sum = wave_sum(sum);
    total = L + log2f(sum) * kLn2C;
  }

  char* orow = p.o + (p.cu_q ? (int64_t)(q_off + i) * p.o_st : (int64_t)b * p.o_sb + (int64_t)i * p.o_st) +
               (int64_t)h * p.o_sh;
  const int64_t o_split_stride = (int64_t)p.total_q * p.hq * p.dv;
  const float* op = p.o_part + (t * p.hq + h) * p.dv;
  for (int d = lane * 2; d < p.dv; d += 128) {
    float a0 = 0.f, a1 = 0.f;
    if (total != -INFINITY) {
      for (int s = 0; s < nsb; ++s) {
        const float w = exp2f((lp[s * lse_split_stride] - total) * kLog2eC);
        const float2 v = *(const float2*)(op + s * o_split_stride + d);
        a0 += w * v.x;
        a1 += w * v.y;
      }
    }
    if (p.out_dtype == DT_F32) {
      *(float2*)(orow + (int64_t)d * 4) = make_float2(a0, a1);
    } else {
      *(uint32_t*)(orow + (int64_t)d * 2) = pack2(a0, a1, p.out_dtype);
    }
  }
  if (p.lse && lane == 0) {
    const int64_t li = p.cu_q ? (int64_t)h * p.lse_sh + q_off + i : (int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + i;
    p.lse[li] = total;
  }
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  const int64_t items = (int64_t)p.max_seqlen_q * p.hq;
  const int64_t gx = (items + kWaves - 1) / kWaves;
  if (gx <= 0 || p.batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(fmha_combine_kernel, dim3((uint32_t)(gx * p.batch)), dim3(64 * kWaves), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fmha
