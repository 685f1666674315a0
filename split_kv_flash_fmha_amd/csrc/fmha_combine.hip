// LSE-weighted combine of split-KV partials (second launch of a split
// forward).  Definition ("[FlyDSL] Enable FP8 FMHA split-K for short
// cached-prefix queries", description: attention followed by a split
// combine): for row (t, h) with partials (O_s, lse_s), s < S_b,
//   L = max_s lse_s;  L = -inf -> O = 0, LSE = -inf;
//   LSE = L + ln sum_s exp(lse_s - L);  O = sum_s exp(lse_s - LSE) O_s.
//
// One 256-thread workgroup per (query row, head, group of cw 16-byte column
// chunks): thread (chunk c, split group g) owns the partial rows of splits
// g, g + 256/cw, ... of its chunk (at most 16).  Every thread issues its
// partial-O loads at once, next to the lse loads, so the workgroup waits for
// one memory round trip; the weights exp(lse_s - LSE) are then formed once in
// LDS and the split groups are summed through LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fmha.h"
#include "fmha_params.h"

namespace fmha {

namespace {

constexpr int kThreads = 256;
constexpr float kLog2eC = 1.4426950408889634f;
constexpr float kLn2C = 0.6931471805599453f;

typedef float f32x4c __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2c __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack2(float a, float b, int out_dtype) {
  if (out_dtype == DT_BF16) {
    __bf16 x = static_cast<__bf16>(a), y = static_cast<__bf16>(b);
    return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
  }
  _Float16 x = static_cast<_Float16>(a), y = static_cast<_Float16>(b);
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

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

template <int MAXL>
__global__ __launch_bounds__(kThreads) void fmha_combine_kernel(CombineParams p) {
  __shared__ float w_s[kThreads];
  __shared__ float red[kThreads / 64];
  __shared__ __attribute__((aligned(16))) f32x4c part[kThreads];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int nchunk = p.dv >> 2;
  const int cw = p.chunks_per_wg;                        // chunks per workgroup
  const int ncg = (nchunk + cw - 1) / cw;                // column groups per row
  const int ngroups = kThreads / cw;                     // split groups
  int64_t item = blockIdx.x;
  const int cg = (int)(item % ncg);
  item /= ncg;
  const int64_t per_b = (int64_t)p.max_seqlen_q * p.hq;
  const int b = (int)(item / per_b);
  const int64_t rem = item % per_b;
  const int i = (int)(rem / p.hq);
  const int h = (int)(rem % p.hq);

  int q_off, sq, sk;
  if (p.cu_q) {
    q_off = p.cu_q[b];
    sq = p.cu_q[b + 1] - q_off;
  } else {
    q_off = b * p.seqlen_q;
    sq = p.seqlen_q;
  }
  sk = p.cu_k ? p.cu_k[b + 1] - p.cu_k[b] : p.seqlen_k;
  if (i >= sq || sk <= 0) return;  // rows of sequences without keys: untouched (uniform)
  const int nsb = min((sk + p.chunk - 1) / p.chunk, p.num_splits);
  const int64_t t = (int64_t)q_off + i;
  const int64_t lse_split_stride = (int64_t)p.hq * p.total_q;

  // issue every load first: this thread's lse and its partial rows
  const float my_lse = tid < nsb ? p.lse_part[(int64_t)tid * lse_split_stride + (int64_t)h * p.total_q + t]
                                 : -INFINITY;
  const int cl = tid % cw, g = tid / cw;
  const int c = cg * cw + cl;
  const bool col_ok = c < nchunk && g < ngroups;
  const int64_t o_split_stride = (int64_t)p.total_q * p.hq * p.dv;
  const float* op = p.o_part + (t * p.hq + h) * p.dv + 4 * c;
  f32x4c v[MAXL];
#pragma unroll
  for (int k = 0; k < MAXL; ++k) {
    const int s = g + k * ngroups;
    v[k] = (col_ok && s < nsb) ? *(const f32x4c*)(op + s * o_split_stride) : f32x4c{0.f, 0.f, 0.f, 0.f};
  }

  // split weights: w_s = exp(lse_s - LSE)
  float mx = wave_max(my_lse);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  const float L = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float e = (L != -INFINITY && tid < nsb) ? exp2f((my_lse - L) * kLog2eC) : 0.f;
  e = wave_sum(e);
  if (lane == 0) red[wave] = e;
  __syncthreads();
  const float sum = red[0] + red[1] + red[2] + red[3];
  const float total = L == -INFINITY ? -INFINITY : L + log2f(sum) * kLn2C;
  w_s[tid] = (tid < nsb && total != -INFINITY) ? exp2f((my_lse - total) * kLog2eC) : 0.f;
  __syncthreads();

  f32x4c acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < MAXL; ++k) {
    const int s = g + k * ngroups;
    if (s < nsb) acc += w_s[s] * v[k];
  }
  part[tid] = acc;
  __syncthreads();
  if (tid < cw && c < nchunk) {
    f32x4c o = part[tid];
    for (int gg = 1; gg < ngroups; ++gg) o += part[gg * cw + tid];
    char* orow = p.o + (p.cu_q ? (int64_t)(q_off + i) * p.o_st : (int64_t)b * p.o_sb + (int64_t)i * p.o_st) +
                 (int64_t)h * p.o_sh;
    if (p.out_dtype == DT_F32) {
      *(f32x4c*)(orow + (int64_t)c * 16) = o;
    } else {
      u32x2c wv = {pack2(o.x, o.y, p.out_dtype), pack2(o.z, o.w, p.out_dtype)};
      *(u32x2c*)(orow + (int64_t)c * 8) = wv;
    }
  }
  if (p.lse && tid == 0 && cg == 0) {
    const int64_t li = p.cu_q ? (int64_t)h * p.lse_sh + q_off + i : (int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + i;
    p.lse[li] = total;
  }
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  const int cw = p.chunks_per_wg, nchunk = p.dv / 4;
  if (cw <= 0) return hipErrorInvalidValue;
  const int64_t items = (int64_t)p.max_seqlen_q * p.hq * p.batch * ((nchunk + cw - 1) / cw);
  if (items <= 0) return hipSuccess;
  const int loads = (p.num_splits + kThreads / cw - 1) / (kThreads / cw);
  const dim3 grid((uint32_t)items), block(kThreads);
  if (loads <= 2) {
    hipLaunchKernelGGL(fmha_combine_kernel<2>, grid, block, 0, stream, p);
  } else if (loads <= 4) {
    hipLaunchKernelGGL(fmha_combine_kernel<4>, grid, block, 0, stream, p);
  } else if (loads <= 8) {
    hipLaunchKernelGGL(fmha_combine_kernel<8>, grid, block, 0, stream, p);
  } else if (loads <= 16) {
    hipLaunchKernelGGL(fmha_combine_kernel<16>, grid, block, 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fmha
