// Device-side check of a cumulative sequence-length array against the
// contract of the varlen interface ("Adds variable sequence lengths to the
// Hopper CuTe DSL FMHA example", section Interface: cumulative int32 lengths
// [0, s0, s0+s1, ...] of sequences packed along the token dimension, with a
// bound on the longest sequence).
// The forward calls never read cu_seqlens on the host, so a caller that gets
// the array from elsewhere can run this check first.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fmha_params.h"

namespace fmha {

namespace {

constexpr int kValidateThreads = 256;

// One workgroup: thread t checks entries t, t + 256, ... and keeps the
// smallest failing index; an LDS reduction takes the minimum and thread 0
// writes 0 (valid) or 1 + that index.  Entry b fails when
//   b == 0 and cu[0] != 0, or
//   b > 0 and cu[b] < cu[b-1] or cu[b] - cu[b-1] > max_seqlen, or
//   b == batch and cu[batch] != total.
__global__ __launch_bounds__(kValidateThreads) void fmha_check_seqlens_kernel(const int32_t* cu, int32_t batch,
                                                                            int32_t total, int32_t max_seqlen,
                                                                            int32_t* result) {
  __shared__ int32_t best[kValidateThreads];
  const int tid = threadIdx.x;
  int32_t first = INT32_MAX;
  for (int32_t b = tid; b <= batch; b += kValidateThreads) {
    const int64_t cur = cu[b];
    bool bad = false;
    if (b == 0) bad = cur != 0;
    if (b > 0) {
      const int64_t prev = cu[b - 1];
      bad = bad || cur < prev || cur - prev > (int64_t)max_seqlen;
    }
    if (b == batch) bad = bad || cur != (int64_t)total;
    if (bad) {
      first = b;
      break;  // later entries of this thread have larger indices
    }
  }
  best[tid] = first;
  __syncthreads();
  for (int s = kValidateThreads / 2; s > 0; s >>= 1) {
    if (tid < s) best[tid] = min(best[tid], best[tid + s]);
    __syncthreads();
  }
  if (tid == 0) *result = best[0] == INT32_MAX ? 0 : best[0] + 1;
}

}  // namespace

hipError_t launch_check_seqlens(const int32_t* cu, int32_t batch, int32_t total, int32_t max_seqlen,
                                int32_t* result, hipStream_t stream) {
  hipLaunchKernelGGL(fmha_check_seqlens_kernel, dim3(1), dim3(kValidateThreads), 0, stream, cu, batch, total,
                     max_seqlen, result);
  return hipGetLastError();
}

}  // namespace fmha
