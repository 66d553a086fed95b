// Measurement helper, not on the layer's path: the sustained rate of the
// int8 matrix-core instruction the fused GEMM kernels use, and the shader
// clock during that run, so that the benchmark can state its roofline
// denominators as measured on the device next to the datasheet figures.
//
// Each wave issues `iters` rounds of four independent
// V_MFMA_I32_16X16X64_I8 chains (independent accumulators, so no round waits
// on the previous one's result) and reads the shader cycle counter
// (s_memtime) before and after.  Lane 0 of each wave stores its cycle count;
// every lane stores a fold of its accumulators so the MFMAs stay live.
#include "gemm_common.h"

namespace mq {
namespace {

__global__ __launch_bounds__(256) void mfma_rate_kernel(int iters, int64_t* cycles, int32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const v4i a = {lane, lane + 1, lane + 2, lane + 3};
  const v4i b = {3 * lane, lane ^ 5, lane + 7, 11};
  v4i c0 = {0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int i = 0; i < iters; ++i) {
    c0 = mfma(a, b, c0);
    c1 = mfma(b, a, c1);
    c2 = mfma(a, a, c2);
    c3 = mfma(b, b, c3);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const int64_t w = (int64_t)blockIdx.x * 4 + wave;
  if (lane == 0) cycles[w] = (int64_t)(t1 - t0);
  const v4i s = c0 + c1 + c2 + c3;
  sink[w * 64 + lane] = s[0] ^ s[1] ^ s[2] ^ s[3];
}

}  // namespace

hipError_t launch_mfma_rate(int blocks, int iters, int64_t* cycles, int32_t* sink, hipStream_t st) {
  hipLaunchKernelGGL(mfma_rate_kernel, dim3((unsigned)blocks), dim3(256), 0, st, iters, cycles, sink);
  return hipGetLastError();
}

}  // namespace mq
