// Outlier migration before the decomposition (SmoothQuant-style balance).
// MosaicQuant technical summary (gist.science/pt/paper/2606.15652),
// Metodologia 1: activation outliers are migrated into the weights first,
// and the migrated weight is then split into the dense 4-bit base and the
// sparse 4-bit residual.  Rule (exponent 1/2):
//   s[k] = sqrt(max_t |Xc[t,k]| / max_n |W[n,k]|)   (fp32; 1 if either max is 0)
//   W'[n,k] = f16(W[n,k] * s[k]),   X'[t,k] = f16(X[t,k] / s[k]).
// Division and square root are IEEE correctly rounded (the build never
// enables fast math), so the scales are bit-reproducible.
#include "mq_internal.h"

namespace mq {
namespace {

constexpr int kRowsPerBlock = 64;

__global__ __launch_bounds__(256) void zero_kernel(float* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// Column max of |A| for fp16 A [R][C] (row stride lda): each thread takes a
// column and kRowsPerBlock rows, then merges with an integer atomic max on
// the float's bits (non-negative floats order like their bit patterns), so
// the result is exact and independent of the merge order.
__global__ __launch_bounds__(256) void colmax_kernel(const uint16_t* a, int64_t R, int64_t C,
                                                     int64_t lda, float* out) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= C) return;
  const int64_t r0 = (int64_t)blockIdx.y * kRowsPerBlock;
  const int64_t r1 = r0 + kRowsPerBlock < R ? r0 + kRowsPerBlock : R;
  float m = 0.f;
  for (int64_t r = r0; r < r1; ++r) m = fmaxf(m, fabsf(h2f(a[r * lda + c])));
  atomicMax(reinterpret_cast<unsigned int*>(out) + c, __float_as_uint(m));
}

__global__ __launch_bounds__(256) void scales_kernel(const float* ax, const float* aw, int64_t K,
                                                     float* s) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k >= K) return;
  const float x = ax[k], w = aw[k];
  s[k] = (x > 0.f && w > 0.f) ? sqrtf(x / w) : 1.f;
}

// out[r][c] = f16(f32(a[r][c]) * s[c])  (divide: f16(f32(a) / s[c])), a
// grid-stride loop so that any R x C fits the launch's 32-bit work-item count
template <bool DIVIDE>
__global__ __launch_bounds__(256) void scale_cols_kernel(const uint16_t* a, int64_t R, int64_t C,
                                                         int64_t lda, const float* s, uint16_t* out) {
  const int64_t n = R * C;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / C, c = i - r * C;
    const float v = h2f(a[r * lda + c]);
    // the fp32 result is materialised before the fp16 rounding: a fused
    // mixed-precision multiply would round the exact product once, not the
    // fp32 product, and differ at fp16 near-ties
    float p = DIVIDE ? v / s[c] : v * s[c];
    asm volatile("" : "+v"(p));
    out[r * C + c] = f2h_bits(p);
  }
}

unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }
// grid of the grid-stride kernels: at most 2^20 workgroups
unsigned strided_blocks(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return (unsigned)(b < ((int64_t)1 << 20) ? b : ((int64_t)1 << 20));
}

}  // namespace

hipError_t launch_smooth_weights(const uint16_t* xc, int64_t T, const uint16_t* w, int64_t N,
                                 int64_t K, float* ax, float* aw, float* s, uint16_t* w_out,
                                 hipStream_t st) {
  hipLaunchKernelGGL(zero_kernel, dim3(blocks_for(K)), dim3(256), 0, st, ax, K);
  hipLaunchKernelGGL(zero_kernel, dim3(blocks_for(K)), dim3(256), 0, st, aw, K);
  hipLaunchKernelGGL(colmax_kernel, dim3(blocks_for(K), (unsigned)((T + kRowsPerBlock - 1) / kRowsPerBlock)),
                     dim3(256), 0, st, xc, T, K, K, ax);
  hipLaunchKernelGGL(colmax_kernel, dim3(blocks_for(K), (unsigned)((N + kRowsPerBlock - 1) / kRowsPerBlock)),
                     dim3(256), 0, st, w, N, K, K, aw);
  hipLaunchKernelGGL(scales_kernel, dim3(blocks_for(K)), dim3(256), 0, st, ax, aw, K, s);
  hipLaunchKernelGGL(scale_cols_kernel<false>, dim3(strided_blocks(N * K)), dim3(256), 0, st, w, N, K, K, s,
                     w_out);
  return hipGetLastError();
}

hipError_t launch_smooth_acts(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const float* s,
                              uint16_t* x_out, hipStream_t st) {
  hipLaunchKernelGGL(scale_cols_kernel<true>, dim3(strided_blocks(M * K)), dim3(256), 0, st, x, M, K, ldx, s,
                     x_out);
  return hipGetLastError();
}

}  // namespace mq
