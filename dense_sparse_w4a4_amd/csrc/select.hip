// Offline block selection: diagonal Hessian, Delta-scores and top-K.
// MosaicQuant technical summary (gist.science/pt/paper/2606.15652),
// Metodologia 2: the Hessian-guided Delta-score approximates each block's
// marginal reduction of output distortion by weighting the residual error
// with the input channels' diagonal Hessian; the top-K blocks get a residual.
//
// Every floating-point step is fixed so the result is bit-identical to a
// plain sequential evaluation: this file is compiled with -ffp-contract=off,
// H sums tokens in order, each Delta row sum runs left to right over the
// block columns and the row sums are added left to right over rows.
#include "blockres.h"

namespace mq {
namespace {

// H[k] = sum_t Xc[t][k]^2, t = 0, 1, ...  One thread per channel; adjacent
// threads read adjacent channels, so every token row is a coalesced read.
__global__ __launch_bounds__(256) void hdiag_kernel(const uint16_t* __restrict__ xc, int64_t T,
                                                    int64_t K, double* __restrict__ H) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= K) return;
  double h = 0.0;
  for (int64_t t = 0; t < T; ++t) {
    const double v = (double)h2f(xc[t * K + k]);
    h = h + v * v;
  }
  H[k] = h;
}

// One wave per block; lane r owns block row r (and r + 64 when b = 128).
__global__ __launch_bounds__(256) void delta_kernel(const uint16_t* __restrict__ w, int64_t N,
                                                    int64_t K, int b,
                                                    const double* __restrict__ H,
                                                    double* __restrict__ delta, int64_t B) {
  __shared__ double rowsum[4][128];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t id = (int64_t)blockIdx.x * 4 + wave;
  const bool live = id < B;
  const int64_t KT = K / b;
  const int64_t nt = live ? id / KT : 0;
  const int64_t kt = live ? id - nt * KT : 0;
  const int64_t kb = kt * b;
  if (live) {
    for (int r = lane; r < b; r += 64) {
      const uint16_t* wrow = w + (nt * b + r) * K;
      const RowScales rs = row_scales(wrow, kb, b);
      double acc = 0.0;
      for (int c = 0; c < b; c += 8) {
        float f[8];
        unpack_h8(*reinterpret_cast<const uint4*>(wrow + kb + c), f);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float e = base_err(f[i], rs.swf);
          const float rh = rs.srf * (float)quant4(e, rs.srf);  // exact
          const double e64 = (double)e;
          const double d = e64 - (double)rh;
          const double gain = e64 * e64 - d * d;
          acc = acc + H[kb + c + i] * gain;
        }
      }
      rowsum[wave][r] = acc;
    }
  }
  __syncthreads();
  if (live && lane == 0) {
    double tot = 0.0;
    for (int r = 0; r < b; ++r) tot = tot + rowsum[wave][r];
    delta[id] = tot;
  }
}

// Order-preserving integer key of a score (higher score -> higher key); -0
// ranks with +0.
__device__ __forceinline__ uint64_t score_key(double d) {
  uint64_t u = __builtin_bit_cast(uint64_t, d);
  if (u == 0x8000000000000000ull) u = 0;
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Single-workgroup top-K: an MSB-first radix select (8 passes of 8-bit
// digits) finds the key T of the n_sel-th largest score and how many of the
// keys equal to T are taken; a stable compaction in id order then writes
// every key > T plus the lowest-id keys == T, which is the (score desc,
// id asc) ranking, already in ascending id order.
__global__ __launch_bounds__(1024) void topk_kernel(const double* __restrict__ delta, int64_t B,
                                                    int n_sel, int32_t* __restrict__ selected) {
  __shared__ unsigned hist[256];
  __shared__ uint64_t s_prefix;
  __shared__ long long s_remaining;
  __shared__ int s_wgt[16], s_weq[16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  if (n_sel <= 0) return;

  uint64_t prefix = 0, mask = 0;
  long long remaining = n_sel;
  for (int shift = 56; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int64_t i = tid; i < B; i += 1024) {
      const uint64_t k = score_key(delta[i]);
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      long long cum = 0;
      int d = 255;
      for (; d > 0; --d) {
        if (cum + (long long)hist[d] >= remaining) break;
        cum += hist[d];
      }
      s_prefix = prefix | ((uint64_t)d << shift);
      s_remaining = remaining - cum;
    }
    __syncthreads();
    prefix = s_prefix;
    remaining = s_remaining;
    mask |= (uint64_t)255 << shift;
    __syncthreads();
  }
  const uint64_t T = prefix;

  long long out_base = 0, eq_seen = 0;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t c0 = 0; c0 < B; c0 += 1024) {
    const int64_t i = c0 + tid;
    const uint64_t k = (i < B) ? score_key(delta[i]) : 0;
    const bool gt = (i < B) && (k > T);
    const bool eq = (i < B) && (k == T);
    const uint64_t beq = __ballot(eq);
    if (lane == 0) s_weq[wave] = __popcll(beq);
    __syncthreads();
    long long eq_before = eq_seen + __popcll(beq & below);
    long long eq_total = 0;
    for (int v = 0; v < 16; ++v) {
      if (v < wave) eq_before += s_weq[v];
      eq_total += s_weq[v];
    }
    const bool take = gt || (eq && eq_before < remaining);
    const uint64_t btk = __ballot(take);
    if (lane == 0) s_wgt[wave] = __popcll(btk);
    __syncthreads();
    long long pos = out_base + __popcll(btk & below);
    long long tk_total = 0;
    for (int v = 0; v < 16; ++v) {
      if (v < wave) pos += s_wgt[v];
      tk_total += s_wgt[v];
    }
    if (take && pos < n_sel) selected[pos] = (int32_t)i;
    out_base += tk_total;
    eq_seen += eq_total;
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_select(const uint16_t* w, const uint16_t* xc, int64_t N, int64_t K,
                         int64_t T, int block, int n_select, int32_t* selected,
                         double* delta, double* hdiag, hipStream_t st) {
  hipLaunchKernelGGL(hdiag_kernel, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st, xc, T,
                     K, hdiag);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t B = (N / block) * (K / block);
  hipLaunchKernelGGL(delta_kernel, dim3((unsigned)((B + 3) / 4)), dim3(256), 0, st, w, N, K,
                     block, hdiag, delta, B);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (n_select > 0) {
    hipLaunchKernelGGL(topk_kernel, dim3(1), dim3(1024), 0, st, delta, B, n_select, selected);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace mq
