// Weight packing: dense 4-bit base (fp16 scale per row and group of 128)
// and the 4-bit residual of the selected blocks, stored CSR by output tile
// row with one fp16 scale per block row.
// MosaicQuant technical summary (gist.science/pt/paper/2606.15652),
// Metodologia 1: W ~ Q(W) + R with both parts 4-bit; Metodologia 2: the
// residual lives on selected blocks only.
#include "blockres.h"

namespace mq {
namespace {

// Base: a 16-lane team per (row, group); lane t handles channels t*8..t*8+7.
__global__ __launch_bounds__(256) void base_pack_kernel(const uint16_t* __restrict__ w,
                                                        int64_t K, uint8_t* __restrict__ qw,
                                                        uint16_t* __restrict__ sw,
                                                        int64_t total_groups) {
  const int64_t gid = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int t = threadIdx.x & 15;
  if (gid >= total_groups) return;
  const int64_t G = K / kGroup;
  const int64_t n = gid / G;
  const int64_t j = gid - n * G;
  float f[8];
  unpack_h8(*reinterpret_cast<const uint4*>(w + n * K + j * kGroup + t * 8), f);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 16));
  const uint16_t sb = f2h_bits(amax / 7.0f);
  const float s = h2f(sb);
  int q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = quant4(f[i], s);
  // slab layout: 16-channel slab n/16, group j, lane 16*(t/4) + n%16,
  // bytes 4*(t%4) .. +3 of that lane's 16
  *reinterpret_cast<uint32_t*>(qw + (n >> 4) * 8 * K + j * 1024 + ((t >> 2) * 16 + (n & 15)) * 16 +
                               (t & 3) * 4) = pack8(q);
  if (t == 0) sw[n * G + j] = sb;
}

// row_ptr[t] = number of selected ids below t*KT (binary search over the
// ascending list); col_idx[i] = id mod KT, or KT (never matched) for an
// id outside [0, B).
__global__ __launch_bounds__(256) void csr_kernel(const int32_t* __restrict__ sel, int n_sel,
                                                  int64_t NT, int64_t KT,
                                                  int32_t* __restrict__ row_ptr,
                                                  int32_t* __restrict__ col_idx) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t B = NT * KT;
  if (i <= NT) {
    const int64_t key = i * KT;
    int lo = 0, hi = n_sel;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)sel[mid] < key) lo = mid + 1; else hi = mid;
    }
    row_ptr[i] = (i == NT) ? n_sel : lo;
  }
  if (i < n_sel) {
    const int64_t id = sel[i];
    col_idx[i] = (id >= 0 && id < B) ? (int32_t)(id % KT) : (int32_t)KT;
  }
}

// Residual: one wave per selected block; lane r owns block row r (and
// r + 64 when b = 128) and writes b/2 bytes of codes and one fp16 scale.
__global__ __launch_bounds__(256) void residual_pack_kernel(
    const uint16_t* __restrict__ w, int64_t K, int b, const int32_t* __restrict__ sel, int n_sel,
    int64_t NT, uint8_t* __restrict__ qr, uint16_t* __restrict__ sr) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * 4 + wave;
  if (i >= n_sel) return;
  const int64_t KT = K / b;
  const int64_t id = sel[i];
  const bool valid = id >= 0 && id < NT * KT;
  const int64_t nt = valid ? id / KT : 0;
  const int64_t kb = valid ? (id - nt * KT) * b : 0;
  for (int r = lane; r < b; r += 64) {
    uint8_t* dst = qr + (i * b + r) * (b / 2);
    if (!valid) {
      for (int c = 0; c < b; c += 8) *reinterpret_cast<uint32_t*>(dst + c / 2) = 0u;
      sr[i * b + r] = 0;
      continue;
    }
    const uint16_t* wrow = w + (nt * b + r) * K;
    const RowScales rs = row_scales(wrow, kb, b);
    for (int c = 0; c < b; c += 8) {
      float f[8];
      unpack_h8(*reinterpret_cast<const uint4*>(wrow + kb + c), f);
      int q[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) q[u] = quant4(base_err(f[u], rs.swf), rs.srf);
      *reinterpret_cast<uint32_t*>(dst + c / 2) = pack8(q);
    }
    sr[i * b + r] = rs.sr_bits;
  }
}

}  // namespace

hipError_t launch_pack(const uint16_t* w, int64_t N, int64_t K, int block,
                       const int32_t* selected, int n_select, uint8_t* qw, uint16_t* sw,
                       int32_t* row_ptr, int32_t* col_idx, uint8_t* qr, uint16_t* sr,
                       hipStream_t st) {
  const int64_t groups = N * (K / kGroup);
  hipLaunchKernelGGL(base_pack_kernel, dim3((unsigned)((groups + 15) / 16)), dim3(256), 0, st, w,
                     K, qw, sw, groups);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t NT = N / block, KT = K / block;
  const int64_t nthreads = (NT + 1 > n_select) ? NT + 1 : n_select;
  hipLaunchKernelGGL(csr_kernel, dim3((unsigned)((nthreads + 255) / 256)), dim3(256), 0, st,
                     selected, n_select, NT, KT, row_ptr, col_idx);
  e = hipGetLastError();
  if (e != hipSuccess || n_select == 0) return e;
  hipLaunchKernelGGL(residual_pack_kernel, dim3((unsigned)((n_select + 3) / 4)), dim3(256), 0, st,
                     w, K, block, selected, n_select, NT, qr, sr);
  return hipGetLastError();
}

}  // namespace mq
