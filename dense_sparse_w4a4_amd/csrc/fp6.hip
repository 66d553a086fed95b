// FP6 operand images for the prefill tile kernel's fp6 route (layout and
// the exactness argument in mq_internal.h).  The 4-bit codes of record are
// unchanged: these kernels only re-encode them, per call, into the
// workspace, so that the tile kernel copies whole operand fragments from
// memory to LDS and runs 32x32x64 FP6 MFMAs on them.
// MosaicQuant technical summary (gist.science/pt/paper/2606.15652),
// Metodologia 3: the online pipeline quantises the activations to 4 bits
// and multiplies them with the 4-bit base and residual.
#include "gemm_common.h"

namespace mq {
namespace {

// Activation quantisation straight into the FP6 image: one 16-lane team per
// token and four consecutive groups (its four 16-byte loads issued first),
// 16 consecutive tokens per workgroup; the scales group-major
// ([K/128][Mpad]).  Per group, lane t
// quantises channels 8t .. 8t+7, i.e. slice u = t/8, half h = (t/4)%2,
// fields 8(t%4) .. +7 (48 bits at bit 48(t%4) of lane m%32 + 32h's six
// dwords); lanes t and t^1 pair their 48-bit chunks and the even one writes
// the three dwords they fill.  Tokens in [M, Mpad) get codes 0, no scale.
constexpr int kActGroups = 4;  // groups per act-quant team

__device__ __forceinline__ void act_quant_fp6_group(const uint4 raw, int64_t m, int t, int64_t G, int64_t j,
                                                    uint8_t* __restrict__ aimg, float* __restrict__ saT,
                                                    int64_t Mpad) {
  float f[8];
  unpack_h8(raw, f);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  amax = row16_max(amax);
  const float s = amax / 7.0f;
  const float r = s == 0.0f ? 0.0f : 1.0f / s;
  const uint64_t own = quant4_fields8(f, s, r);
  const uint32_t plo = (uint32_t)__shfl_xor((int)(uint32_t)own, 1, 16);
  const uint32_t phi = (uint32_t)__shfl_xor((int)(uint32_t)(own >> 32), 1, 16);
  if ((t & 1) == 0) {
    const uint64_t par = ((uint64_t)phi << 32) | plo;
    const uint32_t d0 = (uint32_t)own;
    const uint32_t d1 = (uint32_t)(own >> 32) | (uint32_t)(par << 16);
    const uint32_t d2 = (uint32_t)(par >> 16);
    const int u = t >> 3, h = (t >> 2) & 1, l = (int)(m & 31) + 32 * h;
    uint8_t* img = aimg + ((m >> 5) * G + j) * kFp6Frag;
    if ((t & 2) == 0) {  // fields 0-15: dwords 0-2
      uint32_t* p = reinterpret_cast<uint32_t*>(img + fp6_lo_offset(u, l));
      *reinterpret_cast<uint2*>(p) = make_uint2(d0, d1);
      p[2] = d2;
    } else {  // fields 16-31: dword 3, dwords 4-5
      reinterpret_cast<uint32_t*>(img + fp6_lo_offset(u, l))[3] = d0;
      *reinterpret_cast<uint2*>(img + fp6_hi_offset(u, l)) = make_uint2(d1, d2);
    }
  }
  if (t == 0) saT[j * Mpad + m] = s;  // group-major; padding rows get 0
}

__device__ __forceinline__ void act_quant_fp6_body(const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx,
                                                   uint8_t* __restrict__ aimg, float* __restrict__ saT, int64_t Mpad,
                                                   int64_t bx, int64_t jq) {
  const int64_t m = bx * 16 + (threadIdx.x >> 4);
  const int t = threadIdx.x & 15;
  if (m >= Mpad) return;  // whole 16-lane teams leave together
  const int64_t G = K / kGroup, j0 = jq * kActGroups;
  const int nj = (int)min((int64_t)kActGroups, G - j0);  // the same for the whole workgroup
  uint4 raw[kActGroups];
#pragma unroll
  for (int q = 0; q < kActGroups; ++q) {
    raw[q] = make_uint4(0, 0, 0, 0);  // fp16 zeros: padding rows
    if (m < M && q < nj) raw[q] = *reinterpret_cast<const uint4*>(x + m * ldx + (j0 + q) * kGroup + t * 8);
  }
#pragma unroll
  for (int q = 0; q < kActGroups; ++q)
    if (q < nj) act_quant_fp6_group(raw[q], m, t, G, j0 + q, aimg, saT, Mpad);
}

// A lane's 32 codes (four packed words) -> its two pieces of slice u.
__device__ __forceinline__ void put_lane(uint8_t* img, int u, int l, const uint4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t d[6];
  fp6_fields32(w, d);
  *reinterpret_cast<uint4*>(img + fp6_lo_offset(u, l)) = make_uint4(d[0], d[1], d[2], d[3]);
  *reinterpret_cast<uint2*>(img + fp6_hi_offset(u, l)) = make_uint2(d[4], d[5]);
}

// Packed row-major activation codes [M][K/2] -> image; rows past M zeros.
__global__ __launch_bounds__(256) void acts_fp6_kernel(const uint8_t* __restrict__ qa, int64_t M, int64_t K,
                                                       uint8_t* __restrict__ aimg, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t G = K / kGroup;
  const int l = (int)(i & 63);
  const int u = (int)((i >> 6) & 1);
  const int64_t bj = i >> 7;  // row block * G + group
  const int64_t rb = bj / G, j = bj - rb * G;
  const int64_t m = rb * 32 + (l & 31);
  uint4 v = make_uint4(0, 0, 0, 0);
  if (m < M) v = *reinterpret_cast<const uint4*>(qa + m * (K / 2) + j * 64 + u * 32 + (l >> 5) * 16);
  put_lane(aimg + bj * kFp6Frag, u, l, v);
}

// Base weight codes in the slab layout (row n, group j, codes 32c .. 32c+31
// at qw + (n/16)*8K + j*1024 + (16c + n%16)*16) -> image.
__device__ __forceinline__ uint4 weights_fp6_load(const uint8_t* __restrict__ qw, int64_t K, int64_t i) {
  const int64_t G = K / kGroup;
  const int l = (int)(i & 63);
  const int u = (int)((i >> 6) & 1);
  const int64_t bj = i >> 7;  // column block * G + group
  const int64_t cb = bj / G, j = bj - cb * G;
  const int64_t n = cb * 32 + (l & 31);
  const int c = 2 * u + (l >> 5);
  return *reinterpret_cast<const uint4*>(qw + (n >> 4) * 8 * K + j * 1024 + (16 * c + (n & 15)) * 16);
}

__device__ __forceinline__ void weights_fp6_body(const uint8_t* __restrict__ qw, int64_t K, uint8_t* __restrict__ wimg,
                                                 int64_t total, int64_t bx) {
  const int64_t i = bx * 256 + threadIdx.x;
  if (i >= total) return;
  put_lane(wimg + (i >> 7) * kFp6Frag, (int)((i >> 6) & 1), (int)(i & 63), weights_fp6_load(qw, K, i));
}

// Residual blocks (row r of block e: b/2 bytes at qr + (e*b + r)*(b/2)) ->
// image: one thread per (block, piece, lane); piece p = c*(b/64) + u covers
// rows 32c .. 32c+31 and codes 64u .. 64u+63 of the block.
__device__ __forceinline__ void residual_fp6_body(const uint8_t* __restrict__ qr, int b, uint8_t* __restrict__ rimg,
                                                  int64_t total, int64_t bx) {
  const int64_t i = bx * 256 + threadIdx.x;
  if (i >= total) return;
  const int l = (int)(i & 63);
  const int np = (b / 32) * (b / 64);  // pieces per block
  const int64_t ep = i >> 6;
  const int64_t e = ep / np;
  const int p = (int)(ep - e * np);
  const int c = p / (b / 64), u = p % (b / 64);
  const int64_t r = c * 32 + (l & 31);
  const uint4 v = *reinterpret_cast<const uint4*>(qr + (e * b + r) * (b / 2) + u * 32 + (l >> 5) * 16);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t d[6];
  fp6_fields32(w, d);
  uint8_t* piece = rimg + e * ((int64_t)b * b * 3 / 4) + (int64_t)p * 1536;
  *reinterpret_cast<uint4*>(piece + 16 * l) = make_uint4(d[0], d[1], d[2], d[3]);
  *reinterpret_cast<uint2*>(piece + 1024 + 8 * l) = make_uint2(d[4], d[5]);
}

__global__ __launch_bounds__(256) void weights_fp6_kernel(const uint8_t* __restrict__ qw, int64_t K,
                                                          uint8_t* __restrict__ wimg, int64_t total) {
  weights_fp6_body(qw, K, wimg, total, blockIdx.x);
}
__global__ __launch_bounds__(256) void residual_fp6_kernel(const uint8_t* __restrict__ qr, int b,
                                                           uint8_t* __restrict__ rimg, int64_t total) {
  residual_fp6_body(qr, b, rimg, total, blockIdx.x);
}

// The fp6 layer's three preparations in one launch: blocks [0, na) quantise
// the activations, the next nw convert the base, the rest the residual
// blocks.  They are independent and bound by memory traffic; one grid lets
// them share the machine instead of running back to back.
struct Fp6Prep {
  const uint16_t* x;
  int64_t M, K, ldx, Mpad;
  uint8_t* aimg;
  float* sa;
  const uint8_t* qw;
  const uint16_t* sw;
  int64_t N;
  uint8_t* wimg;
  uint16_t* swT;
  int64_t wtotal;
  const uint8_t* qr;
  int block;
  uint8_t* rimg;
  int64_t rtotal;
  int64_t na_x, na, nw;  // act-quant grid width (Mpad/16), act-quant blocks, base blocks
};
constexpr int kWeightItems = 4;  // base-image items per thread of the preparation launch
__global__ __launch_bounds__(256) void fp6_prep_kernel(Fp6Prep p) {
  const int64_t b = blockIdx.x;
  if (b < p.na) {
    act_quant_fp6_body(p.x, p.M, p.K, p.ldx, p.aimg, p.sa, p.Mpad, b % p.na_x, b / p.na_x);
  } else if (b < p.na + p.nw) {
    // items bw*1024 + 256q + tid, q < 4: the four loads first
    const int64_t i0 = (b - p.na) * (256 * kWeightItems) + threadIdx.x;
    uint4 v[kWeightItems];
#pragma unroll
    for (int q = 0; q < kWeightItems; ++q)
      if (i0 + 256 * q < p.wtotal) v[q] = weights_fp6_load(p.qw, p.K, i0 + 256 * q);
#pragma unroll
    for (int q = 0; q < kWeightItems; ++q) {
      const int64_t i = i0 + 256 * q;
      if (i >= p.wtotal) break;
      const int l = (int)(i & 63), u = (int)((i >> 6) & 1);
      put_lane(p.wimg + (i >> 7) * kFp6Frag, u, l, v[q]);
      // the weight scales group-major: the thread of (column block cb,
      // group j, slice 0, lane l < 32) copies sw[n][j], n = 32 cb + l
      if (u == 0 && l < 32) {
        const int64_t G = p.K / kGroup, bj = i >> 7;
        const int64_t cb = bj / G, j = bj - cb * G, n = cb * 32 + l;
        p.swT[j * p.N + n] = p.sw[n * G + j];
      }
    }
  } else {
    residual_fp6_body(p.qr, p.block, p.rimg, p.rtotal, b - p.na - p.nw);
  }
}

}  // namespace

hipError_t launch_fp6_layer_prep(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* aimg, float* saT,
                                 const uint8_t* qw, const uint16_t* sw, int64_t N, uint8_t* wimg, uint16_t* swT,
                                 const uint8_t* qr, int n_select, int block, uint8_t* rimg, hipStream_t st) {
  Fp6Prep p;
  p.x = x;
  p.M = M;
  p.K = K;
  p.ldx = ldx;
  p.Mpad = wide_rows(M);
  p.aimg = aimg;
  p.sa = saT;
  p.qw = qw;
  p.sw = sw;
  p.N = N;
  p.wimg = wimg;
  p.swT = swT;
  p.wtotal = wimg ? N / 32 * (K / kGroup) * 128 : 0;  // no image: the kernel reads the slabs
  p.qr = qr;
  p.block = block;
  p.rimg = rimg;
  p.rtotal = n_select > 0 ? (int64_t)n_select * (block / 32) * (block / 64) * 64 : 0;
  p.na_x = p.Mpad / 16;
  p.na = p.na_x * ((K / kGroup + kActGroups - 1) / kActGroups);
  p.nw = (p.wtotal + 256 * kWeightItems - 1) / (256 * kWeightItems);
  const int64_t nr = (p.rtotal + 255) / 256;
  hipLaunchKernelGGL(fp6_prep_kernel, dim3((unsigned)(p.na + p.nw + nr)), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_acts_fp6(const uint8_t* qa, int64_t M, int64_t K, uint8_t* aimg, hipStream_t st) {
  const int64_t total = wide_rows(M) / 32 * (K / kGroup) * 128;
  hipLaunchKernelGGL(acts_fp6_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, qa, M, K, aimg,
                     total);
  return hipGetLastError();
}

hipError_t launch_weights_fp6(const uint8_t* qw, int64_t N, int64_t K, uint8_t* wimg, hipStream_t st) {
  const int64_t total = N / 32 * (K / kGroup) * 128;
  hipLaunchKernelGGL(weights_fp6_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, qw, K, wimg,
                     total);
  return hipGetLastError();
}

hipError_t launch_residual_fp6(const uint8_t* qr, int n_select, int block, uint8_t* rimg, hipStream_t st) {
  if (n_select <= 0) return hipSuccess;
  const int64_t total = (int64_t)n_select * (block / 32) * (block / 64) * 64;
  hipLaunchKernelGGL(residual_fp6_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, qr, block,
                     rimg, total);
  return hipGetLastError();
}

}  // namespace mq
