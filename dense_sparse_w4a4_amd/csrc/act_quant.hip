// Activation quantisation Qa(X): per token and group of 128 input channels,
// scale = amax/7 (fp32) and 4-bit codes packed two per byte.
// MosaicQuant technical summary (gist.science/pt/paper/2606.15652),
// Metodologia 3: quantisation is one stage of the online 4-bit pipeline.
//
// Mapping: a team of 16 lanes owns one (token, group); lane t loads 8 fp16
// (one 16-byte load) at channels t*8 .. t*8+7, the team reduces amax across
// its DPP row, and lane t writes one 32-bit word of codes.  A 64-lane wave
// covers 4 groups, so loads and stores are fully coalesced 256-byte / 64-byte
// runs.  The kernel is HBM-bound: 2 bytes read, 0.5 byte written per element.
#include "gemm_common.h"

namespace mq {
namespace {

__global__ __launch_bounds__(256) void act_quant_kernel(const uint16_t* __restrict__ x,
                                                        int64_t K, int64_t ldx,
                                                        uint8_t* __restrict__ qa,
                                                        float* __restrict__ sa,
                                                        int64_t total_groups) {
  const int64_t gid = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int t = threadIdx.x & 15;
  if (gid >= total_groups) return;  // whole 16-lane teams leave together
  const int64_t G = K / kGroup;
  const int64_t m = gid / G;
  const int64_t j = gid - m * G;

  const uint4 v = *reinterpret_cast<const uint4*>(x + m * ldx + j * kGroup + t * 8);
  float f[8];
  unpack_h8(v, f);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  amax = row16_max(amax);  // the team is one DPP row of 16 lanes

  const float s = amax / 7.0f;
  // codes from the reciprocal with one correction step: equal to quant4's
  // IEEE quotient for every fp16 value and every scale amax/7 of an fp16
  // amax >= |value| (checked exhaustively on the host), at three operations
  // per code instead of a division
  const float r = s == 0.0f ? 0.0f : 1.0f / s;
  *reinterpret_cast<uint32_t*>(qa + m * (K / 2) + j * (kGroup / 2) + t * 4) = quant4_word(f, s, r);
  if (t == 0) sa[m * G + j] = s;
}

// The same quantisation, written in the wide fragment order of the prefill
// tile kernel (wide_a_index): codes as int8 16*q, so that kernel copies
// them from memory to LDS without widening them.  One 16-lane team per
// token, 16 consecutive tokens of one group per workgroup, so each 1 KB
// fragment receives 256 contiguous bytes per workgroup.  Tokens in
// [M, Mpad) (the last row block's padding) get codes 0 and no scale.
__global__ __launch_bounds__(256) void act_quant_wide_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                             int64_t K, int64_t ldx, uint8_t* __restrict__ qaw,
                                                             float* __restrict__ sa, int64_t Mpad) {
  const int64_t m = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int t = threadIdx.x & 15;
  if (m >= Mpad) return;  // whole 16-lane teams leave together
  const int64_t G = K / kGroup;
  const int64_t j = blockIdx.y;
  float f[8];
  if (m < M) {
    unpack_h8(*reinterpret_cast<const uint4*>(x + m * ldx + j * kGroup + t * 8), f);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = 0.0f;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  amax = row16_max(amax);
  const float s = amax / 7.0f;
  const float r = s == 0.0f ? 0.0f : 1.0f / s;
  const uint32_t w = quant4_word(f, s, r);  // codes 8t .. 8t+7, low nibble first
  // lane t holds codes 8t .. 8t+7: step t/4, half (t%4)/2, the first or
  // second 8 bytes of that lane chunk: even codes, then odd codes, as 16*q
  uint2 v;
  v.x = (w << 4) & 0xF0F0F0F0u;
  v.y = w & 0xF0F0F0F0u;
  *reinterpret_cast<uint2*>(qaw + wide_a_index(m, j, G, t >> 2, (t >> 1) & 1) + (t & 1) * 8) = v;
  if (t == 0 && m < M) sa[m * G + j] = s;
}

// The same quantisation, written in 16-token tiles for the streaming kernel
// (tiled_a_index): one workgroup per (tile, group) writes that group's 1 KB
// of the tile, so every weight-stream step reads its activation codes as one
// contiguous 1 KB instead of 64 bytes from each of 16 rows.  Tokens in
// [M, Mpad) (the last tile's padding) get codes 0 and no scale.
__global__ __launch_bounds__(256) void act_quant_tiled_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                              int64_t K, int64_t ldx, uint8_t* __restrict__ qat,
                                                              float* __restrict__ sa) {
  const int64_t m = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int t = threadIdx.x & 15;
  const int64_t G = K / kGroup;
  const int64_t j = blockIdx.y;
  float f[8];
  if (m < M) {
    unpack_h8(*reinterpret_cast<const uint4*>(x + m * ldx + j * kGroup + t * 8), f);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = 0.0f;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  amax = row16_max(amax);
  const float s = amax / 7.0f;
  const float r = s == 0.0f ? 0.0f : 1.0f / s;
  *reinterpret_cast<uint32_t*>(qat + tiled_a_index(m, j, G) + t * 4) = quant4_word(f, s, r);
  if (t == 0 && m < M) sa[m * G + j] = s;
}

}  // namespace

hipError_t launch_act_quant_tiled(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* qat,
                                  float* sa, hipStream_t st) {
  hipLaunchKernelGGL(act_quant_tiled_kernel, dim3((unsigned)(tiled_rows(M) / 16), (unsigned)(K / kGroup)),
                     dim3(256), 0, st, x, M, K, ldx, qat, sa);
  return hipGetLastError();
}

hipError_t launch_act_quant_wide(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* qaw,
                                 float* sa, hipStream_t st) {
  const int64_t Mpad = wide_rows(M);
  hipLaunchKernelGGL(act_quant_wide_kernel, dim3((unsigned)(Mpad / 16), (unsigned)(K / kGroup)), dim3(256), 0,
                     st, x, M, K, ldx, qaw, sa, Mpad);
  return hipGetLastError();
}

hipError_t launch_act_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                            uint8_t* qa, float* sa, hipStream_t st) {
  const int64_t groups = M * (K / kGroup);
  const int64_t blocks = (groups + 15) / 16;
  hipLaunchKernelGGL(act_quant_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, K, ldx,
                     qa, sa, groups);
  return hipGetLastError();
}

}  // namespace mq
