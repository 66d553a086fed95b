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
#include "mq_internal.h"

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
  int q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = quant4_rcp(f[i], s, r);
  *reinterpret_cast<uint32_t*>(qa + m * (K / 2) + j * (kGroup / 2) + t * 4) = pack8(q);
  if (t == 0) sa[m * G + j] = s;
}

}  // namespace

hipError_t launch_act_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                            uint8_t* qa, float* sa, hipStream_t st) {
  const int64_t groups = M * (K / kGroup);
  const int64_t blocks = (groups + 15) / 16;
  hipLaunchKernelGGL(act_quant_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, K, ldx,
                     qa, sa, groups);
  return hipGetLastError();
}

}  // namespace mq
