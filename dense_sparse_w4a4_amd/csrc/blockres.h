// Per-row arithmetic of a residual block, shared by the Delta-score kernel and
// the residual packing kernel so both see bit-identical scales and codes.
//
// For output row `wrow` (fp16, K entries) and the block whose first input
// channel is `kb` (block edge b, inside one 128-wide group):
//   sw = f16(max_{k in group} |w_k| / 7)          base scale of the group
//   e_c = w_c - f32(sw) * quant4(w_c, f32(sw))    base error, fp32
//   sr = f16(max_{c<b} |e_c| / 7)                 residual scale of the row
// MosaicQuant technical summary (gist.science/pt/paper/2606.15652),
// Metodologia 1: the 4-bit residual compensates the base's quantisation
// error; Metodologia 2: the residual is allocated per block.
#pragma once

#include "mq_internal.h"

namespace mq {

struct RowScales {
  float swf;         // base scale as fp32
  float srf;         // residual scale as fp32
  uint16_t sr_bits;  // residual scale as fp16 bits
};

__device__ __forceinline__ float base_err(float w, float swf) {
  const float q = (float)quant4(w, swf);
  const float p = swf * q;  // exact: 11-bit x 3-bit significands
  return w - p;
}

__device__ inline RowScales row_scales(const uint16_t* __restrict__ wrow, int64_t kb, int b) {
  const int64_t g0 = (kb / kGroup) * kGroup;
  float amax = 0.0f;
  for (int c = 0; c < kGroup; c += 8) {
    float f[8];
    unpack_h8(*reinterpret_cast<const uint4*>(wrow + g0 + c), f);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  }
  RowScales rs;
  rs.swf = h2f(f2h_bits(amax / 7.0f));
  float ramax = 0.0f;
  for (int c = 0; c < b; c += 8) {
    float f[8];
    unpack_h8(*reinterpret_cast<const uint4*>(wrow + kb + c), f);
#pragma unroll
    for (int i = 0; i < 8; ++i) ramax = fmaxf(ramax, fabsf(base_err(f[i], rs.swf)));
  }
  rs.sr_bits = f2h_bits(ramax / 7.0f);
  rs.srf = h2f(rs.sr_bits);
  return rs;
}

}  // namespace mq
