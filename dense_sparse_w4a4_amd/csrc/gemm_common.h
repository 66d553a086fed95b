// Helpers shared by the fused GEMM kernels.
#pragma once

#include "mq_internal.h"

namespace mq {

// Eight packed two's-complement codes per 32-bit word -> int8 MFMA lanes.
// Each code stays in the high nibble of its byte (byte = 16*q), so no sign
// extension is needed; the even codes of a word go to one 32-bit lane word
// and the odd codes to the next.  Both MFMA operands are widened the same
// way, so the k permutation cancels in the dot product and the accumulator
// holds 256 x the exact integer sum.
__device__ __forceinline__ v4i widen8(uint32_t lo, uint32_t hi) {
  v4i r;
  r[0] = (int)((lo << 4) & 0xF0F0F0F0u);
  r[1] = (int)(lo & 0xF0F0F0F0u);
  r[2] = (int)((hi << 4) & 0xF0F0F0F0u);
  r[3] = (int)(hi & 0xF0F0F0F0u);
  return r;
}

__device__ __forceinline__ v4i mfma(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint4 ld16(const uint8_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

constexpr float kInv256 = 1.0f / 256.0f;

// S_WAITCNT immediate (gfx9 family): vmcnt(4) with expcnt and lgkmcnt left
// unconstrained (vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr unsigned kWaitVm4 = 0x4u | (0x7u << 4) | (0xFu << 8);
constexpr unsigned kWaitVm5 = 0x5u | (0x7u << 4) | (0xFu << 8);

}  // namespace mq
