// Internal helpers shared by the HIP translation units of libmosaicq.
// Device-side numerics here fix the bit-exact conventions of the library:
// IEEE fp32 division (hipcc's default correctly rounded division; the build
// never enables fast-math), rint = round half to even (v_rndne_f32),
// fp32 -> fp16 round to nearest even with subnormals kept (v_cvt_f16_f32
// under the default mode register).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mosaicq.h"

namespace mq {

constexpr int kGroup = 128;
constexpr int kQmax = 7;

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float h2f(uint16_t b) {
  _Float16 h = __builtin_bit_cast(_Float16, b);
  return (float)h;
}

__device__ __forceinline__ uint16_t f2h_bits(float f) {
  _Float16 h = (_Float16)f;  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

// Symmetric 4-bit code: clamp(rint(v / s), -7, 7), 0 when s == 0.
__device__ __forceinline__ int quant4(float v, float s) {
  if (s == 0.0f) return 0;
  float r = rintf(v / s);
  r = fminf(fmaxf(r, -7.0f), 7.0f);
  return (int)r;
}

// Two codes per byte along K, low nibble first, two's complement.
__device__ __forceinline__ uint32_t pack8(const int q[8]) {
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) w |= ((uint32_t)q[i] & 0xFu) << (4 * i);
  return w;
}

// Eight fp16 values held in a uint4 -> floats.
__device__ __forceinline__ void unpack_h8(const uint4& v, float f[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = h2f((uint16_t)(w[i] & 0xFFFFu));
    f[2 * i + 1] = h2f((uint16_t)(w[i] >> 16));
  }
}

}  // namespace mq

// ---------------------------------------------------------------------------
// Host side: error reporting and launchers (defined in the .hip files).
// ---------------------------------------------------------------------------
namespace mq {

void set_error(const char* fmt, ...);
mq_status fail(mq_status s, const char* fmt, ...);

hipError_t launch_act_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                            uint8_t* qa, float* sa, hipStream_t st);

hipError_t launch_select(const uint16_t* w, const uint16_t* xc, int64_t N, int64_t K,
                         int64_t T, int block, int n_select, int32_t* selected,
                         double* delta, double* hdiag, hipStream_t st);

hipError_t launch_pack(const uint16_t* w, int64_t N, int64_t K, int block,
                       const int32_t* selected, int n_select, uint8_t* qw, uint16_t* sw,
                       int32_t* row_ptr, int32_t* col_idx, uint8_t* qr, uint16_t* sr,
                       hipStream_t st);

struct GemmArgs {
  const uint8_t* qa;
  const float* sa;
  int64_t M, N, K;
  const uint8_t* qw;
  const uint16_t* sw;
  int block;
  int n_select;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const uint8_t* qr;
  const uint16_t* sr;
  uint16_t* y;
  int64_t ldy;
  int32_t* acc_dump;  // non-null => dump accumulators
  float* part;        // split-K partial outputs [ksplit][M][N] (tile kernel), or null
  int ksplit;         // K splits of the tile kernel (1 = none)
};

hipError_t launch_fused_gemm(const GemmArgs& a, hipStream_t st);
hipError_t launch_residual_merge(const GemmArgs& a, hipStream_t st);
hipError_t launch_smooth_weights(const uint16_t* xc, int64_t T, const uint16_t* w, int64_t N,
                                 int64_t K, float* ax, float* aw, float* s, uint16_t* w_out,
                                 hipStream_t st);
hipError_t launch_smooth_acts(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const float* s,
                              uint16_t* x_out, hipStream_t st);
bool tile_gemm_fits(const GemmArgs& a);
int tile_gemm_splits(int64_t M, int64_t N, int64_t K);  // K splits the tile kernel would use
hipError_t launch_tile_gemm(const GemmArgs& a, hipStream_t st);

}  // namespace mq
