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

// The same code from the reciprocal r = 1/s (r = 0 when s = 0): q0 = v*r,
// e = v - q0*s (one fma, exact), q1 = q0 + e*r (one fma), which is the
// correctly rounded quotient v/s (Markstein's correction).  An exhaustive
// check over every fp16 v and every scale s = amax/7 with fp16 amax >= |v|
// finds q1 equal to the IEEE quotient except for the sign of a zero
// quotient, so the codes equal quant4's; three operations per code instead
// of a full division.
__device__ __forceinline__ int quant4_rcp(float v, float s, float r) {
  const float q0 = v * r;
  const float e = fmaf(-q0, s, v);
  const float q1 = fmaf(e, r, q0);
  return (int)fminf(fmaxf(rintf(q1), -7.0f), 7.0f);
}

// Max over each row of 16 lanes (DPP: swap neighbours, swap pairs, mirror
// within 8, mirror within 16), for non-negative floats, whose bit patterns
// order like their values.  Every lane of the row must be active.
__device__ __forceinline__ float row16_max(float v) {
  int b = __float_as_int(v);
  b = max(b, __builtin_amdgcn_update_dpp(b, b, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  b = max(b, __builtin_amdgcn_update_dpp(b, b, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  b = max(b, __builtin_amdgcn_update_dpp(b, b, 0x141, 0xF, 0xF, false));  // row_half_mirror
  b = max(b, __builtin_amdgcn_update_dpp(b, b, 0x140, 0xF, 0xF, false));  // row_mirror
  return __int_as_float(b);
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
  const uint16_t* x;  // fp16 activations [M][ldx] to quantise in the streaming
  int64_t ldx;        // kernel (qa, sa unused), or null
};

// In-kernel activation quantisation of the streaming kernel: at most
// kStreamQuantRows tokens, and every (token, group) pair of the tile within
// 4 passes of the workgroup's 16-lane teams.
constexpr int kStreamQuantRows = 4;
// LDS byte offset of the streaming kernel's activation codes: after the
// [G][16] activation scale table, the [G][16*ns + 1] weight scale table
// (rows padded by one slot so that the staging stores, which walk the groups
// of one channel, fall in distinct LDS banks), rounded up to 16 bytes, and
// the spare slots.
__host__ __device__ constexpr int stream_qa_offset(int G, int ns) {
  return 64 * G + (((16 * ns + 1) * G + 3) / 4) * 16 + 16;
}
// Launch shape of the streaming kernel: 16-channel slabs per workgroup,
// waves per workgroup, groups per streamed unit, quantisation passes (0:
// the activations arrive as codes).
struct StreamPlan {
  int ns, ks, u, qp;
};
StreamPlan stream_plan(int64_t M, int64_t N, int64_t K, int block, bool quantise, bool dump);
int stream_waves(int64_t M, int64_t N, int64_t K, int ns);
int stream_quant_passes(int64_t M, int64_t K, int ks);
bool stream_quant_fits(int64_t M, int64_t N, int64_t K);
size_t stream_lds_bytes(int64_t K, int ks, int rows, int ns);

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
