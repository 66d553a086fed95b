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

// Symmetric 4-bit code: clamp(rint(v / s), -7, 7), 0 when s == 0 or when
// the quotient is not a number (inf/inf).
__device__ __forceinline__ int quant4(float v, float s) {
  if (s == 0.0f) return 0;
  float r = rintf(v / s);
  if (r != r) return 0;
  r = fminf(fmaxf(r, -7.0f), 7.0f);
  return (int)r;
}

// The same code from the reciprocal r = 1/s (r = 0 when s = 0): q0 = v*r,
// e = v - q0*s (one fma, exact), q1 = q0 + e*r (one fma), which is the
// correctly rounded quotient v/s (Markstein's correction).  An exhaustive
// check over every finite fp16 amax, every scale s = amax/7 and every fp16
// v with |v| <= amax finds q1 equal to the IEEE quotient except for the
// sign of a zero quotient, so the codes equal quant4's; three operations
// per code instead of a full division.  For an infinite scale (a group
// holding +-inf) the caller replaces the group's codes by quant4's, all 0
// (see quant4_word).
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

// Eight codes of one activation group under scale s (reciprocal r), packed:
// the reciprocal route for a finite scale; for s = +inf (the group holds an
// infinite value) every code is quant4's, 0 (v/inf = 0, inf/inf -> 0).
__device__ __forceinline__ uint32_t quant4_word(const float f[8], float s, float r) {
  int q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = quant4_rcp(f[i], s, r);
  return s < __builtin_inff() ? pack8(q) : 0u;
}

// Wide activation layout of the prefill tile kernel: int8 codes 16*q in the
// kernel's MFMA fragment order, uint8 [Mpad/32][G][4][64][16].  For token m
// (row block m/32, row r = m%32), group j, 32-channel step t and half h, the
// 16 bytes at [m/32][j][t][r + 32h] hold the codes 32t + 16h + (0, 2, 4, 6,
// 1, 3, 5, 7, 8, 10, 12, 14, 9, 11, 13, 15) of the group (the order widen8
// gives for 8 packed bytes), so one row block's group is 4 KB contiguous
// and each 1 KB step fragment is copied to LDS as it is.  Rows past M (up to
// Mpad, a multiple of 32) hold zeros.
__host__ __device__ constexpr int64_t wide_rows(int64_t M) { return (M + 31) / 32 * 32; }
__host__ __device__ inline int64_t wide_a_index(int64_t m, int64_t j, int64_t G, int t, int h) {
  return (((m >> 5) * G + j) * 4 + t) * 1024 + ((m & 31) + 32 * h) * 16;
}

// FP6 operand images of the prefill tile kernel's fp6 route.  The 4-bit
// codes go to the matrix core as FP6 E2M3 fields in sign-magnitude: the
// field of q is |q| (<= 8) with the sign in bit 5.  E2M3 with an exponent
// field of 0 or 1 is linear in its low five bits (n/8 for n <= 15), so the
// field's value is exactly q/8, every product q_a*q_w/64 and every sum of
// them is exact in fp32, and V_MFMA_F32_32X32X64_F8F6F4 returns the exact
// integer dot product / 64 at twice the int8 instruction's K per cycle.
//
// Layout: a 32-row block (tokens or output channels) and one group of 128
// codes take 3 KB, the images of the two 32x32x64 operands (k slices
// u = 0, 1 of 64 codes).  Lane l = r + 32h (row r, half h) holds the codes
// 64u + 32h + i, i = 0..31, as fields at bits 6i of six dwords: dwords 0-3
// at [u * 1024 + 16 l], dwords 4-5 at [2048 + u * 512 + 8 l].  The image of
// a row block's group is copied to LDS as it is (three 1 KB pieces).
constexpr int kFp6Frag = 3072;

// Eight packed two's-complement codes (low nibble first) -> eight fields,
// field i at bits 6i .. 6i+5 of the result.
__device__ __forceinline__ uint64_t fp6_fields8(uint32_t w) {
  const uint32_t s = w & 0x88888888u;           // sign bit of each code
  const uint32_t t = s >> 3;                    // 1 in each negative code
  const uint32_t m = (w ^ ((s - t) + s)) + t;   // |q| in each nibble (no carries: |q| <= 8)
  uint64_t r = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t f = ((m >> (4 * i)) & 0xFu) | (((t >> (4 * i)) & 1u) << 5);
    r |= (uint64_t)f << (6 * i);
  }
  return r;
}

// quant4_word's eight codes written directly as FP6 fields (field i at bits
// 6i of the result): the same reciprocal quotient, rint and clamp, then
// |q| | (q < 0) << 5 (a code of -0.0 counts as 0); every field 0 for an
// infinite scale.
__device__ __forceinline__ uint64_t quant4_fields8(const float f[8], float s, float r) {
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float q0 = f[i] * r;
    const float e = fmaf(-q0, s, f[i]);
    const float q = fminf(fmaxf(rintf(fmaf(e, r, q0)), -7.0f), 7.0f);
    const uint32_t fld = (uint32_t)fabsf(q) | (q < 0.0f ? 32u : 0u);
    if (6 * i + 6 <= 32) {
      lo |= fld << (6 * i);
    } else if (6 * i >= 32) {
      hi |= fld << (6 * i - 32);
    } else {
      lo |= fld << (6 * i);
      hi |= fld >> (32 - 6 * i);
    }
  }
  return s < __builtin_inff() ? ((uint64_t)hi << 32) | lo : 0u;
}

// 32 codes (four words, code i in nibble i % 8 of word i / 8) -> the six
// operand dwords of one lane.
__device__ __forceinline__ void fp6_fields32(const uint32_t w[4], uint32_t d[6]) {
  const uint64_t a = fp6_fields8(w[0]), b = fp6_fields8(w[1]);
  const uint64_t c = fp6_fields8(w[2]), e = fp6_fields8(w[3]);
  d[0] = (uint32_t)a;
  d[1] = (uint32_t)(a >> 32) | (uint32_t)(b << 16);
  d[2] = (uint32_t)(b >> 16);
  d[3] = (uint32_t)c;
  d[4] = (uint32_t)(c >> 32) | (uint32_t)(e << 16);
  d[5] = (uint32_t)(e >> 16);
}

// Byte offsets of a lane's two pieces within a 3 KB row-block group image.
__host__ __device__ constexpr int fp6_lo_offset(int u, int l) { return u * 1024 + 16 * l; }
__host__ __device__ constexpr int fp6_hi_offset(int u, int l) { return 2048 + u * 512 + 8 * l; }

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

// Activation quantisation written in the prefill tile kernel's wide
// fragment order (int8 codes, [ceil(M/32)][K/128][4][64][16] bytes) plus the
// fp32 scales [M][K/128].
// Packed codes of token m, group j (64 bytes) in 16-token tiles: each
// group's codes of a tile are one contiguous 1 KB, rows 64 bytes apart.
__host__ __device__ inline int64_t tiled_a_index(int64_t m, int64_t j, int64_t G) {
  return ((m >> 4) * G + j) * 1024 + (m & 15) * 64;
}
inline int64_t tiled_rows(int64_t M) { return (M + 15) / 16 * 16; }
hipError_t launch_act_quant_tiled(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* qat,
                                  float* sa, hipStream_t st);
hipError_t launch_act_quant_wide(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* qaw,
                                 float* sa, hipStream_t st);

hipError_t launch_select(const uint16_t* w, const uint16_t* xc, int64_t N, int64_t K,
                         int64_t T, int block, int n_select, int32_t* selected,
                         double* delta, double* hdiag, hipStream_t st);

// Exact output distortion and the greedy selection by it (offline study of
// the Delta-score); workspaces in bytes for the given shape.
size_t exact_greedy_workspace(int64_t N, int64_t K, int64_t T, int b);
size_t distortion_workspace(int64_t N, int64_t K, int64_t T, int b);
hipError_t launch_exact_greedy(const uint16_t* w, const uint16_t* x, int64_t N, int64_t K,
                               int64_t T, int b, int n_select, int32_t* selected, int32_t* order,
                               double* gains, double* dist, void* ws, hipStream_t st);
hipError_t launch_distortion(const uint16_t* w, const uint16_t* x, int64_t N, int64_t K,
                             int64_t T, int b, const int32_t* ids, int64_t n_ids, double* dist,
                             void* ws, hipStream_t st);

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
  int split_tail;     // fp6 route: the last split_tail tiles take the K splits
                      // (set by its launcher from the plan)
  const uint16_t* x;  // fp16 activations [M][ldx] to quantise in the streaming
  int64_t ldx;        // kernel (qa, sa unused), or null
  const uint8_t* qaw; // tile kernel: activation codes in the wide fragment order
                      // (wide_a_index), copied to LDS as they are, or null
                      // (packed qa, widened while staged)
  const uint8_t* qat; // streaming kernel: packed activation codes in 16-token
                      // tiles (tiled_a_index), or null (qa row-major)
  // fp6 route of the tile kernel (aimg and rimg set, or none): FP6 images of
  // the activation codes [ceil(M/32)][K/128][3 KB], the base weight codes
  // [N/32][K/128][3 KB] (or null: the kernel reads the packed slabs qw) and
  // the residual blocks [n_select][b*b*3/4]
  const uint8_t* aimg;
  const uint8_t* wimg;
  const uint8_t* rimg;
  // fp6 route, optional: the scales group-major (saT [K/128][saT_ld] fp32,
  // swT [K/128][N] fp16), so that a tile's scales of one group are one
  // contiguous run; null: sa [M][K/128], sw [N][K/128]
  const float* saT;
  const uint16_t* swT;
  int64_t saT_ld;
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
hipError_t launch_mfma_rate(int blocks, int iters, int64_t* cycles, int32_t* sink, hipStream_t st);
bool tile_gemm_fits(const GemmArgs& a);
int tile_gemm_splits(int64_t M, int64_t N, int64_t K);  // K splits the tile kernel would use
hipError_t launch_tile_gemm(const GemmArgs& a, hipStream_t st);
// Packed activation codes qa [M][K/2] -> the wide fragment order.
hipError_t launch_widen_acts(const uint8_t* qa, int64_t M, int64_t K, uint8_t* qaw, hipStream_t st);

// fp6 route: images (layout above) and the tile kernel that reads them.
// Residual block images: b = 64 or 128, one 1.5 KB piece per 32 rows and
// 64-code slice of the block, piece (32-row block c, slice u) at
// (c * (b/64) + u) * 1536, lane l's dwords 0-3 at 16 l and 4-5 at
// 1024 + 8 l of the piece.
inline size_t fp6_rows_bytes(int64_t rows, int64_t K) { return (size_t)((rows + 31) / 32) * (size_t)(K / kGroup) * kFp6Frag; }
inline size_t fp6_residual_bytes(int64_t n_select, int block) { return (size_t)n_select * (size_t)block * block * 3 / 4; }
hipError_t launch_acts_fp6(const uint8_t* qa, int64_t M, int64_t K, uint8_t* aimg, hipStream_t st);
hipError_t launch_weights_fp6(const uint8_t* qw, int64_t N, int64_t K, uint8_t* wimg, hipStream_t st);
hipError_t launch_residual_fp6(const uint8_t* qr, int n_select, int block, uint8_t* rimg, hipStream_t st);
// act-quant into the activation image, base and residual conversion, in one launch
// (the activation scales written group-major, saT [K/128][wide_rows(M)];
// the weight scales sw [N][K/128] copied group-major into swT [K/128][N];
// wimg null: no base conversion and no swT copy)
hipError_t launch_fp6_layer_prep(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* aimg, float* saT,
                                 const uint8_t* qw, const uint16_t* sw, int64_t N, uint8_t* wimg, uint16_t* swT,
                                 const uint8_t* qr, int n_select, int block, uint8_t* rimg, hipStream_t st);
bool tile6_gemm_fits(const GemmArgs& a);
int tile6_gemm_splits(int64_t M, int64_t N, int64_t K);  // K splits of the fp6 route
int64_t tile6_gemm_tail(int64_t M, int64_t N, int64_t K, int ks);  // tiles it splits
hipError_t launch_tile6_gemm(const GemmArgs& a, hipStream_t st);

}  // namespace mq
