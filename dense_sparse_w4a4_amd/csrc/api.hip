// C ABI of libmosaicq: argument validation, then launches on the caller's
// stream.  Nothing is enqueued when validation fails.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "mq_internal.h"

namespace mq {

static thread_local char g_err[512];

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

mq_status fail(mq_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

static mq_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MQ_OK;
  return fail(MQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static bool valid_block(int b) { return b == 32 || b == 64 || b == 128; }

// Number of b x b blocks of an N x K matrix, or INT64_MAX when N or K is
// 2^31 or more (so the callers' block-count limit rejects it without the
// product overflowing).
static int64_t block_count(int64_t N, int64_t K, int b) {
  if (N >= ((int64_t)1 << 31) || K >= ((int64_t)1 << 31)) return INT64_MAX;
  return (N / b) * (K / b);
}

// Sizes the fused GEMM accepts (each below 2^31, packed weights and
// activations each below 4 GiB), checked without overflowing.
static bool gemm_sizes_ok(int64_t M, int64_t N, int64_t K) {
  const int64_t lim = (int64_t)1 << 31;
  return M >= 0 && N >= 0 && K >= 0 && M < lim && N < lim && K < lim &&
         N * (K / 2) < ((int64_t)1 << 32) && M * (K / 2) < ((int64_t)1 << 32);
}

}  // namespace mq

using namespace mq;

#define MQ_REQUIRE(cond, code, ...)      \
  do {                                   \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

extern "C" {

const char* mq_status_str(int s) {
  switch (s) {
    case MQ_OK: return "MQ_OK";
    case MQ_ERR_NULL_PTR: return "MQ_ERR_NULL_PTR";
    case MQ_ERR_SHAPE: return "MQ_ERR_SHAPE";
    case MQ_ERR_ALIGN: return "MQ_ERR_ALIGN";
    case MQ_ERR_BLOCK: return "MQ_ERR_BLOCK";
    case MQ_ERR_BUDGET: return "MQ_ERR_BUDGET";
    case MQ_ERR_CSR: return "MQ_ERR_CSR";
    case MQ_ERR_WORKSPACE: return "MQ_ERR_WORKSPACE";
    case MQ_ERR_HIP: return "MQ_ERR_HIP";
    case MQ_ERR_ARG: return "MQ_ERR_ARG";
    default: return "MQ_ERR_UNKNOWN";
  }
}

const char* mq_last_error(void) { return g_err; }

int mq_version(void) { return (1 << 16) | 0; }

mq_status mq_quantize_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* qa,
                          float* sa, void* stream) {
  g_err[0] = 0;
  MQ_REQUIRE(M >= 0, MQ_ERR_SHAPE, "M = %lld must be >= 0", (long long)M);
  MQ_REQUIRE(K > 0 && K % kGroup == 0, MQ_ERR_SHAPE, "K = %lld must be a positive multiple of 128",
             (long long)K);
  MQ_REQUIRE(ldx >= K, MQ_ERR_SHAPE, "ldx = %lld < K = %lld", (long long)ldx, (long long)K);
  MQ_REQUIRE(M <= (int64_t)1 << 31 && K < (int64_t)1 << 31 && M * (K / kGroup) < (int64_t)1 << 36,
             MQ_ERR_SHAPE, "M x K too large");
  if (M == 0) return MQ_OK;
  MQ_REQUIRE(x && qa && sa, MQ_ERR_NULL_PTR, "x, qa and sa must be non-NULL");
  MQ_REQUIRE(ldx % 8 == 0, MQ_ERR_ALIGN, "ldx = %lld must be a multiple of 8", (long long)ldx);
  MQ_REQUIRE(aligned16(x) && aligned16(qa) && aligned16(sa), MQ_ERR_ALIGN,
             "x, qa and sa must be 16-byte aligned");
  return hip_status(launch_act_quant(x, M, K, ldx, qa, sa, (hipStream_t)stream),
                    "mq_quantize_act launch");
}

mq_status mq_select_blocks(const uint16_t* w, const uint16_t* x_calib, int64_t N, int64_t K,
                           int64_t T, int32_t block, int32_t n_select, int32_t* selected,
                           double* delta_out, double* hdiag_out, void* stream) {
  g_err[0] = 0;
  MQ_REQUIRE(valid_block(block), MQ_ERR_BLOCK, "block = %d must be 32, 64 or 128", block);
  MQ_REQUIRE(N > 0 && N % block == 0, MQ_ERR_SHAPE, "N = %lld must be a positive multiple of %d",
             (long long)N, block);
  MQ_REQUIRE(K > 0 && K % kGroup == 0, MQ_ERR_SHAPE, "K = %lld must be a positive multiple of 128",
             (long long)K);
  MQ_REQUIRE(T >= 0, MQ_ERR_SHAPE, "T = %lld must be >= 0", (long long)T);
  const int64_t B = block_count(N, K, block);
  MQ_REQUIRE(B < ((int64_t)1 << 31), MQ_ERR_SHAPE, "too many blocks (%lld)", (long long)B);
  MQ_REQUIRE(T < ((int64_t)1 << 31) && T * K < ((int64_t)1 << 40), MQ_ERR_SHAPE,
             "T = %lld calibration tokens too many", (long long)T);
  MQ_REQUIRE(n_select >= 0 && n_select <= B, MQ_ERR_BUDGET, "n_select = %d outside [0, %lld]",
             n_select, (long long)B);
  MQ_REQUIRE(w && delta_out && hdiag_out, MQ_ERR_NULL_PTR,
             "w, delta_out and hdiag_out must be non-NULL");
  MQ_REQUIRE(T == 0 || x_calib, MQ_ERR_NULL_PTR, "x_calib must be non-NULL when T > 0");
  MQ_REQUIRE(n_select == 0 || selected, MQ_ERR_NULL_PTR, "selected must be non-NULL");
  MQ_REQUIRE(aligned16(w) && aligned16(x_calib) && aligned16(delta_out) && aligned16(hdiag_out) &&
                 aligned16(selected),
             MQ_ERR_ALIGN, "device pointers must be 16-byte aligned");
  return hip_status(launch_select(w, x_calib, N, K, T, block, n_select, selected, delta_out,
                                  hdiag_out, (hipStream_t)stream),
                    "mq_select_blocks launch");
}

// Shape rules shared by the exact-distortion entry points.
static mq_status exact_check(int64_t N, int64_t K, int64_t T, int32_t block) {
  MQ_REQUIRE(valid_block(block), MQ_ERR_BLOCK, "block = %d must be 32, 64 or 128", block);
  MQ_REQUIRE(N > 0 && N % block == 0, MQ_ERR_SHAPE, "N = %lld must be a positive multiple of %d",
             (long long)N, block);
  MQ_REQUIRE(K > 0 && K % kGroup == 0, MQ_ERR_SHAPE, "K = %lld must be a positive multiple of 128",
             (long long)K);
  MQ_REQUIRE(T >= 0 && T < ((int64_t)1 << 22), MQ_ERR_SHAPE, "T = %lld outside [0, 2^22)",
             (long long)T);
  const int64_t B = block_count(N, K, block);
  MQ_REQUIRE(B < ((int64_t)1 << 24), MQ_ERR_SHAPE, "too many blocks (%lld >= 2^24)", (long long)B);
  MQ_REQUIRE(N * K < ((int64_t)1 << 36) && T * N < ((int64_t)1 << 36), MQ_ERR_SHAPE,
             "N x K or T x N too large");
  return MQ_OK;
}

mq_status mq_select_exact_workspace(int64_t N, int64_t K, int64_t T, int32_t block, size_t* bytes) {
  g_err[0] = 0;
  MQ_REQUIRE(bytes, MQ_ERR_NULL_PTR, "bytes must be non-NULL");
  const mq_status s = exact_check(N, K, T, block);
  if (s != MQ_OK) return s;
  *bytes = exact_greedy_workspace(N, K, T, block);
  return MQ_OK;
}

mq_status mq_select_exact_greedy(const uint16_t* w, const uint16_t* x_calib, int64_t N, int64_t K,
                                 int64_t T, int32_t block, int32_t n_select, int32_t* selected,
                                 int32_t* order, double* gains, double* dist, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  const mq_status s = exact_check(N, K, T, block);
  if (s != MQ_OK) return s;
  const int64_t B = block_count(N, K, block);
  MQ_REQUIRE(n_select >= 0 && n_select <= B, MQ_ERR_BUDGET, "n_select = %d outside [0, %lld]",
             n_select, (long long)B);
  MQ_REQUIRE(w && workspace, MQ_ERR_NULL_PTR, "w and workspace must be non-NULL");
  MQ_REQUIRE(T == 0 || x_calib, MQ_ERR_NULL_PTR, "x_calib must be non-NULL when T > 0");
  MQ_REQUIRE(n_select == 0 || selected, MQ_ERR_NULL_PTR, "selected must be non-NULL");
  MQ_REQUIRE(aligned16(w) && aligned16(x_calib) && aligned16(selected) && aligned16(order) &&
                 aligned16(gains) && aligned16(dist) && aligned16(workspace),
             MQ_ERR_ALIGN, "device pointers must be 16-byte aligned");
  const size_t need = exact_greedy_workspace(N, K, T, block);
  MQ_REQUIRE(workspace_bytes >= need, MQ_ERR_WORKSPACE, "workspace %zu bytes < %zu needed",
             workspace_bytes, need);
  return hip_status(launch_exact_greedy(w, x_calib, N, K, T, block, n_select, selected, order,
                                        gains, dist, workspace, (hipStream_t)stream),
                    "mq_select_exact_greedy launch");
}

mq_status mq_distortion_workspace(int64_t N, int64_t K, int64_t T, int32_t block, size_t* bytes) {
  g_err[0] = 0;
  MQ_REQUIRE(bytes, MQ_ERR_NULL_PTR, "bytes must be non-NULL");
  const mq_status s = exact_check(N, K, T, block);
  if (s != MQ_OK) return s;
  *bytes = distortion_workspace(N, K, T, block);
  return MQ_OK;
}

mq_status mq_distortion(const uint16_t* w, const uint16_t* x, int64_t N, int64_t K, int64_t T,
                        int32_t block, const int32_t* selected, int32_t n_selected, double* dist,
                        void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  const mq_status s = exact_check(N, K, T, block);
  if (s != MQ_OK) return s;
  MQ_REQUIRE(n_selected >= 0, MQ_ERR_BUDGET, "n_selected = %d must be >= 0", n_selected);
  MQ_REQUIRE(w && dist && workspace, MQ_ERR_NULL_PTR, "w, dist and workspace must be non-NULL");
  MQ_REQUIRE(T == 0 || x, MQ_ERR_NULL_PTR, "x must be non-NULL when T > 0");
  MQ_REQUIRE(n_selected == 0 || selected, MQ_ERR_NULL_PTR, "selected must be non-NULL");
  MQ_REQUIRE(aligned16(w) && aligned16(x) && aligned16(selected) && aligned16(dist) &&
                 aligned16(workspace),
             MQ_ERR_ALIGN, "device pointers must be 16-byte aligned");
  const size_t need = distortion_workspace(N, K, T, block);
  MQ_REQUIRE(workspace_bytes >= need, MQ_ERR_WORKSPACE, "workspace %zu bytes < %zu needed",
             workspace_bytes, need);
  return hip_status(launch_distortion(w, x, N, K, T, block, selected, n_selected, dist, workspace,
                                      (hipStream_t)stream),
                    "mq_distortion launch");
}

mq_status mq_pack_weights(const uint16_t* w, int64_t N, int64_t K, int32_t block,
                          const int32_t* selected, int32_t n_select, uint8_t* qw, uint16_t* sw,
                          int32_t* row_ptr, int32_t* col_idx, uint8_t* qr, uint16_t* sr,
                          void* stream) {
  g_err[0] = 0;
  MQ_REQUIRE(valid_block(block), MQ_ERR_BLOCK, "block = %d must be 32, 64 or 128", block);
  MQ_REQUIRE(N > 0 && N % block == 0, MQ_ERR_SHAPE, "N = %lld must be a positive multiple of %d",
             (long long)N, block);
  MQ_REQUIRE(K > 0 && K % kGroup == 0, MQ_ERR_SHAPE, "K = %lld must be a positive multiple of 128",
             (long long)K);
  const int64_t B = block_count(N, K, block);
  MQ_REQUIRE(B < ((int64_t)1 << 31), MQ_ERR_SHAPE, "too many blocks (%lld)", (long long)B);
  MQ_REQUIRE(n_select >= 0 && n_select <= B, MQ_ERR_BUDGET, "n_select = %d outside [0, %lld]",
             n_select, (long long)B);
  MQ_REQUIRE(w && qw && sw && row_ptr, MQ_ERR_NULL_PTR, "w, qw, sw and row_ptr must be non-NULL");
  MQ_REQUIRE(n_select == 0 || (selected && col_idx && qr && sr), MQ_ERR_NULL_PTR,
             "selected, col_idx, qr and sr must be non-NULL when n_select > 0");
  MQ_REQUIRE(aligned16(w) && aligned16(qw) && aligned16(sw) && aligned16(row_ptr) &&
                 aligned16(selected) && aligned16(col_idx) && aligned16(qr) && aligned16(sr),
             MQ_ERR_ALIGN, "device pointers must be 16-byte aligned");
  return hip_status(launch_pack(w, N, K, block, selected, n_select, qw, sw, row_ptr, col_idx, qr,
                                sr, (hipStream_t)stream),
                    "mq_pack_weights launch");
}

static size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

// The fp6 route converts the base weights and the residual blocks on every
// call (one pass over their codes, about 1.9 bytes moved per weight); its
// kernel saves about a fifth of the int8 route's time, which outweighs the
// conversion from about 1000 tokens on (measured on the Qwen3-32B MLP
// shapes: at M = 256 the conversion costs more than it saves).
constexpr int64_t kFp6MinM = 1024;
// Below this many tokens mq_fused_gemm's fp6 route (taken there only when
// the caller asks for it) reads the base codes from the packed slabs,
// re-encoded in the kernel's registers, instead of converting them into an
// image first: measured on the Qwen3-32B MLP shapes at 64-512 tokens it is
// 1-2% faster than the int8 route, against about 30 us for the image
// conversion; from 1024 tokens, where each weight tile serves four or more
// token tiles, the in-kernel re-encoding costs more than the conversion
// (M = 1024: 319 against 260 us).
constexpr int64_t kFp6RawBelow = 1024;
// (MQ_FLAG_FP6_TILE lowers it to the tile kernel's M > 32 for checks.)


// Split-K partials of the tile kernel: [splits][M][N] fp32 when M > 32 and
// the tiles alone would leave compute units idle; 0 otherwise.
static size_t split_workspace(int64_t M, int64_t N, int64_t K) {
  if (M <= 32 || N <= 0 || K < kGroup) return 0;
  const int ks = tile_gemm_splits(M, N, K);
  return ks > 1 ? (size_t)ks * (size_t)M * (size_t)N * sizeof(float) : 0;
}

// Activation codes in the tile kernel's wide fragment order (M > 32):
// one byte per code for ceil(M/32)*32 rows.
static size_t wide_workspace(int64_t M, int64_t K) {
  if (M <= 32 || K < kGroup) return 0;
  return round256((size_t)wide_rows(M) * (size_t)K);
}

// Split-K partials of the fp6 route (its own split rule).
static size_t split6_workspace(int64_t M, int64_t N, int64_t K) {
  if (M <= 32 || N <= 0 || K < kGroup) return 0;
  const int ks = tile6_gemm_splits(M, N, K);
  return ks > 1 ? (size_t)ks * (size_t)M * (size_t)N * sizeof(float) : 0;
}

// mq_fused_gemm's workspace on the int8 route: the wide activation codes,
// then the split-K partials.
static size_t gemm_workspace_i8(int64_t M, int64_t N, int64_t K) {
  return wide_workspace(M, K) + split_workspace(M, N, K);
}

// The fp6 route (M > 32, block 64 or 128): FP6 images of the activation
// codes, the base weights and the residual blocks, then the split-K
// partials.  fp6_images_bytes is exact for (block, n_select); with
// n_select unknown the residual term is bounded by N*K*3/4 (every block
// selected).
static size_t fp6_images_bytes(int64_t M, int64_t N, int64_t K, int block, int64_t n_select) {
  return round256(fp6_rows_bytes(M, K)) + round256(fp6_rows_bytes(N, K)) +
         round256(fp6_residual_bytes(n_select, block));
}
static size_t fp6_images_bound(int64_t M, int64_t N, int64_t K) {
  if (M <= 32 || N <= 0 || K < kGroup) return 0;
  return round256(fp6_rows_bytes(M, K)) + round256(fp6_rows_bytes(N, K)) + round256((size_t)N * (size_t)K * 3 / 4);
}
static size_t gemm_workspace(int64_t M, int64_t N, int64_t K) {
  const size_t i8 = gemm_workspace_i8(M, N, K);
  const size_t f6 = M >= kFp6MinM ? fp6_images_bound(M, N, K) + split6_workspace(M, N, K) : 0;
  return i8 > f6 ? i8 : f6;
}

// Points a at the fp6 images in ws (layout of fp6_images_bytes) and
// enqueues the conversions of the weights (from kFp6RawBelow tokens) and of
// the residual blocks.
static hipError_t fp6_prepare(GemmArgs& a, uint8_t* ws, hipStream_t st) {
  uint8_t* aimg = ws;
  uint8_t* wimg = aimg + round256(fp6_rows_bytes(a.M, a.K));
  uint8_t* rimg = wimg + round256(fp6_rows_bytes(a.N, a.K));
  const bool raw = a.M < kFp6RawBelow;
  hipError_t e = raw ? hipSuccess : launch_weights_fp6(a.qw, a.N, a.K, wimg, st);
  if (e != hipSuccess) return e;
  e = launch_residual_fp6(a.qr, a.n_select, a.block, rimg, st);
  if (e != hipSuccess) return e;
  a.aimg = aimg;
  a.wimg = raw ? nullptr : wimg;
  a.rimg = rimg;
  return hipSuccess;
}

mq_status mq_fused_gemm_workspace(int64_t M, int64_t N, int64_t K, size_t* bytes) {
  g_err[0] = 0;
  MQ_REQUIRE(bytes, MQ_ERR_NULL_PTR, "bytes must be non-NULL");
  MQ_REQUIRE(gemm_sizes_ok(M, N, K), MQ_ERR_SHAPE,
             "sizes must be >= 0 and below 2^31, packed weights and activations below 4 GiB");
  *bytes = gemm_workspace(M, N, K);
  return MQ_OK;
}

mq_status mq_fused_gemm(const uint8_t* qa, const float* sa, int64_t M, int64_t N, int64_t K,
                        const uint8_t* qw, const uint16_t* sw, int32_t block, int32_t n_select,
                        const int32_t* row_ptr, const int32_t* col_idx, const uint8_t* qr,
                        const uint16_t* sr, uint16_t* y, int64_t ldy, void* workspace,
                        size_t workspace_bytes, uint32_t flags, int32_t* acc_dump,
                        void* stream) {
  g_err[0] = 0;
  MQ_REQUIRE((flags & ~(MQ_FLAG_DUMP_ACC | MQ_FLAG_INT8_TILE | MQ_FLAG_FP6_TILE)) == 0, MQ_ERR_ARG,
             "unknown flags 0x%x", flags);
  MQ_REQUIRE(!((flags & MQ_FLAG_INT8_TILE) && (flags & MQ_FLAG_FP6_TILE)), MQ_ERR_ARG,
             "MQ_FLAG_INT8_TILE and MQ_FLAG_FP6_TILE exclude each other");
  MQ_REQUIRE(valid_block(block), MQ_ERR_BLOCK, "block = %d must be 32, 64 or 128", block);
  MQ_REQUIRE(M >= 0, MQ_ERR_SHAPE, "M = %lld must be >= 0", (long long)M);
  MQ_REQUIRE(N > 0 && N % block == 0, MQ_ERR_SHAPE, "N = %lld must be a positive multiple of %d",
             (long long)N, block);
  MQ_REQUIRE(K > 0 && K % kGroup == 0, MQ_ERR_SHAPE, "K = %lld must be a positive multiple of 128",
             (long long)K);
  MQ_REQUIRE(ldy >= N, MQ_ERR_SHAPE, "ldy = %lld < N = %lld", (long long)ldy, (long long)N);
  const int64_t B = block_count(N, K, block);
  MQ_REQUIRE(B < ((int64_t)1 << 31), MQ_ERR_SHAPE, "too many blocks (%lld)", (long long)B);
  MQ_REQUIRE(M < ((int64_t)1 << 31) && N < ((int64_t)1 << 31) && K < ((int64_t)1 << 31),
             MQ_ERR_SHAPE, "sizes must be below 2^31");
  MQ_REQUIRE(N * (K / 2) < ((int64_t)1 << 32) && M * (K / 2) < ((int64_t)1 << 32), MQ_ERR_SHAPE,
             "packed weights and activations must each be below 4 GiB");
  MQ_REQUIRE(n_select >= 0 && n_select <= B, MQ_ERR_BUDGET, "n_select = %d outside [0, %lld]",
             n_select, (long long)B);
  if (M == 0) return MQ_OK;
  MQ_REQUIRE(qa && sa && qw && sw && y, MQ_ERR_NULL_PTR, "qa, sa, qw, sw and y must be non-NULL");
  MQ_REQUIRE(n_select == 0 || (row_ptr && col_idx && qr && sr), MQ_ERR_NULL_PTR,
             "row_ptr, col_idx, qr and sr must be non-NULL when n_select > 0");
  MQ_REQUIRE(!(flags & MQ_FLAG_DUMP_ACC) || acc_dump, MQ_ERR_NULL_PTR,
             "acc_dump must be non-NULL with MQ_FLAG_DUMP_ACC");
  MQ_REQUIRE(ldy % 8 == 0, MQ_ERR_ALIGN, "ldy = %lld must be a multiple of 8", (long long)ldy);
  MQ_REQUIRE(aligned16(qa) && aligned16(sa) && aligned16(qw) && aligned16(sw) && aligned16(y) &&
                 aligned16(row_ptr) && aligned16(col_idx) && aligned16(qr) && aligned16(sr) &&
                 aligned16(acc_dump),
             MQ_ERR_ALIGN, "device pointers must be 16-byte aligned");
  GemmArgs a = {};
  a.qa = qa;
  a.sa = sa;
  a.M = M;
  a.N = N;
  a.K = K;
  a.qw = qw;
  a.sw = sw;
  a.block = block;
  a.n_select = n_select;
  a.row_ptr = n_select ? row_ptr : nullptr;
  a.col_idx = n_select ? col_idx : nullptr;
  a.qr = n_select ? qr : nullptr;
  a.sr = n_select ? sr : nullptr;
  a.y = y;
  a.ldy = ldy;
  a.acc_dump = (flags & MQ_FLAG_DUMP_ACC) ? acc_dump : nullptr;
  // With the whole workspace (tile kernel route, M > 32): the codes are
  // copied once into the wide fragment order, which the tile kernel moves
  // to LDS without widening, and the split-K schedule is used where it
  // applies.  Otherwise one pass over K from the packed codes.
  const size_t split = split_workspace(M, N, K);
  const size_t split6 = split6_workspace(M, N, K);
  const size_t need6 = M > 32 ? fp6_images_bytes(M, N, K, block, n_select) + split6 : 0;
  const size_t need = gemm_workspace_i8(M, N, K);
  const int64_t min_m6 = (flags & MQ_FLAG_FP6_TILE) ? 33 : kFp6MinM;
  const bool fp6 = !(flags & MQ_FLAG_INT8_TILE) && M >= min_m6 && workspace && workspace_bytes >= need6 &&
                   tile6_gemm_fits(a);
  const bool wide = !fp6 && need > 0 && workspace && workspace_bytes >= need && M > 32 && tile_gemm_fits(a);
  if (fp6) {
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    mq_status st = hip_status(fp6_prepare(a, ws, (hipStream_t)stream), "mq_fused_gemm fp6 conversion launch");
    if (st != MQ_OK) return st;
    st = hip_status(launch_acts_fp6(qa, M, K, const_cast<uint8_t*>(a.aimg), (hipStream_t)stream),
                    "mq_fused_gemm fp6 conversion launch");
    if (st != MQ_OK) return st;
    a.part = split6 > 0 ? reinterpret_cast<float*>(ws + need6 - split6) : nullptr;
    a.ksplit = split6 > 0 ? tile6_gemm_splits(M, N, K) : 1;
  } else if (wide) {
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    const mq_status st = hip_status(launch_widen_acts(qa, M, K, ws, (hipStream_t)stream),
                                    "mq_fused_gemm widen launch");
    if (st != MQ_OK) return st;
    a.qaw = ws;
    a.part = split > 0 ? reinterpret_cast<float*>(ws + wide_workspace(M, K)) : nullptr;
    a.ksplit = split > 0 ? tile_gemm_splits(M, N, K) : 1;
  } else {
    a.ksplit = 1;
  }
  return hip_status(launch_fused_gemm(a, (hipStream_t)stream), "mq_fused_gemm launch");
}

// Workspace of mq_fused_layer: none when the streaming kernel quantises the
// activations itself; otherwise the activation codes (packed, in 16-token
// tiles, for the streaming kernel, M <= 32; the wide fragment order for the
// tile kernel, M > 32, whose area also holds the tiled codes when the tile
// kernel does not apply), their scales, then the split-K partials.
static size_t layer_codes_bytes(int64_t M, int64_t K) {
  return M > 32 ? wide_workspace(M, K) : round256((size_t)tiled_rows(M) * (size_t)(K / 2));
}
static size_t layer_workspace_i8(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K < kGroup || stream_quant_fits(M, N, K)) return 0;
  return layer_codes_bytes(M, K) + round256((size_t)M * (size_t)(K / kGroup) * 4) + split_workspace(M, N, K);
}
// The fp6 route: the activation scales group-major [K/128][wide_rows(M)]
// (fp32) and the weight scales group-major [K/128][N] (fp16), the fp6
// images, the split-K partials.
static size_t layer_scales_bytes(int64_t M, int64_t N, int64_t K) {
  return round256((size_t)wide_rows(M) * (size_t)(K / kGroup) * 4) + round256((size_t)N * (size_t)(K / kGroup) * 2);
}
static size_t layer_workspace_fp6(int64_t M, int64_t N, int64_t K, int block, int64_t n_select) {
  return layer_scales_bytes(M, N, K) + fp6_images_bytes(M, N, K, block, n_select) + split6_workspace(M, N, K);
}
static size_t layer_workspace(int64_t M, int64_t N, int64_t K) {
  const size_t i8 = layer_workspace_i8(M, N, K);
  if (M < kFp6MinM || N <= 0 || K < kGroup) return i8;
  const size_t f6 = layer_scales_bytes(M, N, K) + fp6_images_bound(M, N, K) + split6_workspace(M, N, K);
  return i8 > f6 ? i8 : f6;
}

mq_status mq_fused_layer_workspace(int64_t M, int64_t N, int64_t K, size_t* bytes) {
  g_err[0] = 0;
  MQ_REQUIRE(bytes, MQ_ERR_NULL_PTR, "bytes must be non-NULL");
  MQ_REQUIRE(gemm_sizes_ok(M, N, K), MQ_ERR_SHAPE,
             "sizes must be >= 0 and below 2^31, packed weights and activations below 4 GiB");
  *bytes = layer_workspace(M, N, K);
  return MQ_OK;
}

}  // extern "C"

namespace mq {

// Argument checks of the one-call layer (mq_fused_layer and its
// allocation-free variant).  *empty is set for M == 0 (nothing to enqueue);
// *need is the workspace the shape uses.
static mq_status layer_check(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int64_t N,
                             const uint8_t* qw, const uint16_t* sw, int32_t block, int32_t n_select,
                             const int32_t* row_ptr, const int32_t* col_idx, const uint8_t* qr,
                             const uint16_t* sr, uint16_t* y, int64_t ldy, const void* workspace,
                             bool* empty, size_t* need) {
  *empty = false;
  *need = 0;
  MQ_REQUIRE(valid_block(block), MQ_ERR_BLOCK, "block = %d must be 32, 64 or 128", block);
  MQ_REQUIRE(M >= 0, MQ_ERR_SHAPE, "M = %lld must be >= 0", (long long)M);
  MQ_REQUIRE(N > 0 && N % block == 0, MQ_ERR_SHAPE, "N = %lld must be a positive multiple of %d",
             (long long)N, block);
  MQ_REQUIRE(K > 0 && K % kGroup == 0, MQ_ERR_SHAPE, "K = %lld must be a positive multiple of 128",
             (long long)K);
  MQ_REQUIRE(ldx >= K, MQ_ERR_SHAPE, "ldx = %lld < K = %lld", (long long)ldx, (long long)K);
  MQ_REQUIRE(ldy >= N, MQ_ERR_SHAPE, "ldy = %lld < N = %lld", (long long)ldy, (long long)N);
  const int64_t B = block_count(N, K, block);
  MQ_REQUIRE(B < ((int64_t)1 << 31), MQ_ERR_SHAPE, "too many blocks (%lld)", (long long)B);
  MQ_REQUIRE(M < ((int64_t)1 << 31) && N < ((int64_t)1 << 31) && K < ((int64_t)1 << 31),
             MQ_ERR_SHAPE, "sizes must be below 2^31");
  MQ_REQUIRE(N * (K / 2) < ((int64_t)1 << 32) && M * (K / 2) < ((int64_t)1 << 32), MQ_ERR_SHAPE,
             "packed weights and activations must each be below 4 GiB");
  MQ_REQUIRE(n_select >= 0 && n_select <= B, MQ_ERR_BUDGET, "n_select = %d outside [0, %lld]",
             n_select, (long long)B);
  if (M == 0) {
    *empty = true;
    return MQ_OK;
  }
  MQ_REQUIRE(x && qw && sw && y, MQ_ERR_NULL_PTR, "x, qw, sw and y must be non-NULL");
  MQ_REQUIRE(n_select == 0 || (row_ptr && col_idx && qr && sr), MQ_ERR_NULL_PTR,
             "row_ptr, col_idx, qr and sr must be non-NULL when n_select > 0");
  MQ_REQUIRE(ldx % 8 == 0 && ldy % 8 == 0, MQ_ERR_ALIGN,
             "ldx = %lld and ldy = %lld must be multiples of 8", (long long)ldx, (long long)ldy);
  MQ_REQUIRE(aligned16(x) && aligned16(qw) && aligned16(sw) && aligned16(y) &&
                 aligned16(row_ptr) && aligned16(col_idx) && aligned16(qr) && aligned16(sr) &&
                 aligned16(workspace),
             MQ_ERR_ALIGN, "device pointers must be 16-byte aligned");
  *need = layer_workspace_i8(M, N, K);
  return MQ_OK;
}

// Launches of the one-call layer on `ws` of ws_bytes (at least
// layer_workspace_i8's `need`; unused when that is 0): one kernel when the
// streaming GEMM quantises the activations itself; for M > 32 with room for
// the fp6 images, act-quant into the FP6 image, the weight and residual
// conversions and the fp6 tile kernel; else act-quant into the workspace,
// then the fused GEMM with its split-K partials after the codes and scales.
static mq_status layer_run(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int64_t N,
                           const uint8_t* qw, const uint16_t* sw, int32_t block, int32_t n_select,
                           const int32_t* row_ptr, const int32_t* col_idx, const uint8_t* qr,
                           const uint16_t* sr, uint16_t* y, int64_t ldy, uint8_t* ws, size_t need,
                           size_t ws_bytes, hipStream_t st) {
  GemmArgs a = {};
  a.M = M;
  a.N = N;
  a.K = K;
  a.qw = qw;
  a.sw = sw;
  a.block = block;
  a.n_select = n_select;
  a.row_ptr = n_select ? row_ptr : nullptr;
  a.col_idx = n_select ? col_idx : nullptr;
  a.qr = n_select ? qr : nullptr;
  a.sr = n_select ? sr : nullptr;
  a.y = y;
  a.ldy = ldy;
  a.ksplit = 1;
  if (need == 0) {  // one kernel: the streaming GEMM quantises the activations itself
    a.x = x;
    a.ldx = ldx;
    return hip_status(launch_fused_gemm(a, st), "mq_fused_layer launch");
  }
  const size_t split = split_workspace(M, N, K);
  const size_t split6 = split6_workspace(M, N, K);
  if (M >= kFp6MinM && tile6_gemm_fits(a) && ws_bytes >= layer_workspace_fp6(M, N, K, block, n_select)) {
    // fp6 tile kernel: the group-major scales, then the images (act-quant
    // into the activation image and the base and residual conversions in
    // one launch)
    float* saT = reinterpret_cast<float*>(ws);
    uint16_t* swT = reinterpret_cast<uint16_t*>(ws + round256((size_t)wide_rows(M) * (size_t)(K / kGroup) * 4));
    uint8_t* aimg = ws + layer_scales_bytes(M, N, K);
    uint8_t* wimg = aimg + round256(fp6_rows_bytes(M, K));
    uint8_t* rimg = wimg + round256(fp6_rows_bytes(N, K));
    const mq_status s = hip_status(launch_fp6_layer_prep(x, M, K, ldx, aimg, saT, qw, sw, N, wimg, swT, a.qr,
                                                         n_select, block, rimg, st),
                                   "mq_fused_layer fp6 preparation launch");
    if (s != MQ_OK) return s;
    a.aimg = aimg;
    a.wimg = wimg;
    a.rimg = rimg;
    a.saT = saT;
    a.swT = swT;
    a.saT_ld = wide_rows(M);
    if (split6 > 0) {
      a.part = reinterpret_cast<float*>(ws + layer_workspace_fp6(M, N, K, block, n_select) - split6);
      a.ksplit = tile6_gemm_splits(M, N, K);
    }
    return hip_status(launch_fused_gemm(a, st), "mq_fused_layer launch");
  }
  float* sa = reinterpret_cast<float*>(ws + layer_codes_bytes(M, K));
  a.sa = sa;
  if (M > 32 && tile_gemm_fits(a)) {
    // tile kernel: codes quantised straight into the wide fragment order
    const mq_status s = hip_status(launch_act_quant_wide(x, M, K, ldx, ws, sa, st),
                                   "mq_fused_layer act-quant launch");
    if (s != MQ_OK) return s;
    a.qaw = ws;
    if (split > 0) {
      a.part = reinterpret_cast<float*>(ws + need - split);
      a.ksplit = tile_gemm_splits(M, N, K);
    }
  } else if (M > 8 && tiled_rows(M) * (K / 2) < ((int64_t)1 << 32)) {
    // streaming kernel: packed codes in 16-token tiles (each group's codes
    // of a tile one contiguous 1 KB: eight full cache lines instead of 64
    // bytes from each of up to 16 rows; with 8 tokens or fewer the
    // row-major codes touch no more lines than that, and the tile's padding
    // rows would only add bytes)
    const mq_status s = hip_status(launch_act_quant_tiled(x, M, K, ldx, ws, sa, st),
                                   "mq_fused_layer act-quant launch");
    if (s != MQ_OK) return s;
    a.qat = ws;
  } else {
    // streaming kernel: packed codes, row-major
    const mq_status s = hip_status(launch_act_quant(x, M, K, ldx, ws, sa, st),
                                   "mq_fused_layer act-quant launch");
    if (s != MQ_OK) return s;
    a.qa = ws;
  }
  return hip_status(launch_fused_gemm(a, st), "mq_fused_layer launch");
}

// Device scratch of mq_fused_layer_noalloc (each device holds its own copy
// of this array from the time the library's code object is loaded on it
// until the process ends).  In host code `scratch` only names the symbol:
// the address a kernel may use is the one hipGetSymbolAddress returns for
// the current device, looked up once per device and kept in g_scratch.
constexpr size_t kScratchBytes = MQ_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch[kMaxDevices];

static mq_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "mq_fused_layer_noalloc hipGetDevice");
  MQ_REQUIRE(dev >= 0 && dev < kMaxDevices, MQ_ERR_HIP, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "mq_fused_layer_noalloc hipGetSymbolAddress");
    MQ_REQUIRE(p != nullptr, MQ_ERR_HIP, "scratch has no device address");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MQ_OK;
}

}  // namespace mq

extern "C" {

mq_status mq_fused_layer(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int64_t N,
                         const uint8_t* qw, const uint16_t* sw, int32_t block, int32_t n_select,
                         const int32_t* row_ptr, const int32_t* col_idx, const uint8_t* qr,
                         const uint16_t* sr, uint16_t* y, int64_t ldy, void* workspace,
                         size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  bool empty = false;
  size_t need = 0;
  mq_status s = layer_check(x, M, K, ldx, N, qw, sw, block, n_select, row_ptr, col_idx, qr, sr, y,
                            ldy, workspace, &empty, &need);
  if (s != MQ_OK || empty) return s;
  need = layer_workspace(M, N, K);
  MQ_REQUIRE(workspace_bytes >= need && (need == 0 || workspace), MQ_ERR_WORKSPACE,
             "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  return layer_run(x, M, K, ldx, N, qw, sw, block, n_select, row_ptr, col_idx, qr, sr, y, ldy,
                   static_cast<uint8_t*>(workspace), layer_workspace_i8(M, N, K), workspace_bytes,
                   (hipStream_t)stream);
}

mq_status mq_fused_layer_noalloc(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int64_t N,
                                 const uint8_t* qw, const uint16_t* sw, int32_t block,
                                 int32_t n_select, const int32_t* row_ptr, const int32_t* col_idx,
                                 const uint8_t* qr, const uint16_t* sr, uint16_t* y, int64_t ldy,
                                 void* stream) {
  g_err[0] = 0;
  bool empty = false;
  size_t need = 0;
  mq_status s = layer_check(x, M, K, ldx, N, qw, sw, block, n_select, row_ptr, col_idx, qr, sr, y,
                            ldy, nullptr, &empty, &need);
  if (s != MQ_OK || empty) return s;
  MQ_REQUIRE(need <= kScratchBytes, MQ_ERR_WORKSPACE,
             "this shape needs %zu bytes of scratch; the allocation-free entry point has %zu "
             "(use mq_fused_layer with a workspace)", need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    s = scratch_address(&ws);
    if (s != MQ_OK) return s;
  }
  return layer_run(x, M, K, ldx, N, qw, sw, block, n_select, row_ptr, col_idx, qr, sr, y, ldy,
                   static_cast<uint8_t*>(ws), need, need > 0 ? kScratchBytes : 0, (hipStream_t)stream);
}

mq_status mq_residual_merge(const uint8_t* qa, const float* sa, int64_t M, int64_t N, int64_t K,
                            int32_t block, int32_t n_select, const int32_t* row_ptr,
                            const int32_t* col_idx, const uint8_t* qr, const uint16_t* sr,
                            uint16_t* y, int64_t ldy, void* stream) {
  g_err[0] = 0;
  MQ_REQUIRE(valid_block(block), MQ_ERR_BLOCK, "block = %d must be 32, 64 or 128", block);
  MQ_REQUIRE(M >= 0, MQ_ERR_SHAPE, "M = %lld must be >= 0", (long long)M);
  MQ_REQUIRE(N > 0 && N % block == 0, MQ_ERR_SHAPE, "N = %lld must be a positive multiple of %d",
             (long long)N, block);
  MQ_REQUIRE(K > 0 && K % kGroup == 0, MQ_ERR_SHAPE, "K = %lld must be a positive multiple of 128",
             (long long)K);
  MQ_REQUIRE(ldy >= N, MQ_ERR_SHAPE, "ldy = %lld < N = %lld", (long long)ldy, (long long)N);
  const int64_t B = block_count(N, K, block);
  MQ_REQUIRE(M < ((int64_t)1 << 31) && N < ((int64_t)1 << 31) && K < ((int64_t)1 << 31) &&
                 B < ((int64_t)1 << 31),
             MQ_ERR_SHAPE, "sizes must be below 2^31");
  MQ_REQUIRE(n_select >= 0 && n_select <= B, MQ_ERR_BUDGET, "n_select = %d outside [0, %lld]",
             n_select, (long long)B);
  if (M == 0 || n_select == 0) return MQ_OK;
  MQ_REQUIRE(qa && sa && y && row_ptr && col_idx && qr && sr, MQ_ERR_NULL_PTR,
             "qa, sa, y, row_ptr, col_idx, qr and sr must be non-NULL");
  MQ_REQUIRE(aligned16(qa) && aligned16(sa) && aligned16(y) && aligned16(row_ptr) &&
                 aligned16(col_idx) && aligned16(qr) && aligned16(sr),
             MQ_ERR_ALIGN, "device pointers must be 16-byte aligned");
  GemmArgs a = {};
  a.qa = qa;
  a.sa = sa;
  a.M = M;
  a.N = N;
  a.K = K;
  a.block = block;
  a.n_select = n_select;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.qr = qr;
  a.sr = sr;
  a.y = y;
  a.ldy = ldy;
  a.ksplit = 1;
  return hip_status(launch_residual_merge(a, (hipStream_t)stream), "mq_residual_merge launch");
}

mq_status mq_smooth_weights(const uint16_t* x_calib, int64_t T, const uint16_t* w, int64_t N,
                            int64_t K, float* x_absmax, float* w_absmax, float* scales,
                            uint16_t* w_out, void* stream) {
  g_err[0] = 0;
  MQ_REQUIRE(T >= 1 && N >= 1 && K >= 1, MQ_ERR_SHAPE, "T, N and K must be >= 1");
  // (row counts and K below 2^31 keep every launch's work-item count within
  // 32 bits: the column kernels take one thread per channel and one
  // workgroup row per 64 rows; the scaling kernel is a grid-stride loop)
  MQ_REQUIRE(T < ((int64_t)1 << 31) && N < ((int64_t)1 << 31) && K < ((int64_t)1 << 31) &&
                 N * K < ((int64_t)1 << 40) && T * K < ((int64_t)1 << 40),
             MQ_ERR_SHAPE, "sizes too large");
  MQ_REQUIRE(x_calib && w && x_absmax && w_absmax && scales && w_out, MQ_ERR_NULL_PTR,
             "x_calib, w, x_absmax, w_absmax, scales and w_out must be non-NULL");
  MQ_REQUIRE((const void*)w_out != (const void*)w, MQ_ERR_ARG, "w_out must not alias w");
  return hip_status(launch_smooth_weights(x_calib, T, w, N, K, x_absmax, w_absmax, scales, w_out,
                                          (hipStream_t)stream),
                    "mq_smooth_weights launch");
}

mq_status mq_smooth_acts(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                         const float* scales, uint16_t* x_out, void* stream) {
  g_err[0] = 0;
  MQ_REQUIRE(M >= 0 && K >= 1, MQ_ERR_SHAPE, "M must be >= 0 and K >= 1");
  MQ_REQUIRE(ldx >= K, MQ_ERR_SHAPE, "ldx = %lld < K = %lld", (long long)ldx, (long long)K);
  MQ_REQUIRE(M < ((int64_t)1 << 31) && K < ((int64_t)1 << 31) && M * K < ((int64_t)1 << 40),
             MQ_ERR_SHAPE, "sizes too large");
  if (M == 0) return MQ_OK;
  MQ_REQUIRE(x && scales && x_out, MQ_ERR_NULL_PTR, "x, scales and x_out must be non-NULL");
  return hip_status(launch_smooth_acts(x, M, K, ldx, scales, x_out, (hipStream_t)stream),
                    "mq_smooth_acts launch");
}

mq_status mq_measure_mfma(int32_t blocks, int32_t iters, int64_t* cycles, int32_t* sink,
                          void* stream) {
  g_err[0] = 0;
  MQ_REQUIRE(blocks >= 1 && blocks <= (1 << 20) && iters >= 1 && iters <= (1 << 24), MQ_ERR_SHAPE,
             "blocks = %d and iters = %d must be in [1, 2^20] and [1, 2^24]", blocks, iters);
  MQ_REQUIRE(cycles && sink, MQ_ERR_NULL_PTR, "cycles and sink must be non-NULL");
  MQ_REQUIRE(aligned16(cycles) && aligned16(sink), MQ_ERR_ALIGN, "cycles and sink must be 16-byte aligned");
  return hip_status(launch_mfma_rate(blocks, iters, cycles, sink, (hipStream_t)stream),
                    "mq_measure_mfma launch");
}

mq_status mq_validate_csr(const int32_t* row_ptr, const int32_t* col_idx, int64_t N, int64_t K,
                          int32_t block, int32_t n_select, void* stream) {
  g_err[0] = 0;
  MQ_REQUIRE(valid_block(block), MQ_ERR_BLOCK, "block = %d must be 32, 64 or 128", block);
  MQ_REQUIRE(N > 0 && N % block == 0 && K > 0 && K % kGroup == 0, MQ_ERR_SHAPE, "bad N or K");
  MQ_REQUIRE(row_ptr, MQ_ERR_NULL_PTR, "row_ptr must be non-NULL");
  MQ_REQUIRE(n_select >= 0, MQ_ERR_BUDGET, "n_select must be >= 0");
  MQ_REQUIRE(n_select == 0 || col_idx, MQ_ERR_NULL_PTR, "col_idx must be non-NULL");
  const int64_t B = block_count(N, K, block);
  MQ_REQUIRE(B < ((int64_t)1 << 31), MQ_ERR_SHAPE, "too many blocks (%lld)", (long long)B);
  MQ_REQUIRE(n_select <= B, MQ_ERR_BUDGET, "n_select = %d > %lld blocks", n_select, (long long)B);
  const int64_t NT = N / block, KT = K / block;
  std::vector<int32_t> rp(NT + 1), ci(n_select);
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e == hipSuccess)
    e = hipMemcpy(rp.data(), row_ptr, sizeof(int32_t) * (NT + 1), hipMemcpyDeviceToHost);
  if (e == hipSuccess && n_select)
    e = hipMemcpy(ci.data(), col_idx, sizeof(int32_t) * n_select, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_status(e, "mq_validate_csr copy");
  MQ_REQUIRE(rp[0] == 0, MQ_ERR_CSR, "row_ptr[0] = %d", rp[0]);
  MQ_REQUIRE(rp[NT] == n_select, MQ_ERR_CSR, "row_ptr[%lld] = %d != n_select = %d", (long long)NT,
             rp[NT], n_select);
  for (int64_t t = 0; t < NT; ++t) {
    MQ_REQUIRE(rp[t + 1] >= rp[t], MQ_ERR_CSR, "row_ptr decreases at %lld", (long long)t);
    for (int32_t i = rp[t]; i < rp[t + 1]; ++i) {
      MQ_REQUIRE(ci[i] >= 0 && ci[i] < KT, MQ_ERR_CSR, "col_idx[%d] = %d out of range", i, ci[i]);
      MQ_REQUIRE(i == rp[t] || ci[i] > ci[i - 1], MQ_ERR_CSR, "col_idx not ascending at %d", i);
    }
  }
  return MQ_OK;
}


// ---- the fp6 route with prepared operands ----

static mq_status fp6_shape(int64_t M, int64_t N, int64_t K, int32_t block, int32_t n_select) {
  MQ_REQUIRE(block == 64 || block == 128, MQ_ERR_BLOCK, "block = %d: the fp6 route takes 64 or 128", block);
  MQ_REQUIRE(M >= 0 && M < ((int64_t)1 << 31), MQ_ERR_SHAPE, "M = %lld outside [0, 2^31)", (long long)M);
  MQ_REQUIRE(N > 0 && N % block == 0 && N < ((int64_t)1 << 31), MQ_ERR_SHAPE,
             "N = %lld must be a positive multiple of %d below 2^31", (long long)N, block);
  MQ_REQUIRE(K > 0 && K % kGroup == 0 && K < ((int64_t)1 << 31), MQ_ERR_SHAPE,
             "K = %lld must be a positive multiple of 128 below 2^31", (long long)K);
  MQ_REQUIRE(M * K < ((int64_t)1 << 32) && N * K < ((int64_t)1 << 32), MQ_ERR_SHAPE,
             "M*K and N*K must each be below 2^32");
  const int64_t B = block_count(N, K, block);
  MQ_REQUIRE(n_select >= 0 && n_select <= B, MQ_ERR_BUDGET, "n_select = %d outside [0, %lld]", n_select,
             (long long)B);
  MQ_REQUIRE((int64_t)n_select * block * block < ((int64_t)1 << 32), MQ_ERR_SHAPE, "residual too large");
  return MQ_OK;
}

mq_status mq_fp6_sizes(int64_t M, int64_t N, int64_t K, int32_t block, int32_t n_select, size_t* act_bytes,
                       size_t* weight_bytes, size_t* split_bytes) {
  g_err[0] = 0;
  MQ_REQUIRE(act_bytes && weight_bytes && split_bytes, MQ_ERR_NULL_PTR, "size outputs must be non-NULL");
  const mq_status s = fp6_shape(M, N, K, block, n_select);
  if (s != MQ_OK) return s;
  *act_bytes = fp6_rows_bytes(M, K);
  *weight_bytes = round256(fp6_rows_bytes(N, K)) + fp6_residual_bytes(n_select, block);
  *split_bytes = split6_workspace(M, N, K);
  return MQ_OK;
}

mq_status mq_fp6_prepare_acts(const uint8_t* qa, int64_t M, int64_t K, uint8_t* act_img, void* stream) {
  g_err[0] = 0;
  MQ_REQUIRE(K > 0 && K % kGroup == 0 && K < ((int64_t)1 << 31), MQ_ERR_SHAPE,
             "K = %lld must be a positive multiple of 128 below 2^31", (long long)K);
  MQ_REQUIRE(M >= 0 && M < ((int64_t)1 << 31) && M * K < ((int64_t)1 << 32), MQ_ERR_SHAPE,
             "M = %lld: M must be in [0, 2^31) and M*K below 2^32", (long long)M);
  if (M == 0) return MQ_OK;
  MQ_REQUIRE(qa && act_img, MQ_ERR_NULL_PTR, "qa and act_img must be non-NULL");
  MQ_REQUIRE(aligned16(qa) && aligned16(act_img), MQ_ERR_ALIGN, "device pointers must be 16-byte aligned");
  return hip_status(launch_acts_fp6(qa, M, K, act_img, (hipStream_t)stream), "mq_fp6_prepare_acts launch");
}

mq_status mq_fp6_prepare_weights(const uint8_t* qw, int64_t N, int64_t K, int32_t block, int32_t n_select,
                                 const uint8_t* qr, uint8_t* weight_img, void* stream) {
  g_err[0] = 0;
  const mq_status s = fp6_shape(0, N, K, block, n_select);
  if (s != MQ_OK) return s;
  MQ_REQUIRE(qw && weight_img && (n_select == 0 || qr), MQ_ERR_NULL_PTR,
             "qw, weight_img (and qr when n_select > 0) must be non-NULL");
  MQ_REQUIRE(aligned16(qw) && aligned16(qr) && aligned16(weight_img), MQ_ERR_ALIGN,
             "device pointers must be 16-byte aligned");
  hipError_t e = launch_weights_fp6(qw, N, K, weight_img, (hipStream_t)stream);
  if (e == hipSuccess)
    e = launch_residual_fp6(qr, n_select, block, weight_img + round256(fp6_rows_bytes(N, K)), (hipStream_t)stream);
  return hip_status(e, "mq_fp6_prepare_weights launch");
}

mq_status mq_fused_gemm_fp6(const uint8_t* act_img, const float* sa, int64_t M, int64_t N, int64_t K,
                            const uint8_t* weight_img, const uint16_t* sw, int32_t block, int32_t n_select,
                            const int32_t* row_ptr, const int32_t* col_idx, const uint16_t* sr, uint16_t* y,
                            int64_t ldy, void* split_ws, size_t split_bytes, uint32_t flags, int32_t* acc_dump,
                            void* stream) {
  g_err[0] = 0;
  MQ_REQUIRE((flags & ~MQ_FLAG_DUMP_ACC) == 0, MQ_ERR_ARG, "unknown flags 0x%x", flags);
  mq_status s = fp6_shape(M, N, K, block, n_select);
  if (s != MQ_OK) return s;
  MQ_REQUIRE(M == 0 || M > 32, MQ_ERR_SHAPE, "M = %lld: the fp6 route takes M > 32", (long long)M);
  MQ_REQUIRE(ldy >= N && ldy % 8 == 0, MQ_ERR_SHAPE, "ldy = %lld must be >= N and a multiple of 8",
             (long long)ldy);
  if (M == 0) return MQ_OK;
  MQ_REQUIRE(act_img && sa && weight_img && sw && y, MQ_ERR_NULL_PTR,
             "act_img, sa, weight_img, sw and y must be non-NULL");
  MQ_REQUIRE(n_select == 0 || (row_ptr && col_idx && sr), MQ_ERR_NULL_PTR,
             "row_ptr, col_idx and sr must be non-NULL when n_select > 0");
  MQ_REQUIRE(!(flags & MQ_FLAG_DUMP_ACC) || acc_dump, MQ_ERR_NULL_PTR, "acc_dump must be non-NULL with the flag");
  MQ_REQUIRE(aligned16(act_img) && aligned16(sa) && aligned16(weight_img) && aligned16(sw) && aligned16(y) &&
                 aligned16(row_ptr) && aligned16(col_idx) && aligned16(sr) && aligned16(split_ws) &&
                 aligned16(acc_dump),
             MQ_ERR_ALIGN, "device pointers must be 16-byte aligned");
  const size_t split = split6_workspace(M, N, K);
  MQ_REQUIRE(split == 0 || (split_ws && split_bytes >= split), MQ_ERR_WORKSPACE,
             "split-K workspace of %zu bytes given, %zu needed", split_bytes, split);
  GemmArgs a = {};
  a.sa = sa;
  a.M = M;
  a.N = N;
  a.K = K;
  a.qw = nullptr;
  a.sw = sw;
  a.block = block;
  a.n_select = n_select;
  a.row_ptr = n_select ? row_ptr : nullptr;
  a.col_idx = n_select ? col_idx : nullptr;
  a.sr = n_select ? sr : nullptr;
  a.y = y;
  a.ldy = ldy;
  a.acc_dump = (flags & MQ_FLAG_DUMP_ACC) ? acc_dump : nullptr;
  a.aimg = act_img;
  a.wimg = weight_img;
  a.rimg = weight_img + round256(fp6_rows_bytes(N, K));
  MQ_REQUIRE(tile6_gemm_fits(a), MQ_ERR_SHAPE, "K = %lld too long for the fp6 kernel's residual table",
             (long long)K);
  a.part = split > 0 ? static_cast<float*>(split_ws) : nullptr;
  a.ksplit = split > 0 ? tile6_gemm_splits(M, N, K) : 1;
  return hip_status(launch_tile6_gemm(a, (hipStream_t)stream), "mq_fused_gemm_fp6 launch");
}

}  // extern "C"
