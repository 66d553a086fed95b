// C ABI of libmosaicq: argument validation, then launches on the caller's
// stream.  Nothing is enqueued when validation fails.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

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
  MQ_REQUIRE(M <= (int64_t)1 << 31 && M * (K / kGroup) < (int64_t)1 << 36, MQ_ERR_SHAPE,
             "M x K too large");
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
  const int64_t B = (N / block) * (K / block);
  MQ_REQUIRE(B < ((int64_t)1 << 31), MQ_ERR_SHAPE, "too many blocks (%lld)", (long long)B);
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
  const int64_t B = (N / block) * (K / block);
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

// Split-K partials of the tile kernel: [splits][M][N] fp32 when M > 32 and
// the tiles alone would leave compute units idle; 0 otherwise.
static size_t split_workspace(int64_t M, int64_t N, int64_t K) {
  if (M <= 32 || N <= 0 || K < kGroup) return 0;
  const int ks = tile_gemm_splits(M, N, K);
  return ks > 1 ? (size_t)ks * (size_t)M * (size_t)N * sizeof(float) : 0;
}

mq_status mq_fused_gemm_workspace(int64_t M, int64_t N, int64_t K, size_t* bytes) {
  g_err[0] = 0;
  MQ_REQUIRE(bytes, MQ_ERR_NULL_PTR, "bytes must be non-NULL");
  MQ_REQUIRE(M >= 0 && N >= 0 && K >= 0, MQ_ERR_SHAPE, "sizes must be >= 0");
  *bytes = split_workspace(M, N, K);
  return MQ_OK;
}

mq_status mq_fused_gemm(const uint8_t* qa, const float* sa, int64_t M, int64_t N, int64_t K,
                        const uint8_t* qw, const uint16_t* sw, int32_t block, int32_t n_select,
                        const int32_t* row_ptr, const int32_t* col_idx, const uint8_t* qr,
                        const uint16_t* sr, uint16_t* y, int64_t ldy, void* workspace,
                        size_t workspace_bytes, uint32_t flags, int32_t* acc_dump,
                        void* stream) {
  g_err[0] = 0;
  MQ_REQUIRE((flags & ~MQ_FLAG_DUMP_ACC) == 0, MQ_ERR_ARG, "unknown flags 0x%x", flags);
  MQ_REQUIRE(valid_block(block), MQ_ERR_BLOCK, "block = %d must be 32, 64 or 128", block);
  MQ_REQUIRE(M >= 0, MQ_ERR_SHAPE, "M = %lld must be >= 0", (long long)M);
  MQ_REQUIRE(N > 0 && N % block == 0, MQ_ERR_SHAPE, "N = %lld must be a positive multiple of %d",
             (long long)N, block);
  MQ_REQUIRE(K > 0 && K % kGroup == 0, MQ_ERR_SHAPE, "K = %lld must be a positive multiple of 128",
             (long long)K);
  MQ_REQUIRE(ldy >= N, MQ_ERR_SHAPE, "ldy = %lld < N = %lld", (long long)ldy, (long long)N);
  const int64_t B = (N / block) * (K / block);
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
  // split-K only with a large enough workspace; otherwise one pass over K
  const size_t need = split_workspace(M, N, K);
  const bool split = need > 0 && workspace && workspace_bytes >= need && aligned16(workspace);
  a.part = split ? static_cast<float*>(workspace) : nullptr;
  a.ksplit = split ? tile_gemm_splits(M, N, K) : 1;
  return hip_status(launch_fused_gemm(a, (hipStream_t)stream), "mq_fused_gemm launch");
}

static size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

// Workspace of mq_fused_layer: none when the streaming kernel quantises the
// activations itself; otherwise the codes and scales of mq_quantize_act,
// then the fused GEMM's split-K partials.
static size_t layer_workspace(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K < kGroup || stream_quant_fits(M, N, K)) return 0;
  return round256((size_t)M * (size_t)(K / 2)) + round256((size_t)M * (size_t)(K / kGroup) * 4) +
         split_workspace(M, N, K);
}

mq_status mq_fused_layer_workspace(int64_t M, int64_t N, int64_t K, size_t* bytes) {
  g_err[0] = 0;
  MQ_REQUIRE(bytes, MQ_ERR_NULL_PTR, "bytes must be non-NULL");
  MQ_REQUIRE(M >= 0 && N >= 0 && K >= 0, MQ_ERR_SHAPE, "sizes must be >= 0");
  *bytes = layer_workspace(M, N, K);
  return MQ_OK;
}

mq_status mq_fused_layer(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int64_t N,
                         const uint8_t* qw, const uint16_t* sw, int32_t block, int32_t n_select,
                         const int32_t* row_ptr, const int32_t* col_idx, const uint8_t* qr,
                         const uint16_t* sr, uint16_t* y, int64_t ldy, void* workspace,
                         size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  MQ_REQUIRE(valid_block(block), MQ_ERR_BLOCK, "block = %d must be 32, 64 or 128", block);
  MQ_REQUIRE(M >= 0, MQ_ERR_SHAPE, "M = %lld must be >= 0", (long long)M);
  MQ_REQUIRE(N > 0 && N % block == 0, MQ_ERR_SHAPE, "N = %lld must be a positive multiple of %d",
             (long long)N, block);
  MQ_REQUIRE(K > 0 && K % kGroup == 0, MQ_ERR_SHAPE, "K = %lld must be a positive multiple of 128",
             (long long)K);
  MQ_REQUIRE(ldx >= K, MQ_ERR_SHAPE, "ldx = %lld < K = %lld", (long long)ldx, (long long)K);
  MQ_REQUIRE(ldy >= N, MQ_ERR_SHAPE, "ldy = %lld < N = %lld", (long long)ldy, (long long)N);
  const int64_t B = (N / block) * (K / block);
  MQ_REQUIRE(B < ((int64_t)1 << 31), MQ_ERR_SHAPE, "too many blocks (%lld)", (long long)B);
  MQ_REQUIRE(M < ((int64_t)1 << 31) && N < ((int64_t)1 << 31) && K < ((int64_t)1 << 31),
             MQ_ERR_SHAPE, "sizes must be below 2^31");
  MQ_REQUIRE(N * (K / 2) < ((int64_t)1 << 32) && M * (K / 2) < ((int64_t)1 << 32), MQ_ERR_SHAPE,
             "packed weights and activations must each be below 4 GiB");
  MQ_REQUIRE(n_select >= 0 && n_select <= B, MQ_ERR_BUDGET, "n_select = %d outside [0, %lld]",
             n_select, (long long)B);
  if (M == 0) return MQ_OK;
  MQ_REQUIRE(x && qw && sw && y, MQ_ERR_NULL_PTR, "x, qw, sw and y must be non-NULL");
  MQ_REQUIRE(n_select == 0 || (row_ptr && col_idx && qr && sr), MQ_ERR_NULL_PTR,
             "row_ptr, col_idx, qr and sr must be non-NULL when n_select > 0");
  MQ_REQUIRE(ldx % 8 == 0 && ldy % 8 == 0, MQ_ERR_ALIGN,
             "ldx = %lld and ldy = %lld must be multiples of 8", (long long)ldx, (long long)ldy);
  MQ_REQUIRE(aligned16(x) && aligned16(qw) && aligned16(sw) && aligned16(y) &&
                 aligned16(row_ptr) && aligned16(col_idx) && aligned16(qr) && aligned16(sr) &&
                 aligned16(workspace),
             MQ_ERR_ALIGN, "device pointers must be 16-byte aligned");
  const size_t need = layer_workspace(M, N, K);
  MQ_REQUIRE(workspace_bytes >= need && (need == 0 || workspace), MQ_ERR_WORKSPACE,
             "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
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
    return hip_status(launch_fused_gemm(a, (hipStream_t)stream), "mq_fused_layer launch");
  }
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint8_t* qa = ws;
  float* sa = reinterpret_cast<float*>(ws + round256((size_t)M * (size_t)(K / 2)));
  const mq_status st = hip_status(launch_act_quant(x, M, K, ldx, qa, sa, (hipStream_t)stream),
                                  "mq_fused_layer act-quant launch");
  if (st != MQ_OK) return st;
  a.qa = qa;
  a.sa = sa;
  const size_t split = split_workspace(M, N, K);
  if (split > 0) {
    a.part = reinterpret_cast<float*>(ws + need - split);
    a.ksplit = tile_gemm_splits(M, N, K);
  }
  return hip_status(launch_fused_gemm(a, (hipStream_t)stream), "mq_fused_layer launch");
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
  const int64_t B = (N / block) * (K / block);
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
  MQ_REQUIRE(N * K < ((int64_t)1 << 40) && T * K < ((int64_t)1 << 40), MQ_ERR_SHAPE, "sizes too large");
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
  MQ_REQUIRE(M * K < ((int64_t)1 << 40), MQ_ERR_SHAPE, "sizes too large");
  if (M == 0) return MQ_OK;
  MQ_REQUIRE(x && scales && x_out, MQ_ERR_NULL_PTR, "x, scales and x_out must be non-NULL");
  return hip_status(launch_smooth_acts(x, M, K, ldx, scales, x_out, (hipStream_t)stream),
                    "mq_smooth_acts launch");
}

mq_status mq_validate_csr(const int32_t* row_ptr, const int32_t* col_idx, int64_t N, int64_t K,
                          int32_t block, int32_t n_select, void* stream) {
  g_err[0] = 0;
  MQ_REQUIRE(valid_block(block), MQ_ERR_BLOCK, "block = %d must be 32, 64 or 128", block);
  MQ_REQUIRE(N > 0 && N % block == 0 && K > 0 && K % kGroup == 0, MQ_ERR_SHAPE, "bad N or K");
  MQ_REQUIRE(row_ptr, MQ_ERR_NULL_PTR, "row_ptr must be non-NULL");
  MQ_REQUIRE(n_select >= 0, MQ_ERR_BUDGET, "n_select must be >= 0");
  MQ_REQUIRE(n_select == 0 || col_idx, MQ_ERR_NULL_PTR, "col_idx must be non-NULL");
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

}  // extern "C"
