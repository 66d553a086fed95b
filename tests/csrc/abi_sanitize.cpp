// Host-side argument validation of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer (signed overflow, shifts, out-of-bounds):
// every call here either is a pure host query (workspace sizes) or is
// rejected by validation before anything reaches the device, so no GPU is
// needed.  Pointer values are fake and never dereferenced.  Prints the
// number of calls and failures; exits non-zero on a failed expectation.
#include <limits.h>
#include <stdint.h>
#include <stdio.h>

#include <initializer_list>

#include "mosaicq.h"

static int calls = 0, fails = 0;

static void expect(const char* what, int line, mq_status got, int want0, int want1 = -1, int want2 = -1,
                   int want3 = -1) {
  ++calls;
  if (got != want0 && got != want1 && got != want2 && got != want3) {
    printf("FAIL %s (line %d): status %d, detail: %s\n", what, line, (int)got, mq_last_error());
    ++fails;
  }
}
#define EXPECT(call, ...) expect(#call, __LINE__, (call), __VA_ARGS__)

int main() {
  uint8_t* const P8 = reinterpret_cast<uint8_t*>(0x1000);
  uint16_t* const P16 = reinterpret_cast<uint16_t*>(0x1000);
  int32_t* const P32 = reinterpret_cast<int32_t*>(0x1000);
  float* const PF = reinterpret_cast<float*>(0x1000);
  double* const PD = reinterpret_cast<double*>(0x1000);
  uint16_t* const PM16 = reinterpret_cast<uint16_t*>(0x1008);  // misaligned by 8
  void* const PV = reinterpret_cast<void*>(0x1000);
  const int64_t sizes[] = {INT64_MIN, -129, -1, 0, 1, 16, 31, 32, 33, 127, 128, 129, 4096, 25600,
                           (int64_t)1 << 20, ((int64_t)1 << 31) - 1, (int64_t)1 << 31, (int64_t)1 << 32,
                           (int64_t)1 << 40, (int64_t)1 << 62, INT64_MAX};
  const int32_t blocks[] = {INT32_MIN, -64, 0, 16, 32, 48, 64, 128, 256, INT32_MAX};
  const int OK = MQ_OK, SHAPE = MQ_ERR_SHAPE, BLOCK = MQ_ERR_BLOCK;

  // workspace queries: OK or a shape error for every combination, never UB
  size_t bytes = 0;
  for (int64_t M : sizes)
    for (int64_t N : sizes)
      for (int64_t K : sizes) {
        EXPECT(mq_fused_gemm_workspace(M, N, K, &bytes), OK, SHAPE);
        EXPECT(mq_fused_layer_workspace(M, N, K, &bytes), OK, SHAPE);
      }
  for (int64_t N : sizes)
    for (int64_t K : sizes)
      for (int64_t T : sizes)
        for (int32_t b : blocks) {
          EXPECT(mq_select_exact_workspace(N, K, T, b, &bytes), OK, SHAPE, BLOCK);
          EXPECT(mq_distortion_workspace(N, K, T, b, &bytes), OK, SHAPE, BLOCK);
        }
  EXPECT(mq_fused_gemm_workspace(16, 4096, 4096, nullptr), MQ_ERR_NULL_PTR);
  // the fp6 route's size query: OK, a shape, block or budget error, never UB
  size_t ab = 0, wb = 0, pb = 0;
  for (int64_t M : sizes)
    for (int64_t N : sizes)
      for (int64_t K : sizes)
        for (int32_t b : blocks)
          for (int32_t ns : {0, 1, INT32_MAX})
            EXPECT(mq_fp6_sizes(M, N, K, b, ns, &ab, &wb, &pb), OK, SHAPE, BLOCK, MQ_ERR_BUDGET);
  EXPECT(mq_fp6_sizes(4096, 4096, 4096, 64, 0, nullptr, &wb, &pb), MQ_ERR_NULL_PTR);

  // entry points with extreme sizes: rejected before any device work (the
  // other arguments are otherwise valid-looking, so the size checks are
  // what runs)
  for (int64_t big : {(int64_t)1 << 40, (int64_t)1 << 62, INT64_MAX, INT64_MIN, (int64_t)-1}) {
    EXPECT(mq_quantize_act(P16, big, 4096, 4096, P8, PF, nullptr), SHAPE);
    EXPECT(mq_quantize_act(P16, 16, big, big, P8, PF, nullptr), SHAPE);
    EXPECT(mq_select_blocks(P16, P16, big, 4096, 64, 64, 1, P32, PD, PD, nullptr), SHAPE);
    EXPECT(mq_select_blocks(P16, P16, 4096, big, 64, 64, 1, P32, PD, PD, nullptr), SHAPE);
    EXPECT(mq_select_blocks(P16, P16, 4096, 4096, big, 64, 1, P32, PD, PD, nullptr), SHAPE);
    EXPECT(mq_pack_weights(P16, big, 4096, 64, P32, 1, P8, P16, P32, P32, P8, P16, nullptr), SHAPE);
    EXPECT(mq_pack_weights(P16, 4096, big, 64, P32, 1, P8, P16, P32, P32, P8, P16, nullptr), SHAPE);
    EXPECT(mq_fused_gemm(P8, PF, big, 4096, 4096, P8, P16, 64, 1, P32, P32, P8, P16, P16, 4096, nullptr, 0, 0,
                         nullptr, nullptr), SHAPE);
    EXPECT(mq_fused_gemm(P8, PF, 16, big, 4096, P8, P16, 64, 1, P32, P32, P8, P16, P16, 4096, nullptr, 0, 0,
                         nullptr, nullptr), SHAPE);
    EXPECT(mq_fused_gemm(P8, PF, 16, 4096, big, P8, P16, 64, 1, P32, P32, P8, P16, P16, 4096, nullptr, 0, 0,
                         nullptr, nullptr), SHAPE);
    EXPECT(mq_fused_layer(P16, big, 4096, 4096, 4096, P8, P16, 64, 1, P32, P32, P8, P16, P16, 4096, nullptr, 0,
                          nullptr), SHAPE);
    EXPECT(mq_fused_layer(P16, 16, big, big, 4096, P8, P16, 64, 1, P32, P32, P8, P16, P16, 4096, nullptr, 0,
                          nullptr), SHAPE);
    EXPECT(mq_fused_layer(P16, 16, 4096, 4096, big, P8, P16, 64, 1, P32, P32, P8, P16, P16, big, nullptr, 0,
                          nullptr), SHAPE);
    EXPECT(mq_fused_layer_noalloc(P16, big, 4096, 4096, 4096, P8, P16, 64, 1, P32, P32, P8, P16, P16, 4096,
                                  nullptr), SHAPE);
    EXPECT(mq_residual_merge(P8, PF, big, 4096, 4096, 64, 1, P32, P32, P8, P16, P16, 4096, nullptr), SHAPE);
    EXPECT(mq_residual_merge(P8, PF, 16, big, 4096, 64, 1, P32, P32, P8, P16, P16, big, nullptr), SHAPE);
    EXPECT(mq_smooth_weights(P16, big, P16, 4096, 4096, PF, PF, PF, P16, nullptr), SHAPE);
    EXPECT(mq_smooth_weights(P16, 64, P16, big, 4096, PF, PF, PF, P16, nullptr), SHAPE);
    EXPECT(mq_smooth_weights(P16, 64, P16, 4096, big, PF, PF, PF, P16, nullptr), SHAPE);
    EXPECT(mq_smooth_acts(P16, big, 4096, 4096, PF, P16, nullptr), SHAPE);
    EXPECT(mq_smooth_acts(P16, 16, big, big, PF, P16, nullptr), SHAPE);
    EXPECT(mq_select_exact_greedy(P16, P16, big, 4096, 64, 64, 1, P32, nullptr, nullptr, nullptr, PV,
                                  (size_t)1 << 40, nullptr), SHAPE);
    EXPECT(mq_select_exact_greedy(P16, P16, 4096, 4096, big, 64, 1, P32, nullptr, nullptr, nullptr, PV,
                                  (size_t)1 << 40, nullptr), SHAPE);
    EXPECT(mq_distortion(P16, P16, 4096, big, 64, 64, P32, 1, PD, PV, (size_t)1 << 40, nullptr), SHAPE);
    EXPECT(mq_validate_csr(P32, P32, big, 4096, 64, 1, nullptr), SHAPE, MQ_ERR_CSR);
    // the fp6 route's preparation and GEMM: every extreme size rejected
    EXPECT(mq_fp6_prepare_acts(P8, big, 4096, P8, nullptr), SHAPE);
    EXPECT(mq_fp6_prepare_acts(P8, 4096, big, P8, nullptr), SHAPE);
    EXPECT(mq_fp6_prepare_weights(P8, big, 4096, 64, 1, P8, P8, nullptr), SHAPE);
    EXPECT(mq_fp6_prepare_weights(P8, 4096, big, 64, 1, P8, P8, nullptr), SHAPE);
    EXPECT(mq_fused_gemm_fp6(P8, PF, big, 4096, 4096, P8, P16, 64, 1, P32, P32, P16, P16, 4096, nullptr, 0, 0,
                             nullptr, nullptr), SHAPE);
    EXPECT(mq_fused_gemm_fp6(P8, PF, 4096, big, 4096, P8, P16, 64, 1, P32, P32, P16, P16, 4096, nullptr, 0, 0,
                             nullptr, nullptr), SHAPE);
    EXPECT(mq_fused_gemm_fp6(P8, PF, 4096, 4096, big, P8, P16, 64, 1, P32, P32, P16, P16, 4096, nullptr, 0, 0,
                             nullptr, nullptr), SHAPE);
  }

  // budgets, blocks, null and misaligned pointers
  for (int32_t b : blocks) {
    if (b == 32 || b == 64 || b == 128) continue;
    EXPECT(mq_select_blocks(P16, P16, 4096, 4096, 64, b, 1, P32, PD, PD, nullptr), BLOCK);
    EXPECT(mq_fused_layer(P16, 16, 4096, 4096, 4096, P8, P16, b, 1, P32, P32, P8, P16, P16, 4096, nullptr, 0,
                          nullptr), BLOCK);
  }
  for (int32_t b : blocks) {
    if (b == 64 || b == 128) continue;
    EXPECT(mq_fp6_prepare_weights(P8, 4096, 4096, b, 1, P8, P8, nullptr), BLOCK);
    EXPECT(mq_fused_gemm_fp6(P8, PF, 4096, 4096, 4096, P8, P16, b, 1, P32, P32, P16, P16, 4096, nullptr, 0, 0,
                             nullptr, nullptr), BLOCK);
  }
  for (int32_t ns : {INT32_MIN, -1, 4097, INT32_MAX}) {
    EXPECT(mq_fp6_prepare_weights(P8, 4096, 4096, 64, ns, P8, P8, nullptr), MQ_ERR_BUDGET);
    EXPECT(mq_fused_gemm_fp6(P8, PF, 4096, 4096, 4096, P8, P16, 64, ns, P32, P32, P16, P16, 4096, nullptr, 0, 0,
                             nullptr, nullptr), MQ_ERR_BUDGET);
  }
  EXPECT(mq_fused_gemm_fp6(P8, PF, 16, 4096, 4096, P8, P16, 64, 1, P32, P32, P16, P16, 4096, nullptr, 0, 0,
                           nullptr, nullptr), SHAPE);  // M <= 32
  EXPECT(mq_fused_gemm_fp6(P8, PF, 4096, 4096, 4096, P8, P16, 64, 1, P32, P32, P16, PM16, 4096, nullptr, 0, 0,
                           nullptr, nullptr), MQ_ERR_ALIGN);
  for (int32_t ns : {INT32_MIN, -1, 4097, INT32_MAX}) {
    EXPECT(mq_select_blocks(P16, P16, 4096, 4096, 64, 64, ns, P32, PD, PD, nullptr), MQ_ERR_BUDGET);
    EXPECT(mq_fused_gemm(P8, PF, 16, 4096, 4096, P8, P16, 64, ns, P32, P32, P8, P16, P16, 4096, nullptr, 0, 0,
                         nullptr, nullptr), MQ_ERR_BUDGET);
    EXPECT(mq_select_exact_greedy(P16, P16, 4096, 4096, 64, 64, ns, P32, nullptr, nullptr, nullptr, PV,
                                  (size_t)1 << 40, nullptr), MQ_ERR_BUDGET);
  }
  EXPECT(mq_quantize_act(nullptr, 16, 4096, 4096, P8, PF, nullptr), MQ_ERR_NULL_PTR);
  EXPECT(mq_quantize_act(PM16, 16, 4096, 4096, P8, PF, nullptr), MQ_ERR_ALIGN);
  EXPECT(mq_fused_gemm(P8, PF, 16, 4096, 4096, P8, P16, 64, 1, P32, P32, P8, P16, PM16, 4096, nullptr, 0, 0,
                       nullptr, nullptr), MQ_ERR_ALIGN);
  EXPECT(mq_fused_gemm(P8, PF, 16, 4096, 4096, P8, P16, 64, 1, P32, P32, P8, P16, P16, 4096, nullptr, 0, 0x80,
                       nullptr, nullptr), MQ_ERR_ARG);
  EXPECT(mq_measure_mfma(0, 10, reinterpret_cast<int64_t*>(P8), P32, nullptr), SHAPE);
  EXPECT(mq_measure_mfma(INT32_MIN, INT32_MIN, reinterpret_cast<int64_t*>(P8), P32, nullptr), SHAPE);

  // status strings for every code, including unknown ones
  for (int s : {INT_MIN, -1, 0, 1, 5, 9, 10, INT_MAX}) {
    ++calls;
    if (!mq_status_str(s)) ++fails;
  }
  printf("calls %d failures %d\n", calls, fails);
  return fails ? 1 : 0;
}
