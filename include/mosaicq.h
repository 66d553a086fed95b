/*
 * mosaicq.h - C ABI of the MI355X (gfx950) MosaicQuant fused linear layer.
 *
 * The layer computes Y = deq(Qa(X) . Q(W)^T) + deq(Qa(X) . R^T): a dense
 * 4-bit base Q(W) of the whole weight plus a 4-bit residual R kept only on
 * the b x b weight blocks with the largest Hessian-guided Delta-scores.
 *   - decomposition W ~ Q(W) + R, both parts 4-bit: MosaicQuant technical
 *     summary, gist.science/pt/paper/2606.15652, Metodologia 1;
 *   - block-level budget, Delta-score, top-K: same page, Metodologia 2;
 *   - one fused kernel for quantisation, dense compute, sparse compensation
 *     and reduce-sum: same page, Metodologia 3 (ZipperEngine), and the
 *     authors' abstract, fugumt.com/fugumt/paper_check/2606.15652v1.
 *
 * Fixed configuration: groups of 128 input channels; symmetric 4-bit codes
 * in [-7, 7] (code = clamp(rint(v / s), -7, 7), 0 when s == 0, the quotient
 * an IEEE fp32 division rounded half-to-even); scale = amax / 7 in fp32,
 * rounded to fp16 (nearest-even, subnormals kept) for weights and residuals
 * and kept fp32 for activations; residual block edge b in {32, 64, 128}.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked "host".  Matrices are
 *     row-major.  fp16 data is passed as uint16_t bit patterns.
 *   - 4-bit codes are packed two per byte along the input-channel axis,
 *     two's complement: byte i = (q[2i] & 0xF) | ((q[2i+1] & 0xF) << 4).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued on it and the call returns without synchronising;
 *     the caller keeps every buffer alive until the stream has drained.
 *   - The caller owns and allocates every buffer.  The library keeps no
 *     pointer after a call returns and allocates no device memory.
 *   - Every argument is validated before anything is enqueued.  On a
 *     violation nothing is enqueued, the first violation's code is returned
 *     and mq_last_error() describes it.  A failed launch returns
 *     MQ_ERR_HIP.  Faults inside kernels surface at the caller's next
 *     synchronisation.  No call aborts or throws.
 *   - Device pointers must be 16-byte aligned; leading dimensions are in
 *     elements.
 *   - Weights must be finite.  Activations may hold +-inf: a group whose
 *     largest magnitude is infinite gets scale +inf and codes 0 (the IEEE
 *     quotient v/inf is 0; inf/inf, not a number, gives 0 too), so y is
 *     NaN wherever that group contributes.  NaN inputs give unspecified
 *     codes.
 */
#ifndef MOSAICQ_H
#define MOSAICQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MQ_OK = 0,
  MQ_ERR_NULL_PTR = 1,   /* a required pointer is NULL                        */
  MQ_ERR_SHAPE = 2,      /* a size is negative, not a multiple it must be, or
                            a leading dimension is too small                   */
  MQ_ERR_ALIGN = 3,      /* a pointer or leading dimension is misaligned       */
  MQ_ERR_BLOCK = 4,      /* residual block edge not in {32, 64, 128}           */
  MQ_ERR_BUDGET = 5,     /* n_select outside [0, number of blocks]             */
  MQ_ERR_CSR = 6,        /* CSR arrays inconsistent (mq_validate_csr only)     */
  MQ_ERR_WORKSPACE = 7,  /* workspace too small                                */
  MQ_ERR_HIP = 8,        /* the HIP runtime reported an error                  */
  MQ_ERR_ARG = 9         /* any other invalid argument (unknown flag, ...)     */
} mq_status;

/* Human-readable name of a status code (static string). */
const char* mq_status_str(int status);

/* Detail of the most recent failure on the calling thread ("" if none).
   The string stays valid until the next mq_* call on that thread. */
const char* mq_last_error(void);

/* ABI version: (major << 16) | minor. */
int mq_version(void);

/* Group of input channels sharing one scale. */
#define MQ_GROUP 128

/*
 * Activation quantisation Qa(X): per token m and group j of 128 channels,
 *   sa[m][j] = max_k |x[m][k]| / 7         (fp32 division, kept fp32)
 *   qa code  = clamp(rint(x / sa[m][j]), -7, 7)   (0 if sa == 0).
 * [summary-pt Metodologia 3: quantisation is one stage of the fused
 * pipeline; Resultados: W4A4.]
 *   x  : fp16 [M][ldx], ldx >= K, ldx % 8 == 0
 *   qa : uint8 [M][K/2] packed codes (output)
 *   sa : fp32  [M][K/128] (output)
 *   M >= 0 (M == 0 enqueues nothing), K > 0, K % 128 == 0.
 */
mq_status mq_quantize_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                          uint8_t* qa, float* sa, void* stream);

/*
 * Offline block selection.  For W fp16 [N][K] and calibration tokens
 * Xc fp16 [T][K]:
 *   base   sw = f16(amax/7) per (row, group), qw = clamp(rint(W/sw))
 *   error  E = W - sw*qw (fp32)
 *   per b x b block i and block row r: sr = f16(max_c |E| / 7),
 *          R_hat = sr * clamp(rint(E / sr))
 *   H[k]   = sum_t Xc[t][k]^2 in fp64, t = 0, 1, ... in order
 *   Delta_i = sum_r ( sum_c H[k] * (E^2 - (E - R_hat)^2) ) in fp64, each sum
 *            left to right from +0, k = kt*b + c
 *   selected = the n_select ids with the largest Delta (ties: lower id),
 *              written in ascending id order; id = nt*(K/b) + kt.
 * [summary-pt Metodologia 2: Hessian-guided Delta-score weighting the
 * residual error by the input channels' diagonal Hessian; top-K blocks.]
 *   w        : fp16 [N][K];  x_calib: fp16 [T][K]
 *   N % block == 0, K % 128 == 0, block in {32, 64, 128},
 *   0 <= T < 2^31 with T*K < 2^40,
 *   0 <= n_select <= (N/block)*(K/block), (N/block)*(K/block) < 2^31
 *   selected : int32 [n_select] (output; may be NULL when n_select == 0)
 *   delta_out: fp64 [(N/block)*(K/block)] (output, required: also used as
 *              the scores' working storage)
 *   hdiag_out: fp64 [K] (output, required)
 */
mq_status mq_select_blocks(const uint16_t* w, const uint16_t* x_calib,
                           int64_t N, int64_t K, int64_t T, int32_t block,
                           int32_t n_select, int32_t* selected,
                           double* delta_out, double* hdiag_out, void* stream);

/*
 * Pack the dense 4-bit base and the residual of the selected blocks.
 * [summary-pt Metodologia 1: W ~ Q(W) + R, both 4-bit.]
 *   w        : fp16 [N][K]
 *   selected : int32 [n_select], strictly ascending block ids in range
 *              (as written by mq_select_blocks); other contents give
 *              unspecified residual output but every access stays in bounds
 *   qw       : uint8 [N/16][K/128][64][16]  packed base codes in the slab
 *              layout (output): for the 16 channels 16s .. 16s+15 (slab s),
 *              group j and lane l = 16c + r (c < 4, r < 16), the 16 bytes at
 *              [s][j][l] are bytes 16c .. 16c+15 of channel 16s + r's 64
 *              packed bytes of group j (two codes per byte as above).  A
 *              permutation of the row-major [N][K/2] bytes inside each slab
 *              and group, so that one 16-channel x 128-input tile is 1 KB
 *              contiguous, in the order the kernels' lanes read it.  N is a
 *              multiple of 16 (block >= 32 divides it).
 *   sw       : fp16  [N][K/128]     base scales (output)
 *   row_ptr  : int32 [N/block + 1]  CSR by output tile row (output)
 *   col_idx  : int32 [n_select]     block column kt, ascending per row (output)
 *   qr       : uint8 [n_select][block][block/2]  residual codes; row r is
 *              output channel nt*block + r, column c input kt*block + c
 *   sr       : fp16  [n_select][block]  residual scale per block row (output)
 */
mq_status mq_pack_weights(const uint16_t* w, int64_t N, int64_t K, int32_t block,
                          const int32_t* selected, int32_t n_select,
                          uint8_t* qw, uint16_t* sw, int32_t* row_ptr,
                          int32_t* col_idx, uint8_t* qr, uint16_t* sr,
                          void* stream);

/*
 * Exact output distortion of a selection (offline study of the Delta-score).
 *   D(S) = || X (W - deq Q(W) - sum_{i in S} R_hat_i)^T ||_F^2   in fp64,
 * with Q, E = W - deq Q(W) and R_hat exactly as in mq_select_blocks (R_hat of
 * block i is its candidate residual whether or not i is in S).
 * [summary-pt Metodologia 2 and Principais Contribuicoes 2: the Delta-score
 * replaces this costly exact evaluation of the output distortion.]
 *   w        : fp16 [N][K];  x: fp16 [T][K] (the tokens D is measured on)
 *   N % block == 0, K % 128 == 0, 0 <= T < 2^22, block in {32, 64, 128},
 *   (N/block)*(K/block) < 2^24, N*K and T*N < 2^36
 *   selected : int32 [n_selected] block ids; ids outside [0, B) are
 *              ignored and a repeated id counts once
 *   dist     : fp64 [1] (device output)
 *   workspace: device buffer of mq_distortion_workspace's bytes (16-byte
 *              aligned), about 8*N*K bytes; the caller owns it
 * The sum runs in a fixed order, so repeated calls give identical bits.
 */
mq_status mq_distortion_workspace(int64_t N, int64_t K, int64_t T, int32_t block, size_t* bytes);
mq_status mq_distortion(const uint16_t* w, const uint16_t* x, int64_t N, int64_t K, int64_t T,
                        int32_t block, const int32_t* selected, int32_t n_selected, double* dist,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Greedy selection by exact output distortion (offline study of the
 * Delta-score; the packed layer does not use it).  Starting from S = {},
 * n_select times: every unchosen block (nt, kt) has the gain
 *   gain = ||o||^2 - ||o - X[:, kt-block] R_hat_(nt,kt)^T||^2
 * where o = X (E - R_S)^T on the block's output rows nt*block .. +block-1;
 * the block of largest gain joins S (ties: lower id; a NaN gain ranks
 * below every number).  A pick changes only its own row's outputs, so
 * only that row's candidates are evaluated again.  fp64 throughout; each
 * gain sums per 64-token tile, then over tiles in order.
 * [summary-pt Metodologia 2 and Principais Contribuicoes 2, as above.]
 *   w, x_calib, shape rules: as mq_distortion; 0 <= n_select <= B
 *   selected : int32 [n_select] chosen ids, ascending (output)
 *   order    : int32 [n_select] the same ids in the order picked (output,
 *              may be NULL)
 *   gains    : fp64 [n_select] each pick's gain when picked (output, may
 *              be NULL)
 *   dist     : fp64 [2] D({}) and D(S) on x_calib (output, may be NULL)
 *   workspace: device buffer of mq_select_exact_workspace's bytes (16-byte
 *              aligned), about 12*N*K + 8*T*N bytes; the caller owns it
 * Every step runs on `stream` with no host synchronisation: one pick
 * kernel, one update of the picked row's outputs and one re-evaluation
 * of that row per step.
 */
mq_status mq_select_exact_workspace(int64_t N, int64_t K, int64_t T, int32_t block,
                                    size_t* bytes);
mq_status mq_select_exact_greedy(const uint16_t* w, const uint16_t* x_calib, int64_t N, int64_t K,
                                 int64_t T, int32_t block, int32_t n_select, int32_t* selected,
                                 int32_t* order, double* gains, double* dist, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Debug flag for mq_fused_gemm: also store the exact integer accumulators. */
#define MQ_FLAG_DUMP_ACC 1u
/* mq_fused_gemm flags choosing the prefill kernel's route (measurement and
 * cross-checks; both give the same y bits): the int8 route even where the
 * fp6 route would run, or the fp6 route already from M = 33 (by default
 * from M = 1024) when the workspace holds its images and block is 64 or 128.
 * Below M = 1024 that route converts no weight image: the kernel re-encodes
 * the packed base codes as it stages them. */
#define MQ_FLAG_INT8_TILE 2u
#define MQ_FLAG_FP6_TILE 4u

/*
 * Bytes of workspace mq_fused_gemm can use for this shape (host output).
 * Nonzero only for M > 32: the activation codes widened to int8 in the
 * prefill kernel's fragment order (ceil(M/32)*32*K bytes, rounded up to
 * 256), then, when the 256 x 128 output tiles alone would leave compute
 * units idle, fp32 partial outputs [splits][M][N] of the K groups split
 * over several workgroups, summed by a second kernel in split order (so y
 * stays deterministic).  From M = 1024 it is the larger room of the fp6
 * route (see mq_fp6_sizes): the FP6 images of the activation codes, the
 * base and the residual (bounded by every block selected, 0.75*N*K bytes,
 * since block and n_select are not arguments here) and that route's
 * split-K partials (room for [splits][M][N]; that route splits only the
 * tiles of a partial last round when the others fill whole rounds).  Sizes the GEMM does not accept (each below 2^31,
 * packed weights and activations each below 4 GiB) give MQ_ERR_SHAPE.
 */
mq_status mq_fused_gemm_workspace(int64_t M, int64_t N, int64_t K, size_t* bytes);

/*
 * The fused layer (ZipperEngine), one kernel:
 *   acc_base[m][n][j] = sum_{k in group j} qa[m][k] * qw[n][k]        (int32, exact)
 *   acc_res[i][m][r]  = sum_{c<b} qa[m][kt_i*b + c] * qr_i[r][c]      (int32, exact)
 *   y[m][n] = f16( sum_j sa[m][j]*sw[n][j]*acc_base[m][n][j]
 *                + sum_{i in tile row n/b} sa[m][j_i]*sr_i[n - nt*b]*acc_res[i][m][n - nt*b] )
 * with the scale products and the sum in fp32, j_i = kt_i*b/128.  Each
 * residual block reuses the activation tile already staged for the dense
 * base in the same K step.
 * [summary-pt Metodologia 3; abstract: sparse block computation fused into
 * the dense 4-bit GEMM.]
 *   qa, sa   : as written by mq_quantize_act for M x K
 *   qw, sw   : as written by mq_pack_weights for N x K
 *   block, n_select, row_ptr, col_idx, qr, sr: the residual, as written by
 *              mq_pack_weights; n_select == 0 gives the dense-only layer
 *              (row_ptr, col_idx, qr, sr may then be NULL).  A CSR that
 *              points outside [0, n_select) or past K is clipped, never
 *              read out of bounds: row ranges are clipped to [0, n_select]
 *              and made non-decreasing, and an entry whose block column is
 *              outside [0, K/block) contributes nothing.  Other invalid
 *              CSRs (unsorted or repeated columns in a row) give
 *              unspecified but finite y.  Check a CSR with mq_validate_csr.
 *   y        : fp16 [M][ldy], ldy >= N, ldy % 8 == 0 (output)
 *   workspace: device buffer of workspace_bytes (16-byte aligned) or NULL.
 *              With enough for the fp6 route (M >= 1024, block 64 or 128)
 *              the codes, base and residual are re-encoded into it and the
 *              fp6 kernel runs; otherwise, with at least the int8 route's
 *              bytes (M > 32) the codes are widened into it for the int8
 *              kernel; the split-K schedule is used where it applies; with
 *              less, or NULL, the kernel reads the packed codes in one pass
 *              over K (same accumulators, y the same up to fp32 summation
 *              order, slower).
 *              The call owns it until the stream has drained.
 *   Also:      N*K/2 and M*K/2 must each be below 2^32 (MQ_ERR_SHAPE).
 *   flags    : 0 or MQ_FLAG_DUMP_ACC, with at most one of
 *              MQ_FLAG_INT8_TILE / MQ_FLAG_FP6_TILE
 *   acc_dump : with MQ_FLAG_DUMP_ACC, int32 [M*N*(K/128) + n_select*M*block]:
 *              acc_base as [M][N][K/128] followed by acc_res as
 *              [n_select][M][block]; otherwise ignored (may be NULL)
 *   M >= 0 (M == 0 enqueues nothing), N % block == 0, K % 128 == 0.
 */
mq_status mq_fused_gemm(const uint8_t* qa, const float* sa, int64_t M, int64_t N, int64_t K,
                        const uint8_t* qw, const uint16_t* sw,
                        int32_t block, int32_t n_select, const int32_t* row_ptr,
                        const int32_t* col_idx, const uint8_t* qr, const uint16_t* sr,
                        uint16_t* y, int64_t ldy,
                        void* workspace, size_t workspace_bytes,
                        uint32_t flags, int32_t* acc_dump, void* stream);

/*
 * Bytes of workspace mq_fused_layer needs for this shape (host output).
 * 0 when the decode kernel quantises the activations itself (M <= 4 and the
 * shape's (token, group) pairs fit its prologue); otherwise room for the
 * activation codes (in the layout the GEMM kernel reads best: 16-token tiles
 * for the decode kernel above 8 tokens, room for M padded to a multiple of
 * 16 up to M = 32; the wide fragment order for the prefill kernel), their
 * scales and the split-K partials; from M = 1024 the larger room of the fp6
 * route (scales, FP6 images of the activations, base and residual, the
 * residual bounded by 0.75*N*K bytes, and its split-K partials), which
 * mq_fused_layer then uses when block is 64 or 128.
 */
mq_status mq_fused_layer_workspace(int64_t M, int64_t N, int64_t K, size_t* bytes);

/*
 * The whole online layer from fp16 activations: y = mq_fused_gemm applied
 * to mq_quantize_act(x), with results identical to calling the two (same
 * codes, same scales, same y bits).  For M <= 4 (decode), when the shape
 * allows, it is ONE kernel: the streaming GEMM quantises the token tile in
 * its prologue into LDS and never writes codes to memory, which removes the
 * separate launch and the codes' round trip through memory; otherwise the
 * two kernels run back to back on `stream` using the workspace.
 * [summary-pt Metodologia 3: quantisation is one of the stages the fused
 * pipeline overlaps with the GEMM.]
 *   x        : fp16 [M][ldx], ldx >= K, ldx % 8 == 0, finite values
 *   qw .. sr : the packed layer, as for mq_fused_gemm
 *   y        : fp16 [M][ldy], ldy >= N, ldy % 8 == 0 (output)
 *   workspace: device buffer (16-byte aligned) of at least
 *              mq_fused_layer_workspace's bytes (NULL when that is 0);
 *              fewer bytes give MQ_ERR_WORKSPACE.  The call owns it until
 *              the stream has drained.
 *   M >= 0 (M == 0 enqueues nothing); other constraints as mq_fused_gemm.
 */
mq_status mq_fused_layer(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int64_t N,
                         const uint8_t* qw, const uint16_t* sw,
                         int32_t block, int32_t n_select, const int32_t* row_ptr,
                         const int32_t* col_idx, const uint8_t* qr, const uint16_t* sr,
                         uint16_t* y, int64_t ldy, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Device scratch of mq_fused_layer_noalloc, per device: 128 MiB. */
#define MQ_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/*
 * mq_fused_layer for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same launches and the same y bits as mq_fused_layer, with the
 * workspace (activation codes and scales, split-K partials) taken from a
 * device scratch array of MQ_NOALLOC_SCRATCH_BYTES that the library holds on
 * each device from the time its code is loaded there until the process
 * ends.  The call allocates nothing.  Every size with
 * mq_fused_layer_workspace(M, N, K) <= MQ_NOALLOC_SCRATCH_BYTES is accepted
 * (every configured shape up to M = 4096, K = 25600); larger ones return
 * MQ_ERR_WORKSPACE with nothing enqueued.  The first call on a device looks
 * up that device's scratch address (thread-safe).
 * Calls whose launches overlap on one device race on the scratch (for
 * example two streams of one device): the caller serialises them.  Nothing
 * in the scratch needs to start at zero.
 *   Arguments as for mq_fused_layer, without the workspace.
 */
mq_status mq_fused_layer_noalloc(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int64_t N,
                                 const uint8_t* qw, const uint16_t* sw, int32_t block,
                                 int32_t n_select, const int32_t* row_ptr, const int32_t* col_idx,
                                 const uint8_t* qr, const uint16_t* sr, uint16_t* y, int64_t ldy,
                                 void* stream);

/*
 * The prefill kernel's fp6 route with prepared operands.  From M = 1024 on
 * (block 64 or 128), mq_fused_gemm and mq_fused_layer run the LDS-tiled
 * kernel on the FP6 matrix core: the 4-bit codes are re-encoded as FP6
 * E2M3 fields in sign-magnitude, |q| <= 8 in the low five bits, whose value
 * is exactly q/8, so V_MFMA_F32_32X32X64_F8F6F4 returns the exact integer
 * dot products / 64 in fp32, at twice the K per cycle of the int8
 * instruction; y is the int8 route's, bit for bit.  Those calls convert the
 * weights on every call into their workspace; a caller that can keep the
 * converted weights (0.75 byte per weight code, 1.5x the packed base, plus
 * the residual blocks at the same rate) prepares them once here and runs
 * the kernel alone with mq_fused_gemm_fp6.
 * [summary-pt Metodologia 3: the dense 4-bit product and the residual run
 * in one kernel that reuses the staged activation tile.]
 * Image layout (3 KB per 32 rows and group of 128 codes; rows are tokens or
 * output channels): for slice u in {0, 1} (codes 64u .. 64u+63 of the
 * group), lane l = r + 32h (row r, half h) holds codes 64u + 32h + i,
 * i = 0..31, as six-bit fields at bit 6i of six dwords: dwords 0-3 at byte
 * u*1024 + 16l, dwords 4-5 at 2048 + u*512 + 8l.  The weight image is the
 * base, [N/32][K/128][3 KB], then from byte round_up(N*K*3/4, 256) the
 * residual blocks in CSR order, b*b*3/4 bytes each: per 32 rows c and
 * slice u of the block a 1536-byte piece at (c*(b/64) + u)*1536, lane l's
 * dwords 0-3 at 16l, 4-5 at 1024 + 8l.
 */

/* Sizes of the fp6 route's buffers (host outputs): the activation image of
 * M tokens ([ceil(M/32)][K/128][3 KB]), the weight image (base + residual)
 * and mq_fused_gemm_fp6's split-K partials (0 when no split applies).
 * block must be 64 or 128 (MQ_ERR_BLOCK); M*K and N*K below 2^32. */
mq_status mq_fp6_sizes(int64_t M, int64_t N, int64_t K, int32_t block, int32_t n_select,
                       size_t* act_bytes, size_t* weight_bytes, size_t* split_bytes);

/* Packed activation codes qa [M][K/2] (as from mq_quantize_act) -> the
 * activation image act_img (mq_fp6_sizes' act_bytes, 16-byte aligned; rows
 * past M up to a multiple of 32 are written as zeros). */
mq_status mq_fp6_prepare_acts(const uint8_t* qa, int64_t M, int64_t K, uint8_t* act_img,
                              void* stream);

/* Packed base qw (slab layout) and residual qr (as from mq_pack_weights)
 * -> weight_img (mq_fp6_sizes' weight_bytes, 16-byte aligned).  qr may be
 * NULL when n_select == 0. */
mq_status mq_fp6_prepare_weights(const uint8_t* qw, int64_t N, int64_t K, int32_t block,
                                 int32_t n_select, const uint8_t* qr, uint8_t* weight_img,
                                 void* stream);

/* mq_fused_gemm on prepared images: the same accumulators and the same y
 * bits.  M == 0 or M > 32 (the tile kernel's range); block 64 or 128;
 * split_ws holds mq_fp6_sizes' split_bytes (may be NULL when that is 0);
 * flags 0 or MQ_FLAG_DUMP_ACC (acc_dump as for mq_fused_gemm).  A K whose
 * residual table does not fit the kernel's LDS gives MQ_ERR_SHAPE. */
mq_status mq_fused_gemm_fp6(const uint8_t* act_img, const float* sa, int64_t M, int64_t N, int64_t K,
                            const uint8_t* weight_img, const uint16_t* sw, int32_t block,
                            int32_t n_select, const int32_t* row_ptr, const int32_t* col_idx,
                            const uint16_t* sr, uint16_t* y, int64_t ldy, void* split_ws,
                            size_t split_bytes, uint32_t flags, int32_t* acc_dump, void* stream);

/*
 * Unfused ablation (measurement only; the layer's path never needs it): the
 * residual branch as a standalone kernel.  It reloads the activation codes,
 * computes deq(Qa(X) . R^T) for the selected blocks and merges it into the
 * dense output already in y:  y = f16(f32(y) + residual).  Run after
 * mq_fused_gemm with n_select == 0 it reproduces the separate-kernel design
 * that the fused kernel replaces, so the two can be timed on the same data.
 * [summary-pt Metodologia 3: a separate sparse kernel would reload the
 * activations and merge partial outputs.]
 *   Arguments as for mq_fused_gemm (the residual arrays are required when
 *   n_select > 0; n_select == 0 enqueues nothing).  y is read and written.
 */
mq_status mq_residual_merge(const uint8_t* qa, const float* sa, int64_t M, int64_t N, int64_t K,
                            int32_t block, int32_t n_select, const int32_t* row_ptr,
                            const int32_t* col_idx, const uint8_t* qr, const uint16_t* sr,
                            uint16_t* y, int64_t ldy, void* stream);

/*
 * Outlier migration before the decomposition (offline), exponent 1/2:
 *   x_absmax[k] = max_t |x_calib[t][k]|,  w_absmax[k] = max_n |w[n][k]|
 *   scales[k]   = sqrt(x_absmax[k] / w_absmax[k])   (fp32, IEEE division and
 *                 square root; 1 where either maximum is 0)
 *   w_out[n][k] = f16(w[n][k] * scales[k])           (round to nearest even)
 * so that X' W'^T ~ X W^T with X' = mq_smooth_acts(X).  The migrated w_out
 * is what mq_select_blocks / mq_pack_weights then decompose.
 * [summary-pt Metodologia 1: outliers are migrated between activations and
 * weights before the weight is split into base and residual.]
 *   x_calib : fp16 [T][K];  w : fp16 [N][K]
 *   x_absmax, w_absmax, scales : fp32 [K] (outputs)
 *   w_out   : fp16 [N][K] (output; must not alias w)
 *   1 <= T, N, K < 2^31 and N*K, T*K < 2^40 (else MQ_ERR_SHAPE, nothing
 *   enqueued).
 */
mq_status mq_smooth_weights(const uint16_t* x_calib, int64_t T, const uint16_t* w, int64_t N,
                            int64_t K, float* x_absmax, float* w_absmax, float* scales,
                            uint16_t* w_out, void* stream);

/*
 * Migrated activations: x_out[m][k] = f16(x[m][k] / scales[k]).
 *   x : fp16 [M][ldx] (ldx >= K);  scales : fp32 [K] from mq_smooth_weights
 *   x_out : fp16 [M][K] (output).  M == 0 enqueues nothing.
 *   0 <= M < 2^31, 1 <= K < 2^31, M*K < 2^40 (else MQ_ERR_SHAPE).
 */
mq_status mq_smooth_acts(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                         const float* scales, uint16_t* x_out, void* stream);

/*
 * Measurement only (not part of the layer): the sustained rate of the int8
 * matrix-core instruction the fused GEMM kernels use
 * (V_MFMA_I32_16X16X64_I8) and the shader clock, as the roofline
 * denominators measured on the device.  Launches `blocks` workgroups of four
 * waves; each wave runs `iters` rounds of four independent MFMA chains and
 * stores its shader-cycle count (s_memtime delta) in cycles[4*block + wave].
 * Each round is 4 x 2*16*16*64 = 131072 integer ops per wave.  The caller
 * times the launch (e.g. with HIP events) and derives ops/s and cycles/s.
 *   blocks in [1, 2^20], iters in [1, 2^24]
 *   cycles : int64 [4*blocks] (output)
 *   sink   : int32 [256*blocks] (output; keeps the results live)
 */
mq_status mq_measure_mfma(int32_t blocks, int32_t iters, int64_t* cycles, int32_t* sink,
                          void* stream);

/*
 * Synchronous CSR check (copies row_ptr and col_idx to the host and waits
 * for `stream`): row_ptr[0] == 0, non-decreasing, row_ptr[N/block] ==
 * n_select, col_idx strictly ascending within a row and < K/block.
 * N and K below 2^31 with fewer than 2^31 blocks (MQ_ERR_SHAPE) and
 * 0 <= n_select <= number of blocks (MQ_ERR_BUDGET) are checked first.
 * Returns MQ_OK or MQ_ERR_CSR.
 */
mq_status mq_validate_csr(const int32_t* row_ptr, const int32_t* col_idx,
                          int64_t N, int64_t K, int32_t block, int32_t n_select,
                          void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOSAICQ_H */
