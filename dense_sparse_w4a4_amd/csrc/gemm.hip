// ZipperEngine fused layer: dense 4-bit base GEMM + block-sparse 4-bit
// residual + scale/reduce-sum epilogue in one kernel.
// MosaicQuant technical summary (gist.science/pt/paper/2606.15652),
// Metodologia 3: the sparse residual is computed inside the dense 4-bit GEMM
// kernel instead of a separate kernel that would reload the activations and
// merge partial outputs; abstract (fugumt.com/fugumt/paper_check/2606.15652v1):
// sparse block computation fused into the dense GEMM.
//
// CDNA4 mapping.  gfx950 has no 4-bit integer MFMA, so codes are widened to
// int8 in registers and fed to V_MFMA_I32_16X16X64_I8.  Widening keeps each
// code in the high nibble of its byte (byte = 16*q): one AND, or a shift
// and an AND, per 32-bit word, no sign extension.  Both operands get the
// same treatment, so every int32 accumulator holds 256 x the exact dot
// product; the epilogue folds 1/256 into the activation scale and the debug
// dump shifts it out exactly.  Splitting a packed word into its even and odd
// codes permutes k inside a 16-code chunk identically for both operands,
// which leaves the dot product unchanged.
//
// Operand layout per 128-channel group: lane chunk c = lane/16 owns
// group-local channels [32c, 32c+32), i.e. 16 contiguous packed bytes (one
// 16-byte load).  The first 8 bytes feed one MFMA, the last 8 a second, so
// two MFMAs cover the group.  A residual block (edge b in {32, 64, 128},
// always inside one group at a 32-aligned offset) covers whole chunks, so its
// MFMAs take the activation fragment of the same group; chunks outside the
// block feed zeros.
#include "gemm_common.h"

namespace mq {
namespace {

// Streaming kernel for small M (decode): NS 16-channel slabs (16*NS output
// channels, all inside one residual block row) x 16 tokens per workgroup
// (grid.y walks 16-token tiles).  The KS waves of a workgroup split the K
// groups into contiguous runs and reduce their partial sums through LDS in
// wave order.  Activations are the MFMA A operand (rows = tokens), weights
// the B operand (columns = channels): lane l owns channel l%16 of each slab
// and tokens 4*(l/16) + i.  The slabs of a workgroup share one activation
// fragment per group (and, with QP > 0, one in-prologue quantisation).  The
// codes come row-major (qa), or, on the layer route above 8 tokens, in
// 16-token tiles (qat) where a group's fragment is one contiguous 1 KB.
//
// The run of dense groups is streamed in units of U groups with two units
// in flight: the loads of unit t+2 are issued before unit t+1 is computed.
// Every unit issues the same loads (groups past the run re-read its last
// group and get scale 0), so the load counters are waited on exactly, and
// the per-lane offsets are fixed: each unit only moves uniform bases.  The
// tile's activation and weight scales are staged in LDS once.  The residual
// blocks of the tile's block row form a second stream of items against the
// activation fragment of each block's group (the zipper); they are dealt
// round-robin to the waves, so the waves finish together however the
// selected blocks cluster in K.  A wave's first two entries are loaded in
// the prologue beside the first dense units and processed before the dense
// stream, whose run then hides the loads of the next two; any further
// entries follow the dense stream.  A block of edge <= 64 is one MFMA per
// slab on 8-byte operands (only the block's bytes are loaded).
//
// QP > 0 (M <= kStreamQuantRows, one token tile): the activations arrive as
// fp16 and the workgroup quantises them itself before the streams start (the
// act-quant stage fused into the GEMM's prologue).  One (token, group) per
// team of 16 lanes, 8 channels per lane; the scale is the same fp32 amax/7
// as the standalone act-quant kernel and the codes come from the same
// quotient (quant4_rcp), so codes, scales and y are identical to the
// two-kernel path.  QP passes of the teams cover the tile's M x K/128
// pairs.  Codes go to LDS rows of K/2 + 64 bytes (the pad puts the rows on
// different banks) and the A fragments are read from there.  The fp16
// loads are issued before the weight stream, so waiting for them never
// waits on it.
template <int BLK, int KS, bool DUMP, int QP, int U, int NS>
__global__ __launch_bounds__(64 * KS) void gemm_stream_kernel(GemmArgs a) {
  static_assert(16 * NS <= BLK, "the slabs of a workgroup lie in one block row");
  constexpr int CW = 16 * NS;  // channels per workgroup
  extern __shared__ __align__(16) unsigned char smem[];
  const int G = (int)(a.K / kGroup);
  float* sa_t = reinterpret_cast<float*>(smem);  // [G][16]: sa/256 of the tile's tokens
  float* sw_t = sa_t + G * 16;                     // [G][CW+1]: weight scales of the tile's channels
  float* spare = sw_t + G * (CW + 1);              // [2]: target of stores past the tables
  unsigned char* qa_t = smem + stream_qa_offset(G, NS);  // QP > 0: [M][qrow] activation codes
  const int qrow = (int)(a.K / 2) + 64;
  float* red = reinterpret_cast<float*>(smem);   // [KS][16][CW+1] after the streams

  // readfirstlane tells the compiler the wave index is uniform, so loop
  // bounds and bases stay scalar
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int ch = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * CW;
  const int64_t m0 = (int64_t)blockIdx.y * 16;
  const int64_t Kh = a.K / 2;
  const int gb = wave * G / KS;
  const int ng = (wave + 1) * G / KS - gb;

  // per-lane byte offsets (32-bit: the host keeps N*K/2, M*K/2 and the tiled
  // codes' padded size below 2^32)
  // weight codes in the slab layout: each group of a slab is 1 KB, lane l's
  // 16 bytes at l*16, so every weight load of a wave reads 1 KB contiguous;
  // the workgroup's slabs are 16*K/2 bytes apart
  const uint32_t offW = (uint32_t)(n0 * Kh + lane * 16);
  const uint32_t slabW = (uint32_t)(16 * Kh);
  const int64_t mr = m0 + r16;  // token rows past M read row M-1 (computed, never stored)
  // activation codes: row-major qa (group j of token m at m*K/2 + 64j; rows
  // past M read row M-1), or the 16-token tiles of qat (group j's codes of
  // the tile in one contiguous 1 KB at 1024j from the tile's base)
  const bool tiled = a.qat != nullptr;
  const uint8_t* const xb = tiled ? a.qat : a.qa;
  const int64_t xstep = tiled ? 1024 : 64;
  const uint32_t offX = tiled ? (uint32_t)((m0 / 16) * G * 1024 + r16 * 64 + ch * 16)
                              : (uint32_t)((mr < a.M ? mr : a.M - 1) * Kh + ch * 16);
  const int offXl = (int)((mr < a.M ? mr : a.M - 1) - m0) * qrow + ch * 16;  // QP > 0: in qa_t
  auto lds_x = [&](int j) { return *reinterpret_cast<const uint4*>(qa_t + offXl + j * 64); };

  struct Unit {
    uint4 W[U][NS];  // B-operand fragments (weight codes), per group and slab
    uint4 X[U];      // A-operand fragments (activation codes), per group
  };

  // dense unit t: groups gb + t*U + u, clamped to the run
  auto fetch_dense = [&](Unit& D, int t) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = gb + min(t * U + u, ng - 1);
#pragma unroll
      for (int s = 0; s < NS; ++s) D.W[u][s] = ld16(a.qw + (int64_t)j * 1024 + offW + s * slabW);
      if constexpr (QP == 0) D.X[u] = ld16(xb + (int64_t)j * xstep + offX);
    }
  };

  float y[NS][4];
#pragma unroll
  for (int s = 0; s < NS; ++s) y[s][0] = y[s][1] = y[s][2] = y[s][3] = 0.f;
  const v4i zero = {0, 0, 0, 0};

  // one item of slab s: two MFMAs, then y += (sa/256 * sc) * acc for the
  // lane's tokens (sc = the item's weight or residual row scale, 0 for
  // padding)
  auto scale_add = [&](int s, const v4i& acc, float sc, int j, bool valid, int64_t dump_at,
                       bool dump_res) {
    const float4 s4 = *reinterpret_cast<const float4*>(sa_t + j * 16 + 4 * ch);
    y[s][0] = fmaf(s4.x * sc, (float)acc[0], y[s][0]);
    y[s][1] = fmaf(s4.y * sc, (float)acc[1], y[s][1]);
    y[s][2] = fmaf(s4.z * sc, (float)acc[2], y[s][2]);
    y[s][3] = fmaf(s4.w * sc, (float)acc[3], y[s][3]);
    if (DUMP && valid) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + 4 * ch + i;
        if (m < a.M) {
          if (!dump_res)
            a.acc_dump[(m * a.N + n0 + 16 * s + r16) * G + j] = acc[i] >> 8;
          else
            a.acc_dump[dump_at + m * BLK] = acc[i] >> 8;
        }
      }
    }
  };
  auto item = [&](int s, const uint4& W, const uint4& X, float sc, uint32_t rm, int j, bool valid,
                  int64_t dump_at, bool dump_res) {
    v4i acc = mfma(widen8(X.x, X.y), widen8(W.x & rm, W.y & rm), zero);
    acc = mfma(widen8(X.z, X.w), widen8(W.z & rm, W.w & rm), acc);
    scale_add(s, acc, sc, j, valid, dump_at, dump_res);
  };
  auto compute_dense = [&](const Unit& D, int t) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool valid = t * U + u < ng;
      const int j = gb + min(t * U + u, ng - 1);
      const uint4 X = QP > 0 ? lds_x(j) : D.X[u];
#pragma unroll
      for (int s = 0; s < NS; ++s)
        item(s, D.W[u][s], X, valid ? sw_t[j * (CW + 1) + 16 * s + r16] : 0.f, 0xFFFFFFFFu, j, valid, 0,
             false);
    }
  };

  // ---- prologue: the tile's scale loads first, then two dense units and
  // the CSR window in flight; the scales go to LDS (transposed to [G][16]
  // and [G][CW+1]) as soon as they arrive, without waiting for the units ----
  const int nunits = (ng + U - 1) / U;
  // QP > 0: the fp16 activations of the tile's (token, group) pairs, one
  // 16-byte load per pass and lane, all issued first (the launcher picks QP
  // so that the passes cover every pair)
  const int team = (int)(threadIdx.x >> 4), tl = (int)(threadIdx.x & 15);
  const int nrg = QP > 0 ? (int)a.M * G : 0;
  uint4 xv[QP > 0 ? QP : 1];
  if constexpr (QP > 0) {
#pragma unroll
    for (int it = 0; it < QP; ++it) {
      const int rg = min(team + it * 4 * KS, nrg - 1);
      const int row = rg / G, j = rg - row * G;
      xv[it] = *reinterpret_cast<const uint4*>(a.x + (m0 + row) * a.ldx + j * kGroup + tl * 8);
    }
  }
  constexpr int SMAX = 4;       // staged activation scales issued ahead, per thread
  constexpr int WMAX = 4 * NS;  // staged weight scales issued ahead, per thread
  const int nsa = 16 * G, nsw = CW * G;
  const uint8_t* sa_b = reinterpret_cast<const uint8_t*>(a.sa);
  const uint8_t* sw_b = reinterpret_cast<const uint8_t*>(a.sw) + n0 * G * 2;
  float pa[SMAX];
  uint16_t pw[WMAX];
#pragma unroll
  for (int k = 0; k < SMAX; ++k) {
    if constexpr (QP == 0) {
      // activation scales in table order (entry e = group * 16 + token), so
      // consecutive lanes store to consecutive LDS words
      const int e = min((int)threadIdx.x + k * 64 * KS, nsa - 1);
      const int j = e >> 4, mm = e & 15;
      const int64_t m = m0 + mm;
      pa[k] = *reinterpret_cast<const float*>(sa_b + (uint32_t)(((m < a.M ? m : a.M - 1) * G + j) * 4));
    } else {
      pa[k] = 0.f;
    }
  }
#pragma unroll
  for (int k = 0; k < WMAX; ++k) {
    const int i = min((int)threadIdx.x + k * 64 * KS, nsw - 1);
    pw[k] = *reinterpret_cast<const uint16_t*>(sw_b + (uint32_t)(i * 2));
  }
  // (every wave has at least one group: the launcher keeps KS <= G; the
  // loads are unconditional so the waits for the scales above stay exact)
  Unit U0, U1;
  fetch_dense(U0, 0);
  fetch_dense(U1, 1);

  // Residual CSR row of this tile (block row nt; the tile's channels are
  // block rows rrow .. rrow + CW - 1).  The CSR arrays are read through the
  // scalar cache (uniform addresses, a read-only view), so their waits never
  // involve the vector loads in flight.
  typedef const __attribute__((address_space(4))) int32_t* cint_p;
  const cint_p rpc = (cint_p)a.row_ptr;
  const cint_p cic = (cint_p)a.col_idx;
  const int nt = (int)(n0 / BLK);
  const int rrow = (int)(n0 - (int64_t)nt * BLK);
  int rp0 = 0, rp1 = 0;
  if (a.n_select > 0) {
    rp0 = min(max(rpc[nt], 0), a.n_select);
    rp1 = min(max(rpc[nt + 1], rp0), a.n_select);
  }
  // this wave's residual entries are rp0 + wave + KS*k (see below); the
  // first two block columns are fetched now
  const int nres = rp1 > rp0 ? (rp1 - rp0 - wave + KS - 1) / KS : 0;
  auto res_kt = [&](int k) { return cic[rp0 + wave + KS * k]; };
  const int kt_first = nres > 0 ? res_kt(0) : 0;
  const int kt_second = nres > 1 ? res_kt(1) : 0;

  // ---- residual entries: the tile row's entries are dealt round-robin to
  // the waves (entry rp0 + wave + KS*i), so every wave gets the same share
  // whatever the block columns; the reduction below sums them with the
  // dense partials.  The first two entries' loads are issued whether or not
  // the wave has them (past its last entry they read valid dummy addresses:
  // weight codes and scales), so the prologue's load counters are waited on
  // exactly; later entries are loaded only when they exist, so no load is
  // left in flight at the end ----
  // A block of edge b <= 64 is one MFMA per slab: lane chunk c carries the
  // block's channels [16c, 16c + 16) (8 packed bytes of the activation row
  // and of the residual row, chunks past the block edge masked), so its
  // item loads only the block's bytes.  b = 128 covers the whole group and
  // takes the dense items' operand layout (16 bytes, two MFMAs).
  constexpr bool kHalf = BLK <= 64;
  struct Res {
    uint4 W[NS];  // kHalf: .x, .y
    uint4 X;      // kHalf: .x, .y
    uint32_t S[NS];
    uint32_t rm;
    int j;
    int xo;       // kHalf: byte offset of the lane's activation codes in the group
  };
  // (an entry whose block column is outside [0, K/b) contributes nothing:
  // its codes are masked and its group index clipped)
  auto res_ptrs = [&](int k, int kt_in, Res& R) {
    const bool okt = kt_in >= 0 && kt_in < (int)(a.K / BLK);
    const int kt = okt ? kt_in : 0;
    const bool has = k < nres;
    const int e = has ? rp0 + wave + KS * k : 0;
    R.j = kt * BLK / kGroup;
    const int lo = kt * BLK - R.j * kGroup;
    if constexpr (kHalf) {
      const bool act = 16 * ch < BLK && okt;
      R.rm = act ? 0xFFFFFFFFu : 0u;
      R.xo = (lo + (act ? 16 * ch : 0)) / 2;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const uint2 v = *reinterpret_cast<const uint2*>(
            has ? a.qr + (int64_t)e * (BLK * BLK / 2) + (rrow + 16 * s + r16) * (BLK / 2) + (act ? 8 * ch : 0)
                : a.qw + offW);
        R.W[s].x = v.x;
        R.W[s].y = v.y;
        R.S[s] = *(has ? a.sr + (int64_t)e * BLK + rrow + 16 * s + r16 : a.sw);
      }
      if constexpr (QP == 0) {
        const uint2 v = *reinterpret_cast<const uint2*>(xb + (int64_t)R.j * xstep + offX - ch * 16 + R.xo);
        R.X.x = v.x;
        R.X.y = v.y;
      }
    } else {
      const bool act = (32 * ch >= lo) && (32 * ch < lo + BLK) && okt;
      R.rm = act ? 0xFFFFFFFFu : 0u;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        R.W[s] = ld16(has ? a.qr + (int64_t)e * (BLK * BLK / 2) + (rrow + 16 * s + r16) * (BLK / 2) +
                                (act ? 16 * ch - lo / 2 : 0)
                          : a.qw + offW);
        R.S[s] = *(has ? a.sr + (int64_t)e * BLK + rrow + 16 * s + r16 : a.sw);
      }
      if constexpr (QP == 0) R.X = ld16(xb + (int64_t)R.j * xstep + offX);
    }
  };
  // the first two entries are loaded now, before the scale staging, so they
  // arrive during the dense stream
  Res R0, R1;
  res_ptrs(0, kt_first, R0);
  res_ptrs(1, kt_second, R1);

  // (stores past the tables go to the spare slots, so no store is branched
  // and the waits stay exact; with QP > 0 the activation scales of the
  // tile's tokens come from the quantisation below and only the padding
  // rows are written here)
  auto stage_a = [&](int e, float v) {  // e = group * 16 + token
    const int mm = e & 15;
    const bool pad = m0 + mm >= a.M;
    float* const da = e < nsa && (QP == 0 || pad) ? sa_t + e : spare;
    *da = pad ? 0.f : v * kInv256;
  };
  auto stage_w = [&](int i, uint16_t w) {  // i = channel * G + group (source order)
    const int r = i / G, j = i - r * G;
    float* const dw = i < nsw ? sw_t + j * (CW + 1) + r : spare + 1;
    *dw = h2f(w);
  };
#pragma unroll
  for (int k = 0; k < SMAX; ++k) stage_a((int)threadIdx.x + k * 64 * KS, pa[k]);
#pragma unroll
  for (int k = 0; k < WMAX; ++k) stage_w((int)threadIdx.x + k * 64 * KS, pw[k]);
  for (int e = (int)threadIdx.x + SMAX * 64 * KS; e < nsa; e += 64 * KS) {  // long K only
    const int j = e >> 4, mm = e & 15;
    const int64_t m = m0 + mm;
    stage_a(e, QP == 0 ? a.sa[(m < a.M ? m : a.M - 1) * G + j] : 0.f);
  }
  for (int i = (int)threadIdx.x + WMAX * 64 * KS; i < nsw; i += 64 * KS)  // long K only
    stage_w(i, a.sw[(n0 + i / G) * G + i % G]);
  if constexpr (QP > 0) {
    // quantise the tile: pass it covers pairs team + it * (4 KS), clamped
    // to the last pair, so every pass is branch-free and teams past the end
    // rewrite the last pair's codes and scale with identical values
#pragma unroll
    for (int it = 0; it < QP; ++it) {
      const int rg = min(team + it * 4 * KS, nrg - 1);
      const int row = rg / G, j = rg - row * G;
      float f[8];
      unpack_h8(xv[it], f);
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
      amax = row16_max(amax);
      const float sc = amax / 7.0f;
      const float r = sc == 0.0f ? 0.0f : 1.0f / sc;
      *reinterpret_cast<uint32_t*>(qa_t + row * qrow + j * 64 + tl * 4) = quant4_word(f, sc, r);
      if (tl == 0) sa_t[j * 16 + row] = sc * kInv256;
    }
  }
  __syncthreads();

  auto res_item = [&](int k, const Res& R) {
    const int64_t e = rp0 + wave + KS * k;
    if constexpr (kHalf) {
      uint2 X;
      if constexpr (QP > 0) {
        X = *reinterpret_cast<const uint2*>(qa_t + offXl - ch * 16 + R.j * 64 + R.xo);
      } else {
        X = make_uint2(R.X.x, R.X.y);
      }
      const v4i xa = widen8(X.x, X.y);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const v4i acc = mfma(xa, widen8(R.W[s].x & R.rm, R.W[s].y & R.rm), zero);
        scale_add(s, acc, h2f((uint16_t)R.S[s]), R.j, true, a.M * a.N * G + e * a.M * BLK + rrow + 16 * s + r16,
                  true);
      }
    } else {
      const uint4 X = QP > 0 ? lds_x(R.j) : R.X;
#pragma unroll
      for (int s = 0; s < NS; ++s)
        item(s, R.W[s], X, h2f((uint16_t)R.S[s]), R.rm, R.j, true,
             a.M * a.N * G + e * a.M * BLK + rrow + 16 * s + r16, true);
    }
  };
  // ---- the wave's first two residual entries (loaded in the prologue,
  // beside the first dense units), then the loads of the next two, which
  // arrive while the dense stream runs ----
  if (nres > 0) {
    res_item(0, R0);
    if (nres > 2) res_ptrs(2, res_kt(2), R0);
    if (nres > 1) {
      res_item(1, R1);
      if (nres > 3) res_ptrs(3, res_kt(3), R1);
    }
  }
  // ---- dense stream (ping-pong buffers, never copied while in flight) ----
  for (int t = 0; t < nunits; t += 2) {
    compute_dense(U0, t);
    if (t + 2 < nunits) fetch_dense(U0, t + 2);
    if (t + 1 >= nunits) break;
    compute_dense(U1, t + 1);
    if (t + 3 < nunits) fetch_dense(U1, t + 3);
  }

  // ---- residual stream: the same item work against the activation
  // fragment of each block's group, two entries in flight ----
  for (int k = 2; k < nres; k += 2) {
    res_item(k, R0);
    if (k + 2 < nres) res_ptrs(k + 2, res_kt(k + 2), R0);
    if (k + 1 >= nres) break;
    res_item(k + 1, R1);
    if (k + 3 < nres) res_ptrs(k + 3, res_kt(k + 3), R1);
  }

  __syncthreads();  // scales no longer needed: reuse LDS for the reduction
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wave * 16 + 4 * ch + i) * (CW + 1) + 16 * s + r16] = y[s][i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < 16 * CW; idx += 64 * KS) {
    const int mm = idx / CW, nl = idx - mm * CW;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < KS; ++w) sum += red[(w * 16 + mm) * (CW + 1) + nl];
    const int64_t m = m0 + mm;
    if (m < a.M) a.y[m * a.ldy + n0 + nl] = f2h_bits(sum);
  }
}

template <int BLK, int KS, bool DUMP, int QP, int U, int NS>
hipError_t launch_stream_cfg(const GemmArgs& a, hipStream_t st) {
  const size_t lds = stream_lds_bytes(a.K, KS, QP > 0 ? (int)a.M : 0, NS);
  if (lds > 64 * 1024) {
    auto k = gemm_stream_kernel<BLK, KS, DUMP, QP, U, NS>;
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  dim3 grid((unsigned)(a.N / (16 * NS)), (unsigned)((a.M + 15) / 16));
  hipLaunchKernelGGL((gemm_stream_kernel<BLK, KS, DUMP, QP, U, NS>), grid, dim3(64 * KS), lds, st, a);
  return hipGetLastError();
}

template <int BLK, int KS, int NS, int QP>
hipError_t launch_stream_u(const GemmArgs& a, const StreamPlan& p, hipStream_t st) {
  if constexpr (NS == 1) {
    if (p.u == 2) return launch_stream_cfg<BLK, KS, false, QP, 2, NS>(a, st);
  }
  return launch_stream_cfg<BLK, KS, false, QP, 1, NS>(a, st);
}

template <int BLK, int KS, int NS>
hipError_t launch_stream_ks(const GemmArgs& a, const StreamPlan& p, hipStream_t st) {
  if (a.x) {
    switch (p.qp) {
      case 1: return launch_stream_u<BLK, KS, NS, 1>(a, p, st);
      case 2: return launch_stream_u<BLK, KS, NS, 2>(a, p, st);
      default: return launch_stream_u<BLK, KS, NS, 4>(a, p, st);
    }
  }
  if constexpr (NS == 1) {
    if (a.acc_dump) return launch_stream_cfg<BLK, KS, true, 0, 2, 1>(a, st);
  }
  return launch_stream_u<BLK, KS, NS, 0>(a, p, st);
}

template <int BLK, int NS>
hipError_t launch_stream_ns(const GemmArgs& a, const StreamPlan& p, hipStream_t st) {
  switch (p.ks) {
    case 16: return launch_stream_ks<BLK, 16, NS>(a, p, st);
    case 8: return launch_stream_ks<BLK, 8, NS>(a, p, st);
    case 4: return launch_stream_ks<BLK, 4, NS>(a, p, st);
    case 2: return launch_stream_ks<BLK, 2, NS>(a, p, st);
    default: return launch_stream_ks<BLK, 1, NS>(a, p, st);
  }
}

template <int BLK>
hipError_t launch_blk(const GemmArgs& a, hipStream_t st) {
  const StreamPlan p = stream_plan(a.M, a.N, a.K, BLK, a.x != nullptr, a.acc_dump != nullptr);
  if constexpr (BLK >= 64) {
    if (p.ns == 4) return launch_stream_ns<BLK, 4>(a, p, st);
  }
  if (p.ns == 2) return launch_stream_ns<BLK, 2>(a, p, st);
  return launch_stream_ns<BLK, 1>(a, p, st);
}

}  // namespace

size_t stream_lds_bytes(int64_t K, int ks, int rows, int ns) {
  const int64_t G = K / kGroup;
  const size_t stage = (size_t)stream_qa_offset((int)G, ns) + (size_t)rows * (size_t)(K / 2 + 64);
  const size_t reduce = (size_t)ks * 16 * (16 * ns + 1) * 4;
  return stage > reduce ? stage : reduce;
}

// Waves per tile: the most (up to 16) that keep the grid within one
// resident round (<= 4096 waves, 16 per CU) and give every wave at least
// one unit of 4 groups.
int stream_waves(int64_t M, int64_t N, int64_t K, int ns) {
  const int64_t G = K / kGroup;
  const int64_t tiles = (N / (16 * ns)) * ((M + 15) / 16);
  if (tiles * 16 <= 4096 && G >= 64) return 16;
  if (tiles * 8 <= 4096 && G >= 32) return 8;
  if (tiles * 4 <= 4096 && G >= 16) return 4;
  if (G >= 8) return 2;
  return 1;
}

// Passes of the in-prologue quantisation: the power of two (<= 4) that
// covers the tile's M x K/128 (token, group) pairs with the workgroup's
// 4 * ks teams; 0 if 4 passes do not.  Every workgroup quantises the whole
// token tile, so the prologue's cost grows with the passes while the launch
// it saves does not: past 4 passes (measured on the Llama-3-8B and
// Qwen3-32B decode shapes) the two-kernel route is faster.
int stream_quant_passes(int64_t M, int64_t K, int ks) {
  const int64_t pairs = M * (K / kGroup);
  for (int p = 1; p <= 4; p *= 2)
    if (pairs <= (int64_t)p * 4 * ks) return p;
  return 0;
}

// Slabs per workgroup: two when that keeps the grid's wave count and every
// wave still streams eight or more groups, else one.  Measured with
// rotating weights: two slabs (one activation fragment for both) win on the
// Qwen3-32B decode shapes (long per-wave runs; up to 1.3x at M = 16) and
// lose where they halve the waves or shorten the runs (Llama-3-8B shapes).
// Four would need more than the 128 VGPRs that keep 16 waves resident per
// CU.
static int stream_slabs(int64_t M, int64_t N, int64_t K, int block) {
  if (block < 32 || N % 32 != 0) return 1;
  const int64_t mt = (M + 15) / 16;
  const int ks1 = stream_waves(M, N, K, 1), ks2 = stream_waves(M, N, K, 2);
  const bool same_waves = (N / 32) * mt * ks2 >= (N / 16) * mt * ks1;
  return same_waves && (K / kGroup) / ks2 >= 8 ? 2 : 1;
}

// Two slabs also where the one-slab plan's runs are short, with the waves
// per tile cut (to no fewer than four) so that every wave still streams
// eight or more groups, provided the two-slab grid still spans every
// compute unit: measured on Llama-3-8B 4096x14336, M = 16, 11.9 -> 10.9 us
// per launch (the one-slab plan streams four groups per wave there).
// Returns the waves per tile of that plan, 0 when it does not apply.
static int long_run_waves(int64_t M, int64_t N, int64_t K, int block) {
  if (block < 32 || N % 32 != 0) return 0;
  const int64_t G = K / kGroup;
  int ks = 16;
  while (ks > 4 && G / ks < 8) ks /= 2;
  if (G / ks < 8) return 0;
  return (N / 32) * ((M + 15) / 16) >= 256 ? ks : 0;
}

// Four slabs (64 channels) per workgroup for several tokens (M > 4), where
// the block edge allows it and the four-slab grid still spans every compute
// unit, with the long-run rule's waves per tile.  Every workgroup reads its
// token tile's activation fragments once (16 * K/2 bytes, from L2): at
// M = 16 that is half the weight bytes again with two slabs and a quarter
// with four.  Measured on Qwen3-32B 5120x25600, M = 16: 21.0 -> 19.7 us per
// launch; neutral at M = 1, and slower wherever the grid would leave compute
// units idle.  Returns the waves per tile, 0 when it does not apply.
static int four_slab_waves(int64_t M, int64_t N, int64_t K, int block) {
  if (M <= 4 || block < 64 || N % 64 != 0) return 0;
  if ((N / 64) * ((M + 15) / 16) < 256) return 0;
  const int64_t G = K / kGroup;
  int ks = 16;
  while (ks > 4 && G / ks < 8) ks /= 2;
  if (G / ks < 8) return 0;
  // (the tile's scale tables grow with the channels: very long K keeps the
  // two-slab plan, whose tables still fit in LDS)
  return stream_lds_bytes(K, ks, 0, 4) <= 160 * 1024 ? ks : 0;
}

StreamPlan stream_plan(int64_t M, int64_t N, int64_t K, int block, bool quantise, bool dump) {
  StreamPlan p;
  p.ns = dump ? 1 : stream_slabs(M, N, K, block);
  p.ks = stream_waves(M, N, K, p.ns);
  if (!dump && p.ns == 1) {
    const int ks = long_run_waves(M, N, K, block);
    if (ks > 0) {
      p.ns = 2;
      p.ks = ks;
    }
  }
  if (!dump && !quantise) {
    const int ks = four_slab_waves(M, N, K, block);
    if (ks > 0) {
      p.ns = 4;
      p.ks = ks;
    }
  }
  // groups per streamed unit (two units in flight per wave): one when each
  // wave streams six or more groups, else two (slab groups: always one).
  // Shallow units keep fewer weight bytes in flight per wave; measured on
  // the Llama-3-8B decode shapes with rotating weight copies, one-group units
  // are fastest for the long runs and two-group units for the short ones.
  p.u = (p.ns == 1 && (K / kGroup) / p.ks < 6) ? 2 : 1;
  p.qp = quantise ? stream_quant_passes(M, K, p.ks) : 0;
  return p;
}

bool stream_quant_fits(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || M > kStreamQuantRows) return false;
  // whatever the residual block edge, the plan must quantise in the prologue
  for (int block : {32, 64, 128}) {
    if (N % block != 0) continue;
    const StreamPlan p = stream_plan(M, N, K, block, true, false);
    if (p.qp == 0 || stream_lds_bytes(K, p.ks, (int)M, p.ns) > 64 * 1024) return false;
  }
  return true;
}

hipError_t launch_fused_gemm(const GemmArgs& a, hipStream_t st) {
  // fp16 activations (a.x): the streaming kernel quantises them itself (the
  // caller checked stream_quant_fits).  Otherwise, large M: LDS-tiled MFMA
  // kernel (weights read once per 256-token tile); small M, or a K too long
  // for the tile kernel's LDS table: the streaming kernel (weights read once
  // per 16-token tile)
  if (!a.x && a.aimg) return launch_tile6_gemm(a, st);
  if (!a.x && a.M > 32 && tile_gemm_fits(a)) return launch_tile_gemm(a, st);
  switch (a.block) {
    case 32: return launch_blk<32>(a, st);
    case 64: return launch_blk<64>(a, st);
    default: return launch_blk<128>(a, st);
  }
}

}  // namespace mq
