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

// Streaming kernel for small M (decode): 16 output channels x 16 tokens per
// workgroup (grid.y walks 16-token tiles).  The KS waves of a workgroup
// split the K groups into contiguous runs and reduce their partial sums
// through LDS in wave order.  Activations are the MFMA A operand (rows =
// tokens), weights the B operand (columns = channels): lane l owns channel
// n0 + l%16 and tokens 4*(l/16) + i.
//
// The run of dense groups is streamed in units of U groups with two units
// in flight: the loads of unit t+2 are issued before unit t+1 is computed.
// Every unit issues the same loads (groups past the run re-read its last
// group and get scale 0), so the load counters are waited on exactly, and
// the per-lane offsets are fixed: each unit only moves uniform bases.  The
// tile's activation and weight scales are staged in LDS once.  The residual
// blocks of the tile row follow as a second stream with the same item work
// against the activation fragment of each block's group (the zipper); they
// are dealt round-robin to the waves, so the waves finish together however
// the selected blocks cluster in K, and the first one is loaded before the
// dense stream starts.
template <int BLK, int KS, bool DUMP>
__global__ __launch_bounds__(64 * KS) void gemm_stream_kernel(GemmArgs a) {
  constexpr int U = 3;
  extern __shared__ __align__(16) unsigned char smem[];
  const int G = (int)(a.K / kGroup);
  float* sa_t = reinterpret_cast<float*>(smem);  // [G][16]: sa/256 of the tile's tokens
  float* sw_t = sa_t + G * 16;                     // [G][16]: weight scales of the tile's channels
  float* red = reinterpret_cast<float*>(smem);   // [KS][16][17] after the streams

  // readfirstlane tells the compiler the wave index is uniform, so loop
  // bounds and bases stay scalar
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int ch = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t m0 = (int64_t)blockIdx.y * 16;
  const int64_t Kh = a.K / 2;
  const int gb = wave * G / KS;
  const int ng = (wave + 1) * G / KS - gb;

  // per-lane byte offsets (32-bit: the host keeps N*K/2 and M*K/2 below 2^32)
  const uint32_t offW = (uint32_t)((n0 + r16) * Kh + ch * 16);
  const int64_t mr = m0 + r16;  // token rows past M read row M-1 (computed, never stored)
  const uint32_t offX = (uint32_t)((mr < a.M ? mr : a.M - 1) * Kh + ch * 16);

  struct Unit {
    uint4 W[U];  // B-operand fragments (weight codes)
    uint4 X[U];  // A-operand fragments (activation codes)
  };

  // dense unit t: groups gb + t*U + u, clamped to the run
  auto fetch_dense = [&](Unit& D, int t) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = gb + min(t * U + u, ng - 1);
      D.W[u] = ld16(a.qw + (int64_t)j * 64 + offW);
      D.X[u] = ld16(a.qa + (int64_t)j * 64 + offX);
    }
  };

  float y[4] = {0.f, 0.f, 0.f, 0.f};
  const v4i zero = {0, 0, 0, 0};

  // one item: two MFMAs, then y += (sa/256 * s) * acc for the lane's tokens
  // (s = the item's weight or residual row scale, 0 for padding)
  auto item = [&](const uint4& W, const uint4& X, float sc, uint32_t rm, int j, bool valid,
                  int64_t dump_at, bool dump_res) {
    v4i acc = mfma(widen8(X.x, X.y), widen8(W.x & rm, W.y & rm), zero);
    acc = mfma(widen8(X.z, X.w), widen8(W.z & rm, W.w & rm), acc);
    const float4 s4 = *reinterpret_cast<const float4*>(sa_t + j * 16 + 4 * ch);
    y[0] = fmaf(s4.x * sc, (float)acc[0], y[0]);
    y[1] = fmaf(s4.y * sc, (float)acc[1], y[1]);
    y[2] = fmaf(s4.z * sc, (float)acc[2], y[2]);
    y[3] = fmaf(s4.w * sc, (float)acc[3], y[3]);
    if (DUMP && valid) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + 4 * ch + i;
        if (m < a.M) {
          if (!dump_res)
            a.acc_dump[(m * a.N + n0 + r16) * G + j] = acc[i] >> 8;
          else
            a.acc_dump[dump_at + m * BLK] = acc[i] >> 8;
        }
      }
    }
  };
  auto compute_dense = [&](const Unit& D, int t) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool valid = t * U + u < ng;
      const int j = gb + min(t * U + u, ng - 1);
      item(D.W[u], D.X[u], valid ? sw_t[j * 16 + r16] : 0.f, 0xFFFFFFFFu, j, valid, 0, false);
    }
  };

  // ---- prologue: the tile's scale loads first, then two dense units and
  // the CSR window in flight; the scales go to LDS (transposed to [G][16])
  // as soon as they arrive, without waiting for the units ----
  const int nunits = (ng + U - 1) / U;
  constexpr int SMAX = 4;  // staged scale pairs issued ahead, per thread
  const int nst = 16 * G;
  const uint8_t* sa_b = reinterpret_cast<const uint8_t*>(a.sa);
  const uint8_t* sw_b = reinterpret_cast<const uint8_t*>(a.sw) + n0 * G * 2;
  float pa[SMAX];
  uint16_t pw[SMAX];
#pragma unroll
  for (int k = 0; k < SMAX; ++k) {
    const int i = min((int)threadIdx.x + k * 64 * KS, nst - 1);
    const int mm = i / G, j = i - mm * G;
    const int64_t m = m0 + mm;
    pa[k] = *reinterpret_cast<const float*>(sa_b + (uint32_t)(((m < a.M ? m : a.M - 1) * G + j) * 4));
    pw[k] = *reinterpret_cast<const uint16_t*>(sw_b + (uint32_t)(i * 2));
  }
  // (every wave has at least one group: the launcher keeps KS <= G; the
  // loads are unconditional so the waits for the scales above stay exact)
  Unit U0, U1;
  fetch_dense(U0, 0);
  fetch_dense(U1, 1);

  // Residual CSR row of this tile (block row nt, block rows rrow .. rrow+15).
  // The CSR arrays are read through the scalar cache (uniform addresses, a
  // read-only view), so their waits never involve the vector loads in flight.
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
  // first one's block column is fetched now
  const int nres = rp1 > rp0 ? (rp1 - rp0 - wave + KS - 1) / KS : 0;
  auto res_kt = [&](int k) { return cic[rp0 + wave + KS * k]; };
  const int kt_first = nres > 0 ? res_kt(0) : 0;
  const int kt_second = nres > 1 ? res_kt(1) : 0;

  // (stores past the table go to one spare slot, so no store is branched
  // and the waits stay exact)
  auto stage = [&](int i, float v, uint16_t w) {
    const int mm = i / G, j = i - mm * G;
    const int slot = i < nst ? j * 16 + mm : 2 * nst;
    sa_t[slot] = (m0 + mm < a.M) ? v * kInv256 : 0.f;
    sw_t[slot] = h2f(w);
  };
#pragma unroll
  for (int k = 0; k < SMAX; ++k) stage((int)threadIdx.x + k * 64 * KS, pa[k], pw[k]);
  for (int i = (int)threadIdx.x + SMAX * 64 * KS; i < nst; i += 64 * KS) {  // long K only
    const int mm = i / G, j = i - mm * G;
    const int64_t m = m0 + mm;
    stage(i, a.sa[(m < a.M ? m : a.M - 1) * G + j], a.sw[(n0 + mm) * G + j]);
  }
  __syncthreads();

  // ---- residual entries: the tile row's entries are dealt round-robin to
  // the waves (entry rp0 + wave + KS*i), so every wave gets the same share
  // whatever the block columns; the reduction below sums them with the
  // dense partials ----
  auto res_ptrs = [&](int k, int kt, uint4& W, uint4& X, uint32_t& S, uint32_t& rm, int& j) {
    const int e = rp0 + wave + KS * k;
    j = kt * BLK / kGroup;
    const int lo = kt * BLK - j * kGroup;
    const bool act = (32 * ch >= lo) && (32 * ch < lo + BLK);
    rm = act ? 0xFFFFFFFFu : 0u;
    W = ld16(a.qr + (int64_t)e * (BLK * BLK / 2) + (rrow + r16) * (BLK / 2) + (act ? 16 * ch - lo / 2 : 0));
    X = ld16(a.qa + (int64_t)j * 64 + offX);
    S = a.sr[(int64_t)e * BLK + rrow + r16];
  };
  auto res_item = [&](int k, const uint4& W, const uint4& X, uint32_t S, uint32_t rm, int j) {
    const int64_t e = rp0 + wave + KS * k;
    item(W, X, h2f((uint16_t)S), rm, j, true, a.M * a.N * G + e * a.M * BLK + rrow + r16, true);
  };
  // the first two entries are loaded now, so they arrive during the dense
  // stream
  uint4 W0, X0, W1, X1;
  uint32_t S0 = 0, S1 = 0, rm0 = 0, rm1 = 0;
  int j0 = 0, j1 = 0;
  if (nres > 0) res_ptrs(0, kt_first, W0, X0, S0, rm0, j0);
  if (nres > 1) res_ptrs(1, kt_second, W1, X1, S1, rm1, j1);

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
  for (int k = 0; k < nres; k += 2) {
    res_item(k, W0, X0, S0, rm0, j0);
    if (k + 2 < nres) res_ptrs(k + 2, res_kt(k + 2), W0, X0, S0, rm0, j0);
    if (k + 1 >= nres) break;
    res_item(k + 1, W1, X1, S1, rm1, j1);
    if (k + 3 < nres) res_ptrs(k + 3, res_kt(k + 3), W1, X1, S1, rm1, j1);
  }

  __syncthreads();  // scales no longer needed: reuse LDS for the reduction
#pragma unroll
  for (int i = 0; i < 4; ++i) red[(wave * 16 + 4 * ch + i) * 17 + r16] = y[i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < 256; idx += 64 * KS) {
    const int mm = idx >> 4, nl = idx & 15;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < KS; ++w) s += red[(w * 16 + mm) * 17 + nl];
    const int64_t m = m0 + mm;
    if (m < a.M) a.y[m * a.ldy + n0 + nl] = f2h_bits(s);
  }
}

template <int BLK, int KS, bool DUMP>
hipError_t launch_stream_cfg(const GemmArgs& a, hipStream_t st) {
  const int64_t G = a.K / kGroup;
  const size_t stage = (size_t)G * 16 * 4 * 2 + 4 * 16 * 4 + 16;
  const size_t reduce = (size_t)KS * 16 * 17 * 4;
  const size_t lds = stage > reduce ? stage : reduce;
  dim3 grid((unsigned)(a.N / 16), (unsigned)((a.M + 15) / 16));
  hipLaunchKernelGGL((gemm_stream_kernel<BLK, KS, DUMP>), grid, dim3(64 * KS), lds, st, a);
  return hipGetLastError();
}

// Waves per tile: the most (up to 16) that keep the grid within one
// resident round (<= 4096 waves, 16 per CU) and give every wave at least
// one unit of 4 groups.
template <int BLK, bool DUMP>
hipError_t launch_stream(const GemmArgs& a, hipStream_t st) {
  const int64_t G = a.K / kGroup;
  const int64_t tiles = (a.N / 16) * ((a.M + 15) / 16);
  if (tiles * 16 <= 4096 && G >= 64) return launch_stream_cfg<BLK, 16, DUMP>(a, st);
  if (tiles * 8 <= 4096 && G >= 32) return launch_stream_cfg<BLK, 8, DUMP>(a, st);
  if (tiles * 4 <= 4096 && G >= 16) return launch_stream_cfg<BLK, 4, DUMP>(a, st);
  if (G >= 8) return launch_stream_cfg<BLK, 2, DUMP>(a, st);
  return launch_stream_cfg<BLK, 1, DUMP>(a, st);
}

template <int BLK>
hipError_t launch_blk(const GemmArgs& a, hipStream_t st) {
  return a.acc_dump ? launch_stream<BLK, true>(a, st) : launch_stream<BLK, false>(a, st);
}

}  // namespace

hipError_t launch_fused_gemm(const GemmArgs& a, hipStream_t st) {
  // large M: LDS-tiled MFMA kernel (weights read once per 256-token tile);
  // small M, or a K too long for the tile kernel's LDS table: the streaming
  // kernel (weights read once per 16-token tile)
  if (a.M > 32 && tile_gemm_fits(a)) return launch_tile_gemm(a, st);
  switch (a.block) {
    case 32: return launch_blk<32>(a, st);
    case 64: return launch_blk<64>(a, st);
    default: return launch_blk<128>(a, st);
  }
}

}  // namespace mq
