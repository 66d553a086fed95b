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
// MFMAs reuse the activation registers already loaded for the dense base in
// the same group (the "zipper"); chunks outside the block feed zeros.
#include "gemm_common.h"

namespace mq {
namespace {


// Streaming tile for small M: 16 output channels x 16 tokens per workgroup
// (grid.y walks 16-token tiles).  The KS waves of a workgroup split the K
// groups into contiguous runs; partial sums are reduced through LDS in wave
// order.  Activations are the MFMA A operand (rows = tokens), weights the B
// operand (columns = channels): lane l owns channel n0 + l%16 and tokens
// 4*(l/16) + i.
//
// Each wave consumes one stream of items: first its dense groups, then the
// residual blocks of its tile row whose block column lies in its groups,
// then padding.  Every item, dense or residual, is the same work - one
// 16-byte B fragment (weight or residual codes), one 16-byte A fragment
// (the activation codes of the item's group), one 2-byte scale (sw[n][j] or
// sr[e][r]), two MFMAs and a scale-and-add - so the zipper is literally the
// same instruction stream applied to the residual, against the activation
// codes of the same group.  Items are processed in units of U, and the next
// unit's loads are in flight while the current unit computes.  Because every
// unit issues exactly the same loads (padding items read a cached valid
// address and are masked to zero), the hardware load counters are waited on
// exactly, and nothing in the loop depends on the CSR lookup, which is read
// from a register window only when the stream reaches its residual items.
template <int BLK, int KS, int U, bool DUMP>
__global__ __launch_bounds__(64 * KS) void gemm_stream_kernel(GemmArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int G = (int)(a.K / kGroup);
  float* sa_t = reinterpret_cast<float*>(smem);  // [G][16]: sa/256 of the tile's tokens
  float* red = reinterpret_cast<float*>(smem);   // [KS][16][17] after the stream

  // readfirstlane tells the compiler the wave index is uniform, so loop
  // bounds and item metadata stay scalar
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int ch = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t m0 = (int64_t)blockIdx.y * 16;
  const int64_t Kh = a.K / 2;
  const int gb = wave * G / KS;
  const int ng = (wave + 1) * G / KS - gb;

  const uint8_t* wrow = a.qw + (n0 + r16) * Kh + ch * 16;
  // token rows past M read row M-1 (computed, never stored)
  const int64_t mr = m0 + r16;
  const uint8_t* xrow = a.qa + (mr < a.M ? mr : a.M - 1) * Kh + ch * 16;
  const uint16_t* swrow = a.sw + (n0 + r16) * G;

  // Residual CSR row of this tile (block row nt, block rows rrow .. rrow+15).
  // Lane l of the window holds the block column of entry wbase + l.
  const int nt = (int)(n0 / BLK);
  const int rrow = (int)(n0 - (int64_t)nt * BLK);
  int rp0 = 0, rp1 = 0;
  if (a.n_select > 0) {
    rp0 = a.row_ptr[nt];
    rp1 = a.row_ptr[nt + 1];
  }
  int wbase = 0;
  int kt_win = 0;

  struct Unit {
    uint4 A[U];     // B-operand fragments (weights or residual codes)
    uint4 X[U];     // A-operand fragments (activation codes)
    uint32_t S[U];  // scale bits (fp16 in the low half)
    float4 sa[U];   // activation scales of the lane's 4 tokens (from LDS)
  };
  struct Meta {
    int j[U];       // group of the item (for the activation scale)
    int e[U];       // residual entry, or -1 for a dense item, -2 for padding
    uint32_t rm[U]; // lane mask for the B fragment
  };

  // ---- the wave's residual items: [e_first, e_first + nr) ----
  // Register work only (the window was loaded once in the prologue), so no
  // load in the stream depends on it.  Entries the single window cannot
  // show run after the stream (see below).
  int nr = -1, e_first = rp0;
  bool window_full = false;
  auto ensure_nr = [&]() {
    if (nr >= 0) return;
    nr = 0;
    if (rp1 <= rp0 || ng <= 0) return;
    const int kt0 = gb * kGroup / BLK;
    const int kt1 = (gb + ng) * kGroup / BLK;
    const bool valid = wbase + lane < rp1;
    const int below = __popcll(__ballot(valid && kt_win < kt0));
    const int inside = __popcll(__ballot(valid && kt_win >= kt0 && kt_win < kt1));
    e_first = wbase + below;
    nr = inside;
    window_full = (below + inside == 64) && (wbase + 64 < rp1);
  };

  auto item_meta = [&](int i, Meta& M, int u, const uint8_t*& ap, const uint16_t*& sp) {
    if (i < ng) {
      const int j = gb + i;
      M.j[u] = j;
      M.e[u] = -1;
      M.rm[u] = 0xFFFFFFFFu;
      ap = wrow + (int64_t)j * 64;
      sp = swrow + j;
    } else if (i < ng + nr) {
      const int e = e_first + (i - ng);
      const int kt = __builtin_amdgcn_readlane(kt_win, e - wbase);
      const int j = kt * BLK / kGroup;
      const int lo = kt * BLK - j * kGroup;
      const bool act = (32 * ch >= lo) && (32 * ch < lo + BLK);
      M.j[u] = j;
      M.e[u] = e;
      M.rm[u] = act ? 0xFFFFFFFFu : 0u;
      ap = a.qr + (int64_t)e * (BLK * BLK / 2) + (rrow + r16) * (BLK / 2) + (act ? 16 * ch - lo / 2 : 0);
      sp = a.sr + (int64_t)e * BLK + rrow + r16;
    } else {
      M.j[u] = gb;
      M.e[u] = -2;
      M.rm[u] = 0u;
      ap = wrow;
      sp = swrow;
    }
  };

  // issue the U items of unit t (exactly 3U loads, always)
  auto fetch = [&](Unit& D, Meta& M, int t) {
    if ((t + 1) * U > ng) ensure_nr();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint8_t* ap;
      const uint16_t* sp;
      item_meta(t * U + u, M, u, ap, sp);
      D.A[u] = ld16(ap);
      D.X[u] = ld16(xrow + (int64_t)M.j[u] * 64);
      D.S[u] = *sp;
    }
  };
  // activation scales of a unit, read from LDS one unit ahead of use
  auto fetch_sa = [&](Unit& D, const Meta& M) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      D.sa[u] = *reinterpret_cast<const float4*>(sa_t + M.j[u] * 16 + 4 * ch);
  };

  float y[4] = {0.f, 0.f, 0.f, 0.f};
  const v4i zero = {0, 0, 0, 0};

  auto compute = [&](const Unit& D, const Meta& M) {
    const float4* sa4 = D.sa;
    v4i acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t rm = M.rm[u];
      acc[u] = mfma(widen8(D.X[u].x, D.X[u].y), widen8(D.A[u].x & rm, D.A[u].y & rm), zero);
      acc[u] = mfma(widen8(D.X[u].z, D.X[u].w), widen8(D.A[u].z & rm, D.A[u].w & rm), acc[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float sc = (M.e[u] == -2) ? 0.f : h2f((uint16_t)D.S[u]);
      y[0] = fmaf(sa4[u].x * sc, (float)acc[u][0], y[0]);
      y[1] = fmaf(sa4[u].y * sc, (float)acc[u][1], y[1]);
      y[2] = fmaf(sa4[u].z * sc, (float)acc[u][2], y[2]);
      y[3] = fmaf(sa4[u].w * sc, (float)acc[u][3], y[3]);
      if (DUMP && M.e[u] != -2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t m = m0 + 4 * ch + i;
          if (m < a.M) {
            if (M.e[u] == -1)
              a.acc_dump[(m * a.N + n0 + r16) * G + M.j[u]] = acc[u][i] >> 8;
            else
              a.acc_dump[a.M * a.N * G + ((int64_t)M.e[u] * a.M + m) * BLK + rrow + r16] =
                  acc[u][i] >> 8;
          }
        }
      }
    }
  };

  // ---- prologue: unit 0 in flight, then the activation scales to LDS ----
  Unit U0, U1;
  Meta M0, M1;
  // unit 0 holds only dense items unless the wave has fewer than U groups;
  // in that case the CSR lookup happens first
  if (ng > 0 && ng >= U) fetch(U0, M0, 0);
  if (a.n_select > 0) {
    rp0 = min(max(rp0, 0), a.n_select);
    rp1 = min(max(rp1, rp0), a.n_select);
    wbase = rp0;
    if (rp1 > rp0) kt_win = a.col_idx[min(rp0 + lane, rp1 - 1)];
  }
  if (ng > 0 && ng < U) fetch(U0, M0, 0);
  {
    const int bd = 64 * KS;
    for (int i0 = threadIdx.x; i0 < 16 * G; i0 += 4 * bd) {
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int idx = min(i0 + q * bd, 16 * G - 1);
        const int mm = idx / G;
        v[q] = a.sa[(m0 + mm < a.M ? m0 + mm : a.M - 1) * G + (idx - mm * G)];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int idx = i0 + q * bd;
        if (idx < 16 * G) {
          const int mm = idx / G, j = idx - mm * G;
          sa_t[j * 16 + mm] = (m0 + mm < a.M) ? v[q] * kInv256 : 0.f;
        }
      }
    }
  }
  __syncthreads();

  // ---- the stream (ping-pong buffers, never copied while in flight) ----
  if (ng > 0) {
    fetch_sa(U0, M0);
    for (int t = 0;; t += 2) {
      bool more = (t + 1) * U < ng + max(nr, 0) || (t + 1) * U < ng;
      if (!more && (t + 1) * U >= ng) {
        ensure_nr();
        more = (t + 1) * U < ng + nr;
      }
      fetch(U1, M1, t + 1);
      fetch_sa(U1, M1);
      compute(U0, M0);
      if (!more) break;
      bool more2 = (t + 2) * U < ng + max(nr, 0) || (t + 2) * U < ng;
      if (!more2 && (t + 2) * U >= ng) {
        ensure_nr();
        more2 = (t + 2) * U < ng + nr;
      }
      fetch(U0, M0, t + 2);
      fetch_sa(U0, M0);
      compute(U1, M1);
      if (!more2) break;
    }
  }

  // ---- residual entries the window did not show (rows with more than 64
  // entries up to this wave's last block column; rare): one at a time ----
  if (ng > 0 && window_full) {
    const int kt0 = gb * kGroup / BLK;
    const int kt1 = (gb + ng) * kGroup / BLK;
    for (int e = wbase + 64; e < rp1; ++e) {
      const int kt = a.col_idx[e];
      if (kt >= kt1) break;
      if (kt < kt0) continue;
      const int j = kt * BLK / kGroup;
      const int lo = kt * BLK - j * kGroup;
      const bool act = (32 * ch >= lo) && (32 * ch < lo + BLK);
      Unit D;
      Meta M;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        M.j[u] = j;
        M.e[u] = u == 0 ? e : -2;
        M.rm[u] = (u == 0 && act) ? 0xFFFFFFFFu : 0u;
        D.A[u] = ld16(a.qr + (int64_t)e * (BLK * BLK / 2) + (rrow + r16) * (BLK / 2) +
                      (act ? 16 * ch - lo / 2 : 0));
        D.X[u] = ld16(xrow + (int64_t)j * 64);
        D.S[u] = a.sr[(int64_t)e * BLK + rrow + r16];
      }
      fetch_sa(D, M);
      compute(D, M);
    }
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

template <int BLK, int KS, int U, bool DUMP>
hipError_t launch_stream_cfg(const GemmArgs& a, hipStream_t st) {
  const int64_t G = a.K / kGroup;
  const size_t stage = (size_t)G * 16 * 4;
  const size_t reduce = (size_t)KS * 16 * 17 * 4;
  const size_t lds = stage > reduce ? stage : reduce;
  dim3 grid((unsigned)(a.N / 16), (unsigned)((a.M + 15) / 16));
  hipLaunchKernelGGL((gemm_stream_kernel<BLK, KS, U, DUMP>), grid, dim3(64 * KS), lds, st, a);
  return hipGetLastError();
}

// Waves per tile: enough workgroups to fill the machine, at least one unit
// of items per wave.
template <int BLK, bool DUMP>
hipError_t launch_stream(const GemmArgs& a, hipStream_t st) {
  const int64_t G = a.K / kGroup;
  const int64_t tiles = (a.N / 16) * ((a.M + 15) / 16);
  if (tiles >= 768 && G >= 8) return launch_stream_cfg<BLK, 4, 4, DUMP>(a, st);
  if (G >= 32) return launch_stream_cfg<BLK, 8, 4, DUMP>(a, st);
  if (G >= 8) return launch_stream_cfg<BLK, 4, 4, DUMP>(a, st);
  return launch_stream_cfg<BLK, 2, 4, DUMP>(a, st);
}

template <int BLK>
hipError_t launch_blk(const GemmArgs& a, hipStream_t st) {
  return a.acc_dump ? launch_stream<BLK, true>(a, st) : launch_stream<BLK, false>(a, st);
}

}  // namespace

hipError_t launch_fused_gemm(const GemmArgs& a, hipStream_t st) {
  // large M: LDS-tiled MFMA kernel (weights read once per 128-token tile);
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
