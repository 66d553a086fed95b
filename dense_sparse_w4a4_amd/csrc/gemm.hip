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
// product; the epilogue folds 1/256 into the scale and the debug dump shifts
// it out exactly.  Splitting a packed word into its even and odd codes
// permutes k inside a 16-code chunk identically for both operands, which
// leaves the dot product unchanged.
//
// Per 128-channel group j the two MFMAs cover group-local k in [0, 64) and
// [64, 128); lane chunk c (lane/16) holds k = 16c .. 16c+15 of each half.
// A residual block (edge b in {32, 64, 128}) of the current group lies in
// one or both halves at a chunk-aligned offset, so its MFMA reuses the same
// activation registers (the "zipper"); lanes outside a 32-wide block feed
// zeros.
#include "mq_internal.h"

namespace mq {
namespace {

__device__ __forceinline__ v4i widen8(uint2 p) {
  v4i r;
  r[0] = (int)((p.x << 4) & 0xF0F0F0F0u);
  r[1] = (int)(p.x & 0xF0F0F0F0u);
  r[2] = (int)((p.y << 4) & 0xF0F0F0F0u);
  r[3] = (int)(p.y & 0xF0F0F0F0u);
  return r;
}

__device__ __forceinline__ uint2 ld8(const uint8_t* p) {
  return *reinterpret_cast<const uint2*>(p);
}

__device__ __forceinline__ v4i mfma(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

constexpr float kInv256 = 1.0f / 256.0f;

// Skinny tile: 16 output channels x 16 tokens per workgroup, K split across
// the KS waves of the workgroup (contiguous runs of groups), partial sums
// reduced through LDS in wave order.  Weights are the MFMA A operand (rows =
// output channels), activations the B operand (columns = tokens).  Output
// lane layout: token m = m0 + lane%16, channels n0 + 4*(lane/16) + i.
template <int BLK, int KS, bool DUMP>
__global__ __launch_bounds__(64 * KS) void gemm_skinny_kernel(GemmArgs a) {
  constexpr int U = 4;  // groups whose loads are issued together
  __shared__ float red[KS][16][17];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int ch = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t m0 = (int64_t)blockIdx.y * 16;
  const int64_t G = a.K / kGroup;
  const int64_t Kh = a.K / 2;
  const int64_t gb = (int64_t)wave * G / KS;
  const int64_t ge = (int64_t)(wave + 1) * G / KS;

  const uint8_t* wrow = a.qw + (n0 + r16) * Kh + ch * 8;
  const int64_t m = m0 + r16;
  const bool mval = m < a.M;
  const uint8_t* xrow = a.qa + (mval ? m : 0) * Kh + ch * 8;
  const float* sarow = a.sa + (mval ? m : 0) * G;
  const uint16_t* swrow = a.sw + (n0 + 4 * ch) * G;

  // CSR cursor of this tile's block row, advanced group by group.
  const int64_t nt = n0 / BLK;
  const int rrow = (int)(n0 - nt * BLK);  // first block row covered by this tile
  int e = 0, e_end = 0;
  if (a.n_select > 0) {
    int rp0 = a.row_ptr[nt], rp1 = a.row_ptr[nt + 1];
    rp0 = min(max(rp0, 0), a.n_select);
    rp1 = min(max(rp1, rp0), a.n_select);
    e = rp0;
    e_end = rp1;
    const int kt0 = (int)(gb * kGroup / BLK);
    while (e < e_end && a.col_idx[e] < kt0) ++e;
  }

  float yacc[4] = {0.f, 0.f, 0.f, 0.f};
  const v4i zero = {0, 0, 0, 0};

  for (int64_t jb = gb; jb < ge; jb += U) {
    uint2 w0[U], w1[U], x0[U], x1[U];
    float sav[U];
    float swv[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = jb + u;
      if (j < ge) {
        w0[u] = ld8(wrow + j * 64);
        w1[u] = ld8(wrow + j * 64 + 32);
        if (mval) {
          x0[u] = ld8(xrow + j * 64);
          x1[u] = ld8(xrow + j * 64 + 32);
          sav[u] = sarow[j] * kInv256;
        } else {
          x0[u] = make_uint2(0, 0);
          x1[u] = make_uint2(0, 0);
          sav[u] = 0.f;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) swv[u][i] = h2f(swrow[i * G + j]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = jb + u;
      if (j >= ge) break;
      const v4i X0 = widen8(x0[u]);
      const v4i X1 = widen8(x1[u]);
      v4i acc = mfma(widen8(w0[u]), X0, zero);
      acc = mfma(widen8(w1[u]), X1, acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) yacc[i] = fmaf(sav[u] * swv[u][i], (float)acc[i], yacc[i]);
      if (DUMP && mval) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a.acc_dump[(m * a.N + n0 + 4 * ch + i) * G + j] = acc[i] >> 8;
      }
      // Zipper: residual blocks of this tile row inside group j.
      const int kt_lo = (int)(j * kGroup / BLK);
      const int kt_hi = (int)((j + 1) * kGroup / BLK);
      while (e < e_end) {
        const int kt = a.col_idx[e];
        if (kt >= kt_hi) break;
        if (kt >= kt_lo) {
          const int lo = kt * BLK - (int)(j * kGroup);  // group-local first channel
          const uint8_t* rb = a.qr + (int64_t)e * (BLK * BLK / 2) + (rrow + r16) * (BLK / 2);
          v4i racc;
          if (BLK == 128) {
            racc = mfma(widen8(ld8(rb + ch * 8)), X0, zero);
            racc = mfma(widen8(ld8(rb + 32 + ch * 8)), X1, racc);
          } else if (BLK == 64) {
            racc = mfma(widen8(ld8(rb + ch * 8)), lo == 0 ? X0 : X1, zero);
          } else {
            const int c0 = ((lo & 63) >> 5) * 2;  // first active lane chunk
            const bool act = (ch >> 1) == (c0 >> 1);
            const v4i R = act ? widen8(ld8(rb + (ch - c0) * 8)) : zero;
            racc = mfma(R, lo < 64 ? X0 : X1, zero);
          }
          const uint16_t* srp = a.sr + (int64_t)e * BLK + rrow + 4 * ch;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            yacc[i] = fmaf(sav[u] * h2f(srp[i]), (float)racc[i], yacc[i]);
          if (DUMP && mval) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              a.acc_dump[a.M * a.N * G + ((int64_t)e * a.M + m) * BLK + rrow + 4 * ch + i] =
                  racc[i] >> 8;
          }
        }
        ++e;
      }
    }
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][4 * ch + i][r16] = yacc[i];
  __syncthreads();
  for (int t = threadIdx.x; t < 256; t += 64 * KS) {
    const int ml = t >> 4, nl = t & 15;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < KS; ++w) s += red[w][nl][ml];
    if (m0 + ml < a.M) a.y[(m0 + ml) * a.ldy + n0 + nl] = f2h_bits(s);
  }
}

template <int BLK, bool DUMP>
hipError_t launch_skinny(const GemmArgs& a, hipStream_t st) {
  const int64_t G = a.K / kGroup;
  dim3 grid((unsigned)(a.N / 16), (unsigned)((a.M + 15) / 16));
  if (G >= 16) {
    hipLaunchKernelGGL((gemm_skinny_kernel<BLK, 8, DUMP>), grid, dim3(512), 0, st, a);
  } else {
    hipLaunchKernelGGL((gemm_skinny_kernel<BLK, 4, DUMP>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

template <int BLK>
hipError_t launch_blk(const GemmArgs& a, hipStream_t st) {
  return a.acc_dump ? launch_skinny<BLK, true>(a, st) : launch_skinny<BLK, false>(a, st);
}

}  // namespace

hipError_t launch_fused_gemm(const GemmArgs& a, hipStream_t st) {
  switch (a.block) {
    case 32: return launch_blk<32>(a, st);
    case 64: return launch_blk<64>(a, st);
    default: return launch_blk<128>(a, st);
  }
}

}  // namespace mq
