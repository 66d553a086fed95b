// Unfused ablation of the residual branch: a standalone residual GEMM that
// reloads the activations and merges its partial output into y, i.e. the
// design the ZipperEngine replaces.  MosaicQuant technical summary
// (gist.science/pt/paper/2606.15652), Metodologia 3: computing the sparse
// compensation in a separate kernel would reload the activations and merge
// partial outputs; the fused kernel avoids both.  This kernel exists so the
// two designs can be timed against each other on the same data; the layer's
// path never uses it.
//
// Grid: (N/b block rows, 16-token tiles); one wave per 16 channels of the
// block row.  For each selected block of its row the wave loads the block's
// codes for its 16 channels and the activation codes of the block's group
// for its 16 tokens (again, from L2/HBM), runs the same two int8 MFMAs as the
// fused kernel's residual item, and accumulates sa*sr*acc; at the end it
// adds that to the dense output already in y: y = f16(f32(y) + residual).
#include "gemm_common.h"

namespace mq {
namespace {

template <int BLK>
__global__ __launch_bounds__(64 * (BLK / 16)) void residual_merge_kernel(GemmArgs a) {
  const int G = (int)(a.K / kGroup);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int ch = lane >> 4;
  const int nt = blockIdx.x;
  const int64_t m0 = (int64_t)blockIdx.y * 16;
  const int rrow = wave * 16;  // this wave's 16 channels inside the block row
  const int64_t Kh = a.K / 2;
  const int64_t mr = m0 + r16;
  const uint8_t* xrow = a.qa + (mr < a.M ? mr : a.M - 1) * Kh + ch * 16;
  const int e0 = min(max(a.row_ptr[nt], 0), a.n_select);
  const int e1 = min(max(a.row_ptr[nt + 1], e0), a.n_select);
  const v4i zero = {0, 0, 0, 0};
  float y[4] = {0.f, 0.f, 0.f, 0.f};
  // entries in chunks of four, all loads of a chunk in flight together
  constexpr int C = 4;
  for (int eb = e0; eb < e1; eb += C) {
    uint4 W[C], X[C];
    uint32_t rm[C];
    int jj[C];
    float sr[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int e = min(eb + c, e1 - 1);
      const int kt_in = a.col_idx[e];
      const bool okt = kt_in >= 0 && kt_in < (int)(a.K / BLK);  // else the entry adds nothing
      const int kt = okt ? kt_in : 0;
      const int j = kt * BLK / kGroup;
      const int lo = kt * BLK - j * kGroup;
      const bool act = (32 * ch >= lo) && (32 * ch < lo + BLK) && (eb + c < e1) && okt;
      rm[c] = act ? 0xFFFFFFFFu : 0u;
      jj[c] = j;
      W[c] = ld16(a.qr + (int64_t)e * (BLK * BLK / 2) + (rrow + r16) * (BLK / 2) + (act ? 16 * ch - lo / 2 : 0));
      X[c] = ld16(xrow + (int64_t)j * 64);
      sr[c] = h2f(a.sr[(int64_t)e * BLK + rrow + r16]);
    }
#pragma unroll
    for (int c = 0; c < C; ++c) {
      v4i acc = mfma(widen8(X[c].x, X[c].y), widen8(W[c].x & rm[c], W[c].y & rm[c]), zero);
      acc = mfma(widen8(X[c].z, X[c].w), widen8(W[c].z & rm[c], W[c].w & rm[c]), acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + 4 * ch + i;
        const float sa = a.sa[(m < a.M ? m : a.M - 1) * G + jj[c]] * kInv256;
        y[i] = fmaf(sa * sr[c], (float)acc[i], y[i]);
      }
    }
  }
  const int64_t n = (int64_t)nt * BLK + rrow + r16;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + 4 * ch + i;
    if (m < a.M) {
      uint16_t* p = a.y + m * a.ldy + n;
      *p = f2h_bits(h2f(*p) + y[i]);
    }
  }
}

template <int BLK>
hipError_t launch_res(const GemmArgs& a, hipStream_t st) {
  dim3 grid((unsigned)(a.N / BLK), (unsigned)((a.M + 15) / 16));
  hipLaunchKernelGGL(residual_merge_kernel<BLK>, grid, dim3(64 * (BLK / 16)), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_residual_merge(const GemmArgs& a, hipStream_t st) {
  switch (a.block) {
    case 32: return launch_res<32>(a, st);
    case 64: return launch_res<64>(a, st);
    default: return launch_res<128>(a, st);
  }
}

}  // namespace mq
