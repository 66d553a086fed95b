// ZipperEngine fused layer for large M (prefill): LDS-tiled int8-MFMA GEMM.
// MosaicQuant technical summary (gist.science/pt/paper/2606.15652),
// Metodologia 3: one kernel runs the dense 4-bit GEMM, the sparse residual
// compensation and the scale/reduce-sum epilogue, the residual reusing the
// activation tile of the dense product.
//
// Tile: 128 tokens x 128 output channels per workgroup of four waves (2 x 2,
// 64 x 64 each, sixteen 16x16 MFMA tiles per wave).  One K step is one
// 128-channel group.  Per group the workgroup stages, in a register buffer
// and then in LDS:
//   A  activation codes, 128 rows x 64 bytes
//   B  weight codes,     128 rows x 64 bytes
//   R  residual codes for the same 128 channels (zero where no block is
//      selected), 128 rows x 64 bytes
//   the activation scales (x 1/256), weight scales and residual row scales.
// LDS holds each 16x16 fragment in MFMA lane order (slot = tile*64 + lane,
// 16 bytes), so every fragment read is one conflict-free 16-byte LDS read.
//
// K layout inside a group: lane chunk c = lane/16 feeds the first MFMA with
// channels [16c, 16c+16) and the second with [64+16c, 64+16c+16).  A 64-wide
// residual block therefore lines up with exactly one of the two MFMAs, a
// 32-wide block with one MFMA on half of the lanes, a 128-wide block with
// both, and each block keeps its own accumulator and row scale.
//
// Pipeline: group g passes through register buffer g%2 and LDS stage g%2.
// While the waves compute group j from LDS, the loads of groups j+1 and j+2
// are in flight; each group's loads have about two compute steps to arrive.
// Every step issues the same loads (groups past the end re-read the last
// group), so the hardware load counters are waited on exactly.
#include "gemm_common.h"

namespace mq {
namespace {

constexpr int TBM = 128;  // tokens per tile
constexpr int TBN = 128;  // output channels per tile

template <int BLK>
struct TileCfg {
  static constexpr int NBR = TBN / BLK;                    // block rows in a tile
  static constexpr int NBC = kGroup / BLK;                 // block columns in a group
  static constexpr int NSR = (TBN * NBC + 255) / 256;      // scale loads per thread
  static constexpr int SRS = NSR * 256;                    // residual-scale slots per stage
};

struct Stage {
  uint4 A[2], B[2], R[2];
  uint32_t rm[2];        // residual piece present (all-ones) or absent (zero)
  uint32_t sc;           // activation scale bits (waves 0-1) or weight scale (2-3)
  uint32_t sr[2];        // residual row scale bits (raw load)
  uint32_t srm[2];       // all-ones where that residual scale exists
};

template <int BLK, bool DUMP>
__global__ __launch_bounds__(256, 1) void gemm_tile_kernel(GemmArgs a) {
  using C = TileCfg<BLK>;
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int SA = 64 * 8 * 16;  // bytes of one staged operand tile (8 tiles x 64 lanes x 16 B)
  constexpr int STAGE = 3 * SA + TBM * 4 + TBN * 2 + C::SRS * 2;
  const int G = (int)(a.K / kGroup);
  const int KT = (int)(a.K / BLK);
  uint16_t* tab = reinterpret_cast<uint16_t*>(smem + 2 * STAGE);  // [NBR][KT]: entry-rp+1, 0 = none
  __shared__ int rp_row[C::NBR];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int r16 = lane & 15;
  const int ch = lane >> 4;

  // XCD-aware tile order: consecutive tiles (same token rows, adjacent
  // channel tiles) go to the same XCD so its L2 serves the shared A rows.
  const int tiles_n = (int)((a.N + TBN - 1) / TBN);
  const int tiles = (int)gridDim.x;
  const int xcd = blockIdx.x % 8;
  const int per = tiles / 8, rem = tiles % 8;
  const int tile = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + blockIdx.x / 8;
  const int64_t m0 = (int64_t)(tile / tiles_n) * TBM;
  const int64_t n0 = (int64_t)(tile % tiles_n) * TBN;
  const int64_t Kh = a.K / 2;
  const int nt0 = (int)(n0 / BLK);
  const int nrows_b = (int)(a.N / BLK);

  // ---- entry table of the tile's block rows: tab[rb][kt] ----
  for (int i = tid; i < C::NBR * KT; i += 256) tab[i] = 0;
  if (tid < C::NBR) {
    int r0 = 0;
    if (a.n_select > 0 && nt0 + tid < nrows_b) r0 = min(max(a.row_ptr[nt0 + tid], 0), a.n_select);
    rp_row[tid] = r0;
  }
  __syncthreads();
  if (a.n_select > 0) {
#pragma unroll
    for (int rb = 0; rb < C::NBR; ++rb) {
      if (nt0 + rb >= nrows_b) break;
      const int b0 = rp_row[rb];
      const int b1 = min(max(a.row_ptr[nt0 + rb + 1], b0), a.n_select);
      for (int e = b0 + tid; e < b1 && e - b0 < 0xFFFF; e += 256) {
        const int kt = a.col_idx[e];
        if (kt >= 0 && kt < KT) tab[rb * KT + kt] = (uint16_t)(e - b0 + 1);
      }
    }
  }
  __syncthreads();

  // ---- staging: global -> registers (fixed load count) ----
  auto load = [&](Stage& S, int j) {
    j = min(j, G - 1);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + 256 * i;
      const int r = q >> 2, p = q & 3;
      const int64_t m = min(m0 + r, a.M - 1);
      const int64_t n = min(n0 + r, a.N - 1);
      S.A[i] = ld16(a.qa + m * Kh + j * 64 + p * 16);
      S.B[i] = ld16(a.qw + n * Kh + j * 64 + p * 16);
      const int rb = (int)(n / BLK) - nt0;
      const int kg = j * kGroup + p * 32;
      const int kt = kg / BLK;
      const int ent = (a.n_select > 0) ? (int)tab[rb * KT + kt] : 0;
      const uint8_t* rp = a.qw;
      if (ent > 0) {
        const int64_t e = rp_row[rb] + ent - 1;
        rp = a.qr + e * (BLK * BLK / 2) + (n - (int64_t)(nt0 + rb) * BLK) * (BLK / 2) + (kg - kt * BLK) / 2;
      }
      S.R[i] = ld16(rp);
      S.rm[i] = ent > 0 ? 0xFFFFFFFFu : 0u;
    }
    if (wave < 2) {
      S.sc = __float_as_uint(a.sa[min(m0 + tid, a.M - 1) * G + j]);
    } else {
      S.sc = a.sw[min(n0 + (tid - 128), a.N - 1) * G + j];
    }
#pragma unroll
    for (int i = 0; i < C::NSR; ++i) {
      const int idx = tid + 256 * i;
      const int r = idx / C::NBC, c = idx % C::NBC;
      const int64_t n = min(n0 + min(r, TBN - 1), a.N - 1);
      const int rb = (int)(n / BLK) - nt0;
      const int ent = (a.n_select > 0 && idx < TBN * C::NBC) ? (int)tab[rb * KT + j * C::NBC + c] : 0;
      const uint16_t* sp = a.sw;
      if (ent > 0) sp = a.sr + (int64_t)(rp_row[rb] + ent - 1) * BLK + (n - (int64_t)(nt0 + rb) * BLK);
      S.sr[i] = (uint32_t)(*sp);  // combined with the mask at the LDS store, not here,
      S.srm[i] = ent > 0 ? 0xFFFFFFFFu : 0u;  // so the load is not waited on early
    }
  };

  // registers -> LDS stage (fragment lane order)
  auto store = [&](unsigned char* st, const Stage& S) {
    unsigned char* As = st;
    unsigned char* Bs = st + SA;
    unsigned char* Rs = st + 2 * SA;
    float* sas = reinterpret_cast<float*>(st + 3 * SA);
    uint16_t* sws = reinterpret_cast<uint16_t*>(st + 3 * SA + TBM * 4);
    uint16_t* srs = reinterpret_cast<uint16_t*>(st + 3 * SA + TBM * 4 + TBN * 2);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + 256 * i;
      const int r = q >> 2, p = q & 3;
      const int h = p >> 1, c0 = (p & 1) * 2;
      const int slot = (r >> 4) * 64 + (r & 15) + 16 * c0;
      const int o0 = slot * 16 + h * 8, o1 = (slot + 16) * 16 + h * 8;
      *reinterpret_cast<uint2*>(As + o0) = make_uint2(S.A[i].x, S.A[i].y);
      *reinterpret_cast<uint2*>(As + o1) = make_uint2(S.A[i].z, S.A[i].w);
      *reinterpret_cast<uint2*>(Bs + o0) = make_uint2(S.B[i].x, S.B[i].y);
      *reinterpret_cast<uint2*>(Bs + o1) = make_uint2(S.B[i].z, S.B[i].w);
      const uint32_t rm = S.rm[i];
      *reinterpret_cast<uint2*>(Rs + o0) = make_uint2(S.R[i].x & rm, S.R[i].y & rm);
      *reinterpret_cast<uint2*>(Rs + o1) = make_uint2(S.R[i].z & rm, S.R[i].w & rm);
    }
    if (wave < 2) {
      sas[tid] = (m0 + tid < a.M) ? __uint_as_float(S.sc) * kInv256 : 0.f;
    } else {
      sws[tid - 128] = (uint16_t)S.sc;
    }
#pragma unroll
    for (int i = 0; i < C::NSR; ++i) {
      const int idx = tid + 256 * i;
      srs[idx] = (uint16_t)(S.sr[i] & S.srm[i]);  // slots past TBN*NBC are padding
    }
  };

  const int wm = wave >> 1, wn = wave & 1;
  float y[4][4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) y[i][q][e] = 0.f;
  const v4i zero = {0, 0, 0, 0};

  auto compute = [&](const unsigned char* st, int j) {
    const unsigned char* As = st;
    const unsigned char* Bs = st + SA;
    const unsigned char* Rs = st + 2 * SA;
    const float* sas = reinterpret_cast<const float*>(st + 3 * SA);
    const uint16_t* sws = reinterpret_cast<const uint16_t*>(st + 3 * SA + TBM * 4);
    const uint16_t* srs = reinterpret_cast<const uint16_t*>(st + 3 * SA + TBM * 4 + TBN * 2);
    v4i Alo[4], Ahi[4];
    float4 sa4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tm = wm * 4 + i;
      const uint4 v = *reinterpret_cast<const uint4*>(As + (tm * 64 + lane) * 16);
      Alo[i] = widen8(v.x, v.y);
      Ahi[i] = widen8(v.z, v.w);
      sa4[i] = *reinterpret_cast<const float4*>(sas + tm * 16 + 4 * ch);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int tn = wn * 4 + q;
      const uint4 v = *reinterpret_cast<const uint4*>(Bs + (tn * 64 + lane) * 16);
      const v4i Blo = widen8(v.x, v.y), Bhi = widen8(v.z, v.w);
      const float sw = h2f(sws[tn * 16 + r16]);
      v4i acc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] = mfma(Alo[i], Blo, zero);
        acc[i] = mfma(Ahi[i], Bhi, acc[i]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        y[i][q][0] = fmaf(sa4[i].x * sw, (float)acc[i][0], y[i][q][0]);
        y[i][q][1] = fmaf(sa4[i].y * sw, (float)acc[i][1], y[i][q][1]);
        y[i][q][2] = fmaf(sa4[i].z * sw, (float)acc[i][2], y[i][q][2]);
        y[i][q][3] = fmaf(sa4[i].w * sw, (float)acc[i][3], y[i][q][3]);
        if (DUMP) {
          const int64_t n = n0 + tn * 16 + r16;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t m = m0 + (wm * 4 + i) * 16 + 4 * ch + e;
            if (m < a.M && n < a.N) a.acc_dump[(m * a.N + n) * G + j] = acc[i][e] >> 8;
          }
        }
      }
      // zipper: residual blocks of these 16 channels in group j
      const int nt = (int)((n0 + tn * 16) / BLK);
      const int rb = nt - nt0;
      if (a.n_select > 0 && nt < nrows_b) {
        const uint4 rv = *reinterpret_cast<const uint4*>(Rs + (tn * 64 + lane) * 16);
#pragma unroll
        for (int c = 0; c < C::NBC; ++c) {
          const int ent = __builtin_amdgcn_readfirstlane((int)tab[rb * KT + j * C::NBC + c]);
          if (ent == 0) continue;
          const float srf = h2f(srs[(tn * 16 + r16) * C::NBC + c]);
          v4i racc[4];
          if (BLK == 128) {
            const v4i Rlo = widen8(rv.x, rv.y), Rhi = widen8(rv.z, rv.w);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              racc[i] = mfma(Alo[i], Rlo, zero);
              racc[i] = mfma(Ahi[i], Rhi, racc[i]);
            }
          } else if (BLK == 64) {
            const v4i R = (c == 0) ? widen8(rv.x, rv.y) : widen8(rv.z, rv.w);
#pragma unroll
            for (int i = 0; i < 4; ++i) racc[i] = mfma(c == 0 ? Alo[i] : Ahi[i], R, zero);
          } else {
            // 32-wide block c: MFMA half c/2, lane chunks 2*(c%2), 2*(c%2)+1
            const uint32_t msk = ((ch >> 1) == (c & 1)) ? 0xFFFFFFFFu : 0u;
            const v4i R = (c < 2) ? widen8(rv.x & msk, rv.y & msk) : widen8(rv.z & msk, rv.w & msk);
#pragma unroll
            for (int i = 0; i < 4; ++i) racc[i] = mfma(c < 2 ? Alo[i] : Ahi[i], R, zero);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            y[i][q][0] = fmaf(sa4[i].x * srf, (float)racc[i][0], y[i][q][0]);
            y[i][q][1] = fmaf(sa4[i].y * srf, (float)racc[i][1], y[i][q][1]);
            y[i][q][2] = fmaf(sa4[i].z * srf, (float)racc[i][2], y[i][q][2]);
            y[i][q][3] = fmaf(sa4[i].w * srf, (float)racc[i][3], y[i][q][3]);
            if (DUMP) {
              const int64_t e_g = rp_row[rb] + ent - 1;
              const int rr = (int)(n0 + tn * 16 + r16 - (int64_t)nt * BLK);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int64_t m = m0 + (wm * 4 + i) * 16 + 4 * ch + e;
                if (m < a.M)
                  a.acc_dump[a.M * a.N * G + (e_g * a.M + m) * BLK + rr] = racc[i][e] >> 8;
              }
            }
          }
        }
      }
    }
  };

  unsigned char* st0 = smem;
  unsigned char* st1 = smem + STAGE;
  Stage R0, R1;
  load(R0, 0);
  load(R1, 1);
  store(st0, R0);
  load(R0, 2);
  __syncthreads();
  for (int j = 0; j < G; j += 2) {
    compute(st0, j);
    store(st1, R1);   // group j+1
    load(R1, j + 3);
    __syncthreads();
    if (j + 1 >= G) break;
    compute(st1, j + 1);
    store(st0, R0);   // group j+2
    load(R0, j + 4);
    __syncthreads();
  }

  // ---- output ----
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t n = n0 + (wn * 4 + q) * 16 + r16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t m = m0 + (wm * 4 + i) * 16 + 4 * ch + e;
        if (m < a.M && n < a.N) a.y[m * a.ldy + n] = f2h_bits(y[i][q][e]);
      }
    }
}

template <int BLK, bool DUMP>
hipError_t launch_tile_cfg(const GemmArgs& a, hipStream_t st) {
  using C = TileCfg<BLK>;
  constexpr int SA = 64 * 8 * 16;
  constexpr int STAGE = 3 * SA + TBM * 4 + TBN * 2 + C::SRS * 2;
  const size_t lds = 2 * (size_t)STAGE + (size_t)C::NBR * (size_t)(a.K / BLK) * 2;
  const int64_t tiles = ((a.M + TBM - 1) / TBM) * ((a.N + TBN - 1) / TBN);
  hipLaunchKernelGGL((gemm_tile_kernel<BLK, DUMP>), dim3((unsigned)tiles), dim3(256), lds, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tile_gemm(const GemmArgs& a, hipStream_t st) {
  const bool d = a.acc_dump != nullptr;
  switch (a.block) {
    case 32: return d ? launch_tile_cfg<32, true>(a, st) : launch_tile_cfg<32, false>(a, st);
    case 64: return d ? launch_tile_cfg<64, true>(a, st) : launch_tile_cfg<64, false>(a, st);
    default: return d ? launch_tile_cfg<128, true>(a, st) : launch_tile_cfg<128, false>(a, st);
  }
}

}  // namespace mq
