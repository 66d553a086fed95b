// ZipperEngine fused layer for large M (prefill), fp6 route: the LDS-tiled
// GEMM of gemm_tile.hip with its operands on the FP6 matrix core.
// MosaicQuant technical summary (gist.science/pt/paper/2606.15652),
// Metodologia 3: one kernel runs the dense 4-bit GEMM, the sparse residual
// compensation and the scale/reduce-sum epilogue, the residual reusing the
// activation tile of the dense product.
//
// The 4-bit codes reach this kernel re-encoded as FP6 E2M3 images (fp6.hip,
// layout in mq_internal.h): each field's value is exactly q/8, so one
// V_MFMA_F32_32X32X64_F8F6F4 gives the exact integer dot product of 64
// codes / 64, in fp32.  On gfx950 that instruction takes as long as one
// V_MFMA_I32_32X32X32_I8 for twice the K, and its fp32 result needs no
// conversion before the per-group scaling: per 32 x 32 sub-tile and group
// two FP6 MFMAs, one scale-product MFMA and 16 FMAs per lane, where the int8
// route has four int8 MFMAs, one scale-product MFMA, 16 converts and 16 FMAs.
//
// Tile: 256 tokens x 128 output channels per workgroup of eight waves (wave
// w computes the 64 x 64 quarter (w % 4, w / 4), four 32 x 32 sub-tiles).
// Per 128-channel group the workgroup's LDS stage holds
//   A  eight 32-token row blocks' images (24 KB), copied from memory by LDS
//      DMA (wave w: row block w, three 1 KB pieces);
//   B  four 32-channel column blocks' weight images (12 KB), by LDS DMA
//      (pieces w and w + 8 of the twelve);
//   R  the residual images of the tile's selected blocks in this group, in
//      the column blocks' layout (12 KB; wave w stages column block w / 2,
//      slice w % 2 through registers; rows of unselected blocks hold unused
//      data);
//   the scale operands: per token sa * 64 and per channel sw (and the
//      residual row scales) as (hi, lo) bf16 pairs; one
//      V_MFMA_F32_32X32X8_BF16 forms each sub-tile's 32 x 32 products
//      sa * sw (exact in sw, within 2^-16 in sa), and the factor 64 undoes
//      the fields' 1/8 on both operands.
// Every product S * D equals the int8 route's (both are sa * sw * dot up to
// the same bf16 split, scaled by powers of two), so the two routes give the
// same fp32 partial sums and the same fp16 outputs.
//
// Pipeline and residual table as in gemm_tile.hip: two LDS stages, one
// LDS-only barrier per group, register buffers two groups ahead, every step
// issuing the same loads (dummy offsets where no residual block is selected)
// so that the DMA wait counts them exactly.  Work order: banded and
// XCD-aware as there, but K is split only for the tiles of a partial last
// round (all tiles when there are fewer than one round), the others taking
// all of K first, so the partials' HBM round trip covers only those tiles.
#include "gemm_common.h"

namespace mq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));

constexpr int TBM = 256;
constexpr int TBN = 128;
constexpr int NTHR = 512;
constexpr size_t kMaxLds = 160 * 1024;

// Origin of tile t in the banded order: bands of four token tiles, channel
// tiles outer within a band, so that consecutive tiles share weight tiles.
__device__ __forceinline__ void tile6_origin(int t, int tiles_m, int tiles_n, int64_t& m0, int64_t& n0) {
  constexpr int kBand = 4;
  const int band = t / (kBand * tiles_n);
  const int bh = min(kBand, tiles_m - band * kBand);
  const int rbi = t - band * kBand * tiles_n;
  m0 = (int64_t)(band * kBand + rbi % bh) * TBM;
  n0 = (int64_t)(rbi / bh) * TBN;
}

template <int BLK>
struct Tile6Cfg {
  static constexpr int NBR = TBN / BLK;      // block rows in a tile
  static constexpr int NBC = kGroup / BLK;   // block columns in a group
  static constexpr int NS = BLK / 64;        // 64-code slices of a block
  static constexpr int NSRS = TBN * NBC;     // residual-scale slots (<= NTHR)
  static constexpr int A_OFF = 0;                     // 8 row blocks x 3 KB
  static constexpr int B_OFF = 8 * kFp6Frag;          // 4 column blocks x 3 KB
  static constexpr int R_OFF = B_OFF + 4 * kFp6Frag;  // 4 column blocks x 3 KB
  static constexpr int SA_OFF = R_OFF + 4 * kFp6Frag; // [8 row blocks][32 lanes] x 8 bytes
  static constexpr int SW_OFF = SA_OFF + 8 * 256;     // [4 column blocks][32 lanes] x 8 bytes
  static constexpr int SR_OFF = SW_OFF + 4 * 256;     // [4 column blocks][NBC][32 lanes] x 8 bytes
  static constexpr int STAGE = SR_OFF + 4 * NBC * 256;
  static constexpr int ZERO_OFF = 2 * STAGE;          // 16 zero bytes
  static constexpr int TAB_OFF = ZERO_OFF + 16;
  static size_t lds(int64_t K) {
    return (size_t)TAB_OFF + (size_t)NBR * (size_t)(K / BLK) * 2 + (size_t)(K / kGroup);
  }
};

typedef __attribute__((address_space(3))) v4i lds_v4i;
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x2 lds_u2;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ v4i lds_ld16(uint32_t a) { return *(const lds_v4i*)(uintptr_t)a; }
__device__ __forceinline__ v4s lds_ld8(uint32_t a) { return *(const lds_v4s*)(uintptr_t)a; }
__device__ __forceinline__ u32x2 lds_ld8u(uint32_t a) { return *(const lds_u2*)(uintptr_t)a; }
__device__ __forceinline__ void lds_st16(uint32_t a, v4i v) { *(lds_v4i*)(uintptr_t)a = v; }
__device__ __forceinline__ void lds_st8(uint32_t a, uint32_t lo, uint32_t hi) {
  const u32x2 v = {lo, hi};
  *(lds_u2*)(uintptr_t)a = v;
}

// This wave's LDS writes complete, then s_barrier (the global loads of later
// groups stay in flight; LDS DMA is waited for separately, before it).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// One lane's FP6 operand: its dwords 0-3 at LDS address lo, 4-5 at hi.
// Callers pass bases that already hold the lane's offsets (fp6_lo_offset /
// fp6_hi_offset at u = 0) plus compile-time offsets of the fragment, which
// fold into the instructions' offset fields.
__device__ __forceinline__ v8i frag6(uint32_t lo_a, uint32_t hi_a) {
  const v4i lo = lds_ld16(lo_a);
  const u32x2 hi = lds_ld8u(hi_a);
  const v8i r = {lo[0], lo[1], lo[2], lo[3], (int)hi[0], (int)hi[1], 0, 0};
  return r;
}
// D = A . B + C on FP6 E2M3 operands (format code 2 for both).
__device__ __forceinline__ v16f mfma6(v8i a, v8i b, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 2, 2, 0, 0, 0, 0);
}
__device__ __forceinline__ v16f mfma_scale(v4s a, v4s b) {
  const v16f z = {};
  return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a, b, z, 0, 0, 0);
}

__device__ __forceinline__ uint32_t bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_value(uint32_t b) { return __uint_as_float(b << 16); }
// (hi, lo) bf16 pair with hi + lo = x to within 2^-16 relative (exactly for
// an fp16 x).
__device__ __forceinline__ uint32_t split_bf16(float x) {
  const uint32_t hi = bf16_bits(x);
  const uint32_t lo = bf16_bits(x - bf16_value(hi));
  return hi | (lo << 16);
}

struct Stage6 {
  v4i W;  // raw base codes (weights without an image): 32 codes of one lane slice
  v4i Rlo;
  u32x2 Rhi;
  uint32_t sc;  // activation scale bits (waves 0-3) or weight scale bits (waves 4-5)
  uint32_t sr;  // residual row scale bits
};

// WRAW: no weight image; the base codes are read from the packed slab
// layout into registers (one lane slice, 32 codes, per thread and group),
// re-encoded there and stored to LDS like the residual pieces.
template <int BLK, bool DUMP, bool WRAW>
__global__ __launch_bounds__(NTHR, 1) void gemm_tile6_kernel(GemmArgs a) {
  using C = Tile6Cfg<BLK>;
  extern __shared__ __align__(16) unsigned char smem[];
  const int G = (int)(a.K / kGroup);
  const int KT = (int)(a.K / BLK);
  uint16_t* tab = reinterpret_cast<uint16_t*>(smem + C::TAB_OFF);  // [NBR][KT]: entry-rp+1, 0 = none
  uint8_t* anyr = smem + C::TAB_OFF + C::NBR * KT * 2;              // [G]: a selected block in group j
  __shared__ int rp_row[C::NBR];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & 7;
  const int lane = tid & 63;

  // work order: the first `full` tiles (banded order) take all of K, the
  // last `tail` tiles are split ksplit ways (tail = every tile: split-K as in
  // the int8 route).  Workgroup b runs on XCD b % 8; each XCD takes a
  // contiguous share of the full tiles and then a contiguous share of the
  // split units, so the short units fill the last round everywhere.
  const int tiles_n = (int)((a.N + TBN - 1) / TBN);
  const int tiles_m = (int)((a.M + TBM - 1) / TBM);
  const int tiles = tiles_m * tiles_n;
  const int tail = a.ksplit > 1 ? a.split_tail : 0;
  const int full = tiles - tail;
  const int items = (int)gridDim.x;  // full + tail * ksplit
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int nfull = full / 8 + (xcd < full % 8 ? 1 : 0);
  const int fbase = xcd * (full / 8) + min(xcd, full % 8);
  int tile, split, jb, je;
  if (slot < nfull) {
    tile = fbase + slot;
    split = -1;
    jb = 0;
    je = G;
  } else {
    const int unit = xcd * (items / 8) + min(xcd, items % 8) - fbase + (slot - nfull);
    split = unit / tail;
    tile = full + (unit - split * tail);
    jb = (int)((int64_t)split * G / a.ksplit);
    je = (int)((int64_t)(split + 1) * G / a.ksplit);
  }
  int64_t m0, n0;
  tile6_origin(tile, tiles_m, tiles_n, m0, n0);
  const int nt0 = (int)(n0 / BLK);
  const int nrows_b = (int)(a.N / BLK);

  // ---- entry table of the tile's block rows: tab[rb][kt]; anyr[j] ----
  for (int i = tid; i < C::NBR * KT; i += NTHR) tab[i] = 0;
  for (int i = tid; i < G; i += NTHR) anyr[i] = 0;
  if (tid < 4) reinterpret_cast<uint32_t*>(smem + C::ZERO_OFF)[tid] = 0u;
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
      for (int e = b0 + tid; e < b1 && e - b0 < 0xFFFF; e += NTHR) {
        const int kt = a.col_idx[e];
        if (kt >= 0 && kt < KT) {
          tab[rb * KT + kt] = (uint16_t)(e - b0 + 1);
          anyr[kt / C::NBC] = 1;  // (benign race: every writer stores 1)
        }
      }
    }
  }
  __syncthreads();

  // ---- operand copies by LDS DMA ----
  // A: wave w copies row block w of the tile (row blocks past the last one
  // of M re-read the last one).  B: wave w copies pieces w and, for w < 4,
  // w + 8 of the twelve 1 KB pieces (column block p / 3, piece p % 3) of the
  // four column blocks (past N: the last one).
  const int64_t nrb = wide_rows(a.M) / 32;
  const int64_t ncb = a.N / 32;
  const uint8_t* srcA = a.aimg + min(m0 / 32 + wave, nrb - 1) * G * kFp6Frag + lane * 16;
  const int pB0 = wave, pB1 = wave + 8;
  const uint8_t* wimg = WRAW ? a.qw : a.wimg;  // (no image: B pointers unused)
  const uint8_t* srcB0 = wimg + min(n0 / 32 + pB0 / 3, ncb - 1) * G * kFp6Frag + (pB0 % 3) * 1024 + lane * 16;
  const uint8_t* srcB1 =
      wimg + min(n0 / 32 + (pB1 < 12 ? pB1 : 0) / 3, ncb - 1) * G * kFp6Frag + (pB1 % 3) * 1024 + lane * 16;
  const uint32_t dstB0 = (uint32_t)(C::B_OFF + (pB0 / 3) * kFp6Frag + (pB0 % 3) * 1024);
  const uint32_t dstB1 = (uint32_t)(C::B_OFF + ((pB1 < 12 ? pB1 : 0) / 3) * kFp6Frag + (pB1 % 3) * 1024);
  typedef __attribute__((address_space(3))) void* lds_ptr;
  auto dma = [&](uint32_t st, int j) {
    j = min(j, je - 1);
    const int64_t jo = (int64_t)j * kFp6Frag;
#pragma unroll
    for (int p = 0; p < 3; ++p)
      __builtin_amdgcn_global_load_lds(srcA + jo + p * 1024,
                                       (lds_ptr)(uintptr_t)(st + C::A_OFF + (uint32_t)wave * kFp6Frag + p * 1024), 16,
                                       0, 0);
    if (!WRAW) {
      __builtin_amdgcn_global_load_lds(srcB0 + jo, (lds_ptr)(uintptr_t)(st + dstB0), 16, 0, 0);
      if (wave < 4) __builtin_amdgcn_global_load_lds(srcB1 + jo, (lds_ptr)(uintptr_t)(st + dstB1), 16, 0, 0);
    }
  };
  // raw base codes: thread tid makes lane lw = tid % 64 of slice uw6 =
  // (tid / 64) % 2 of the tile's column block cw = tid / 128 (past N: the
  // last one), codes 32c .. 32c+31 of row n, c = 2 uw6 + lw / 32, at
  // qw + (n/16)*8K + j*1024 + (16c + n%16)*16 in the slab layout
  const int cw = tid >> 7, uw6 = (tid >> 6) & 1, lw = tid & 63;
  const int64_t nw = min(n0 / 32 + cw, ncb - 1) * 32 + (lw & 31);
  const uint8_t* srcW = a.qw + (nw >> 4) * 8 * a.K + (16 * (2 * uw6 + (lw >> 5)) + (nw & 15)) * 16;
  const uint32_t dstWlo = (uint32_t)(C::B_OFF + cw * kFp6Frag + fp6_lo_offset(uw6, lw));
  const uint32_t dstWhi = (uint32_t)(C::B_OFF + cw * kFp6Frag + fp6_hi_offset(uw6, lw));
  // after a step's loads: the step's DMA (issued before the step's four
  // register loads: scale, residual pieces, residual scale) has completed.
  // The builtin (vmcnt 4; expcnt, lgkmcnt unconstrained) rather than inline
  // asm, so that the compiler's own wait analysis knows every older load is
  // done and adds no vmcnt(0) before the next step's stores.
  auto dma_wait = [&]() {
    __builtin_amdgcn_s_waitcnt(WRAW ? kWaitVm5 : kWaitVm4);  // WRAW: five register loads a step
    asm volatile("" ::: "memory");
  };

  // ---- register staging: scales, residual pieces ----
  // Residual: wave w stages column block cbw = w / 2, slice uw = w % 2 of
  // the tile's selected block there (block row cbw*32/BLK, block column
  // uw*64/BLK of the group; its piece (cbw*32 % BLK)/32 * NS + (uw*64 % BLK)/64).
  const uint8_t* rbase = a.n_select > 0 ? a.rimg : a.wimg;
  const uint8_t* sbase = a.n_select > 0 ? reinterpret_cast<const uint8_t*>(a.sr)
                                        : reinterpret_cast<const uint8_t*>(a.sw);
  const int cbw = wave >> 1, uw = wave & 1;
  const int rbtw = (cbw * 32) / BLK;
  const int tabR = rbtw * KT + (uw * 64) / BLK;  // (rows past N: table zero, dummy loads)
  const int64_t rblk = (int64_t)BLK * BLK * 3 / 4;
  const int64_t roff = (int64_t)((((cbw * 32) % BLK) / 32) * C::NS + ((uw * 64) % BLK) / 64) * 1536;
  const int rrp = rp_row[rbtw] - 1;
  const uint32_t dstRlo = (uint32_t)(C::R_OFF + cbw * kFp6Frag + fp6_lo_offset(uw, lane));
  const uint32_t dstRhi = (uint32_t)(C::R_OFF + cbw * kFp6Frag + fp6_hi_offset(uw, lane));
  int tabS, baseS;
  uint32_t slotS;
  {
    // residual scale slot tid: channel r = tid / NBC, block column c = tid % NBC
    const int r = min(tid / C::NBC, TBN - 1), c = tid % C::NBC;
    const int64_t n = min(n0 + r, a.N - 1);
    const int rb = (int)(n / BLK) - nt0;
    tabS = tid < C::NSRS ? rb * KT + c : -1;
    baseS = ((rp_row[rb] - 1) * BLK + (int)(n - (int64_t)(nt0 + rb) * BLK)) * 2;
    slotS = (uint32_t)(C::SR_OFF + (((r >> 5) * C::NBC + c) * 32 + (r & 31)) * 8);
  }
  // scale of this lane for group 0 and the step to the next group: waves 0-3
  // token m0 + tid's sa, waves 4-7 channel n0 + tid - 256's sw (past the
  // end: the last one), group-major when the caller gives saT / swT (one
  // contiguous run per group), else [M][G] / [N][G]
  const int64_t msc = wave < 4 ? min(m0 + tid, (a.saT ? a.saT_ld : a.M) - 1) : 0;
  const int64_t nsc = min(n0 + min(tid - 256, TBN - 1), a.N - 1);
  const uint8_t* scb = wave < 4 ? (a.saT ? reinterpret_cast<const uint8_t*>(a.saT) + msc * 4
                                         : reinterpret_cast<const uint8_t*>(a.sa) + msc * G * 4)
                                : (a.swT ? reinterpret_cast<const uint8_t*>(a.swT) + nsc * 2
                                         : reinterpret_cast<const uint8_t*>(a.sw) + nsc * G * 2);
  const int64_t sc_step = wave < 4 ? (a.saT ? a.saT_ld * 4 : 4) : (a.swT ? a.N * 2 : 2);

  auto load = [&](Stage6& S, int j) {
    j = min(j, je - 1);
    if (WRAW) S.W = *reinterpret_cast<const v4i*>(srcW + (int64_t)j * 1024);
    if (wave < 4) {
      S.sc = *reinterpret_cast<const uint32_t*>(scb + j * sc_step);
    } else {
      S.sc = *reinterpret_cast<const uint16_t*>(scb + j * sc_step);
    }
    // residual pieces and row scales: loaded in every step, from offset 0 of
    // a valid buffer where no block is selected, so the DMA wait is exact
    const int entR = (int)tab[tabR + j * C::NBC];
    const int entS = (int)tab[max(tabS, 0) + j * C::NBC];
    const uint8_t* rp = rbase + (entR > 0 ? (int64_t)(rrp + entR) * rblk + roff : 0);
    S.Rlo = *reinterpret_cast<const v4i*>(rp + lane * 16);
    S.Rhi = *reinterpret_cast<const u32x2*>(rp + 1024 + lane * 8);
    const int es = tabS >= 0 ? entS : 0;
    S.sr = *reinterpret_cast<const uint16_t*>(sbase + (uint32_t)(es > 0 ? es * (BLK * 2) + baseS : 0));
  };

  auto store = [&](uint32_t st, const Stage6& S, int j) {
    if (WRAW) {
      const uint32_t w[4] = {(uint32_t)S.W[0], (uint32_t)S.W[1], (uint32_t)S.W[2], (uint32_t)S.W[3]};
      uint32_t d[6];
      fp6_fields32(w, d);
      v4i lo;
      lo[0] = (int)d[0];
      lo[1] = (int)d[1];
      lo[2] = (int)d[2];
      lo[3] = (int)d[3];
      lds_st16(st + dstWlo, lo);
      lds_st8(st + dstWhi, d[4], d[5]);
    }
    if (wave < 4) {
      // activation scale * 64 (the fields' 1/8 on both operands): (hi, lo, hi, lo)
      const float s = (m0 + tid < a.M) ? __uint_as_float(S.sc) * 64.0f : 0.f;
      const uint32_t p = split_bf16(s);
      lds_st8(st + C::SA_OFF + (uint32_t)tid * 8, p, p);
    } else if (wave < 6) {
      // weight scale: (hi, hi, lo, lo)
      const uint32_t p = split_bf16(h2f((uint16_t)S.sc));
      const uint32_t hi = p & 0xFFFFu, lo = p >> 16;
      lds_st8(st + C::SW_OFF + (uint32_t)(tid - 256) * 8, hi | (hi << 16), lo | (lo << 16));
    }
    if (anyr[j]) {
      lds_st16(st + dstRlo, S.Rlo);
      lds_st8(st + dstRhi, S.Rhi[0], S.Rhi[1]);
      if (tid < C::NSRS) {
        const uint32_t p = split_bf16(h2f((uint16_t)S.sr));
        const uint32_t hi = p & 0xFFFFu, lo = p >> 16;
        lds_st8(st + slotS, hi | (hi << 16), lo | (lo << 16));
      }
    }
  };

  const int wm = wave & 3, wn = wave >> 2;
  float y[2][2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int e = 0; e < 16; ++e) y[i][q][e] = 0.f;
  const v16f zero16 = {};

  auto epi = [](float (&yt)[16], const v16f& S, const v16f& d) {
#pragma unroll
    for (int e = 0; e < 16; ++e) yt[e] = fmaf(S[e], d[e], yt[e]);
  };

  // residual-table lookups of this wave for group j: lane q*NBC + c holds
  // the entry of the wave's column block q, block column c (0 = none)
  const int tq = min(lane / C::NBC, 1), tc = lane % C::NBC;
  const int tnt = (int)((n0 + (wn * 2 + tq) * 32) / BLK);
  const bool tvalid = lane < 2 * C::NBC && tnt < nrows_b;
  const int tidx = tvalid ? (tnt - nt0) * KT + tc : 0;
  const uint32_t zaddr = lds_addr(smem) + C::ZERO_OFF;

  auto compute = [&](uint32_t st, int j) {
    // lane bases of the wave's row / column blocks (and of its residual
    // column blocks), recomputed from opaque copies in every step so that
    // only compile-time constants remain in the fragment addresses
    uint32_t la = st + C::A_OFF + (uint32_t)wm * (2 * kFp6Frag) + (uint32_t)lane * 16u;
    uint32_t ha = st + C::A_OFF + (uint32_t)wm * (2 * kFp6Frag) + 2048u + (uint32_t)lane * 8u;
    uint32_t lb = st + C::B_OFF + (uint32_t)wn * (2 * kFp6Frag) + (uint32_t)lane * 16u;
    uint32_t hb = st + C::B_OFF + (uint32_t)wn * (2 * kFp6Frag) + 2048u + (uint32_t)lane * 8u;
    uint32_t sa_b = lane < 32 ? st + C::SA_OFF + (uint32_t)lane * 8u + (uint32_t)wm * 512u : zaddr;
    uint32_t sw_b = lane < 32 ? st + C::SW_OFF + (uint32_t)lane * 8u + (uint32_t)wn * 512u : zaddr;
    const uint32_t sstep = lane < 32 ? 256u : 0u;
    asm volatile("" : "+v"(la), "+v"(ha), "+v"(lb), "+v"(hb), "+v"(sa_b), "+v"(sw_b));
    int ent_raw = (int)tab[tidx + j * C::NBC];
    v8i B[2][2], A[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int u = 0; u < 2; ++u) B[cb][u] = frag6(lb + cb * kFp6Frag + u * 1024, hb + cb * kFp6Frag + u * 512);
    const v4s sa0 = lds_ld8(sa_b), sw0 = lds_ld8(sw_b);
    const v4s sw1 = lds_ld8(sw_b + sstep), sa1 = lds_ld8(sa_b + sstep);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int u = 0; u < 2; ++u) A[u] = frag6(la + rb * kFp6Frag + u * 1024, ha + rb * kFp6Frag + u * 512);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const v16f S = mfma_scale(rb ? sa1 : sa0, cb ? sw1 : sw0);
        v16f d = mfma6(A[0], B[cb][0], zero16);
        d = mfma6(A[1], B[cb][1], d);
        epi(y[rb][cb], S, d);
        if (DUMP) {
          const int64_t n = n0 + (wn * 2 + cb) * 32 + (lane & 31);
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int64_t m = m0 + (wm * 2 + rb) * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
            if (m < a.M && n < a.N) a.acc_dump[(m * a.N + n) * G + j] = (int)(d[e] * 64.0f);
          }
        }
      }
    }

    // zipper: residual blocks of the wave's column blocks in group j, against
    // the same activation images
    asm volatile("" : "+v"(ent_raw));
    const int ent_l = tvalid ? ent_raw : 0;
    const uint64_t pres = __builtin_amdgcn_ballot_w64(ent_l > 0);
    if (pres) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        if (!((pres >> (q * C::NBC)) & ((1u << C::NBC) - 1u))) continue;
        const int cbg = wn * 2 + q;
        const int nt = (int)((n0 + cbg * 32) / BLK);
        const int rb_t = nt - nt0;
#pragma unroll
        for (int c = 0; c < C::NBC; ++c) {
          if (!((pres >> (q * C::NBC + c)) & 1u)) continue;
          // (rare path: the residual bases are formed here)
          const uint32_t lr = st + C::R_OFF + (uint32_t)cbg * kFp6Frag + (uint32_t)lane * 16u;
          const uint32_t hr = st + C::R_OFF + (uint32_t)cbg * kFp6Frag + 2048u + (uint32_t)lane * 8u;
          v8i Rf[C::NS];
#pragma unroll
          for (int s = 0; s < C::NS; ++s) Rf[s] = frag6(lr + (c * C::NS + s) * 1024, hr + (c * C::NS + s) * 512);
          const uint32_t sr_a = lane < 32 ? st + C::SR_OFF + (uint32_t)((cbg * C::NBC + c) * 256 + lane * 8) : zaddr;
          const v4s srq = lds_ld8(sr_a);
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            v16f d = zero16;
#pragma unroll
            for (int s = 0; s < C::NS; ++s)
              d = mfma6(frag6(la + rb * kFp6Frag + (c * C::NS + s) * 1024, ha + rb * kFp6Frag + (c * C::NS + s) * 512),
                        Rf[s], d);
            const v16f SR = mfma_scale(rb ? sa1 : sa0, srq);
            epi(y[rb][q], SR, d);
            if (DUMP) {
              const int ent = __builtin_amdgcn_readlane(ent_l, q * C::NBC + c);
              const int64_t e_g = rp_row[rb_t] + ent - 1;
              const int rr = (int)(n0 + cbg * 32 + (lane & 31) - (int64_t)nt * BLK);
#pragma unroll
              for (int e = 0; e < 16; ++e) {
                const int64_t m = m0 + (wm * 2 + rb) * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                if (m < a.M) a.acc_dump[a.M * a.N * G + (e_g * a.M + m) * BLK + rr] = (int)(d[e] * 64.0f);
              }
            }
          }
        }
      }
    }
  };

  // Two LDS stages, one barrier per group; register buffers R0/R1 hold the
  // scales and residual pieces of groups j+2 and j+3 in flight.
  const uint32_t st0 = lds_addr(smem);
  const uint32_t st1 = st0 + C::STAGE;
  Stage6 R0, R1;
  dma(st0, jb);
  load(R0, jb);
  load(R1, jb + 1);
  store(st0, R0, jb);
  load(R0, jb + 2);
  dma_wait();
  lds_barrier();
  // Each step first stores the next group's register-staged pieces (their
  // loads were issued two steps earlier and no DMA is in flight), then
  // issues the next group's DMA, then computes: a store after the DMA would
  // make the compiler wait for every outstanding load (vmcnt(0)) before its
  // LDS writes, the DMA included, exposing its whole latency in every step.
  int j = jb;
  for (; j + 1 < je; j += 2) {
    store(st1, R1, min(j + 1, je - 1));
    dma(st1, j + 1);
    compute(st0, j);
    load(R1, j + 3);
    dma_wait();
    lds_barrier();
    store(st0, R0, min(j + 2, je - 1));
    dma(st0, j + 2);
    compute(st1, j + 1);
    load(R0, j + 4);
    dma_wait();
    lds_barrier();
  }
  if (j < je) compute(st0, j);  // odd group count: the last group

  // ---- output ----
  // fp16 output in 4-byte stores: lanes 2i and 2i+1 hold channels n and n+1
  // of the same rows, and of each row pair (e, e+1) they swap one value (a
  // DPP move within lane pairs), so the even lane writes row e at (n, n+1)
  // and the odd lane row e+1 at (n-1, n).  Every such store is aligned (y
  // 16-byte aligned, ldy a multiple of 8) and n < N implies n+1 < N (N is a
  // multiple of 32).
  const bool odd = lane & 1;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int64_t n = n0 + (wn * 2 + cb) * 32 + (lane & 31);
      if (split >= 0) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t m = m0 + (wm * 2 + rb) * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          if (m < a.M && n < a.N) a.part[((int64_t)split * a.M + m) * a.N + n] = y[rb][cb][e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          const float v0 = y[rb][cb][e], v1 = y[rb][cb][e + 1];
          // quad_perm (1, 0, 3, 2): each lane reads its pair partner
          const float r = __int_as_float(
              __builtin_amdgcn_update_dpp(0, __float_as_int(odd ? v0 : v1), 0xB1, 0xF, 0xF, false));
          const int64_t m = m0 + (wm * 2 + rb) * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3) + (odd ? 1 : 0);
          const uint32_t lo = f2h_bits(odd ? r : v0), hi = f2h_bits(odd ? v1 : r);
          if (m < a.M && n < a.N)
            *reinterpret_cast<uint32_t*>(a.y + m * a.ldy + (n & ~(int64_t)1)) = lo | (hi << 16);
        }
      }
    }
}

// Split-K reduce over the split tiles only: y = fp16(sum of the splits' fp32
// partials, in split order).  32 workgroups per tile, four consecutive
// outputs per thread (N is a multiple of 32): 16-byte partial loads, one
// 8-byte store.
__global__ __launch_bounds__(256) void split_reduce6_kernel(const float* __restrict__ part, int ksplit, int64_t M,
                                                            int64_t N, uint16_t* y, int64_t ldy, int full) {
  const int tiles_n = (int)((N + TBN - 1) / TBN), tiles_m = (int)((M + TBM - 1) / TBM);
  int64_t m0, n0;
  tile6_origin(full + (int)(blockIdx.x / 32), tiles_m, tiles_n, m0, n0);
  const int e = ((int)(blockIdx.x % 32) * 256 + (int)threadIdx.x) * 4;  // < TBM * TBN
  const int64_t m = m0 + e / TBN, n = n0 + e % TBN;
  if (m >= M || n >= N) return;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k = 0; k < ksplit; ++k) {
    const float4 v = *reinterpret_cast<const float4*>(part + ((int64_t)k * M + m) * N + n);
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  const uint32_t lo = (uint32_t)f2h_bits(s.x) | ((uint32_t)f2h_bits(s.y) << 16);
  const uint32_t hi = (uint32_t)f2h_bits(s.z) | ((uint32_t)f2h_bits(s.w) << 16);
  *reinterpret_cast<uint2*>(y + m * ldy + n) = make_uint2(lo, hi);
}

template <int BLK, bool DUMP, bool WRAW>
hipError_t launch_tile6_cfg(const GemmArgs& a, hipStream_t st) {
  using C = Tile6Cfg<BLK>;
  const size_t lds = C::lds(a.K);
  auto kern = gemm_tile6_kernel<BLK, DUMP, WRAW>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t tiles = ((a.M + TBM - 1) / TBM) * ((a.N + TBN - 1) / TBN);
  GemmArgs b = a;
  b.split_tail = a.ksplit > 1 ? (int)tile6_gemm_tail(a.M, a.N, a.K, a.ksplit) : 0;
  if (b.ksplit > 1 && b.part == nullptr) return hipErrorInvalidValue;
  const int64_t full = tiles - b.split_tail;
  hipLaunchKernelGGL(kern, dim3((unsigned)(full + (int64_t)b.split_tail * b.ksplit)), dim3(NTHR), lds, st, b);
  e = hipGetLastError();
  if (e != hipSuccess || b.ksplit == 1) return e;
  hipLaunchKernelGGL(split_reduce6_kernel, dim3((unsigned)(b.split_tail * 32)), dim3(256), 0, st, b.part, b.ksplit,
                     b.M, b.N, b.y, b.ldy, (int)full);
  return hipGetLastError();
}

}  // namespace

// Work plan of the fp6 route: K splits and how many tiles take them.  The
// estimate counts rounds of one 512-thread workgroup per CU times groups per
// workgroup (about 1.4 us per group) plus the split tiles' fp32 partials'
// round trip through HBM (written once, read once, at about 5 TB/s).  With
// `tail` split tiles the other tiles fill whole rounds first (full is a
// multiple of the CU count) and the split units share what is left.  Plain
// split-K (every tile split) is the tail = tiles case.
namespace {
constexpr int64_t kPlanCUs = 256;

double tile6_estimate(int64_t M, int64_t N, int64_t tiles, int64_t G, int ks, int64_t tail) {
  constexpr double kGroupSec = 1.4e-6, kHbm = 5.0e12;
  if (ks == 1) return (double)((tiles + kPlanCUs - 1) / kPlanCUs) * (double)G * kGroupSec;
  const int64_t full = tiles - tail, gs = (G + ks - 1) / ks;
  const double groups = (double)(full / kPlanCUs * G) + (double)((tail * ks + kPlanCUs - 1) / kPlanCUs * gs);
  const double outs = std::min((double)tail * TBM * TBN, (double)M * (double)N);
  return groups * kGroupSec + (double)(ks + 1) * outs * 4.0 / kHbm;
}

// The best tail for ks splits: every tile, or all but whole rounds of tiles.
int64_t tile6_best_tail(int64_t M, int64_t N, int64_t tiles, int64_t G, int ks, double* est) {
  int64_t bt = tiles;
  double best = tile6_estimate(M, N, tiles, G, ks, tiles);
  for (int64_t full = kPlanCUs; full < tiles; full += kPlanCUs) {
    const double t = tile6_estimate(M, N, tiles, G, ks, tiles - full);
    if (t < best) {
      best = t;
      bt = tiles - full;
    }
  }
  if (est) *est = best;
  return bt;
}
}  // namespace

// The fewest splits within 3% of the best estimate, at least 8 groups per
// split (Qwen3-32B 25600 x 5120 at M = 4096: 640 tiles, 2.5 rounds -> 512
// tiles over all of K in two rounds, the last 128 split two ways).
int tile6_gemm_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ((M + TBM - 1) / TBM) * ((N + TBN - 1) / TBN);
  const int64_t G = K / kGroup;
  double best = 0.0;
  int bk = 1;
  for (int ks = 1; ks <= 8 && (ks == 1 || G / ks >= 8); ++ks) {
    double t = 0.0;
    if (ks == 1)
      t = tile6_estimate(M, N, tiles, G, 1, 0);
    else
      tile6_best_tail(M, N, tiles, G, ks, &t);
    if (ks == 1 || t < best * 0.97) {
      best = t;
      bk = ks;
    }
  }
  return bk;
}

// Tiles split ks ways under the plan above (the last ones in the banded
// order); 0 for ks = 1.
int64_t tile6_gemm_tail(int64_t M, int64_t N, int64_t K, int ks) {
  if (ks <= 1) return 0;
  const int64_t tiles = ((M + TBM - 1) / TBM) * ((N + TBN - 1) / TBN);
  return tile6_best_tail(M, N, tiles, K / kGroup, ks, nullptr);
}

// The fp6 route covers blocks of 64 and 128 (a block of 32 is half a 64-code
// slice, whose other half would belong to another block) and K whose
// residual table fits in LDS.
bool tile6_gemm_fits(const GemmArgs& a) {
  if (a.block != 64 && a.block != 128) return false;
  if (a.M <= 32 || a.N % 32 != 0) return false;
  const int64_t lim = (int64_t)1 << 32;
  if (a.M * a.K >= lim || a.N * a.K >= lim || (int64_t)a.n_select * a.block * a.block >= lim) return false;
  return a.block == 64 ? Tile6Cfg<64>::lds(a.K) <= kMaxLds : Tile6Cfg<128>::lds(a.K) <= kMaxLds;
}

hipError_t launch_tile6_gemm(const GemmArgs& a, hipStream_t st) {
  const bool d = a.acc_dump != nullptr;
  if (a.wimg == nullptr) {  // base codes from the packed slabs
    if (a.block == 64) return d ? launch_tile6_cfg<64, true, true>(a, st) : launch_tile6_cfg<64, false, true>(a, st);
    return d ? launch_tile6_cfg<128, true, true>(a, st) : launch_tile6_cfg<128, false, true>(a, st);
  }
  if (a.block == 64) return d ? launch_tile6_cfg<64, true, false>(a, st) : launch_tile6_cfg<64, false, false>(a, st);
  return d ? launch_tile6_cfg<128, true, false>(a, st) : launch_tile6_cfg<128, false, false>(a, st);
}

}  // namespace mq
