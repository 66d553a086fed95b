// ZipperEngine fused layer for large M (prefill): LDS-tiled int8-MFMA GEMM.
// MosaicQuant technical summary (gist.science/pt/paper/2606.15652),
// Metodologia 3: one kernel runs the dense 4-bit GEMM, the sparse residual
// compensation and the scale/reduce-sum epilogue, the residual reusing the
// activation tile of the dense product.
//
// Tile: 256 tokens x 128 output channels per workgroup of eight waves (4 x 2,
// 64 x 64 each, four 32 x 32 sub-tiles per wave).  One K step is one
// 128-channel group, four V_MFMA_I32_32X32X32_I8 per sub-tile.  Per group
// the workgroup stages, through a register buffer into LDS:
//   A   activation codes, 256 rows x 64 bytes
//   B   weight codes,     128 rows x 64 bytes
//   R   residual codes of the block columns selected in these 128 channels,
//       128 rows x 64 bytes (only when the tile has a selected block in the
//       group; rows of unselected blocks hold unused data)
//   the scale operands (below).
// Codes are widened to int8 once, while being written to LDS (byte = 16*q,
// so every accumulator is 256 x the exact integer sum), and LDS holds each
// MFMA operand fragment in lane order (1 KB per fragment, lane l's 16 bytes
// at 16*l), so every operand read is one conflict-free 16-byte read.
//
// Operand layout of a 32 x 32 x 32 step t (channels 32t .. 32t+31 of the
// group): lane l holds row (token, or output channel) l % 32 and the 16
// codes 32t + 16*(l/32) .. +15, i.e. 8 packed bytes; both operands use the
// same layout, so the products pair up whatever order the instruction
// gives the 16 bytes.  A residual block (edge 32, 64 or 128, inside one
// group at a multiple of 32) covers whole steps: its MFMAs take the
// activation fragments of exactly those steps.
//
// Scale products on the matrix core: the epilogue needs, per element and
// group, S = sa[m] * sw[n] (fp32).  One V_MFMA_F32_32X32X8_BF16 forms a
// whole 32 x 32 tile of them: lanes 0-31 hold (sa_hi, sa_lo, sa_hi, sa_lo)
// for their row and (sw_hi, sw_hi, sw_lo, sw_lo) for their column, lanes
// 32-63 zeros, where x_hi = bf16(x) and x_lo = bf16(x - x_hi), so the
// product is (sa_hi + sa_lo)(sw_hi + sw_lo): sw exactly (an fp16 value is
// the sum of two bf16), sa to within 2^-16 relative.  The vector unit then
// does two operations per element and group, y += S * float(acc), where it
// would otherwise need three; a 32 x 32 product costs one instruction of 32
// cycles against 128 cycles of int8 MFMAs per sub-tile and group.  The
// factor 1/256 of the widened codes is folded into sa_hi/sa_lo.  The same
// instruction with the residual row scales forms the residual's products.
//
// Pipeline: group g passes through register buffer g%2 and LDS stage g%2.
// While the waves compute group j from LDS, the loads of groups j+1 and j+2
// are in flight.  Every step issues the same loads (activation DMA,
// weight codes and scales, residual codes and row scales, the last from a
// dummy offset where no block is selected; groups past the end re-read the
// last group), so the hardware load counters are waited on exactly.  Within a group a wave runs its four sub-tiles one
// after the other (scale product and int8 MFMAs, then the epilogue); the
// two waves of each SIMD overlap one's MFMAs with the other's epilogue.
#include "gemm_common.h"

namespace mq {
namespace {

typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));

constexpr int TBM = 256;    // tokens per tile
constexpr int TBN = 128;    // output channels per tile
constexpr int NTHR = 512;   // eight waves: 4 (tokens) x 2 (channels), 64 x 64 each
constexpr size_t kMaxLds = 160 * 1024;

template <int BLK>
struct TileCfg {
  static constexpr int NBR = TBN / BLK;      // block rows in a tile
  static constexpr int NBC = kGroup / BLK;   // block columns in a group
  static constexpr int NSRS = TBN * NBC;     // residual-scale slots (<= NTHR)
  static constexpr int OPA = 8 * 4 * 1024;   // widened activation fragments: 8 row blocks x 4 steps
  static constexpr int OPB = 4 * 4 * 1024;   // widened weight / residual fragments: 4 column blocks x 4 steps
  static constexpr int A_OFF = 0;
  static constexpr int B_OFF = OPA;
  static constexpr int R_OFF = OPA + OPB;
  static constexpr int SA_OFF = OPA + 2 * OPB;    // [8 row blocks][32 lanes] x 8 bytes
  static constexpr int SW_OFF = SA_OFF + 8 * 256;  // [4 column blocks][32 lanes] x 8 bytes
  static constexpr int SR_OFF = SW_OFF + 4 * 256;  // [4 column blocks][NBC][32 lanes] x 8 bytes
  static constexpr int STAGE = SR_OFF + 4 * NBC * 256;
  static constexpr int ZERO_OFF = 2 * STAGE;       // 16 zero bytes (lanes 32-63 of the scale operands)
  static constexpr int TAB_OFF = ZERO_OFF + 16;
  static size_t lds(int64_t K) {
    return (size_t)TAB_OFF + (size_t)NBR * (size_t)(K / BLK) * 2 + (size_t)(K / kGroup);
  }
};

// Register buffer of one group.  Residual pieces and scales of blocks that
// are not selected are loaded from offset 0 of a valid buffer; compute reads
// the residual operand and scale of a block column only when the block is
// selected, so that data is never used and needs no mask.
struct Stage {
  uint4 A[2], B, R;
  uint32_t sc;  // activation scale bits (waves 0-3) or weight scale bits (waves 4-5)
  uint32_t sr;  // residual row scale bits
};

// LDS access through 32-bit LDS addresses, so that constant offsets fold
// into the instructions' offset fields.
typedef __attribute__((address_space(3))) v4i lds_v4i;
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x2 lds_u2;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ v4i lds_ld16(uint32_t a) { return *(const lds_v4i*)(uintptr_t)a; }
__device__ __forceinline__ v4s lds_ld8(uint32_t a) { return *(const lds_v4s*)(uintptr_t)a; }
__device__ __forceinline__ void lds_st16(uint32_t a, v4i v) { *(lds_v4i*)(uintptr_t)a = v; }
__device__ __forceinline__ void lds_st8(uint32_t a, uint32_t lo, uint32_t hi) {
  const u32x2 v = {lo, hi};
  *(lds_u2*)(uintptr_t)a = v;
}

// Workgroup barrier for the K loop's LDS hand-over: this wave's LDS writes
// complete (lgkmcnt), then s_barrier.  Unlike __syncthreads it does not
// wait for the wave's outstanding global loads (a release fence waits
// vmcnt(0)), so the register buffers' loads for later groups stay in
// flight across it; the "memory" clobber keeps the compiler from moving LDS
// accesses across it.  LDS DMA into a stage is waited for separately
// (vmcnt) before this barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ v16i mfma32(v4i a, v4i b, v16i c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v16f mfma_scale(v4s a, v4s b) {
  const v16f z = {};
  return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a, b, z, 0, 0, 0);
}

// bf16 bits of x, round to nearest even (NaN stays NaN, overflow -> inf).
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_value(uint32_t b) { return __uint_as_float(b << 16); }

// (hi, lo) bf16 pair with hi + lo = x to within 2^-16 relative (exactly
// for an fp16 x).
__device__ __forceinline__ uint32_t split_bf16(float x) {
  const uint32_t hi = bf16_bits(x);
  const uint32_t lo = bf16_bits(x - bf16_value(hi));
  return hi | (lo << 16);
}

template <int BLK, bool DUMP, bool AW>
__global__ __launch_bounds__(NTHR, 1) void gemm_tile_kernel(GemmArgs a) {
  using C = TileCfg<BLK>;
  extern __shared__ __align__(16) unsigned char smem[];
  const int G = (int)(a.K / kGroup);
  const int KT = (int)(a.K / BLK);
  uint16_t* tab = reinterpret_cast<uint16_t*>(smem + C::TAB_OFF);  // [NBR][KT]: entry-rp+1, 0 = none
  uint8_t* anyr = smem + C::TAB_OFF + C::NBR * KT * 2;              // [G]: a selected block in group j
  __shared__ int rp_row[C::NBR];

  const int tid = threadIdx.x;
  // (& 7 makes the range known, so LDS offsets fold into the instructions)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & 7;
  const int lane = tid & 63;
  const int r16 = lane & 15;
  const int ch = lane >> 4;

  // XCD-aware order: consecutive work items (same K split, neighbouring
  // tiles in the banded order below) go to the same XCD so its L2 serves
  // the rows and weight tiles they share.  With split-K, work item =
  // split * tiles + tile.
  const int tiles_n = (int)((a.N + TBN - 1) / TBN);
  const int items = (int)gridDim.x;
  const int tiles = items / a.ksplit;
  const int xcd = blockIdx.x % 8;
  const int per = items / 8, rem = items % 8;
  const int item = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + blockIdx.x / 8;
  const int split = item / tiles;
  const int tile = item - split * tiles;
  const int jb = (int)((int64_t)split * G / a.ksplit);        // this split's groups
  const int je = (int)((int64_t)(split + 1) * G / a.ksplit);  // [jb, je)
  // Bands of kBand token tiles: consecutive tiles walk down a band's token
  // tiles for one channel tile, then move to the next channel tile, so the
  // workgroups an XCD runs together share weight tiles as well as token rows.
  constexpr int kBand = 4;
  const int tiles_m = tiles / tiles_n;
  const int band = tile / (kBand * tiles_n);
  const int bh = min(kBand, tiles_m - band * kBand);
  const int rb = tile - band * kBand * tiles_n;
  const int64_t m0 = (int64_t)(band * kBand + rb % bh) * TBM;
  const int64_t n0 = (int64_t)(rb / bh) * TBN;
  const int64_t Kh = a.K / 2;
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

  // ---- staging: global -> registers (fixed load count for A, B, scales) ----
  // Lane l of wave w handles row l%16 of a 16-row slab and 16-byte piece
  // l/16 (k step t = l/16), so the 16 lanes of a piece write 256 consecutive
  // LDS bytes.  A: slabs w and w + 8 (rows 16w + r16 and 128 + 16w + r16);
  // B and R: slab w of the tile's channels (weight codes in the slab layout:
  // 1 KB per group, lane l's bytes at 16*l).  Per-thread offsets are fixed
  // for the whole K loop; each group adds a uniform step to a uniform base
  // (32-bit offsets: the host routes operands of 4 GiB or more to the
  // streaming kernel).
  const uint8_t* rbase = a.n_select > 0 ? a.qr : a.qw;
  const uint8_t* sbase = a.n_select > 0 ? reinterpret_cast<const uint8_t*>(a.sr)
                                        : reinterpret_cast<const uint8_t*>(a.sw);
  uint32_t offA[2], slotA[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 16 * (wave + 8 * i) + r16;  // token row in the tile
    offA[i] = (uint32_t)(min(m0 + r, a.M - 1) * Kh + ch * 16);
    slotA[i] = (uint32_t)((((r >> 5) * 4 + ch) * 64 + (r & 31)) * 16);
  }
  const int rw = 16 * wave + r16;  // channel row in the tile
  const int64_t nw = min(n0 + rw, a.N - 1);
  const int64_t slab = min(n0 / 16 + wave, a.N / 16 - 1);
  const uint32_t offB = (uint32_t)(slab * 16 * Kh + lane * 16);
  const uint32_t slotB = (uint32_t)((((rw >> 5) * 4 + ch) * 64 + (rw & 31)) * 16);
  const int rbw = (int)(nw / BLK) - nt0;
  const int tabR = rbw * KT + (ch * 32) / BLK;
  const int baseR = (rp_row[rbw] - 1) * (BLK * BLK / 2) + (int)(nw - (int64_t)(nt0 + rbw) * BLK) * (BLK / 2) +
                    ((ch * 32) % BLK) / 2;
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
  const uint32_t offS = wave < 4 ? (uint32_t)(min(m0 + tid, a.M - 1) * G * 4)
                                 : (uint32_t)(min(n0 + min(tid - 256, TBN - 1), a.N - 1) * G * 2);

  auto load = [&](Stage& S, int j) {
    j = min(j, je - 1);
    if constexpr (!AW) {
      const uint8_t* qa_j = a.qa + j * 64;
      S.A[0] = ld16(qa_j + offA[0]);
      S.A[1] = ld16(qa_j + offA[1]);
    }
    S.B = ld16(a.qw + j * 1024 + offB);
    if (wave < 4) {
      S.sc = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(a.sa) + j * 4 + offS);
    } else {
      S.sc = *reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(a.sw) + j * 2 + offS);
    }
    // residual codes and row scales: loaded in every step, from offset 0
    // of a valid buffer where no block is selected (tab is zero-filled), so
    // every step issues the same loads and the DMA wait below is exact
    const int entR = (int)tab[tabR + j * C::NBC];
    const int entS = (int)tab[max(tabS, 0) + j * C::NBC];
    S.R = ld16(rbase + (uint32_t)(entR > 0 ? entR * (BLK * BLK / 2) + baseR : 0));
    const int es = tabS >= 0 ? entS : 0;
    S.sr = *reinterpret_cast<const uint16_t*>(sbase + (uint32_t)(es > 0 ? es * (BLK * 2) + baseS : 0));
  };

  // registers -> LDS stage, in four parts: widened operands in lane order,
  // scale operands as (hi, lo) bf16 pairs in the scale-MFMA lane order
  auto store_part = [&](uint32_t st, const Stage& S, int j, int part) {
    if (part < 2) {
      if constexpr (AW) return;  // (the activation fragments arrive by DMA)
      const uint32_t b = st + C::A_OFF + slotA[part];
      lds_st16(b, widen8(S.A[part].x, S.A[part].y));
      lds_st16(b + 512, widen8(S.A[part].z, S.A[part].w));
    } else if (part == 2) {
      const uint32_t b = st + C::B_OFF + slotB;
      lds_st16(b, widen8(S.B.x, S.B.y));
      lds_st16(b + 512, widen8(S.B.z, S.B.w));
      if (wave < 4) {
        // activation scale / 256 (the widened codes' factor): (hi, lo, hi, lo)
        const float s = (m0 + tid < a.M) ? __uint_as_float(S.sc) * kInv256 : 0.f;
        const uint32_t p = split_bf16(s);
        lds_st8(st + C::SA_OFF + (uint32_t)tid * 8, p, p);
      } else if (wave < 6) {
        // weight scale: (hi, hi, lo, lo)
        const uint32_t p = split_bf16(h2f((uint16_t)S.sc));
        const uint32_t hi = p & 0xFFFFu, lo = p >> 16;
        lds_st8(st + C::SW_OFF + (uint32_t)(tid - 256) * 8, hi | (hi << 16), lo | (lo << 16));
      }
    } else if (anyr[j]) {
      const uint32_t b = st + C::R_OFF + slotB;
      lds_st16(b, widen8(S.R.x, S.R.y));
      lds_st16(b + 512, widen8(S.R.z, S.R.w));
      if (tid < C::NSRS) {
        const uint32_t p = split_bf16(h2f((uint16_t)S.sr));
        const uint32_t hi = p & 0xFFFFu, lo = p >> 16;
        lds_st8(st + slotS, hi | (hi << 16), lo | (lo << 16));
      }
    }
  };

  // Wave w computes the 64-token x 64-channel quarter (wm, wn) = (w % 4, w / 4)
  // of the tile.  The hardware places waves w and w + 4 of a workgroup on one
  // SIMD (measured with the hardware wave-id register), so every SIMD holds
  // one wave of each 64-channel half: residual blocks, whose work falls on
  // the waves of their own channels only, load all four SIMDs alike instead
  // of two of them twice.
  const int wm = wave & 3, wn = wave >> 2;
  float y[2][2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int e = 0; e < 16; ++e) y[i][q][e] = 0.f;
  const v16i zero16 = {};

  auto epi = [](float (&yt)[16], const v16f& S, const v16i& acc) {
#pragma unroll
    for (int e = 0; e < 16; ++e) yt[e] = fmaf(S[e], (float)acc[e], yt[e]);
  };

  // residual-table lookups of this wave for group j: lane q*NBC + c holds
  // the entry of column block q (32 channels), block column c (0 = not
  // selected)
  const int tq = min(lane / C::NBC, 1), tc = lane % C::NBC;
  const int tnt = (int)((n0 + (wn * 2 + tq) * 32) / BLK);
  const bool tvalid = lane < 2 * C::NBC && tnt < nrows_b;
  const int tidx = tvalid ? (tnt - nt0) * KT + tc : 0;
  const uint32_t zaddr = lds_addr(smem) + C::ZERO_OFF;

  auto compute = [&](uint32_t st, int j) {
    // Bases include the wave's row / column blocks and are recomputed from
    // an opaque copy in every step, so only compile-time constants remain
    // in the per-fragment LDS addresses and fold into the offsets.
    uint32_t la = st + C::A_OFF + (uint32_t)lane * 16u + (uint32_t)wm * 8192u;
    uint32_t lb = st + C::B_OFF + (uint32_t)lane * 16u + (uint32_t)wn * 8192u;
    // scale operands: lanes 0-31 read their row's / column's pair, lanes
    // 32-63 the zero slot
    uint32_t sa_b = lane < 32 ? st + C::SA_OFF + (uint32_t)lane * 8u + (uint32_t)wm * 512u : zaddr;
    uint32_t sw_b = lane < 32 ? st + C::SW_OFF + (uint32_t)lane * 8u + (uint32_t)wn * 512u : zaddr;
    const uint32_t sstep = lane < 32 ? 256u : 0u;
    asm volatile("" : "+v"(la), "+v"(lb), "+v"(sa_b), "+v"(sw_b));
    // its value is first used after the dense sub-tiles
    int ent_raw = (int)tab[tidx + j * C::NBC];
    // operands: the row block's activation fragments (one register set,
    // reloaded for the second row block once the first one's MFMAs have
    // been issued) and both column blocks' weight fragments
    v4i A[4], B0[4], B1[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) A[t] = lds_ld16(la + t * 1024);
#pragma unroll
    for (int t = 0; t < 4; ++t) B0[t] = lds_ld16(lb + t * 1024);
    const v4s sa0 = lds_ld8(sa_b), sw0 = lds_ld8(sw_b);
#pragma unroll
    for (int t = 0; t < 4; ++t) B1[t] = lds_ld16(lb + 4096 + t * 1024);
    const v4s sw1 = lds_ld8(sw_b + sstep);
    const v4s sa1 = lds_ld8(sa_b + sstep);

    // four sub-tiles (0,0), (0,1), (1,0), (1,1): per sub-tile the scale
    // product and the four int8 MFMAs, then its epilogue; the two waves of a
    // SIMD overlap one wave's MFMAs with the other's epilogue
    auto sub = [&](int s, const v4i (&Bc)[4], v4s sa, v4s sw) {
      const v16f S = mfma_scale(sa, sw);
      v16i acc = mfma32(A[0], Bc[0], zero16);
      acc = mfma32(A[1], Bc[1], acc);
      acc = mfma32(A[2], Bc[2], acc);
      acc = mfma32(A[3], Bc[3], acc);
      const int rb = s >> 1, cb = s & 1;
      epi(y[rb][cb], S, acc);
      if (DUMP) {
        const int64_t n = n0 + (wn * 2 + cb) * 32 + (lane & 31);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t m = m0 + (wm * 2 + rb) * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          if (m < a.M && n < a.N) a.acc_dump[(m * a.N + n) * G + j] = acc[e] >> 8;
        }
      }
    };
    sub(0, B0, sa0, sw0);
    sub(1, B1, sa0, sw1);
#pragma unroll
    for (int t = 0; t < 4; ++t) A[t] = lds_ld16(la + 4096 + t * 1024);
    sub(2, B0, sa1, sw0);
    sub(3, B1, sa1, sw1);

    // zipper: residual blocks of the wave's column blocks in group j, against
    // the same activation fragments (lane q*NBC + c of the ballot: column
    // block q, block column c)
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
          // (rare path: the residual addresses are formed here)
          constexpr int NS = BLK / 32;  // 32-channel steps of a block
          const uint32_t lr = st + C::R_OFF + (uint32_t)lane * 16u + (uint32_t)cbg * 4096u;
          v4i Rf[NS];
#pragma unroll
          for (int u = 0; u < NS; ++u) Rf[u] = lds_ld16(lr + (uint32_t)(c * NS + u) * 1024u);
          const uint32_t sr_a = lane < 32 ? st + C::SR_OFF + (uint32_t)((cbg * C::NBC + c) * 256 + lane * 8) : zaddr;
          const v4s srq = lds_ld8(sr_a);
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            v4i Ar[NS];  // the row block's activation fragments of the block's steps
#pragma unroll
            for (int u = 0; u < NS; ++u) Ar[u] = lds_ld16(la + (uint32_t)rb * 4096u + (uint32_t)(c * NS + u) * 1024u);
            v16i racc = mfma32(Ar[0], Rf[0], zero16);
#pragma unroll
            for (int u = 1; u < NS; ++u) racc = mfma32(Ar[u], Rf[u], racc);
            const v16f SR = mfma_scale(rb ? sa1 : sa0, srq);
            epi(y[rb][q], SR, racc);
            if (DUMP) {
              const int ent = __builtin_amdgcn_readlane(ent_l, q * C::NBC + c);
              const int64_t e_g = rp_row[rb_t] + ent - 1;
              const int rr = (int)(n0 + cbg * 32 + (lane & 31) - (int64_t)nt * BLK);
#pragma unroll
              for (int e = 0; e < 16; ++e) {
                const int64_t m = m0 + (wm * 2 + rb) * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                if (m < a.M) a.acc_dump[a.M * a.N * G + (e_g * a.M + m) * BLK + rr] = racc[e] >> 8;
              }
            }
          }
        }
      }
    }
  };

  // Wide activations (AW): wave w copies row block w of the tile, group j
  // (4 KB, four 1 KB step fragments) from memory straight into LDS stage st
  // (LDS DMA: lane l's 16 bytes land at the fragment base + 16*l, the lane
  // order the fragments are stored in).  Issued at the start of a step for
  // the next group, so the copy runs under the current group's MFMAs; a
  // wave waits for its own copies (vmcnt) before the barrier that ends the
  // step.  Row blocks past the last one of M re-read the last one.
  const int64_t nrb = wide_rows(a.M) / 32;
  const uint8_t* dma_src = AW ? a.qaw + min((int64_t)(m0 / 32 + wave), nrb - 1) * G * 4096 + lane * 16 : nullptr;
  auto dma = [&](uint32_t st, int j) {
    if constexpr (AW) {
      j = min(j, je - 1);
      typedef __attribute__((address_space(3))) void* lds_ptr;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        __builtin_amdgcn_global_load_lds(dma_src + (int64_t)j * 4096 + t * 1024,
                                         (lds_ptr)(uintptr_t)(st + C::A_OFF + (uint32_t)wave * 4096u + t * 1024),
                                         16, 0, 0);
    }
  };
  // after a step's loads: the step's DMA (issued before the step's four
  // register loads: weights, scale, residual codes, residual scale) has
  // completed
  auto dma_wait = [&]() {
    if constexpr (AW) {
      // the builtin rather than inline asm, so that the compiler's own wait
      // analysis knows every older load is done
      __builtin_amdgcn_s_waitcnt(kWaitVm4);
      asm volatile("" ::: "memory");
    }
  };

  // Two LDS stages: group j is computed from stage j%2 while the waves
  // write group j+1 into the other stage; one barrier per group.  Register
  // buffers R0/R1 hold groups j+2 and j+3 in flight.
  const uint32_t st0 = lds_addr(smem);
  const uint32_t st1 = st0 + C::STAGE;
  Stage R0, R1;
  R0.R = R1.R = make_uint4(0, 0, 0, 0);
  R0.sr = R1.sr = 0;
  dma(st0, jb);
  load(R0, jb);
  load(R1, jb + 1);
#pragma unroll
  for (int part = 0; part < 4; ++part) store_part(st0, R0, jb, part);
  load(R0, jb + 2);
  dma_wait();
  lds_barrier();
  // one exit only, so the accumulators need no copies on the back edge
  // Each step first stores the next group's register-staged operands (their
  // loads were issued two steps earlier and no DMA is in flight), then
  // issues the next group's activation DMA, then computes: a store after the
  // DMA would make the compiler wait for every outstanding load (vmcnt(0))
  // before its LDS writes, the DMA included, exposing its latency in every
  // step.
  int j = jb;
  for (; j + 1 < je; j += 2) {
#pragma unroll
    for (int part = 0; part < 4; ++part) store_part(st1, R1, min(j + 1, je - 1), part);  // group j+1
    dma(st1, j + 1);
    compute(st0, j);
    load(R1, j + 3);
    dma_wait();
    lds_barrier();
#pragma unroll
    for (int part = 0; part < 4; ++part) store_part(st0, R0, min(j + 2, je - 1), part);  // group j+2
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
  // multiple of the block edge, so of 32).
  const bool odd = lane & 1;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int64_t n = n0 + (wn * 2 + cb) * 32 + (lane & 31);
      if (a.part) {
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

// Split-K reduce: y = fp16(sum of the splits' fp32 partials, in split order),
// so the result does not depend on the order the workgroups ran in.
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ part, int ksplit,
                                                           int64_t M, int64_t N, uint16_t* y, int64_t ldy) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * N) return;
  const int64_t m = idx / N, n = idx - m * N;
  float s = 0.f;
  for (int k = 0; k < ksplit; ++k) s += part[((int64_t)k * M + m) * N + n];
  y[m * ldy + n] = f2h_bits(s);
}

template <int BLK, bool DUMP, bool AW>
hipError_t launch_tile_cfg(const GemmArgs& a, hipStream_t st) {
  using C = TileCfg<BLK>;
  const size_t lds = C::lds(a.K);
  auto kern = gemm_tile_kernel<BLK, DUMP, AW>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t tiles = ((a.M + TBM - 1) / TBM) * ((a.N + TBN - 1) / TBN);
  hipLaunchKernelGGL(kern, dim3((unsigned)(tiles * a.ksplit)), dim3(NTHR), lds, st, a);
  e = hipGetLastError();
  if (e != hipSuccess || a.ksplit == 1) return e;
  hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((a.M * a.N + 255) / 256)), dim3(256), 0, st,
                     a.part, a.ksplit, a.M, a.N, a.y, a.ldy);
  return hipGetLastError();
}

}  // namespace

// K splits: when the tiles alone leave CUs idle (one 512-thread workgroup
// per CU), split K so that tiles x splits fills at most one round, keeping
// at least 8 groups per split.
int tile_gemm_splits(int64_t M, int64_t N, int64_t K) {
  constexpr int64_t kCUs = 256;
  const int64_t tiles = ((M + TBM - 1) / TBM) * ((N + TBN - 1) / TBN);
  const int64_t G = K / kGroup;
  int64_t ks = kCUs / (tiles > 0 ? tiles : 1);
  ks = ks < 8 ? ks : 8;
  ks = ks < G / 8 ? ks : G / 8;
  return ks > 1 ? (int)ks : 1;
}

bool tile_gemm_fits(const GemmArgs& a) {
  const int64_t lim = (int64_t)1 << 32;
  const int64_t G = a.K / kGroup;
  if (a.M * (a.K / 2) >= lim || a.N * (a.K / 2) >= lim || a.M * G * 4 >= lim ||
      (int64_t)a.n_select * a.block * a.block / 2 >= ((int64_t)1 << 31))
    return false;
  switch (a.block) {
    case 32: return TileCfg<32>::lds(a.K) <= kMaxLds;
    case 64: return TileCfg<64>::lds(a.K) <= kMaxLds;
    default: return TileCfg<128>::lds(a.K) <= kMaxLds;
  }
}

namespace {

template <int BLK>
hipError_t launch_tile_blk(const GemmArgs& a, hipStream_t st) {
  const bool d = a.acc_dump != nullptr;
  if (a.qaw) return d ? launch_tile_cfg<BLK, true, true>(a, st) : launch_tile_cfg<BLK, false, true>(a, st);
  return d ? launch_tile_cfg<BLK, true, false>(a, st) : launch_tile_cfg<BLK, false, false>(a, st);
}

// Packed activation codes -> the wide fragment order: thread i writes the
// 16 bytes at i*16 of the wide array (row block, group, step, lane), read
// as 8 packed bytes of one token and widened.
__global__ __launch_bounds__(256) void widen_acts_kernel(const uint8_t* __restrict__ qa, int64_t M, int64_t K,
                                                         uint8_t* __restrict__ qaw, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t G = K / kGroup;
  const int l = (int)(i & 63);
  const int t = (int)((i >> 6) & 3);
  const int64_t jr = i >> 8;  // row block * G + group
  const int64_t rb = jr / G, j = jr - rb * G;
  const int64_t m = rb * 32 + (l & 31);
  v4i v = {0, 0, 0, 0};
  if (m < M) {
    const uint2 p = *reinterpret_cast<const uint2*>(qa + m * (K / 2) + j * 64 + t * 16 + (l >> 5) * 8);
    v = widen8(p.x, p.y);
  }
  *reinterpret_cast<v4i*>(qaw + i * 16) = v;
}

}  // namespace

hipError_t launch_widen_acts(const uint8_t* qa, int64_t M, int64_t K, uint8_t* qaw, hipStream_t st) {
  const int64_t total = wide_rows(M) * (K / kGroup) * 8;  // 16-byte pieces
  hipLaunchKernelGGL(widen_acts_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, qa, M, K, qaw,
                     total);
  return hipGetLastError();
}

hipError_t launch_tile_gemm(const GemmArgs& a, hipStream_t st) {
  switch (a.block) {
    case 32: return launch_tile_blk<32>(a, st);
    case 64: return launch_tile_blk<64>(a, st);
    default: return launch_tile_blk<128>(a, st);
  }
}

}  // namespace mq
