// ZipperEngine fused layer for large M (prefill): LDS-tiled int8-MFMA GEMM.
// MosaicQuant technical summary (gist.science/pt/paper/2606.15652),
// Metodologia 3: one kernel runs the dense 4-bit GEMM, the sparse residual
// compensation and the scale/reduce-sum epilogue, the residual reusing the
// activation tile of the dense product.
//
// Tile: 256 tokens x 128 output channels per workgroup of eight waves (4 x 2,
// 64 x 64 each, sixteen 16x16 MFMA tiles per wave).  One K step is one
// 128-channel group.  Per group the workgroup stages, through a register
// buffer into LDS:
//   A  activation codes, 256 rows x 64 bytes
//   B  weight codes,     128 rows x 64 bytes
//   R  residual codes of the block columns selected in these 128 channels,
//      128 rows x 64 bytes (rows of unselected blocks hold unused data)
//   the activation scales, weight scales and residual row scales.
// Codes are widened to int8 once, while being written to LDS, and LDS holds
// each MFMA operand in lane order (slot = (tile*2 + half)*64 + lane, 16
// bytes), so every operand read is one conflict-free 16-byte LDS read.  In
// staging, lane l of a wave handles row l%16 of a 16-row slab and 16-byte
// piece l/16, so the 16 lanes of a piece write 256 consecutive bytes.
//
// K layout inside a group: lane chunk c = lane/16 feeds the first MFMA with
// channels [16c, 16c+16) and the second with [64+16c, 64+16c+16).  A 64-wide
// residual block therefore lines up with exactly one of the two MFMAs, a
// 32-wide block with one MFMA on half of the lanes, a 128-wide block with
// both, and each block keeps its own accumulator and row scale.
//
// Epilogue: per 16x16 tile and group, y += (sa[m]*sw[n]) * acc[m][n] on the
// vector unit: one multiply, one int->float conversion and one FMA per
// element and group (the scales are staged in LDS as fp32; a lane reads the
// four token scales of its rows as one 16-byte read).  Measured on this
// part, the multiply costs less issue time than forming the tile's outer
// product of scales on the matrix core.  The factor 256 carried by the
// widened codes is removed once, at the final store.
//
// Pipeline: group g passes through register buffer g%2 and LDS stage g%2.
// While the waves compute group j from LDS, the loads of groups j+1 and j+2
// are in flight; each group's loads have about two compute steps to arrive.
// Every step issues the same loads (groups past the end re-read the last
// group), so the hardware load counters are waited on exactly.  Within a
// group, a wave's 16 dense tiles run as one software pipeline (the MFMAs of
// tile t, then the epilogue of tile t-2), and its residual blocks follow.
#include "gemm_common.h"

namespace mq {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int TBM = 256;    // tokens per tile
constexpr int TBN = 128;    // output channels per tile
constexpr int NTHR = 512;   // eight waves: 4 (tokens) x 2 (channels), 64 x 64 each
constexpr size_t kMaxLds = 160 * 1024;

template <int BLK>
struct TileCfg {
  static constexpr int NBR = TBN / BLK;      // block rows in a tile
  static constexpr int NBC = kGroup / BLK;   // block columns in a group
  static constexpr int NSRS = TBN * NBC;     // residual-scale slots (<= NTHR)
  static constexpr int OPA = 16 * 2 * 1024;  // widened activation operands (16 row tiles)
  static constexpr int OPB = 8 * 2 * 1024;   // widened weight / residual operands (8 column tiles)
  static constexpr int A_OFF = 0;
  static constexpr int B_OFF = OPA;
  static constexpr int R_OFF = OPA + OPB;
  static constexpr int SA_OFF = OPA + 2 * OPB;
  static constexpr int SW_OFF = SA_OFF + TBM * 16;
  static constexpr int SR_OFF = SW_OFF + TBN * 16;
  static constexpr int STAGE = SR_OFF + NSRS * 16;
  static size_t lds(int64_t K) { return 2 * (size_t)STAGE + (size_t)NBR * (size_t)(K / BLK) * 2; }
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
typedef __attribute__((address_space(3))) float lds_f32;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ v4i lds_ld16(uint32_t a) { return *(const lds_v4i*)(uintptr_t)a; }
__device__ __forceinline__ void lds_st16(uint32_t a, v4i v) { *(lds_v4i*)(uintptr_t)a = v; }
__device__ __forceinline__ float lds_ldf(uint32_t a) { return *(const lds_f32*)(uintptr_t)a; }
__device__ __forceinline__ void lds_stf(uint32_t a, float v) { *(lds_f32*)(uintptr_t)a = v; }

template <int BLK, bool DUMP>
__global__ __launch_bounds__(NTHR, 1) void gemm_tile_kernel(GemmArgs a) {
  using C = TileCfg<BLK>;
  extern __shared__ __align__(16) unsigned char smem[];
  const int G = (int)(a.K / kGroup);
  const int KT = (int)(a.K / BLK);
  uint16_t* tab = reinterpret_cast<uint16_t*>(smem + 2 * C::STAGE);  // [NBR][KT]: entry-rp+1, 0 = none
  __shared__ int rp_row[C::NBR];

  const int tid = threadIdx.x;
  // (& 7 makes the range known, so LDS offsets fold into the instructions)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & 7;
  const int lane = tid & 63;
  const int r16 = lane & 15;
  const int ch = lane >> 4;

  // XCD-aware order: consecutive work items (same K split, same token rows,
  // adjacent channel tiles) go to the same XCD so its L2 serves the shared
  // A rows.  With split-K, work item = split * tiles + tile.
  const int tiles_n = (int)((a.N + TBN - 1) / TBN);
  const int items = (int)gridDim.x;
  const int tiles = items / a.ksplit;
  const int xcd = blockIdx.x % 8;
  const int per = items / 8, rem = items % 8;
  const int item = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + blockIdx.x / 8;
  const int split = item / tiles;
  const int tile = item - split * tiles;
  const int jb = (int)((int64_t)split * G / a.ksplit);             // this split's groups
  const int je = (int)((int64_t)(split + 1) * G / a.ksplit);       // [jb, je)
  const int64_t m0 = (int64_t)(tile / tiles_n) * TBM;
  const int64_t n0 = (int64_t)(tile % tiles_n) * TBN;
  const int64_t Kh = a.K / 2;
  const int nt0 = (int)(n0 / BLK);
  const int nrows_b = (int)(a.N / BLK);

  // ---- entry table of the tile's block rows: tab[rb][kt] ----
  for (int i = tid; i < C::NBR * KT; i += NTHR) tab[i] = 0;
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
        if (kt >= 0 && kt < KT) tab[rb * KT + kt] = (uint16_t)(e - b0 + 1);
      }
    }
  }
  __syncthreads();

  // ---- staging: global -> registers (fixed load count) ----
  // Lane l of a wave handles row l%16 of a 16-row slab and 16-byte piece
  // l/16, so the 16 lanes of a piece write 256 consecutive LDS bytes.
  // Per-thread offsets are fixed for the whole K loop; each group adds a
  // uniform step to a uniform base (32-bit offsets: the host routes
  // operands of 4 GiB or more to the streaming kernel).  Pieces and scales
  // of blocks that are not selected read offset 0 of a valid buffer.
  const uint8_t* rbase = a.n_select > 0 ? a.qr : a.qw;
  const uint8_t* sbase = a.n_select > 0 ? reinterpret_cast<const uint8_t*>(a.sr)
                                        : reinterpret_cast<const uint8_t*>(a.sw);
  uint32_t offA[2], slotA[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 16 * (wave + 8 * i) + r16;  // token row in the tile
    offA[i] = (uint32_t)(min(m0 + r, a.M - 1) * Kh + ch * 16);
    slotA[i] = (uint32_t)((((r >> 4) * 2 + (ch >> 1)) * 64 + r16 + 32 * (ch & 1)) * 16);
  }
  const int rw = 16 * wave + r16;  // channel row in the tile
  const int64_t nw = min(n0 + rw, a.N - 1);
  // weight codes in the slab layout: wave w stages slab n0/16 + w (the last
  // slab for tiles past N), 1 KB per group with lane l's bytes at l*16
  const int64_t slab = min(n0 / 16 + wave, a.N / 16 - 1);
  const uint32_t offB = (uint32_t)(slab * 16 * Kh + lane * 16);
  const uint32_t slotB = (uint32_t)((((rw >> 4) * 2 + (ch >> 1)) * 64 + r16 + 32 * (ch & 1)) * 16);
  const int rbw = (int)(nw / BLK) - nt0;
  const int tabR = rbw * KT + (ch * 32) / BLK;
  const int baseR = (rp_row[rbw] - 1) * (BLK * BLK / 2) + (int)(nw - (int64_t)(nt0 + rbw) * BLK) * (BLK / 2) +
                    ((ch * 32) % BLK) / 2;
  int tabS, baseS;
  {
    const int r = min(tid / C::NBC, TBN - 1), c = tid % C::NBC;
    const int64_t n = min(n0 + r, a.N - 1);
    const int rb = (int)(n / BLK) - nt0;
    tabS = tid < C::NSRS ? rb * KT + c : -1;
    baseS = ((rp_row[rb] - 1) * BLK + (int)(n - (int64_t)(nt0 + rb) * BLK)) * 2;
  }
  const uint32_t offS = wave < 4 ? (uint32_t)(min(m0 + tid, a.M - 1) * G * 4)
                                 : (uint32_t)(min(n0 + min(tid - 256, TBN - 1), a.N - 1) * G * 2);

  auto load = [&](Stage& S, int j) {
    j = min(j, je - 1);
    // table entries first (tab is zero-filled, so unguarded reads are safe)
    const int entR = (int)tab[tabR + j * C::NBC];
    const int entS = (int)tab[max(tabS, 0) + j * C::NBC];
    const uint8_t* qa_j = a.qa + j * 64;
    S.A[0] = ld16(qa_j + offA[0]);
    S.A[1] = ld16(qa_j + offA[1]);
    S.B = ld16(a.qw + j * 1024 + offB);
    if (wave < 4) {
      S.sc = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(a.sa) + j * 4 + offS);
    } else {
      S.sc = *reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(a.sw) + j * 2 + offS);
    }
    S.R = ld16(rbase + (uint32_t)(entR > 0 ? entR * (BLK * BLK / 2) + baseR : 0));
    const int es = tabS >= 0 ? entS : 0;
    S.sr = *reinterpret_cast<const uint16_t*>(sbase + (uint32_t)(es > 0 ? es * (BLK * 2) + baseS : 0));
  };

  // registers -> LDS stage: widened operands in lane order, scale operands
  auto store = [&](uint32_t st, const Stage& S) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t b = st + C::A_OFF + slotA[i];
      lds_st16(b, widen8(S.A[i].x, S.A[i].y));
      lds_st16(b + 256, widen8(S.A[i].z, S.A[i].w));
    }
    const uint32_t b = st + C::B_OFF + slotB;
    lds_st16(b, widen8(S.B.x, S.B.y));
    lds_st16(b + 256, widen8(S.B.z, S.B.w));
    lds_st16(b + C::OPB, widen8(S.R.x, S.R.y));
    lds_st16(b + C::OPB + 256, widen8(S.R.z, S.R.w));
    if (wave < 4) {
      lds_stf(st + C::SA_OFF + (uint32_t)tid * 4, (m0 + tid < a.M) ? __uint_as_float(S.sc) : 0.f);
    } else if (wave < 6) {
      lds_stf(st + C::SW_OFF + (uint32_t)(tid - 256) * 4, h2f((uint16_t)S.sc));
    }
    if (tid < C::NSRS) lds_stf(st + C::SR_OFF + (uint32_t)tid * 4, h2f((uint16_t)S.sr));
  };

  const int wm = wave >> 1, wn = wave & 1;  // 64-row x 64-channel quarter of the tile
  float y[4][4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) y[i][q][e] = 0.f;
  const v4i zero = {0, 0, 0, 0};
  // One tile step: its MFMAs first, then an earlier tile's epilogue (whose
  // products finished during the MFMAs), then a fence for the scheduler.
  auto tile_order = [](bool with_epi) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
    if (with_epi) __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);  // VALU
    __builtin_amdgcn_sched_barrier(0);
  };

  // y += (sa[m] * s) * acc: the scale product on the vector unit (one
  // multiply per element, cheaper here than a matrix-core step per tile)
  auto epi = [](float (&yt)[4], const float4& sa4, float s, const v4i& acc) {
    yt[0] = fmaf(sa4.x * s, (float)acc[0], yt[0]);
    yt[1] = fmaf(sa4.y * s, (float)acc[1], yt[1]);
    yt[2] = fmaf(sa4.z * s, (float)acc[2], yt[2]);
    yt[3] = fmaf(sa4.w * s, (float)acc[3], yt[3]);
  };

  // residual-table lookups of this wave for group j: lane q*NBC + c holds
  // the entry of column tile q, block column c (0 = not selected)
  const int tq = min(lane / C::NBC, 3), tc = lane % C::NBC;
  const int tnt = (int)((n0 + (wn * 4 + tq) * 16) / BLK);
  const bool tvalid = lane < 4 * C::NBC && tnt < nrows_b;
  const int tidx = tvalid ? (tnt - nt0) * KT + tc : 0;

  auto compute = [&](uint32_t st, int j) {
    // Bases include the wave's tile row / column and are recomputed from an
    // opaque copy in every step, so only compile-time constants remain in
    // the per-tile LDS addresses and fold into the instructions' offsets.
    uint32_t la = st + C::A_OFF + (uint32_t)lane * 16u + (uint32_t)wm * 8192u;
    uint32_t lb = st + C::B_OFF + (uint32_t)lane * 16u + (uint32_t)wn * 8192u;
    uint32_t sa_b = st + C::SA_OFF + (uint32_t)ch * 16u + (uint32_t)wm * 256u;
    uint32_t sw_b = st + C::SW_OFF + (uint32_t)r16 * 4u + (uint32_t)wn * 256u;
    asm volatile("" : "+v"(la), "+v"(lb), "+v"(sa_b), "+v"(sw_b));
    // tab is zero-filled and always allocated, so the read needs no guard;
    // its value is first used after the dense tiles
    int ent_raw = (int)tab[tidx + j * C::NBC];
    // operands in the order the first tiles need them
    v4i Bc0 = lds_ld16(lb), Bc1 = lds_ld16(lb + 1024);
    v4i A0[4], A1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      A0[i] = lds_ld16(la + (i * 2 + 0) * 1024);
      A1[i] = lds_ld16(la + (i * 2 + 1) * 1024);
    }
    float4 sa4[4];  // sa of the lane's four tokens in each 16-row tile
#pragma unroll
    for (int i = 0; i < 4; ++i) sa4[i] = __builtin_bit_cast(float4, lds_ld16(sa_b + i * 64));
    float sw[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) sw[q] = lds_ldf(sw_b + q * 64);
    v4i Bn0 = lds_ld16(lb + 2048), Bn1 = lds_ld16(lb + 3072);

    // Dense tiles t = 4q + i (column q, row tile i) as one software
    // pipeline: the MFMAs of tile t are issued before the epilogue of tile
    // t-2, so three tiles' products are live at most.
    v4i acc[16];
    auto finish = [&](int t) {
      const int q = t >> 2, i = t & 3;
      epi(y[i][q], sa4[i], sw[q], acc[t]);
      if (DUMP) {
        const int64_t n = n0 + (wn * 4 + q) * 16 + r16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t m = m0 + (wm * 4 + i) * 16 + 4 * ch + e;
          if (m < a.M && n < a.N) a.acc_dump[(m * a.N + n) * G + j] = acc[t][e] >> 8;
        }
      }
    };
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int q = t >> 2, i = t & 3;
      if (i == 0 && q > 0) {  // next column; prefetch the one after
        Bc0 = Bn0;
        Bc1 = Bn1;
        if (q < 3) {
          Bn0 = lds_ld16(lb + ((q + 1) * 2 + 0) * 1024);
          Bn1 = lds_ld16(lb + ((q + 1) * 2 + 1) * 1024);
        }
      }
      acc[t] = mfma(A1[i], Bc1, mfma(A0[i], Bc0, zero));
      if (t >= 2) finish(t - 2);
      tile_order(t >= 2);
    }
    finish(14);
    finish(15);

    // zipper: residual blocks of the wave's columns in group j, against the
    // same activation operands (lane q*NBC + c of the ballot: column q,
    // block column c)
    asm volatile("" : "+v"(ent_raw));
    const int ent_l = tvalid ? ent_raw : 0;
    const uint64_t pres = __builtin_amdgcn_ballot_w64(ent_l > 0);
    if (pres) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (!((pres >> (q * C::NBC)) & ((1u << C::NBC) - 1u))) continue;
        const int tn = wn * 4 + q;
        const int nt = (int)((n0 + tn * 16) / BLK);
        const int rb = nt - nt0;
#pragma unroll
        for (int c = 0; c < C::NBC; ++c) {
          if (!((pres >> (q * C::NBC + c)) & 1u)) continue;
          // (rare path: the residual addresses are formed here)
          const float srq = lds_ldf(st + C::SR_OFF + (uint32_t)((tn * 16 + r16) * C::NBC + c) * 4);
          const uint32_t lr = st + C::R_OFF + (uint32_t)lane * 16u + (uint32_t)tn * 2048u;
          const v4i R0 = lds_ld16(lr);
          const v4i R1 = lds_ld16(lr + 1024);
          v4i racc[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (BLK == 128) {
              racc[i] = mfma(A1[i], R1, mfma(A0[i], R0, zero));
            } else if (BLK == 64) {
              racc[i] = (c == 0) ? mfma(A0[i], R0, zero) : mfma(A1[i], R1, zero);
            } else {
              // 32-wide block c: MFMA half c/2, lane chunks 2*(c%2), 2*(c%2)+1
              const int msk = ((ch >> 1) == (c & 1)) ? -1 : 0;
              const v4i Rm = ((c < 2) ? R0 : R1) & msk;
              racc[i] = mfma((c < 2) ? A0[i] : A1[i], Rm, zero);
            }
            if (i > 0) epi(y[i - 1][q], sa4[i - 1], srq, racc[i - 1]);
            __builtin_amdgcn_sched_barrier(0);
          }
          epi(y[3][q], sa4[3], srq, racc[3]);
          if (DUMP) {
            const int ent = __builtin_amdgcn_readlane(ent_l, q * C::NBC + c);
            const int64_t e_g = rp_row[rb] + ent - 1;
            const int rr = (int)(n0 + tn * 16 + r16 - (int64_t)nt * BLK);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int64_t m = m0 + (wm * 4 + i) * 16 + 4 * ch + e;
                if (m < a.M) a.acc_dump[a.M * a.N * G + (e_g * a.M + m) * BLK + rr] = racc[i][e] >> 8;
              }
          }
        }
      }
    }
  };

  // Two LDS stages: group j is computed from stage j%2 while the waves
  // write group j+1 into the other stage; one barrier per group.  Register
  // buffers R0/R1 hold groups j+2 and j+3 in flight.
  const uint32_t st0 = lds_addr(smem);
  const uint32_t st1 = st0 + C::STAGE;
  Stage R0, R1;
  load(R0, jb);
  load(R1, jb + 1);
  store(st0, R0);
  load(R0, jb + 2);
  __syncthreads();
  // one exit only, so the accumulators need no copies on the back edge
  int j = jb;
  for (; j + 1 < je; j += 2) {
    compute(st0, j);
    store(st1, R1);  // group j+1
    load(R1, j + 3);
    __syncthreads();
    compute(st1, j + 1);
    store(st0, R0);  // group j+2
    load(R0, j + 4);
    __syncthreads();
  }
  if (j < je) compute(st0, j);  // odd group count: the last group

  // ---- output (the widened codes carry a factor 256) ----
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t n = n0 + (wn * 4 + q) * 16 + r16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t m = m0 + (wm * 4 + i) * 16 + 4 * ch + e;
        if (m < a.M && n < a.N) {
          if (a.part)
            a.part[((int64_t)split * a.M + m) * a.N + n] = y[i][q][e] * kInv256;
          else
            a.y[m * a.ldy + n] = f2h_bits(y[i][q][e] * kInv256);
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

template <int BLK, bool DUMP>
hipError_t launch_tile_cfg(const GemmArgs& a, hipStream_t st) {
  using C = TileCfg<BLK>;
  const size_t lds = C::lds(a.K);
  auto kern = gemm_tile_kernel<BLK, DUMP>;
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

hipError_t launch_tile_gemm(const GemmArgs& a, hipStream_t st) {
  const bool d = a.acc_dump != nullptr;
  switch (a.block) {
    case 32: return d ? launch_tile_cfg<32, true>(a, st) : launch_tile_cfg<32, false>(a, st);
    case 64: return d ? launch_tile_cfg<64, true>(a, st) : launch_tile_cfg<64, false>(a, st);
    default: return d ? launch_tile_cfg<128, true>(a, st) : launch_tile_cfg<128, false>(a, st);
  }
}

}  // namespace mq
