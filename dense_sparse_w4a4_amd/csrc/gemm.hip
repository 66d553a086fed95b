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
#include "mq_internal.h"

namespace mq {
namespace {

__device__ __forceinline__ v4i widen8(uint32_t lo, uint32_t hi) {
  v4i r;
  r[0] = (int)((lo << 4) & 0xF0F0F0F0u);
  r[1] = (int)(lo & 0xF0F0F0F0u);
  r[2] = (int)((hi << 4) & 0xF0F0F0F0u);
  r[3] = (int)(hi & 0xF0F0F0F0u);
  return r;
}

__device__ __forceinline__ v4i mfma(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint4 ld16(const uint8_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

constexpr float kInv256 = 1.0f / 256.0f;

// Skinny tile: 16 output channels x (16*MT) tokens per workgroup.  The KS
// waves split the K groups into contiguous runs and their partial sums are
// reduced through LDS in wave order.  Activations are the MFMA A operand
// (rows = tokens), weights the B operand (columns = channels): lane l holds
// channel n0 + l%16 and tokens 4*(l/16) + i of each 16-token tile.
//
// Memory pipeline per wave (all loads are unconditional so the hardware
// counters never wait on a load that is not needed yet):
//   * dense fragments (weights + activations) of batch t+1 (U groups) are
//     issued before batch t is computed (register double buffer);
//   * the tile row's CSR entries sit in a register window (lane l holds the
//     block column of entry wbase + l), so locating a batch's residual blocks
//     is a ballot, not a chain of dependent loads;
//   * up to RB residual blocks of batch t are fetched right after batch t's
//     dense MFMAs and consumed one batch later, together with the activation
//     fragments of batch t that are kept for that purpose (the zipper reuses
//     them instead of reloading activations); any further blocks of the batch
//     are loaded and consumed at once.
// Scales are staged in LDS once per workgroup (activation scales transposed
// to [group][token] and pre-multiplied by 1/256).
template <int BLK, int KS, int MT, int U, bool DUMP>
__global__ __launch_bounds__(64 * KS) void gemm_skinny_kernel(GemmArgs a) {
  constexpr int RB = 4;
  constexpr int TM = 16 * MT;
  extern __shared__ __align__(16) unsigned char smem[];
  const int G = (int)(a.K / kGroup);
  const int KT = (int)(a.K / BLK);
  float* sa_t = reinterpret_cast<float*>(smem);                            // [G][TM]
  uint16_t* sw_t = reinterpret_cast<uint16_t*>(smem + (size_t)G * TM * 4);  // [G][16]
  int* csr_l = reinterpret_cast<int*>(smem + (size_t)G * TM * 4 + (size_t)G * 32);  // [<= KT]
  float* red = reinterpret_cast<float*>(smem);                             // [KS][TM][17]

  // readfirstlane tells the compiler the wave index is uniform, so loop
  // bounds and guards below stay scalar branches (no exec-masked loads)
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int ch = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t m0 = (int64_t)blockIdx.y * TM;
  const int64_t Kh = a.K / 2;
  const int gb = wave * G / KS;
  const int ge = (wave + 1) * G / KS;
  const int nb = (ge - gb + U - 1) / U;

  const uint8_t* wp = a.qw + (n0 + r16) * Kh + ch * 16;
  // Token rows past M read row M-1 instead (their results are never stored).
  const uint8_t* xp[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int64_t m = m0 + t * 16 + r16;
    xp[t] = a.qa + (m < a.M ? m : a.M - 1) * Kh + ch * 16;
  }

  // This tile's rows lie in block row nt, block rows rrow .. rrow+15.
  const int nt = (int)(n0 / BLK);
  const int rrow = (int)(n0 - (int64_t)nt * BLK);
  int rp0 = 0, rp1 = 0;
  if (a.n_select > 0) {
    rp0 = min(max(a.row_ptr[nt], 0), a.n_select);
    rp1 = min(max(a.row_ptr[nt + 1], rp0), a.n_select);
  }
  const bool has_res = rp1 > rp0;

  struct Dense {
    uint4 W[U];
    uint4 X[MT][U];
  };
  struct Slots {
    uint4 R[RB];
    uint32_t M[RB];  // all-ones where the lane's chunk lies inside the block
    uint16_t S[RB];  // residual scale bits (converted where used)
    int e[RB], j[RB];
    int n;
  };

  auto fetch_dense = [&](Dense& D, int jb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = min(jb + u, ge - 1);
      D.W[u] = ld16(wp + (int64_t)j * 64);
#pragma unroll
      for (int t = 0; t < MT; ++t) D.X[t][u] = ld16(xp[t] + (int64_t)j * 64);
    }
  };

  float y[MT][4];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) y[t][i] = 0.f;
  const v4i zero = {0, 0, 0, 0};

  auto load_sa4 = [&](int j, float (&sa4)[MT][4]) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const float4 s4 = *reinterpret_cast<const float4*>(sa_t + j * TM + t * 16 + 4 * ch);
      sa4[t][0] = s4.x;
      sa4[t][1] = s4.y;
      sa4[t][2] = s4.z;
      sa4[t][3] = s4.w;
    }
  };

  auto residual = [&](uint4 R, uint32_t rm, float srf, int e, int j, const uint4 (&Xg)[MT]) {
    float sa4[MT][4];
    load_sa4(j, sa4);
    const v4i Rlo = widen8(R.x & rm, R.y & rm);
    const v4i Rhi = widen8(R.z & rm, R.w & rm);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      v4i racc = mfma(widen8(Xg[t].x, Xg[t].y), Rlo, zero);
      racc = mfma(widen8(Xg[t].z, Xg[t].w), Rhi, racc);
#pragma unroll
      for (int i = 0; i < 4; ++i) y[t][i] = fmaf(sa4[t][i] * srf, (float)racc[i], y[t][i]);
      if (DUMP) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t m = m0 + t * 16 + 4 * ch + i;
          if (m < a.M)
            a.acc_dump[a.M * a.N * G + ((int64_t)e * a.M + m) * BLK + rrow + r16] = racc[i] >> 8;
        }
      }
    }
  };

  // residual block against the activation fragments of group u of a batch
  // (u is uniform; the unrolled select keeps register indices static)
  auto residual_in = [&](const uint4 (&X)[MT][U], int u, uint4 R, uint32_t rm, float srf, int e,
                         int j) {
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      if (uu == u) {
        uint4 Xg[MT];
#pragma unroll
        for (int tt = 0; tt < MT; ++tt) Xg[tt] = X[tt][uu];
        residual(R, rm, srf, e, j, Xg);
      }
    }
  };

  auto res_ptr = [&](int e, int kt, uint32_t& rm) {
    const int js = kt * BLK / kGroup;
    const int lo = kt * BLK - js * kGroup;
    const bool act = (32 * ch >= lo) && (32 * ch < lo + BLK);
    rm = act ? 0xFFFFFFFFu : 0u;
    return a.qr + (int64_t)e * (BLK * BLK / 2) + (rrow + r16) * (BLK / 2) +
           (act ? 16 * ch - lo / 2 : 0);
  };

  auto compute_dense = [&](const Dense& D, int jb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jb + u;
      if (j >= ge) break;
      float sa4[MT][4];
      load_sa4(j, sa4);
      const float swf = h2f(sw_t[j * 16 + r16]);
      const v4i Wlo = widen8(D.W[u].x, D.W[u].y);
      const v4i Whi = widen8(D.W[u].z, D.W[u].w);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        v4i acc = mfma(widen8(D.X[t][u].x, D.X[t][u].y), Wlo, zero);
        acc = mfma(widen8(D.X[t][u].z, D.X[t][u].w), Whi, acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) y[t][i] = fmaf(sa4[t][i] * swf, (float)acc[i], y[t][i]);
        if (DUMP) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t m = m0 + t * 16 + 4 * ch + i;
            if (m < a.M) a.acc_dump[(m * a.N + n0 + r16) * G + j] = acc[i] >> 8;
          }
        }
      }
    }
  };

  // ---- prologue: batch 0, scale staging loads, CSR window ----
  Dense cur, nxt;
  if (nb > 0) fetch_dense(cur, gb);

  const int bd = 64 * KS;
  const int na = TM * G, nw = 16 * G;
  float sav[4];
  uint16_t swv[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int ia = min((int)threadIdx.x + q * bd, na - 1);
    const int ma = ia / G;
    sav[q] = a.sa[(m0 + ma < a.M ? m0 + ma : a.M - 1) * G + (ia - ma * G)];
    const int iw = min((int)threadIdx.x + q * bd, nw - 1);
    swv[q] = a.sw[(n0 + iw / G) * G + (iw - (iw / G) * G)];
  }

  // the tile row's CSR entries (block columns) are copied to LDS, so the
  // residual bookkeeping in the loop never waits on global memory
  const int row_len = min(rp1 - rp0, KT);
  int ktv[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    ktv[q] = has_res ? a.col_idx[min(rp0 + min((int)threadIdx.x + q * bd, row_len - 1),
                                     a.n_select - 1)]
                     : 0;

#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int ia = (int)threadIdx.x + q * bd;
    if (ia < na) {
      const int ma = ia / G, j = ia - ma * G;
      sa_t[j * TM + ma] = (m0 + ma < a.M) ? sav[q] * kInv256 : 0.f;
    }
    const int iw = (int)threadIdx.x + q * bd;
    if (iw < nw) {
      const int r = iw / G, j = iw - r * G;
      sw_t[j * 16 + r] = swv[q];
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if ((int)threadIdx.x + q * bd < row_len) csr_l[threadIdx.x + q * bd] = ktv[q];
  // tails of very long K or rows (more than four elements per thread)
  for (int i = (int)threadIdx.x + 4 * bd; i < row_len; i += bd) csr_l[i] = a.col_idx[rp0 + i];
  for (int ia = (int)threadIdx.x + 4 * bd; ia < na; ia += bd) {
    const int ma = ia / G, j = ia - ma * G;
    sa_t[j * TM + ma] = (m0 + ma < a.M) ? a.sa[(m0 + ma) * G + j] * kInv256 : 0.f;
  }
  for (int iw = (int)threadIdx.x + 4 * bd; iw < nw; iw += bd) {
    const int r = iw / G, j = iw - r * G;
    sw_t[j * 16 + r] = a.sw[(n0 + r) * G + j];
  }
  __syncthreads();

  // ---- main loop ----
  // row-relative index of the first entry not yet assigned to a batch:
  // lower bound of the wave's first block column in the sorted row
  int e_next = 0;
  if (has_res) {
    const int kt0 = gb * kGroup / BLK;
    for (int c = 0; c < row_len; c += 64) {
      const int i = c + lane;
      const int below = __popcll(__ballot(i < row_len && csr_l[i] < kt0));
      e_next = c + below;
      if (below < 64) break;
    }
  }
  const int e_first = e_next;
  bool any_overflow = false;
  uint4 Xprev[MT][U];
  int jprev = gb;

  // residual blocks held in slots P, from the batch whose activations are in Xprev
  auto residual_slots = [&](const Slots& P) {
#pragma unroll
    for (int s = 0; s < RB; ++s) {
      if (s < P.n) {
        const int u = P.j[s] - jprev;
        if (u >= 0 && u < U && P.j[s] < ge)
          residual_in(Xprev, u, P.R[s], P.M[s], h2f(P.S[s]), P.e[s], P.j[s]);
      }
    }
  };

  // One pipeline step for batch t held in Dc: prefetch batch t+1 into Dn,
  // compute batch t, fetch batch t's residual blocks into Sc, then consume
  // the previous batch's blocks from Sp.  Buffers alternate between steps,
  // so registers that are still being loaded are never copied.
  auto step = [&](Dense& Dc, Dense& Dn, Slots& Sc, Slots& Sp, int t) {
    const int jb = gb + t * U;
    // Every step issues the same loads (the last prefetch re-reads the final
    // batch, which is cached), so the compiler's load counters are exact and
    // computing batch t never waits for batch t+1.
    fetch_dense(Dn, min(jb + U, gb + (nb - 1) * U));
    compute_dense(Dc, jb);

    Sc.n = 0;
    int n_in = 0;
    if (has_res) {
      // entries of this batch: [e_next, e_next + n_in) (kt < kt_hi)
      const int kt_hi = min(jb + U, ge) * kGroup / BLK;
      for (int c = e_next; c < row_len; c += 64) {
        const int i = c + lane;
        const int cnt = __popcll(__ballot(i < row_len && csr_l[i] < kt_hi));
        n_in += cnt;
        if (cnt < 64) break;
      }
      Sc.n = min(n_in, RB);
    }
    // RB slot loads every step (unused slots read a valid cached address)
#pragma unroll
    for (int s = 0; s < RB; ++s) {
      const bool live = s < Sc.n;
      const int e = rp0 + e_next + s;
      const int kt = live ? csr_l[e_next + s] : 0;
      uint32_t rm = 0;
      const uint8_t* rp = live ? res_ptr(e, kt, rm) : wp;
      Sc.R[s] = ld16(rp);
      Sc.M[s] = rm;
      Sc.S[s] = *(live ? a.sr + (int64_t)e * BLK + rrow + r16 : a.sw);
      Sc.e[s] = e;
      Sc.j[s] = kt * BLK / kGroup;
    }
    if (has_res) {
      any_overflow |= n_in > RB;  // blocks past the slots run after the loop
      e_next += n_in;
    }
    residual_slots(Sp);
#pragma unroll
    for (int tt = 0; tt < MT; ++tt)
#pragma unroll
      for (int u = 0; u < U; ++u) Xprev[tt][u] = Dc.X[tt][u];
    jprev = jb;
  };

  Slots S0, S1;
  S0.n = 0;
  S1.n = 0;
  for (int t = 0; t < nb; t += 2) {
    step(cur, nxt, S0, S1, t);
    if (t + 1 >= nb) {
      residual_slots(S0);
      break;
    }
    step(nxt, cur, S1, S0, t + 1);
    if (t + 2 >= nb) residual_slots(S1);
  }

  // Cleanup (rare): batches with more than RB residual blocks.  Replays the
  // batch bookkeeping and runs the blocks past the slots, reloading their
  // activation fragments (kept out of the pipelined loop so the loop's loads
  // all have fixed counts).
  if (any_overflow) {
    int e = e_first;
    for (int t = 0; t < nb; ++t) {
      const int jb = gb + t * U;
      const int kt_hi = min(jb + U, ge) * kGroup / BLK;
      int n_in = 0;
      for (int c = e; c < row_len; c += 64) {
        const int i = c + lane;
        const int cnt = __popcll(__ballot(i < row_len && csr_l[i] < kt_hi));
        n_in += cnt;
        if (cnt < 64) break;
      }
      for (int s = RB; s < n_in; ++s) {
        const int eg = rp0 + e + s;
        const int kt = csr_l[e + s];
        const int js = kt * BLK / kGroup;
        if (js < jb || js >= jb + U || js >= ge) continue;
        uint32_t rm;
        const uint4 R = ld16(res_ptr(eg, kt, rm));
        uint4 Xg[MT];
#pragma unroll
        for (int tt = 0; tt < MT; ++tt) Xg[tt] = ld16(xp[tt] + (int64_t)js * 64);
        residual(R, rm, h2f(a.sr[(int64_t)eg * BLK + rrow + r16]), eg, js, Xg);
      }
      e += n_in;
    }
  }

  __syncthreads();  // scales no longer needed: reuse LDS for the reduction
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wave * TM + t * 16 + 4 * ch + i) * 17 + r16] = y[t][i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < TM * 16; idx += 64 * KS) {
    const int mm = idx >> 4, nl = idx & 15;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < KS; ++w) s += red[(w * TM + mm) * 17 + nl];
    const int64_t m = m0 + mm;
    if (m < a.M) a.y[m * a.ldy + n0 + nl] = f2h_bits(s);
  }
}

template <int BLK, int KS, int MT, int U, bool DUMP>
hipError_t launch_skinny_cfg(const GemmArgs& a, hipStream_t st) {
  constexpr int TM = 16 * MT;
  const int64_t G = a.K / kGroup;
  const size_t stage = (size_t)G * TM * 4 + (size_t)G * 16 * 2 + (size_t)(a.K / BLK) * 4;
  const size_t reduce = (size_t)KS * TM * 17 * 4;
  const size_t lds = stage > reduce ? stage : reduce;
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  dim3 grid((unsigned)(a.N / 16), (unsigned)((a.M + TM - 1) / TM));
  hipLaunchKernelGGL((gemm_skinny_kernel<BLK, KS, MT, U, DUMP>), grid, dim3(64 * KS), lds, st, a);
  return hipGetLastError();
}

template <int BLK, bool DUMP>
hipError_t launch_skinny(const GemmArgs& a, hipStream_t st) {
  const int64_t G = a.K / kGroup;
  if (a.M <= 16) {
    if (G >= 32) return launch_skinny_cfg<BLK, 8, 1, 4, DUMP>(a, st);
    return launch_skinny_cfg<BLK, 4, 1, 4, DUMP>(a, st);
  }
  if (a.M <= 32) return launch_skinny_cfg<BLK, 4, 2, 2, DUMP>(a, st);
  return launch_skinny_cfg<BLK, 4, 4, 2, DUMP>(a, st);
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
