// Exact output distortion of a block selection, and the greedy selection that
// lowers it one block at a time.
//
// MosaicQuant technical summary (gist.science/pt/paper/2606.15652),
// Metodologia 2 and Principais Contribuições 2: the Hessian-guided Delta-score
// stands in for a costly exact evaluation of the output distortion
//   D(S) = || X (W - deq Q(W) - sum_{i in S} R_hat_i)^T ||_F^2 .
// These kernels make that evaluation on the GPU, so the Delta top-K can be
// set against it on full-size layers.
//
// Greedy step: with o = X (E - R_S)^T restricted to the b outputs of block
// row nt, every unchosen block (nt, kt) has the gain
//   gain = ||o||^2 - ||o - X_kt R_hat_(nt,kt)^T||^2 ,
// the block with the largest gain (ties: lower id) joins S, the outputs of its
// row are updated, and only that row's candidates are evaluated again (a pick
// changes no other row's outputs).  fp64 throughout: X (fp16), E and R_hat
// (fp32, from the same per-row scales as the packed residual) are exact in
// fp64.
//
// Outputs o are kept in HBM as [N/b][T][b] fp64, so one block row's outputs
// for a run of tokens are contiguous.
#include "blockres.h"

namespace mq {
namespace {

constexpr int kTok = 64;   // tokens per tile (candidate and GEMM kernels)
constexpr int kGN = 64;    // outputs per GEMM tile
constexpr int kGK = 32;    // inputs per GEMM step

// Sum of one double per thread over a 256-thread workgroup, in a fixed order
// (so a result never depends on scheduling).  Every thread must call it.
__device__ double wg_sum256(double v, double* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

// Fill kernel (no memset nodes, so the sequence may be captured in a graph).
__global__ void fill_u8_kernel(uint8_t* __restrict__ p, int64_t n, uint8_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// ids -> 0/1 mask over the B blocks; ids outside [0, B) are ignored.
__global__ void scatter_mask_kernel(const int32_t* __restrict__ ids, int64_t n, int64_t B,
                                    uint8_t* __restrict__ mask) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int32_t id = ids[i];
    if (id >= 0 && id < B) mask[id] = 1;
  }
}

// Per (row n, block column kt): rem[n][k] = E (fp64), minus R_hat where the
// block is in `mask`; rhat[n][k] = R_hat (fp32) when requested.  E = W - sw*q
// is exact in fp32 (both terms share the group's binade scale), and so is
// R_hat = sr * code; the fp64 difference is exact too.
__global__ __launch_bounds__(256) void prep_kernel(const uint16_t* __restrict__ w, int64_t N,
                                                   int64_t K, int b, const uint8_t* __restrict__ mask,
                                                   double* __restrict__ rem,
                                                   float* __restrict__ rhat) {
  const int64_t KT = K / b;
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= N * KT) return;
  const int64_t n = u / KT, kt = u - n * KT;
  const int64_t kb = kt * b;
  const uint16_t* wrow = w + n * K;
  const RowScales rs = row_scales(wrow, kb, b);
  const bool sub = mask && mask[(n / b) * KT + kt];
  for (int c = 0; c < b; ++c) {
    const float e = base_err(h2f(wrow[kb + c]), rs.swf);
    const float rh = rs.srf * (float)quant4(e, rs.srf);
    rem[n * K + kb + c] = sub ? (double)e - (double)rh : (double)e;
    if (rhat) rhat[n * K + kb + c] = rh;
  }
}

// out[t][n] = sum_k X[t][k] * rem[n][k] in fp64, 64 tokens x 64 outputs per
// workgroup, 4 x 4 per thread.  `out` (optional) is stored as [N/b][T][b];
// `partial` (optional) gets each workgroup's sum of out^2.
__global__ __launch_bounds__(256) void xrem_gemm_kernel(const uint16_t* __restrict__ x, int64_t T,
                                                        int64_t K, const double* __restrict__ rem,
                                                        int64_t N, int b, double* __restrict__ out,
                                                        double* __restrict__ partial) {
  __shared__ __align__(16) double Xs[kGK][kTok + 2];
  __shared__ __align__(16) double Ws[kGK][kGN + 2];
  __shared__ double red[4];
  const int tid = threadIdx.x;
  const int64_t n0 = (int64_t)blockIdx.x * kGN;
  const int64_t t0 = (int64_t)blockIdx.y * kTok;
  const int tg = tid & 15, ng = tid >> 4;
  const int lr = tid >> 2, lk = (tid & 3) * 8;  // load role: one row, 8 inputs
  double acc[4][4] = {};
  for (int64_t k0 = 0; k0 < K; k0 += kGK) {
    {
      const int64_t t = t0 + lr;
      float f[8] = {};
      if (t < T) unpack_h8(*reinterpret_cast<const uint4*>(x + t * K + k0 + lk), f);
#pragma unroll
      for (int e = 0; e < 8; ++e) Xs[lk + e][lr] = (double)f[e];
      const int64_t n = n0 + lr;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        double2 v = make_double2(0.0, 0.0);
        if (n < N) v = *reinterpret_cast<const double2*>(rem + n * K + k0 + lk + e);
        Ws[lk + e][lr] = v.x;
        Ws[lk + e + 1][lr] = v.y;
      }
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < kGK; ++kk) {
      const double2 a0 = *reinterpret_cast<const double2*>(&Xs[kk][tg * 4]);
      const double2 a1 = *reinterpret_cast<const double2*>(&Xs[kk][tg * 4 + 2]);
      const double2 b0 = *reinterpret_cast<const double2*>(&Ws[kk][ng * 4]);
      const double2 b1 = *reinterpret_cast<const double2*>(&Ws[kk][ng * 4 + 2]);
      const double av[4] = {a0.x, a0.y, a1.x, a1.y};
      const double bv[4] = {b0.x, b0.y, b1.x, b1.y};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fma(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t t = t0 + tg * 4 + i;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + ng * 4 + j;
      if (t < T && n < N) {
        if (out) out[((n / b) * T + t) * b + (n % b)] = acc[i][j];
        s = s + acc[i][j] * acc[i][j];
      }
    }
  }
  if (partial) {
    const double tot = wg_sum256(s, red);
    if (tid == 0) partial[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = tot;
  }
}

// One candidate block (nt, kt) against one tile of 64 tokens:
//   d[t][r] = sum_c X[t][kt*BLK + c] * R_hat[nt*BLK + r][kt*BLK + c]
// GAIN: parts[id][tile] = (sum o^2, sum (o - d)^2) over the tile's outputs.
// UPDATE: o -= d (the block has just been picked).
// The candidate is `id0 + blockIdx.x`, or, with `pick`, block row *pick / KT
// and column blockIdx.x (GAIN) or *pick % KT (UPDATE).
template <int BLK, bool UPDATE>
__global__ __launch_bounds__(256) void cand_kernel(const uint16_t* __restrict__ x, int64_t T,
                                                   int64_t K, const float* __restrict__ rhat,
                                                   double* __restrict__ out, int64_t KT,
                                                   const int32_t* __restrict__ pick,
                                                   const uint8_t* __restrict__ chosen,
                                                   double* __restrict__ parts, int64_t id0) {
  constexpr int RPT = BLK / 16;
  __shared__ __align__(16) float Xs[BLK][kTok + 4];  // [c][t]
  __shared__ __align__(16) float Rs[BLK][BLK + 4];   // [c][r]
  __shared__ double red[4];
  int64_t nt, kt;
  if (pick) {
    const int64_t p = *pick;
    nt = p / KT;
    kt = UPDATE ? p - nt * KT : (int64_t)blockIdx.x;
  } else {
    const int64_t id = id0 + blockIdx.x;
    nt = id / KT;
    kt = id - nt * KT;
  }
  const int64_t id = nt * KT + kt;
  if (!UPDATE && chosen[id]) return;  // uniform over the workgroup
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.y * kTok;
  const int64_t kb = kt * BLK;
  for (int e = tid; e < BLK * BLK; e += 256) {
    const int r = e / BLK, c = e - r * BLK;
    Rs[c][r] = rhat[(nt * BLK + r) * K + kb + c];
  }
  for (int e = tid; e < kTok * BLK; e += 256) {
    const int t = e / BLK, c = e - t * BLK;
    Xs[c][t] = (t0 + t < T) ? h2f(x[(t0 + t) * K + kb + c]) : 0.0f;
  }
  __syncthreads();
  const int tg = tid & 15, rg = tid >> 4;
  double d[4][RPT] = {};
  for (int c = 0; c < BLK; ++c) {
    const float4 xa = *reinterpret_cast<const float4*>(&Xs[c][tg * 4]);
    const double xv[4] = {(double)xa.x, (double)xa.y, (double)xa.z, (double)xa.w};
    double rv[RPT];
    if constexpr (RPT == 2) {
      const float2 r2 = *reinterpret_cast<const float2*>(&Rs[c][rg * 2]);
      rv[0] = r2.x;
      rv[1] = r2.y;
    } else {
#pragma unroll
      for (int q = 0; q < RPT; q += 4) {
        const float4 r4 = *reinterpret_cast<const float4*>(&Rs[c][rg * RPT + q]);
        rv[q] = r4.x;
        rv[q + 1] = r4.y;
        rv[q + 2] = r4.z;
        rv[q + 3] = r4.w;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < RPT; ++j) d[i][j] = fma(xv[i], rv[j], d[i][j]);
  }
  double base = 0.0, sq = 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t t = t0 + tg * 4 + i;
    if (t < T) {
      double* po = out + (nt * T + t) * BLK + rg * RPT;
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        const double o = po[j];
        if constexpr (UPDATE) {
          po[j] = o - d[i][j];
        } else {
          const double e = o - d[i][j];
          base = base + o * o;
          sq = sq + e * e;
        }
      }
    }
  }
  if constexpr (!UPDATE) {
    const double tb = wg_sum256(base, red);
    const double ts = wg_sum256(sq, red);
    if (tid == 0) {
      double* p = parts + (id * gridDim.y + blockIdx.y) * 2;
      p[0] = tb;
      p[1] = ts;
    }
  }
}

// gain = sum over tiles of ||o||^2  -  sum over tiles of ||o - d||^2.
__device__ __forceinline__ double finish_gain(const double* __restrict__ parts, int64_t id,
                                              int64_t ntile) {
  double b = 0.0, s = 0.0;
  for (int64_t q = 0; q < ntile; ++q) {
    b = b + parts[(id * ntile + q) * 2];
    s = s + parts[(id * ntile + q) * 2 + 1];
  }
  return b - s;
}

__global__ void finish_all_kernel(const double* __restrict__ parts, int64_t ntile, int64_t B,
                                  double* __restrict__ gain) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < B;
       i += (int64_t)gridDim.x * blockDim.x)
    gain[i] = finish_gain(parts, i, ntile);
}

// Ranking key of a gain: larger gain -> larger key, -0 with +0, NaN below
// every number; 0 is kept for "no candidate".
__device__ __forceinline__ uint64_t gain_key(double g) {
  if (g != g) return 1;
  uint64_t u = __builtin_bit_cast(uint64_t, g);
  if (u == 0x8000000000000000ull) u = 0;
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// One greedy step, one workgroup: refresh the gains of the row the previous
// pick changed, then take the unchosen block of largest gain (ties: lower id).
__global__ __launch_bounds__(1024) void pick_kernel(double* __restrict__ gain,
                                                    uint8_t* __restrict__ chosen,
                                                    const double* __restrict__ parts,
                                                    int64_t ntile, int64_t B, int64_t KT,
                                                    int32_t* __restrict__ order,
                                                    double* __restrict__ gains_out, int step) {
  __shared__ uint64_t sk[16];
  __shared__ int64_t si[16];
  const int tid = threadIdx.x;
  if (step > 0) {
    const int64_t nt = order[step - 1] / KT;
    for (int64_t kt = tid; kt < KT; kt += 1024) {
      const int64_t id = nt * KT + kt;
      if (!chosen[id]) gain[id] = finish_gain(parts, id, ntile);
    }
    __syncthreads();
  }
  uint64_t bk = 0;
  int64_t bi = INT64_MAX;
  for (int64_t i = tid; i < B; i += 1024) {
    if (chosen[i]) continue;
    const uint64_t k = gain_key(gain[i]);
    if (k > bk) {  // ids rise along a thread's walk: equal keys keep the lower id
      bk = k;
      bi = i;
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint64_t ok = __shfl_xor(bk, m);
    const int64_t oi = __shfl_xor(bi, m);
    if (ok > bk || (ok == bk && oi < bi)) {
      bk = ok;
      bi = oi;
    }
  }
  if ((tid & 63) == 0) {
    sk[tid >> 6] = bk;
    si[tid >> 6] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int v = 1; v < 16; ++v)
      if (sk[v] > bk || (sk[v] == bk && si[v] < bi)) {
        bk = sk[v];
        bi = si[v];
      }
    order[step] = (int32_t)bi;
    gains_out[step] = gain[bi];
    chosen[bi] = 1;
  }
}

// Ids of the chosen blocks in ascending order (one workgroup).
__global__ __launch_bounds__(1024) void compact_kernel(const uint8_t* __restrict__ chosen,
                                                       int64_t B, int n_sel,
                                                       int32_t* __restrict__ selected) {
  __shared__ int cnt[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int64_t base = 0;
  for (int64_t c0 = 0; c0 < B; c0 += 1024) {
    const int64_t i = c0 + tid;
    const bool take = i < B && chosen[i];
    const uint64_t bal = __ballot(take);
    if (lane == 0) cnt[wave] = __popcll(bal);
    __syncthreads();
    int64_t pos = base + __popcll(bal & below);
    int64_t tot = 0;
    for (int v = 0; v < 16; ++v) {
      if (v < wave) pos += cnt[v];
      tot += cnt[v];
    }
    if (take && pos < n_sel) selected[pos] = (int32_t)i;
    base += tot;
    __syncthreads();
  }
}

// Sum of squares in two fixed-order stages: 256 workgroups over contiguous
// chunks, then one workgroup over the partials.
constexpr int kSumParts = 256;

__global__ __launch_bounds__(256) void sumsq_partial_kernel(const double* __restrict__ v,
                                                            int64_t n, double* __restrict__ partial) {
  __shared__ double red[4];
  const int64_t chunk = (n + kSumParts - 1) / kSumParts;
  const int64_t lo = blockIdx.x * chunk;
  const int64_t hi = lo + chunk < n ? lo + chunk : n;
  double s = 0.0;
  for (int64_t i = lo + threadIdx.x; i < hi; i += 256) s = s + v[i] * v[i];
  const double tot = wg_sum256(s, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = tot;
}

__global__ __launch_bounds__(256) void sum_final_kernel(const double* __restrict__ partial,
                                                        int64_t n, double* __restrict__ dst) {
  __shared__ double red[4];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += 256) s = s + partial[i];
  const double tot = wg_sum256(s, red);
  if (threadIdx.x == 0) *dst = tot;
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

struct GreedyWs {
  double* rem;
  float* rhat;
  double* out;
  double* gain;
  double* parts;
  uint8_t* chosen;
  int32_t* order;
  double* gains;
  double* sums;
  size_t bytes;
};

GreedyWs greedy_layout(void* ws, int64_t N, int64_t K, int64_t T, int b) {
  const int64_t B = (N / b) * (K / b);
  const int64_t ntile = (T + kTok - 1) / kTok;
  char* p = static_cast<char*>(ws);
  size_t off = 0;
  GreedyWs g{};
  auto take = [&](size_t n) {
    char* q = p ? p + off : nullptr;
    off += align256(n);
    return q;
  };
  g.rem = reinterpret_cast<double*>(take((size_t)N * K * sizeof(double)));
  g.rhat = reinterpret_cast<float*>(take((size_t)N * K * sizeof(float)));
  g.out = reinterpret_cast<double*>(take((size_t)T * N * sizeof(double)));
  g.gain = reinterpret_cast<double*>(take((size_t)B * sizeof(double)));
  g.parts = reinterpret_cast<double*>(take((size_t)B * ntile * 2 * sizeof(double)));
  g.chosen = reinterpret_cast<uint8_t*>(take((size_t)B));
  g.order = reinterpret_cast<int32_t*>(take((size_t)B * sizeof(int32_t)));
  g.gains = reinterpret_cast<double*>(take((size_t)B * sizeof(double)));
  g.sums = reinterpret_cast<double*>(take((size_t)(kSumParts + 2) * sizeof(double)));
  g.bytes = off;
  return g;
}

struct DistWs {
  double* rem;
  uint8_t* mask;
  double* partial;
  double* sums;
  size_t bytes;
};

int64_t gemm_tiles(int64_t N, int64_t T) {
  return ((N + kGN - 1) / kGN) * ((T + kTok - 1) / kTok);
}

DistWs dist_layout(void* ws, int64_t N, int64_t K, int64_t T, int b) {
  const int64_t B = (N / b) * (K / b);
  char* p = static_cast<char*>(ws);
  size_t off = 0;
  DistWs d{};
  auto take = [&](size_t n) {
    char* q = p ? p + off : nullptr;
    off += align256(n);
    return q;
  };
  d.rem = reinterpret_cast<double*>(take((size_t)N * K * sizeof(double)));
  d.mask = reinterpret_cast<uint8_t*>(take((size_t)B));
  d.partial = reinterpret_cast<double*>(take((size_t)gemm_tiles(N, T) * sizeof(double)));
  d.sums = reinterpret_cast<double*>(take((size_t)kSumParts * sizeof(double)));
  d.bytes = off;
  return d;
}

unsigned grid_for(int64_t n, int per) {
  const int64_t g = (n + per - 1) / per;
  return (unsigned)(g < 65536 ? (g > 0 ? g : 1) : 65536);
}

template <int BLK>
hipError_t greedy_blk(const uint16_t* x, int64_t N, int64_t K, int64_t T, int n_select,
                      const GreedyWs& g, hipStream_t st) {
  const int64_t KT = K / BLK;
  const int64_t B = (N / BLK) * KT;
  const int64_t ntile = (T + kTok - 1) / kTok;
  if (ntile > 0) {
    hipLaunchKernelGGL((cand_kernel<BLK, false>), dim3((unsigned)B, (unsigned)ntile), dim3(256), 0,
                       st, x, T, K, g.rhat, g.out, KT, nullptr, g.chosen, g.parts, (int64_t)0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(finish_all_kernel, dim3(grid_for(B, 256)), dim3(256), 0, st, g.parts, ntile,
                     B, g.gain);
  hipError_t e = hipGetLastError();
  for (int s = 0; s < n_select && e == hipSuccess; ++s) {
    hipLaunchKernelGGL(pick_kernel, dim3(1), dim3(1024), 0, st, g.gain, g.chosen, g.parts, ntile,
                       B, KT, g.order, g.gains, s);
    e = hipGetLastError();
    if (e != hipSuccess || ntile == 0) continue;
    // the outputs are needed after the last pick too (the final distortion)
    hipLaunchKernelGGL((cand_kernel<BLK, true>), dim3(1, (unsigned)ntile), dim3(256), 0, st, x, T,
                       K, g.rhat, g.out, KT, g.order + s, g.chosen, g.parts, (int64_t)0);
    e = hipGetLastError();
    if (e != hipSuccess || s + 1 == n_select) continue;
    hipLaunchKernelGGL((cand_kernel<BLK, false>), dim3((unsigned)KT, (unsigned)ntile), dim3(256), 0,
                       st, x, T, K, g.rhat, g.out, KT, g.order + s, g.chosen, g.parts, (int64_t)0);
    e = hipGetLastError();
  }
  return e;
}

hipError_t sumsq(const double* v, int64_t n, double* partial, double* dst, hipStream_t st) {
  hipLaunchKernelGGL(sumsq_partial_kernel, dim3(kSumParts), dim3(256), 0, st, v, n, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sum_final_kernel, dim3(1), dim3(256), 0, st, partial, (int64_t)kSumParts, dst);
  return hipGetLastError();
}

}  // namespace

size_t exact_greedy_workspace(int64_t N, int64_t K, int64_t T, int b) {
  return greedy_layout(nullptr, N, K, T, b).bytes;
}

size_t distortion_workspace(int64_t N, int64_t K, int64_t T, int b) {
  return dist_layout(nullptr, N, K, T, b).bytes;
}

hipError_t launch_exact_greedy(const uint16_t* w, const uint16_t* x, int64_t N, int64_t K,
                               int64_t T, int b, int n_select, int32_t* selected, int32_t* order,
                               double* gains, double* dist, void* ws, hipStream_t st) {
  const GreedyWs g = greedy_layout(ws, N, K, T, b);
  const int64_t KT = K / b;
  const int64_t B = (N / b) * KT;
  hipLaunchKernelGGL(fill_u8_kernel, dim3(grid_for(B, 256)), dim3(256), 0, st, g.chosen, B,
                     (uint8_t)0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(prep_kernel, dim3((unsigned)((N * KT + 255) / 256)), dim3(256), 0, st, w, N, K,
                     b, nullptr, g.rem, g.rhat);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (T > 0) {
    hipLaunchKernelGGL(xrem_gemm_kernel, dim3((unsigned)((N + kGN - 1) / kGN),
                                              (unsigned)((T + kTok - 1) / kTok)),
                       dim3(256), 0, st, x, T, K, g.rem, N, b, g.out, nullptr);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (dist && (e = sumsq(g.out, T * N, g.sums, dist, st)) != hipSuccess) return e;
  switch (b) {
    case 32: e = greedy_blk<32>(x, N, K, T, n_select, g, st); break;
    case 64: e = greedy_blk<64>(x, N, K, T, n_select, g, st); break;
    default: e = greedy_blk<128>(x, N, K, T, n_select, g, st); break;
  }
  if (e != hipSuccess) return e;
  if (dist && (e = sumsq(g.out, T * N, g.sums, dist + 1, st)) != hipSuccess) return e;
  if (n_select > 0) {
    hipLaunchKernelGGL(compact_kernel, dim3(1), dim3(1024), 0, st, g.chosen, B, n_select, selected);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (order) {
      e = hipMemcpyAsync(order, g.order, (size_t)n_select * sizeof(int32_t),
                         hipMemcpyDeviceToDevice, st);
      if (e != hipSuccess) return e;
    }
    if (gains)
      e = hipMemcpyAsync(gains, g.gains, (size_t)n_select * sizeof(double),
                         hipMemcpyDeviceToDevice, st);
  }
  return e;
}

hipError_t launch_distortion(const uint16_t* w, const uint16_t* x, int64_t N, int64_t K,
                             int64_t T, int b, const int32_t* ids, int64_t n_ids, double* dist,
                             void* ws, hipStream_t st) {
  const DistWs d = dist_layout(ws, N, K, T, b);
  const int64_t KT = K / b;
  const int64_t B = (N / b) * KT;
  hipLaunchKernelGGL(fill_u8_kernel, dim3(grid_for(B, 256)), dim3(256), 0, st, d.mask, B,
                     (uint8_t)0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (n_ids > 0) {
    hipLaunchKernelGGL(scatter_mask_kernel, dim3(grid_for(n_ids, 256)), dim3(256), 0, st, ids,
                       n_ids, B, d.mask);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(prep_kernel, dim3((unsigned)((N * KT + 255) / 256)), dim3(256), 0, st, w, N, K,
                     b, d.mask, d.rem, nullptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t tiles = gemm_tiles(N, T);
  if (T > 0) {
    hipLaunchKernelGGL(xrem_gemm_kernel, dim3((unsigned)((N + kGN - 1) / kGN),
                                              (unsigned)((T + kTok - 1) / kTok)),
                       dim3(256), 0, st, x, T, K, d.rem, N, b, nullptr, d.partial);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(sum_final_kernel, dim3(1), dim3(256), 0, st, d.partial, T > 0 ? tiles : 0,
                     dist);
  return hipGetLastError();
}

}  // namespace mq
