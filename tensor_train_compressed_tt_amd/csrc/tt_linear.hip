// TT-linear layer on gfx950: merged-halves contraction order, fused streaming
// kernels with MFMA on the dense (tokens x modes) . (modes x rank) products.
//
// Method (CoMERA project page, "Learn the ranks while training" and "Making
// small tensor operations fast on GPUs", one contraction order for both
// passes): W = L diag(D_s) R, where L is the product of the cores on one side
// of the link s between the output-side and the input-side modes and R the
// product of the cores on the other side, each with its internal link
// diagonals.  With A = diag(D_s) R (rank x N_in) and B = L (N_out x rank)
// (output modes first in the chain; transposed roles otherwise):
//   forward   Z = x A^T (kept), Y = Z B^T
//   backward  dZ = dY B, dB = dY^T Z, dX = dZ A, dA = dZ^T x,
//             then the core gradients by a reverse sweep through each half.
// Rank adaptivity: the entries of D_s that are exactly zero are dropped on the
// device (the live slices are compacted), so the skinny products run over the
// live rank only; zero entries of the inner links zero their slices by plain
// multiplication.
//
// Kernels (one stream, no host synchronisation, no allocation):
//   k_merge      one work-group per row of a left prefix product / column of
//                a right suffix product; writes the compacted A, B (and
//                transposes) in the activation dtype plus the fp32 prefix and
//                suffix products used by the backward sweep
//   k_fwd        per 64-token tile: Z = x A^T with the K range split over the
//                4 waves, Z summed in LDS and saved, then Y^T = B Z^T
//   k_bwd_dy     per (column group, token group): dZ partials over its column
//                range, dB^T partials over its token range, dY read once
//   k_bwd_dx     per (column group, token group): dZ = sum of partials,
//                dX^T = A^T dZ^T, dA partials; x read once, dX written once
//   k_reduce     sums the partials into the gradients of the two half products
//   k_core_step  one step of the reverse sweep on both halves at once
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include "tt_plan.hpp"
#include "ttc_device.hpp"
#include "ttc_trace.hpp"

namespace ttc {

struct ChainPtrs {
  const float* G[kMaxCores];
  const float* D[kMaxCores];
};

// ------------------------------------------------------------------------------
// merge
// ------------------------------------------------------------------------------
struct MergeArgs {
  ChainPtrs c;
  int d, s, rs, Rpad, in_first;
  int modes[kMaxCores];
  int ranks[kMaxCores + 1];
  int64_t item_off[kMaxCores + 1];
  int64_t chain_off[kMaxCores];
  int64_t N_in, N_out;
  int* meta;
  void* Ac;
  void* AcT;
  void* Bc;
  void* BcT;
  float* chain;
};

template <typename T>
__global__ __launch_bounds__(128) void k_merge(MergeArgs a) {
  typedef typename Elem<T>::type E;
  __shared__ float v[TTC_MAX_RANK];
  __shared__ float w[TTC_MAX_RANK];
  __shared__ int live[TTC_MAX_RANK];
  __shared__ int reff_s;
  const int tid = threadIdx.x;
  const int64_t item = blockIdx.x;
  const int d = a.d, s = a.s;

  // live entries of the split link's diagonal, in increasing link index
  const float* Ds = a.c.D[s - 1];
  if (tid == 0) {
    int cnt = 0;
    for (int b = 0; b < a.rs; ++b)
      if (Ds[b] != 0.0f) live[cnt++] = b;
    reff_s = cnt;
    for (int j = cnt; j < TTC_MAX_RANK; ++j) live[j] = -1;
  }
  __syncthreads();
  const int reff = reff_s;
  if (item == 0) {
    for (int j = tid; j < TTC_MAX_RANK; j += blockDim.x) {
      a.meta[kMetaLive + j] = live[j];
      a.meta[kMetaPos + j] = -1;
    }
    __syncthreads();
    for (int j = tid; j < reff; j += blockDim.x) a.meta[kMetaPos + live[j]] = j;
    if (tid == 0) a.meta[kMetaReff] = reff;
  }

  // which core's item range holds this item
  int k = -1;
  for (int kk = 0; kk < d; ++kk) {
    int64_t hi;
    if (kk < s)
      hi = (kk + 1 < s) ? a.item_off[kk + 1] : (s < d ? a.item_off[d - 1] : a.item_off[d]);
    else
      hi = (kk - 1 >= s) ? a.item_off[kk - 1] : a.item_off[d];
    if (item >= a.item_off[kk] && item < hi) k = kk;
  }
  if (k < 0) return;
  int64_t idx = item - a.item_off[k];

  if (k < s) {
    // row idx of the prefix product M_k = G_0 D_0 G_1 ... G_k (digits j_0..j_k)
    int dig[kMaxCores];
    int64_t rem = idx;
    for (int t = k; t >= 0; --t) {
      dig[t] = (int)(rem % a.modes[t]);
      rem /= a.modes[t];
    }
    const int r1 = a.ranks[1];
    if (tid < r1) v[tid] = a.c.G[0][(int64_t)dig[0] * r1 + tid];
    __syncthreads();
    for (int t = 1; t <= k; ++t) {
      const int r0 = a.ranks[t], rn = a.ranks[t + 1], n = a.modes[t];
      const float* G = a.c.G[t];
      const float* D = a.c.D[t - 1];
      if (tid < rn) {
        float acc = 0.f;
        for (int aa = 0; aa < r0; ++aa) acc += (v[aa] * D[aa]) * G[((int64_t)aa * n + dig[t]) * rn + tid];
        w[tid] = acc;
      }
      __syncthreads();
      if (tid < rn) v[tid] = w[tid];
      __syncthreads();
    }
    const int rk = a.ranks[k + 1];
    if (k < s - 1) {
      if (tid < rk) a.chain[a.chain_off[k] + idx * rk + tid] = v[tid];
      return;
    }
    // a row of L (length rs)
    for (int j = tid; j < a.Rpad; j += blockDim.x) {
      const int b = j < reff ? live[j] : -1;
      if (!a.in_first) {  // B row idx
        const E val = (E)Mma<T>::from_f32(b >= 0 ? v[b] : 0.f);
        ((E*)a.Bc)[idx * a.Rpad + j] = val;
        ((E*)a.BcT)[(int64_t)j * a.N_out + idx] = val;
      } else {  // A column idx
        const E val = (E)Mma<T>::from_f32(b >= 0 ? Ds[b] * v[b] : 0.f);
        ((E*)a.Ac)[(int64_t)j * a.N_in + idx] = val;
        ((E*)a.AcT)[idx * a.Rpad + j] = val;
      }
    }
  } else {
    // column idx of the suffix product N_k = G_k D_k ... G_{d-1} (digits j_k..j_{d-1})
    int dig[kMaxCores];
    int64_t rem = idx;
    for (int t = d - 1; t >= k; --t) {
      dig[t] = (int)(rem % a.modes[t]);
      rem /= a.modes[t];
    }
    const int rl = a.ranks[d - 1];
    if (tid < rl) v[tid] = a.c.G[d - 1][(int64_t)tid * a.modes[d - 1] + dig[d - 1]];
    __syncthreads();
    for (int t = d - 2; t >= k; --t) {
      const int r0 = a.ranks[t], rn = a.ranks[t + 1], n = a.modes[t];
      const float* G = a.c.G[t];
      const float* D = a.c.D[t];
      if (tid < r0) {
        const float* row = G + ((int64_t)tid * n + dig[t]) * rn;
        float acc = 0.f;
        for (int b = 0; b < rn; ++b) acc += row[b] * (D[b] * v[b]);
        w[tid] = acc;
      }
      __syncthreads();
      if (tid < r0) v[tid] = w[tid];
      __syncthreads();
    }
    const int rk = a.ranks[k];
    if (k > s) {
      int64_t cols = 1;
      for (int t = k; t < d; ++t) cols *= a.modes[t];
      if (tid < rk) a.chain[a.chain_off[k] + (int64_t)tid * cols + idx] = v[tid];
      return;
    }
    // a column of R (length rs)
    for (int j = tid; j < a.Rpad; j += blockDim.x) {
      const int b = j < reff ? live[j] : -1;
      if (!a.in_first) {  // A column idx
        const E val = (E)Mma<T>::from_f32(b >= 0 ? Ds[b] * v[b] : 0.f);
        ((E*)a.Ac)[(int64_t)j * a.N_in + idx] = val;
        ((E*)a.AcT)[idx * a.Rpad + j] = val;
      } else {  // B row idx
        const E val = (E)Mma<T>::from_f32(b >= 0 ? v[b] : 0.f);
        ((E*)a.Bc)[idx * a.Rpad + j] = val;
        ((E*)a.BcT)[(int64_t)j * a.N_out + idx] = val;
      }
    }
  }
}

// ------------------------------------------------------------------------------
// shared tile helpers
// ------------------------------------------------------------------------------
// 64 x 64 tile of a row-major matrix into LDS (leading dimension LD), zeros
// outside [0,nrows) x [0,ncols).
template <typename T, int LD>
__device__ __forceinline__ void load_tile64(typename Elem<T>::type* lds, const typename Elem<T>::type* src,
                                            int64_t r0, int64_t nrows, int64_t c0, int64_t ncols, int64_t ld,
                                            bool vec) {
  typedef typename Mma<T>::frag frag;
  constexpr int EPV = Mma<T>::EPV;
  constexpr int PER_ROW = 64 / EPV;  // 16-byte groups per row
  for (int i = threadIdx.x; i < 64 * PER_ROW; i += 256) {
    const int rr = i / PER_ROW, pp = i % PER_ROW;
    frag f = load_frag<T>(src, r0 + rr, nrows, c0 + pp * EPV, ncols, ld, vec);
    *reinterpret_cast<frag*>(lds + rr * LD + pp * EPV) = f;
  }
}

// store 4 consecutive values of one row; `vec` says the 4-element group is
// aligned and fully in range
template <typename T>
__device__ __forceinline__ void store4(typename Elem<T>::type* p, f32x4 v, int valid, bool vec);

template <>
__device__ __forceinline__ void store4<bf16_t>(unsigned short* p, f32x4 v, int valid, bool vec) {
  if (vec && valid >= 4) {
    u16x4 o = {f32_to_bf16(v[0]), f32_to_bf16(v[1]), f32_to_bf16(v[2]), f32_to_bf16(v[3])};
    *reinterpret_cast<u16x4*>(p) = o;
  } else {
    for (int e = 0; e < 4 && e < valid; ++e) p[e] = f32_to_bf16(v[e]);
  }
}
template <>
__device__ __forceinline__ void store4<float>(float* p, f32x4 v, int valid, bool vec) {
  if (vec && valid >= 4) {
    *reinterpret_cast<f32x4*>(p) = v;
  } else {
    for (int e = 0; e < 4 && e < valid; ++e) p[e] = v[e];
  }
}

template <int NR>
struct BwdShape {
  static constexpr int CWC = (16 / NR) > 8 ? 8 : ((16 / NR) < 1 ? 1 : 16 / NR);
};

// ------------------------------------------------------------------------------
// forward
// ------------------------------------------------------------------------------
template <typename T, int NR>
__global__ __launch_bounds__(256) void k_fwd(const typename Elem<T>::type* __restrict__ x,
                                             const typename Elem<T>::type* __restrict__ Ac,
                                             const typename Elem<T>::type* __restrict__ Bc,
                                             float* __restrict__ Z, typename Elem<T>::type* __restrict__ y,
                                             int64_t T_, int64_t N_in, int64_t N_out, int vin, int vout) {
  typedef typename Elem<T>::type E;
  typedef typename Mma<T>::frag frag;
  constexpr int Rpad = 16 * NR;
  constexpr int EPV = Mma<T>::EPV, KSTEP = Mma<T>::KSTEP;
  constexpr int ZLD = Rpad + 8;
  extern __shared__ __align__(16) char smem[];
  float* zred = reinterpret_cast<float*>(smem);  // [4 waves][64 tokens][Rpad]
  E* zl = reinterpret_cast<E*>(smem);            // [64][ZLD], reuses zred after the sum

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int64_t t0 = (int64_t)blockIdx.x * 64;

  f32x4 acc[4][NR];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int n = 0; n < NR; ++n) acc[u][n] = zero4();

  const int nks = (int)((N_in + KSTEP - 1) / KSTEP);
  for (int ks = w; ks < nks; ks += 4) {
    const int64_t col = (int64_t)ks * KSTEP + g * EPV;
    frag fa[4], fb[NR];
#pragma unroll
    for (int u = 0; u < 4; ++u) fa[u] = load_frag<T>(x, t0 + 16 * u + c, T_, col, N_in, N_in, vin);
#pragma unroll
    for (int n = 0; n < NR; ++n) fb[n] = load_frag<T>(Ac, 16 * n + c, Rpad, col, N_in, N_in, vin);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int n = 0; n < NR; ++n) acc[u][n] = Mma<T>::mma(fa[u], fb[n], acc[u][n]);
  }
  // lane (g, c) holds Z rows 4g+v of token tile u, rank column 16n+c
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int n = 0; n < NR; ++n)
#pragma unroll
      for (int vv = 0; vv < 4; ++vv) zred[(w * 64 + 16 * u + 4 * g + vv) * Rpad + 16 * n + c] = acc[u][n][vv];
  __syncthreads();
  constexpr int PER = 64 * Rpad / 256;
  float zs[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = threadIdx.x + 256 * i;
    zs[i] = ((zred[idx] + zred[64 * Rpad + idx]) + zred[2 * 64 * Rpad + idx]) + zred[3 * 64 * Rpad + idx];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = threadIdx.x + 256 * i;
    const int tt = idx / Rpad, j = idx % Rpad;
    if (t0 + tt < T_) Z[(t0 + tt) * Rpad + j] = zs[i];
    zl[tt * ZLD + j] = (E)Mma<T>::from_f32(zs[i]);
  }
  __syncthreads();

  // Y^T = B Z^T: M = output column, N = token, K = rank
  const int not_ = (int)((N_out + 15) / 16);
  for (int ot = w; ot < not_; ot += 4) {
    f32x4 acc2[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc2[u] = zero4();
#pragma unroll
    for (int ks = 0; ks < Rpad / KSTEP; ++ks) {
      const int kc = ks * KSTEP + g * EPV;
      const frag fa = load_frag<T>(Bc, (int64_t)ot * 16 + c, N_out, kc, Rpad, Rpad, true);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const frag fz = lds_frag<T>(zl + (16 * u + c) * ZLD + kc);
        acc2[u] = Mma<T>::mma(fa, fz, acc2[u]);
      }
    }
    const int64_t o0 = (int64_t)ot * 16 + 4 * g;
    const int valid = (int)std::min<int64_t>(4, N_out - o0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t t = t0 + 16 * u + c;
      if (t < T_ && valid > 0) store4<T>(y + t * N_out + o0, acc2[u], valid, vout);
    }
  }
}

// ------------------------------------------------------------------------------
// backward, dY pass
// ------------------------------------------------------------------------------
template <typename T, int NR>
__global__ __launch_bounds__(256) void k_bwd_dy(const typename Elem<T>::type* __restrict__ dy,
                                                const typename Elem<T>::type* __restrict__ BcT,
                                                const float* __restrict__ Z, float* __restrict__ dZp,
                                                float* __restrict__ dBp, int64_t T_, int64_t N_out, int ncc,
                                                int tpg, int ntiles, int vout) {
  typedef typename Elem<T>::type E;
  typedef typename Mma<T>::frag frag;
  constexpr int Rpad = 16 * NR;
  constexpr int CWC = BwdShape<NR>::CWC;
  constexpr int EPV = Mma<T>::EPV, KSTEP = Mma<T>::KSTEP;
  constexpr int LD = 64 + 8;
  __shared__ __align__(16) E dyl[64 * LD];
  __shared__ __align__(16) E ztl[Rpad * LD];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int gc = blockIdx.x, gt = blockIdx.y;
  const int64_t col_lo = (int64_t)gc * ncc * 64;

  f32x4 accB[CWC][NR];
#pragma unroll
  for (int cc = 0; cc < CWC; ++cc)
#pragma unroll
    for (int n = 0; n < NR; ++n) accB[cc][n] = zero4();

  const int tt_lo = gt * tpg;
  const int tt_hi = min(ntiles, tt_lo + tpg);
  for (int tt = tt_lo; tt < tt_hi; ++tt) {
    const int64_t t0 = (int64_t)tt * 64;
    __syncthreads();
    for (int idx = threadIdx.x; idx < 64 * Rpad; idx += 256) {
      const int tl = idx / Rpad, j = idx % Rpad;
      const float z = (t0 + tl < T_) ? Z[(t0 + tl) * Rpad + j] : 0.f;
      ztl[j * LD + tl] = (E)Mma<T>::from_f32(z);
    }
    f32x4 accZ[NR];
#pragma unroll
    for (int n = 0; n < NR; ++n) accZ[n] = zero4();
#pragma unroll
    for (int cc = 0; cc < CWC; ++cc) {
      const int64_t ob = col_lo + cc * 64;
      if (cc < ncc && ob < N_out) {
        if (cc > 0) __syncthreads();
        load_tile64<T, LD>(dyl, dy, t0, T_, ob, N_out, N_out, vout);
        __syncthreads();
        // dZ: M = token (tile w), N = rank, K = column
#pragma unroll
        for (int ks = 0; ks < 64 / KSTEP; ++ks) {
          const int kc = ks * KSTEP + g * EPV;
          const frag fa = lds_frag<T>(dyl + (16 * w + c) * LD + kc);
#pragma unroll
          for (int n = 0; n < NR; ++n) {
            const frag fb = load_frag<T>(BcT, 16 * n + c, Rpad, ob + kc, N_out, N_out, vout);
            accZ[n] = Mma<T>::mma(fa, fb, accZ[n]);
          }
        }
        // dB^T: M = rank, N = column (tile w of the chunk), K = token
#pragma unroll
        for (int ks = 0; ks < 64 / KSTEP; ++ks) {
          const int kt = ks * KSTEP + g * EPV;
          const frag fb = lds_col_frag<T>(dyl + kt * LD + 16 * w + c, LD);
#pragma unroll
          for (int n = 0; n < NR; ++n) {
            const frag fa = lds_frag<T>(ztl + (16 * n + c) * LD + kt);
            accB[cc][n] = Mma<T>::mma(fa, fb, accB[cc][n]);
          }
        }
      }
    }
    // dZ partial of this column group: tokens t0+16w+4g+v, rank 16n+c
#pragma unroll
    for (int n = 0; n < NR; ++n)
#pragma unroll
      for (int vv = 0; vv < 4; ++vv) {
        const int64_t t = t0 + 16 * w + 4 * g + vv;
        if (t < T_) dZp[((int64_t)gc * T_ + t) * Rpad + 16 * n + c] = accZ[n][vv];
      }
  }
  // dB^T partial of this token group: rank 16n+4g+v, column ob+16w+c
#pragma unroll
  for (int cc = 0; cc < CWC; ++cc) {
    const int64_t o = col_lo + cc * 64 + 16 * w + c;
    if (cc < ncc && o < N_out) {
#pragma unroll
      for (int n = 0; n < NR; ++n)
#pragma unroll
        for (int vv = 0; vv < 4; ++vv)
          dBp[((int64_t)gt * Rpad + 16 * n + 4 * g + vv) * N_out + o] = accB[cc][n][vv];
    }
  }
}

// ------------------------------------------------------------------------------
// backward, dX pass
// ------------------------------------------------------------------------------
template <typename T, int NR>
__global__ __launch_bounds__(256) void k_bwd_dx(const typename Elem<T>::type* __restrict__ x,
                                                const typename Elem<T>::type* __restrict__ AcT,
                                                const float* __restrict__ dZp, int ngc, float* __restrict__ dAp,
                                                typename Elem<T>::type* __restrict__ dx, int64_t T_, int64_t N_in,
                                                int ncc, int tpg, int ntiles, int vin) {
  typedef typename Elem<T>::type E;
  typedef typename Mma<T>::frag frag;
  constexpr int Rpad = 16 * NR;
  constexpr int CWC = BwdShape<NR>::CWC;
  constexpr int EPV = Mma<T>::EPV, KSTEP = Mma<T>::KSTEP;
  constexpr int LD = 64 + 8;
  constexpr int ZLD = Rpad + 8;
  __shared__ __align__(16) E xl[64 * LD];
  __shared__ __align__(16) E dzl[64 * ZLD];
  __shared__ __align__(16) E dztl[Rpad * LD];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int gc = blockIdx.x, gt = blockIdx.y;
  const int64_t col_lo = (int64_t)gc * ncc * 64;

  f32x4 accA[CWC][NR];
#pragma unroll
  for (int cc = 0; cc < CWC; ++cc)
#pragma unroll
    for (int n = 0; n < NR; ++n) accA[cc][n] = zero4();

  const int tt_lo = gt * tpg;
  const int tt_hi = min(ntiles, tt_lo + tpg);
  for (int tt = tt_lo; tt < tt_hi; ++tt) {
    const int64_t t0 = (int64_t)tt * 64;
    __syncthreads();
    for (int idx = threadIdx.x; idx < 64 * Rpad; idx += 256) {
      const int tl = idx / Rpad, j = idx % Rpad;
      float z = 0.f;
      if (t0 + tl < T_)
        for (int q = 0; q < ngc; ++q) z += dZp[((int64_t)q * T_ + t0 + tl) * Rpad + j];
      const E e = (E)Mma<T>::from_f32(z);
      dzl[tl * ZLD + j] = e;
      dztl[j * LD + tl] = e;
    }
#pragma unroll
    for (int cc = 0; cc < CWC; ++cc) {
      const int64_t ib = col_lo + cc * 64;
      if (cc < ncc && ib < N_in) {
        if (cc > 0) __syncthreads();
        load_tile64<T, LD>(xl, x, t0, T_, ib, N_in, N_in, vin);
        __syncthreads();
        if (dx) {
          // dX^T = A^T dZ^T: M = input column (tile w), N = token, K = rank
          f32x4 accX[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) accX[u] = zero4();
#pragma unroll
          for (int ks = 0; ks < Rpad / KSTEP; ++ks) {
            const int kc = ks * KSTEP + g * EPV;
            const frag fa = load_frag<T>(AcT, ib + 16 * w + c, N_in, kc, Rpad, Rpad, true);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const frag fz = lds_frag<T>(dzl + (16 * u + c) * ZLD + kc);
              accX[u] = Mma<T>::mma(fa, fz, accX[u]);
            }
          }
          const int64_t i0 = ib + 16 * w + 4 * g;
          const int valid = (int)std::min<int64_t>(4, N_in - i0);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int64_t t = t0 + 16 * u + c;
            if (t < T_ && valid > 0) store4<T>(dx + t * N_in + i0, accX[u], valid, vin);
          }
        }
        // dA: M = rank, N = input column (tile w of the chunk), K = token
#pragma unroll
        for (int ks = 0; ks < 64 / KSTEP; ++ks) {
          const int kt = ks * KSTEP + g * EPV;
          const frag fb = lds_col_frag<T>(xl + kt * LD + 16 * w + c, LD);
#pragma unroll
          for (int n = 0; n < NR; ++n) {
            const frag fa = lds_frag<T>(dztl + (16 * n + c) * LD + kt);
            accA[cc][n] = Mma<T>::mma(fa, fb, accA[cc][n]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int cc = 0; cc < CWC; ++cc) {
    const int64_t i = col_lo + cc * 64 + 16 * w + c;
    if (cc < ncc && i < N_in) {
#pragma unroll
      for (int n = 0; n < NR; ++n)
#pragma unroll
        for (int vv = 0; vv < 4; ++vv)
          dAp[((int64_t)gt * Rpad + 16 * n + 4 * g + vv) * N_in + i] = accA[cc][n][vv];
    }
  }
}

// ------------------------------------------------------------------------------
// partial sums -> gradients of the two half products (full rank, fp32)
// ------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_reduce(const float* __restrict__ dBp, int gtB, const float* __restrict__ dAp,
                                                int gtA, const int* __restrict__ meta,
                                                const float* __restrict__ Ds, float* __restrict__ dL,
                                                float* __restrict__ dR, int64_t N_out, int64_t N_in, int rs,
                                                int Rpad, int in_first) {
  const int64_t nB = (int64_t)rs * N_out, nA = (int64_t)rs * N_in;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < nB + nA;
       idx += (int64_t)gridDim.x * blockDim.x) {
    if (idx < nB) {
      const int b = (int)(idx / N_out);
      const int64_t o = idx % N_out;
      const int j = meta[kMetaPos + b];
      float acc = 0.f;
      if (j >= 0)
        for (int q = 0; q < gtB; ++q) acc += dBp[((int64_t)q * Rpad + j) * N_out + o];
      if (!in_first)
        dL[o * rs + b] = acc;
      else
        dR[(int64_t)b * N_out + o] = acc;
    } else {
      const int64_t id2 = idx - nB;
      const int b = (int)(id2 / N_in);
      const int64_t i = id2 % N_in;
      const int j = meta[kMetaPos + b];
      float acc = 0.f;
      if (j >= 0) {
        for (int q = 0; q < gtA; ++q) acc += dAp[((int64_t)q * Rpad + j) * N_in + i];
        acc *= Ds[b];
      }
      if (!in_first)
        dR[(int64_t)b * N_in + i] = acc;
      else
        dL[i * rs + b] = acc;
    }
  }
}

// ------------------------------------------------------------------------------
// reverse sweep for the core gradients
// ------------------------------------------------------------------------------
struct StepArgs {
  ChainPtrs c;
  float* dG[kMaxCores];
  int d;
  int modes[kMaxCores];
  int ranks[kMaxCores + 1];
  int64_t chain_off[kMaxCores];
  const float* chain;
  int kL, kR;          // cores of this step on the left / right half, -1 = none
  const float* dM;     // gradient of the left prefix M_kL (rowsL x r_{kL+1})
  float* dMn;          // gradient of M_{kL-1}
  const float* dN;     // gradient of the right suffix N_kR (r_kR x colsR)
  float* dNn;          // gradient of N_{kR+1}
  int64_t rowsL, colsR;
};

// Left core k, M_k[(alpha, m), c] = sum_a P[alpha, a] G_k[a, m, c] with
// P = M_{k-1} diag(D_{k-1}):
//   dG_k[a, m, c]   = sum_alpha P[alpha, a] dM_k[(alpha, m), c]
//   dM_{k-1}[alpha, a] = D_{k-1}[a] sum_{m, c} dM_k[(alpha, m), c] G_k[a, m, c]
// Right core k, N_k[a, (m, beta)] = sum_c G_k[a, m, c] Q[c, beta] with
// Q = diag(D_k) N_{k+1}:
//   dG_k[a, m, c]   = sum_beta dN_k[a, (m, beta)] Q[c, beta]
//   dN_{k+1}[c, beta] = D_k[c] sum_{a, m} G_k[a, m, c] dN_k[a, (m, beta)]
__global__ __launch_bounds__(256) void k_core_step(StepArgs a) {
  int64_t nL1 = 0, nL2 = 0, nR1 = 0, nR2 = 0;
  if (a.kL >= 0) {
    const int k = a.kL;
    nL1 = (int64_t)a.ranks[k] * a.modes[k] * a.ranks[k + 1];
    if (k > 0) nL2 = (a.rowsL / a.modes[k]) * a.ranks[k];
  }
  if (a.kR >= 0) {
    const int k = a.kR;
    nR1 = (int64_t)a.ranks[k] * a.modes[k] * a.ranks[k + 1];
    if (k < a.d - 1) nR2 = (int64_t)a.ranks[k + 1] * (a.colsR / a.modes[k]);
  }
  const int64_t total = nL1 + nL2 + nR1 + nR2;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    if (idx < nL1 + nL2) {
      const int k = a.kL;
      const int n = a.modes[k], r0 = a.ranks[k], r1 = a.ranks[k + 1];
      const int64_t alphas = a.rowsL / n;
      if (idx < nL1) {
        const int cc = (int)(idx % r1);
        const int m = (int)((idx / r1) % n);
        const int aa = (int)(idx / ((int64_t)r1 * n));
        float acc = 0.f;
        if (k == 0) {
          acc = a.dM[(int64_t)m * r1 + cc];
        } else {
          const float* Mp = a.chain + a.chain_off[k - 1];
          const float dk = a.c.D[k - 1][aa];
          for (int64_t al = 0; al < alphas; ++al)
            acc += (Mp[al * r0 + aa] * dk) * a.dM[(al * n + m) * r1 + cc];
        }
        a.dG[k][idx] = acc;
      } else {
        const int64_t id2 = idx - nL1;
        const int aa = (int)(id2 % r0);
        const int64_t al = id2 / r0;
        const float* Gk = a.c.G[k];
        float acc = 0.f;
        for (int m = 0; m < n; ++m) {
          const float* dm = a.dM + (al * n + m) * r1;
          const float* gk = Gk + ((int64_t)aa * n + m) * r1;
          for (int cc = 0; cc < r1; ++cc) acc += dm[cc] * gk[cc];
        }
        a.dMn[al * r0 + aa] = a.c.D[k - 1][aa] * acc;
      }
    } else {
      const int64_t id3 = idx - nL1 - nL2;
      const int k = a.kR;
      const int n = a.modes[k], r0 = a.ranks[k], r1 = a.ranks[k + 1];
      const int64_t betas = a.colsR / n;
      if (id3 < nR1) {
        const int cc = (int)(id3 % r1);
        const int m = (int)((id3 / r1) % n);
        const int aa = (int)(id3 / ((int64_t)r1 * n));
        float acc = 0.f;
        if (k == a.d - 1) {
          acc = a.dN[(int64_t)aa * a.colsR + m];
        } else {
          const float* Nn = a.chain + a.chain_off[k + 1];
          const float dk = a.c.D[k][cc];
          const float* dn = a.dN + (int64_t)aa * a.colsR + (int64_t)m * betas;
          for (int64_t be = 0; be < betas; ++be) acc += dn[be] * (dk * Nn[(int64_t)cc * betas + be]);
        }
        a.dG[k][id3] = acc;
      } else {
        const int64_t id4 = id3 - nR1;
        const int64_t be = id4 % betas;
        const int cc = (int)(id4 / betas);
        const float* Gk = a.c.G[k];
        float acc = 0.f;
        for (int aa = 0; aa < r0; ++aa)
          for (int m = 0; m < n; ++m)
            acc += Gk[((int64_t)aa * n + m) * r1 + cc] * a.dN[(int64_t)aa * a.colsR + (int64_t)m * betas + be];
        a.dNn[(int64_t)cc * betas + be] = a.c.D[k][cc] * acc;
      }
    }
  }
}

__global__ void k_zero(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

// ------------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------------
static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

static ttc_status check_chain(const LinearPlan& P, const float* const* G, const float* const* D) {
  if (!G) return TTC_ERR_NULL;
  if (P.d > 1 && !D) return TTC_ERR_NULL;
  for (int k = 0; k < P.d; ++k)
    if (!G[k]) return TTC_ERR_NULL;
  for (int k = 0; k < P.d - 1; ++k)
    if (!D[k]) return TTC_ERR_NULL;
  return TTC_OK;
}

static ChainPtrs chain_ptrs(const LinearPlan& P, const float* const* G, const float* const* D) {
  ChainPtrs c;
  memset(&c, 0, sizeof(c));
  for (int k = 0; k < P.d; ++k) c.G[k] = G[k];
  for (int k = 0; k < P.d - 1; ++k) c.D[k] = D[k];
  return c;
}

static ttc_status hip_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? TTC_OK : TTC_ERR_HIP;
}

template <typename T, int NR>
static void launch_fwd(const LinearPlan& P, const void* x, char* saved, void* y, hipStream_t st) {
  typedef typename Elem<T>::type E;
  const size_t lds = size_t(4) * 64 * 16 * NR * sizeof(float);
  auto kern = k_fwd<T, NR>;
  static bool lds_set = false;  // set once, before any graph capture can see it
  if (!lds_set) {
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    lds_set = true;
  }
  const int vin = (P.N_in % Mma<T>::EPV) == 0 && aligned16(x);
  const int vout = (P.N_out % 4) == 0 && aligned16(y);
  TraceScope ts("fwd", st);
  hipLaunchKernelGGL(kern, dim3(P.ntiles), dim3(256), lds, st, (const E*)x, (const E*)(saved + P.sv_Ac),
                     (const E*)(saved + P.sv_Bc), (float*)(saved + P.sv_Z), (E*)y, P.T, P.N_in, P.N_out, vin,
                     vout);
}

template <typename T, int NR>
static void launch_bwd_main(const LinearPlan& P, const void* x, const void* dy, const char* saved, void* dx,
                            char* scratch, hipStream_t st) {
  typedef typename Elem<T>::type E;
  const int vout = (P.N_out % Mma<T>::EPV) == 0 && aligned16(dy);
  {
    TraceScope ts("bwd_dy", st);
    hipLaunchKernelGGL((k_bwd_dy<T, NR>), dim3(P.dy_gc, P.dy_gt), dim3(256), 0, st, (const E*)dy,
                     (const E*)(saved + P.sv_BcT), (const float*)(saved + P.sv_Z), (float*)(scratch + P.sc_dZp),
                     (float*)(scratch + P.sc_dBp), P.T, P.N_out, P.dy_ncc, P.dy_tpg, P.ntiles, vout);
  }
  const int vin = (P.N_in % Mma<T>::EPV) == 0 && aligned16(x) && (dx == nullptr || aligned16(dx));
  TraceScope ts("bwd_dx", st);
  hipLaunchKernelGGL((k_bwd_dx<T, NR>), dim3(P.dx_gc, P.dx_gt), dim3(256), 0, st, (const E*)x,
                     (const E*)(saved + P.sv_AcT), (const float*)(scratch + P.sc_dZp), P.dy_gc,
                     (float*)(scratch + P.sc_dAp), (E*)dx, P.T, P.N_in, P.dx_ncc, P.dx_tpg, P.ntiles, vin);
}

template <typename T>
static bool dispatch_fwd(const LinearPlan& P, const void* x, char* saved, void* y, hipStream_t st) {
  switch (P.NR) {
    case 2: launch_fwd<T, 2>(P, x, saved, y, st); return true;
    case 4: launch_fwd<T, 4>(P, x, saved, y, st); return true;
    case 6: launch_fwd<T, 6>(P, x, saved, y, st); return true;
    case 8: launch_fwd<T, 8>(P, x, saved, y, st); return true;
  }
  return false;
}

template <typename T>
static bool dispatch_bwd(const LinearPlan& P, const void* x, const void* dy, const char* saved, void* dx,
                         char* scratch, hipStream_t st) {
  switch (P.NR) {
    case 2: launch_bwd_main<T, 2>(P, x, dy, saved, dx, scratch, st); return true;
    case 4: launch_bwd_main<T, 4>(P, x, dy, saved, dx, scratch, st); return true;
    case 6: launch_bwd_main<T, 6>(P, x, dy, saved, dx, scratch, st); return true;
    case 8: launch_bwd_main<T, 8>(P, x, dy, saved, dx, scratch, st); return true;
  }
  return false;
}

}  // namespace ttc

using namespace ttc;

extern "C" ttc_status tt_linear_workspace(const tt_linear_desc* desc, int64_t T, size_t* saved_bytes,
                                          size_t* scratch_bytes) {
  if (!saved_bytes || !scratch_bytes) return TTC_ERR_NULL;
  LinearPlan P;
  const ttc_status st = make_linear_plan(desc, T, &P);
  if (st != TTC_OK) return st;
  *saved_bytes = P.sv_total;
  *scratch_bytes = P.sc_total;
  return TTC_OK;
}

extern "C" ttc_status tt_linear_fwd(const tt_linear_desc* desc, int64_t T, const void* x, const float* const* G,
                                    const float* const* D, void* y, void* saved, size_t saved_bytes, void* scratch,
                                    size_t scratch_bytes, ttc_stream_t stream) {
  (void)scratch;
  (void)scratch_bytes;
  LinearPlan P;
  ttc_status st = make_linear_plan(desc, T, &P);
  if (st != TTC_OK) return st;
  if ((st = check_chain(P, G, D)) != TTC_OK) return st;
  if (T == 0) return TTC_OK;
  if (!x || !y || !saved) return TTC_ERR_NULL;
  if (!aligned16(x) || !aligned16(y) || !aligned16(saved)) return TTC_ERR_ALIGN;
  if (saved_bytes < P.sv_total) return TTC_ERR_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  char* sv = static_cast<char*>(saved);
  MergeArgs m;
  memset(&m, 0, sizeof(m));
  m.c = chain_ptrs(P, G, D);
  m.d = P.d;
  m.s = P.s;
  m.rs = P.rs;
  m.Rpad = P.Rpad;
  m.in_first = P.in_first;
  for (int k = 0; k < P.d; ++k) {
    m.modes[k] = P.modes[k];
    m.chain_off[k] = P.chain_off[k];
  }
  for (int k = 0; k <= P.d; ++k) {
    m.ranks[k] = P.ranks[k];
    m.item_off[k] = P.item_off[k];
  }
  m.N_in = P.N_in;
  m.N_out = P.N_out;
  m.meta = reinterpret_cast<int*>(sv + P.sv_meta);
  m.Ac = sv + P.sv_Ac;
  m.AcT = sv + P.sv_AcT;
  m.Bc = sv + P.sv_Bc;
  m.BcT = sv + P.sv_BcT;
  m.chain = reinterpret_cast<float*>(sv + P.sv_chain);
  {
    TraceScope ts("merge", s);
    if (P.act == TTC_BF16)
      hipLaunchKernelGGL(k_merge<bf16_t>, dim3((unsigned)P.item_off[P.d]), dim3(128), 0, s, m);
    else
      hipLaunchKernelGGL(k_merge<float>, dim3((unsigned)P.item_off[P.d]), dim3(128), 0, s, m);
  }
  const bool ok = P.act == TTC_BF16 ? dispatch_fwd<bf16_t>(P, x, sv, y, s) : dispatch_fwd<float>(P, x, sv, y, s);
  if (!ok) return TTC_ERR_UNSUPPORTED;
  return hip_status();
}

extern "C" ttc_status tt_linear_bwd(const tt_linear_desc* desc, int64_t T, const void* x, const void* dy,
                                    const float* const* G, const float* const* D, const void* saved,
                                    size_t saved_bytes, void* dx, float* const* dG, void* scratch,
                                    size_t scratch_bytes, ttc_stream_t stream) {
  LinearPlan P;
  ttc_status st = make_linear_plan(desc, T, &P);
  if (st != TTC_OK) return st;
  if ((st = check_chain(P, G, D)) != TTC_OK) return st;
  if (!dG) return TTC_ERR_NULL;
  for (int k = 0; k < P.d; ++k)
    if (!dG[k]) return TTC_ERR_NULL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (T == 0) {
    for (int k = 0; k < P.d; ++k) {
      const int64_t n = (int64_t)P.ranks[k] * P.modes[k] * P.ranks[k + 1];
      TraceScope ts("zero", s);
      hipLaunchKernelGGL(k_zero, dim3((unsigned)std::min<int64_t>(1024, (n + 255) / 256)), dim3(256), 0, s, dG[k], n);
    }
    return hip_status();
  }
  if (!x || !dy || !saved || !scratch) return TTC_ERR_NULL;
  if (!aligned16(x) || !aligned16(dy) || !aligned16(saved) || !aligned16(scratch) || (dx && !aligned16(dx)))
    return TTC_ERR_ALIGN;
  if (saved_bytes < P.sv_total || scratch_bytes < P.sc_total) return TTC_ERR_WORKSPACE;
  const char* sv = static_cast<const char*>(saved);
  char* sc = static_cast<char*>(scratch);
  const bool ok = P.act == TTC_BF16 ? dispatch_bwd<bf16_t>(P, x, dy, sv, dx, sc, s)
                                    : dispatch_bwd<float>(P, x, dy, sv, dx, sc, s);
  if (!ok) return TTC_ERR_UNSUPPORTED;
  // partial sums -> dL, dR
  {
    const int64_t n = (int64_t)P.rs * (P.N_out + P.N_in);
    const unsigned blocks = (unsigned)std::min<int64_t>(2048, (n + 255) / 256);
    TraceScope ts("reduce", s);
    hipLaunchKernelGGL(k_reduce, dim3(blocks), dim3(256), 0, s, (const float*)(sc + P.sc_dBp), P.dy_gt,
                       (const float*)(sc + P.sc_dAp), P.dx_gt, (const int*)(sv + P.sv_meta), D[P.s - 1],
                       (float*)(sc + P.sc_dL), (float*)(sc + P.sc_dR), P.N_out, P.N_in, P.rs, P.Rpad, P.in_first);
  }
  // reverse sweep through both halves
  StepArgs a;
  memset(&a, 0, sizeof(a));
  a.c = chain_ptrs(P, G, D);
  for (int k = 0; k < P.d; ++k) {
    a.dG[k] = dG[k];
    a.modes[k] = P.modes[k];
    a.chain_off[k] = P.chain_off[k];
  }
  for (int k = 0; k <= P.d; ++k) a.ranks[k] = P.ranks[k];
  a.d = P.d;
  a.chain = reinterpret_cast<const float*>(sv + P.sv_chain);
  const float* curL = reinterpret_cast<const float*>(sc + P.sc_dL);
  const float* curR = reinterpret_cast<const float*>(sc + P.sc_dR);
  int64_t rowsL = P.NL, colsR = P.NRt;
  const int steps = std::max(P.s, P.d - P.s);
  for (int i = 0; i < steps; ++i) {
    float* buf = reinterpret_cast<float*>(sc + ((i & 1) ? P.sc_w1 : P.sc_w0));
    a.kL = (P.s - 1 - i >= 0) ? P.s - 1 - i : -1;
    a.kR = (P.s + i < P.d) ? P.s + i : -1;
    a.dM = curL;
    a.dMn = buf;
    a.dN = curR;
    a.dNn = buf + P.wl_floats;
    a.rowsL = rowsL;
    a.colsR = colsR;
    int64_t total = 0;
    if (a.kL >= 0) {
      const int k = a.kL;
      total += (int64_t)P.ranks[k] * P.modes[k] * P.ranks[k + 1];
      if (k > 0) total += (rowsL / P.modes[k]) * P.ranks[k];
    }
    if (a.kR >= 0) {
      const int k = a.kR;
      total += (int64_t)P.ranks[k] * P.modes[k] * P.ranks[k + 1];
      if (k < P.d - 1) total += (int64_t)P.ranks[k + 1] * (colsR / P.modes[k]);
    }
    const unsigned blocks = (unsigned)std::max<int64_t>(1, std::min<int64_t>(4096, (total + 255) / 256));
    {
      TraceScope ts("core_step", s);
      hipLaunchKernelGGL(k_core_step, dim3(blocks), dim3(256), 0, s, a);
    }
    if (a.kL >= 0) {
      curL = a.dMn;
      rowsL /= P.modes[a.kL];
    }
    if (a.kR >= 0) {
      curR = a.dNn;
      colsR /= P.modes[a.kR];
    }
  }
  return hip_status();
}

extern "C" ttc_status tt_linear_explain(const tt_linear_desc* desc, int64_t T, char* buf, size_t n) {
  if (!buf || n == 0) return TTC_ERR_NULL;
  LinearPlan P;
  const ttc_status st = make_linear_plan(desc, T, &P);
  if (st != TTC_OK) return st;
  double macs[4], bytes[4];
  linear_path_costs(P, macs, bytes);
  snprintf(buf, n,
           "path=merged split=%d rank=%d rpad=%d N_out=%lld N_in=%lld T=%lld "
           "merged_macs=%.6g merged_bytes=%.6g sequential_macs=%.6g sequential_bytes=%.6g "
           "dense_macs=%.6g dense_bytes=%.6g dy_grid=%dx%d dx_grid=%dx%d saved=%zu scratch=%zu",
           P.s, P.rs, P.Rpad, (long long)P.N_out, (long long)P.N_in, (long long)T, macs[1], bytes[1], macs[2],
           bytes[2], macs[3], bytes[3], P.dy_gc, P.dy_gt, P.dx_gc, P.dx_gt, P.sv_total, P.sc_total);
  return TTC_OK;
}

extern "C" ttc_status tt_linear_path_cost(const tt_linear_desc* desc, int64_t T, int32_t path, double* macs,
                                          double* bytes) {
  if (!macs || !bytes) return TTC_ERR_NULL;
  if (path < TTC_PATH_MERGED || path > TTC_PATH_DENSE) return TTC_ERR_UNSUPPORTED;
  // cost the path regardless of whether it is implemented
  tt_linear_desc dd = *desc;
  dd.path = TTC_PATH_AUTO;
  LinearPlan P;
  const ttc_status st = make_linear_plan(&dd, T, &P);
  if (st != TTC_OK) return st;
  double m[4], b[4];
  linear_path_costs(P, m, b);
  *macs = m[path];
  *bytes = b[path];
  return TTC_OK;
}

extern "C" const char* ttc_status_str(ttc_status s) {
  switch (s) {
    case TTC_OK: return "ok";
    case TTC_ERR_NULL: return "null pointer";
    case TTC_ERR_SHAPE: return "bad shape";
    case TTC_ERR_RANK: return "bad ranks";
    case TTC_ERR_DTYPE: return "bad dtype";
    case TTC_ERR_ALIGN: return "pointer not 16-byte aligned";
    case TTC_ERR_WORKSPACE: return "workspace too small";
    case TTC_ERR_UNSUPPORTED: return "unsupported";
    case TTC_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

extern "C" const char* ttc_version(void) { return "ttc 0.1 gfx950"; }
