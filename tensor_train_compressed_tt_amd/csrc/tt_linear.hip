// TT-linear layer on gfx950: merged-halves contraction order, streaming
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
// live rank; zero entries of the inner links zero their slices by plain
// multiplication, which keeps dead-slice gradients exactly 0.
//
// Kernels (one stream, no host synchronisation, no allocation):
//   k_merge      both halves of the chain multiplied out, one prefix of the
//                walk from each chain end per work-group: the prefix products
//                kept for the sweep, the compacted A, B (and transposes) in
//                the activation dtype
//   k_fwd        per 64-token tile: Z = x A^T with the K range split over the
//                waves (two load batches in flight; x of wide inputs read as
//                whole 256-byte row pieces and staged through LDS), Z summed
//                in LDS and kept, then Y^T = B Z^T with the B fragments
//                prefetched
//   k_bwd_dy     per (column group, token group): 64 x 256-byte slabs of dY
//                stream through LDS with register prefetch; dZ (or its
//                partials over the column groups), dB^T partials over the
//                token group
//   k_dz_sum     sums the dZ partials of the column groups in group order
//                (skipped where the dX pass sums two partials itself)
//   k_bwd_dx     per (column group, token group): slabs of x stream through
//                LDS; dX^T = A^T dZ^T written per slab, dA partials
//   k_reduce     sums the partials into the gradients of the two half products
//   k_sweep      one level of the reverse sweep through both halves: the
//                small GEMMs of that level as 32 x 32 fp32-MFMA tiles spread
//                over work-groups (one launch per level)
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <type_traits>
#include <vector>

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
// Each half of the chain is multiplied out one row (left half) or one column
// (right half) at a time, walking from the chain's end towards the split
// link s:
//   left   v_0 = G_0[0, i_0, :],     v_t = (v_{t-1} diag(D_{t-1})) G_t[:, i_t, :]
//   right  w_0 = G_{d-1}[:, j, 0],   w_t = G_k[:, j_k, :] diag(D_k) w_{t-1}   (k = d-1-t)
// The walk's last step is the core next to the split; every other step
// belongs to a prefix (the digits of the cores before it).  A work-group owns
// kMergePG consecutive prefixes: it forms their prefix products once (the
// chain area the backward sweep reads: rows M_t of the left half, columns N_k
// of the right half, each written by exactly one work-group), then loops over
// the last core's mode with that core's slices staged in LDS.  The rows and
// columns of the two half products go straight into the MFMA operands in the
// activation dtype, keeping only the live slices of the split link:
// B = L and A = diag(D_s) R (roles swapped when the chain starts with the
// input modes), each also transposed, zero-padded to Rpad.  One launch per
// activation dtype for up to kMaxMerge layers.
// Layers per launch of the batched reductions.
constexpr int kMaxBatch = 8;

struct MergeLayer {
  const float* G[kMaxCores];
  const float* D[kMaxCores];  // D[k] on the link between cores k and k+1
  float* chain;               // prefix / suffix products (fp32)
  int chain_off[kMaxCores];   // float offsets (the plan keeps them below 2^31)
  int lstride[kMaxCores];     // stride of each position's mode in its kind's listed index
  int modes[kMaxCores];
  int ranks[kMaxCores + 1];
  void* Ac;
  void* AcT;
  void* Bc;
  void* BcT;
  int* meta;
  int64_t N_in, N_out;
  int64_t npl, npr;  // prefixes of the left and the right half
  int64_t wgl;       // work-groups of the left half (the rest: right half)
  int d, s, in_first, rs, Rpad;
};
constexpr int kMaxMerge = 6;
struct MergeBatch {
  MergeLayer l[kMaxMerge];
  int64_t first[kMaxMerge + 1];
  int n;
};
static_assert(sizeof(MergeBatch) <= 4000, "MergeBatch too large for a kernel argument");

constexpr int kMergeThreads = 512;
constexpr int kMergePG = 8;      // prefixes per work-group
constexpr int kMergeOut = 8192;  // floats of staged outputs ([pg][mode chunk][rank])
constexpr int kMergeX = 32;      // core values per thread loaded before they are used

// A batch of core values g[(x0 + u) * sx], u < kMergeX, zero past rin.  With
// unit stride (the right half's walk: each lane reads its own contiguous run,
// the lanes' runs far apart) the batch comes as 16- or 8-byte loads when the
// run is aligned (rin a multiple of 4 or 2), not as kMergeX scalar loads that
// each touch as many cache lines as there are lanes.
__device__ __forceinline__ void merge_batch(float (&gv)[kMergeX], const float* __restrict__ g, int64_t sx, int x0,
                                            int rin) {
  const uintptr_t adr = (uintptr_t)(g + x0);
  if (sx == 1 && (rin & 3) == 0 && (adr & 15) == 0) {
#pragma unroll
    for (int u = 0; u < kMergeX; u += 4) {
      const f32x4 v = x0 + u < rin ? *reinterpret_cast<const f32x4*>(g + x0 + u) : zero4();
#pragma unroll
      for (int e = 0; e < 4; ++e) gv[u + e] = v[e];
    }
  } else if (sx == 1 && (rin & 1) == 0 && (adr & 7) == 0) {
#pragma unroll
    for (int u = 0; u < kMergeX; u += 2) {
      const f32x2 v = x0 + u < rin ? *reinterpret_cast<const f32x2*>(g + x0 + u) : f32x2{0.f, 0.f};
      gv[u] = v[0];
      gv[u + 1] = v[1];
    }
  } else {
#pragma unroll
    for (int u = 0; u < kMergeX; ++u) gv[u] = x0 + u < rin ? g[(int64_t)(x0 + u) * sx] : 0.f;
  }
}

// One output of a walk step for up to kMergePG prefixes at once:
//   acc[pg] += sum_x v[pg][x] * G(x), x < rin,
// with the rin core values G(x) = g[x * sx] requested in batches of kMergeX
// (a plain loop would wait for each load in turn) and v read from LDS.
__device__ __forceinline__ void merge_dot(float (&acc)[kMergePG], const float* __restrict__ g, int64_t sx,
                                          int rin, const float* v) {
  for (int x0 = 0; x0 < rin; x0 += kMergeX) {
    float gv[kMergeX];
    merge_batch(gv, g, sx, x0, rin);
#pragma unroll
    for (int u = 0; u < kMergeX; ++u) {
      if (x0 + u < rin) {
#pragma unroll
        for (int pg = 0; pg < kMergePG; ++pg) acc[pg] = fmaf(v[pg * TTC_MAX_RANK + x0 + u], gv[u], acc[pg]);
      }
    }
  }
}

// store 4 consecutive values of one row (defined with the streaming helpers)
template <typename T>
__device__ __forceinline__ void store4(typename Elem<T>::type* p, f32x4 v, int valid, bool vec);

// Digit of walk step t of prefix p (step 0 most significant on the left,
// least significant on the right).  Prefix counts are below 2^24 (the plan
// bounds N_in and N_out), so the index arithmetic of the merge is 32-bit.
__device__ __forceinline__ int merge_digit(const MergeLayer& a, bool left, int S, int t, int p) {
  int div = 1;
  if (left) {
    for (int u = t + 1; u <= S - 2; ++u) div *= a.modes[u];
    return (p / div) % a.modes[t];
  }
  for (int u = 0; u < t; ++u) div *= a.modes[a.d - 1 - u];
  return (p / div) % a.modes[a.d - 1 - t];
}

// Eight core values g[(x0 + u) * sx], u < 8, zero at or past rin (16- or
// 8-byte loads where the run is contiguous and aligned).
__device__ __forceinline__ void merge_load8(float (&o)[8], const float* __restrict__ g, int64_t sx, int x0, int rin) {
  const uintptr_t adr = (uintptr_t)(g + x0);
  if (sx == 1 && (rin & 3) == 0 && (adr & 15) == 0) {
#pragma unroll
    for (int u = 0; u < 8; u += 4) {
      const f32x4 v = x0 + u < rin ? *reinterpret_cast<const f32x4*>(g + x0 + u) : zero4();
#pragma unroll
      for (int e = 0; e < 4; ++e) o[u + e] = v[e];
    }
  } else if (sx == 1 && (rin & 1) == 0 && (adr & 7) == 0) {
#pragma unroll
    for (int u = 0; u < 8; u += 2) {
      const f32x2 v = x0 + u < rin ? *reinterpret_cast<const f32x2*>(g + x0 + u) : f32x2{0.f, 0.f};
      o[u] = v[0];
      o[u + 1] = v[1];
    }
  } else {
#pragma unroll
    for (int u = 0; u < 8; ++u) o[u] = x0 + u < rin ? g[(int64_t)(x0 + u) * sx] : 0.f;
  }
}

// FAST (every layer of the launch: at most three cores per half, ranks up to
// kMergeX, a last core's mode times the split rank up to kMergeThreads): each
// thread forms at most one output of every walk step, and the last step is
// one fp32-MFMA product [prefix x rin] x [rin x (mode index, rank)], so every
// core value and diagonal entry a thread reads is requested at the start and
// the work-group waits for memory once instead of once or twice per step
// (each wait is a round trip to memory beyond the L2).
template <typename T, bool FAST>
__global__ __launch_bounds__(kMergeThreads) void k_merge(MergeBatch mb) {
  typedef typename Elem<T>::type E;
  __shared__ float ob[kMergeOut];                          // [pg][ii][rout] outputs of the last step
  __shared__ float vb[2][kMergePG * TTC_MAX_RANK];         // prefix vectors (D applied)
  __shared__ int live[TTC_MAX_RANK], pos[TTC_MAX_RANK];
  __shared__ float dlive[TTC_MAX_RANK];  // D_s at the live entries, compacted
  __shared__ int s_reff;
  int q = 0;
  while (q < mb.n - 1 && (int64_t)blockIdx.x >= mb.first[q + 1]) ++q;
  const MergeLayer& a = mb.l[q];
  const int tid = threadIdx.x;
  int64_t wg = (int64_t)blockIdx.x - mb.first[q];
  const bool left = wg < a.wgl;
  if (!left) wg -= a.wgl;
  const int d = a.d, s = a.s;
  const int S = left ? s : d - s;  // cores in this half
  const int NP = (int)(left ? a.npl : a.npr);
  const int p0 = (int)wg * kMergePG;
  const int npg = NP - p0 < kMergePG ? NP - p0 : kMergePG;
  const float* Ds = a.D[s - 1];
  float gw0[kMergeX], gw1[kMergeX];
  float bl[kMergeThreads / 128][8];  // FAST last step: B values of this lane's output tiles
  float dn0 = 0.f, dn1 = 0.f;
  // FAST: the walk steps' fields, read with the first loads
  int wn[2] = {1, 1}, wrin[2] = {0, 0}, wrout[2] = {0, 0}, wls[2] = {0, 0};
  float* wch[2] = {nullptr, nullptr};
  const int lane = tid & 63, wv = tid >> 6;
  if constexpr (FAST) {
    // walk step t: output (pg, y) = (tid / rout, tid % rout)
    auto walk_load = [&](int t, float (&gv)[kMergeX], float& dn) {
      const int k = left ? t : d - 1 - t;
      const int n = a.modes[k];
      const int rin = left ? a.ranks[k] : a.ranks[k + 1];
      const int rout = left ? a.ranks[k + 1] : a.ranks[k];
      wn[t] = n;
      wrin[t] = rin;
      wrout[t] = rout;
      wls[t] = a.lstride[k];
      wch[t] = a.chain + a.chain_off[k];
      if (tid < npg * rout) {
        const int pg = tid / rout, y = tid - pg * rout;
        const int dg = merge_digit(a, left, S, t, p0 + pg);
        const float* g = left ? a.G[k] + (int64_t)dg * rout + y : a.G[k] + ((int64_t)y * n + dg) * rin;
        merge_batch(gv, g, left ? (int64_t)n * rout : 1, 0, rin);
        dn = (left ? a.D[k] : a.D[k - 1])[y];
      }
    };
    if (S >= 2) walk_load(0, gw0, dn0);
    if (S >= 3) walk_load(1, gw1, dn1);
    // last step: the B operand of the product, column c = (mode index ii,
    // rank y) = (c / rs, c % rs), row x; wave wv takes the 16-column tiles
    // wv, wv + 8, ..., and lane group gq of a tile supplies rows 8gq .. 8gq+7
    // (the same order of K for both operands)
    const int kf = left ? s - 1 : s;
    const int n = a.modes[kf];
    const int rin = left ? a.ranks[kf] : a.ranks[kf + 1];
    const int NC = n * a.rs;
#pragma unroll
    for (int u = 0; u < kMergeThreads / 128; ++u) {
      const int c = 16 * (wv + 8 * u) + (lane & 15);
      if (c < NC) {
        const int ii = c / a.rs, y = c - ii * a.rs;
        const float* g = left ? a.G[kf] + c : a.G[kf] + ((int64_t)y * n + ii) * rin;
        merge_load8(bl[u], g, left ? (int64_t)NC : 1, 8 * (lane >> 4), rin);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) bl[u][e] = 0.f;
      }
    }
  }
  // live entries of the split link's diagonal, in increasing link index
  if (tid < 64) {
    const int lane = tid;
    const float d0 = lane < a.rs ? Ds[lane] : 0.f, d1 = lane + 64 < a.rs ? Ds[lane + 64] : 0.f;
    const bool f0 = d0 != 0.0f, f1 = d1 != 0.0f;
    const uint64_t m0 = __ballot(f0), m1 = __ballot(f1);
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    const int c0 = __popcll(m0);
    const int i0 = __popcll(m0 & below), i1 = c0 + __popcll(m1 & below);
    pos[lane] = f0 ? i0 : -1;
    pos[lane + 64] = f1 ? i1 : -1;
    live[lane] = -1;
    live[lane + 64] = -1;
    __builtin_amdgcn_wave_barrier();
    if (f0) {
      live[i0] = lane;
      dlive[i0] = d0;
    }
    if (f1) {
      live[i1] = lane + 64;
      dlive[i1] = d1;
    }
    if (lane == 0) s_reff = c0 + __popcll(m1);
  }
  for (int e = tid; e < kMergePG; e += kMergeThreads) vb[0][e * TTC_MAX_RANK] = 1.0f;
  __syncthreads();
  const int reff = s_reff;
  if (left && wg == 0) {
    for (int j = tid; j < TTC_MAX_RANK; j += kMergeThreads) {
      a.meta[kMetaLive + j] = live[j];
      a.meta[kMetaPos + j] = pos[j];
    }
    if (tid == 0) a.meta[kMetaReff] = reff;
  }

  // Prefix walk, steps 0..S-2: thread (y, pg-group) forms output y of the
  // step for every prefix of the work-group; the digit of step t of prefix p
  // has step 0 most significant on the left and least significant on the
  // right.  The next step's input is this output times the link diagonal.
  int cur = 0;
  int divL = 1;  // left: product of the modes of steps t+1..S-2
  for (int t = 1; t <= S - 2; ++t) divL *= a.modes[t];
  int mulR = 1;  // right: product of the modes of steps 0..t
  if constexpr (FAST) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (t < S - 1) {
        const int rin = wrin[t], rout = wrout[t];
        if (!left) mulR *= wn[t];
        if (tid < npg * rout) {
          const int pg = tid / rout, y = tid - pg * rout;
          const float* v = vb[cur] + pg * TTC_MAX_RANK;
          float acc = 0.f;
#pragma unroll
          for (int u = 0; u < kMergeX; ++u)
            if (u < rin) acc = fmaf(v[u], t == 0 ? gw0[u] : gw1[u], acc);
          vb[cur ^ 1][pg * TTC_MAX_RANK + y] = acc * (t == 0 ? dn0 : dn1);
          // one writer per chain row: the prefix whose later digits are all 0
          const int p = p0 + pg;
          if (left) {
            if (p % divL == 0) wch[t][(int64_t)(p / divL) * rout + y] = acc;
          } else if (p < mulR) {
            wch[t][(int64_t)y * mulR + p] = acc;
          }
        }
        __syncthreads();
        cur ^= 1;
        if (left && t == 0 && S == 3) divL /= wn[1];
      }
    }
  } else for (int t = 0; t < S - 1; ++t) {
    const int k = left ? t : d - 1 - t;
    const int n = a.modes[k];
    const int rin = left ? a.ranks[k] : a.ranks[k + 1];
    const int rout = left ? a.ranks[k + 1] : a.ranks[k];
    if (!left) mulR *= n;
    const float* G = a.G[k];
    // diagonal applied to this step's output before the next step
    const float* Dn = left ? a.D[k] : a.D[k - 1];
    float* ch = a.chain + a.chain_off[k];
    // one writer per chain row: the prefix whose later digits are all 0
    auto chain_put = [&](int p, int y, float acc) {
      if (left) {
        if (p % divL == 0) ch[(int64_t)(p / divL) * rout + y] = acc;
      } else if (p < mulR) {
        ch[(int64_t)y * mulR + p] = acc;
      }
    };
    for (int e = tid; e < npg * rout; e += kMergeThreads) {
      const int pg = e / rout, y = e - pg * rout;
      const int p = p0 + pg;
      const int dg = left ? (p / divL) % n : (p / (mulR / n)) % n;
      const float* g = left ? G + (int64_t)dg * rout + y : G + ((int64_t)y * n + dg) * rin;
      const int64_t sx = left ? (int64_t)n * rout : 1;
      const float* v = vb[cur] + pg * TTC_MAX_RANK;
      float acc = 0.f;
      for (int x0 = 0; x0 < rin; x0 += kMergeX) {
        float gv[kMergeX];
        merge_batch(gv, g, sx, x0, rin);
#pragma unroll
        for (int u = 0; u < kMergeX; ++u)
          if (x0 + u < rin) acc = fmaf(v[x0 + u], gv[u], acc);
      }
      vb[cur ^ 1][pg * TTC_MAX_RANK + y] = acc * Dn[y];
      chain_put(p, y, acc);
    }
    __syncthreads();
    cur ^= 1;
    if (left && t + 1 <= S - 2) divL /= a.modes[t + 1];
  }

  // Last step: the core next to the split, all its mode indices for all the
  // prefixes, in chunks of ci mode indices; outputs staged in LDS, then
  // written as rows of the packed operand and of its transpose.
  const int kf = left ? s - 1 : s;
  const int n = a.modes[kf];
  const int rin = left ? a.ranks[kf] : a.ranks[kf + 1];
  const int rout = a.rs;
  const float* G = a.G[kf];
  const bool is_b = left != (a.in_first != 0);
  // B is kept as [N_out][Rpad] (Bc) and [Rpad][N_out] (BcT), A as [Rpad][N_in]
  // (Ac) and [N_in][Rpad] (AcT): `out` is the [N][Rpad] one, `outT` the other
  E* out = reinterpret_cast<E*>(is_b ? a.Bc : a.AcT);
  E* outT = reinterpret_cast<E*>(is_b ? a.BcT : a.Ac);
  const int64_t Nlong = is_b ? a.N_out : a.N_in;
  const int Rpad = a.Rpad;
  int ci = kMergeOut / (kMergePG * rout);
  if (ci > n) ci = n;
  const float* v = vb[cur];
  // the operand row of (prefix, mode index i) is its listed index: the sum of
  // every chain digit times that mode's stride in the listed order (the chain
  // index itself when each half lists its modes in chain order)
  __shared__ int64_t lbase[kMergePG];
  if (tid < npg) {
    int rem = p0 + tid;
    int64_t b = 0;
    if (FAST) {
      // the walk's digits, least significant first
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int t = left ? S - 2 - u : u;
        if (t >= 0 && t <= S - 2) {
          const int mt = t == 0 ? wn[0] : wn[1], st = t == 0 ? wls[0] : wls[1];
          b += (int64_t)(rem % mt) * st;
          rem /= mt;
        }
      }
    } else if (left) {
      for (int t = S - 2; t >= 0; --t) {
        b += (rem % a.modes[t]) * a.lstride[t];
        rem /= a.modes[t];
      }
    } else {
      for (int t = 0; t <= S - 2; ++t) {
        const int k = d - 1 - t;
        b += (rem % a.modes[k]) * a.lstride[k];
        rem /= a.modes[k];
      }
    }
    lbase[tid] = b;
  }
  const int64_t lsf = a.lstride[kf];
  __syncthreads();
  for (int i0 = 0; i0 < n; i0 += ci) {
    const int ni = n - i0 < ci ? n - i0 : ci;
    if constexpr (FAST) {
      // one chunk (ci = n): out[pg][c] = sum_x v[pg][x] B[x][c] as 16 x 16
      // fp32-MFMA tiles (M = prefix, rows past npg zero; K = x in the lane
      // groups' order of the B values loaded at the start; N = c)
      const int NC = n * rout;
      const int m = lane & 15, gq = lane >> 4;
      f32x4 a0 = zero4(), a1 = zero4();
      if (m < npg) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a0[e] = 8 * gq + e < rin ? v[m * TTC_MAX_RANK + 8 * gq + e] : 0.f;
          a1[e] = 8 * gq + 4 + e < rin ? v[m * TTC_MAX_RANK + 8 * gq + 4 + e] : 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < kMergeThreads / 128; ++u) {
        const int c = 16 * (wv + 8 * u) + m;
        if (16 * (wv + 8 * u) < NC) {
          f32x4 acc = zero4();
          acc = Mma<float>::mma(a0, f32x4{bl[u][0], bl[u][1], bl[u][2], bl[u][3]}, acc);
          acc = Mma<float>::mma(a1, f32x4{bl[u][4], bl[u][5], bl[u][6], bl[u][7]}, acc);
          // lane (gq, m) holds rows 4gq .. 4gq+3 of column c
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * gq + e < npg && c < NC) ob[(4 * gq + e) * NC + c] = acc[e];
        }
      }
    } else {
      for (int e = tid; e < ni * rout; e += kMergeThreads) {
        const int ii = e / rout, y = e - ii * rout;
        const float* g = left ? G + (int64_t)(i0 + ii) * rout + y : G + ((int64_t)y * n + i0 + ii) * rin;
        float acc[kMergePG];
#pragma unroll
        for (int pg = 0; pg < kMergePG; ++pg) acc[pg] = 0.f;
        merge_dot(acc, g, left ? (int64_t)n * rout : 1, rin, v);
#pragma unroll
        for (int pg = 0; pg < kMergePG; ++pg)
          if (pg < npg) ob[(pg * ci + ii) * rout + y] = acc[pg];
      }
    }
    __syncthreads();
    // packed operand rows [idx][Rpad] and the transpose [Rpad][Nlong], four
    // consecutive entries of a row per thread and store where they are
    // contiguous in memory
    auto packed = [&](int pg, int ii, int j) {
      const int b = j < reff ? live[j] : -1;
      const float val = b >= 0 ? ob[(pg * ci + ii) * rout + b] : 0.f;
      return b >= 0 && !is_b ? dlive[j] * val : val;
    };
    // (left: rows of one prefix, consecutive mode indices adjacent; right:
    // consecutive prefixes adjacent, the order in which their rows follow
    // one another when the chain end's mode is least significant)
    for (int e = 4 * tid; e < npg * ni * Rpad; e += 4 * kMergeThreads) {
      const int r = e / Rpad, j = e - r * Rpad;  // Rpad is a multiple of 4
      const int pg = left ? r / ni : r % npg;
      const int ii = left ? r - pg * ni : r / npg;
      const int64_t idx = lbase[pg] + (int64_t)(i0 + ii) * lsf;
      const f32x4 v = {packed(pg, ii, j), packed(pg, ii, j + 1), packed(pg, ii, j + 2), packed(pg, ii, j + 3)};
      store4<T>(out + idx * Rpad + j, v, 4, true);
    }
    // left half, last mode least significant in the listed order: four
    // consecutive mode indices of one prefix are four consecutive columns
    if (left && lsf == 1 && (ni & 3) == 0 && (i0 & 3) == 0 && (n & 3) == 0 && (Nlong & 3) == 0) {
      for (int e = 4 * tid; e < npg * ni * Rpad; e += 4 * kMergeThreads) {
        const int j = e / (npg * ni);
        const int r = e - j * npg * ni;
        const int pg = r / ni, ii = r % ni;
        const int64_t idx = lbase[pg] + i0 + ii;
        const f32x4 v = {packed(pg, ii, j), packed(pg, ii + 1, j), packed(pg, ii + 2, j), packed(pg, ii + 3, j)};
        store4<T>(outT + (int64_t)j * Nlong + idx, v, 4, true);
      }
    } else if (!left && S >= 2 && a.lstride[d - 1] == 1 && (a.modes[d - 1] & 3) == 0 && (npg & 3) == 0 &&
               (Nlong & 3) == 0) {
      // right half, its chain end's mode least significant in the listed
      // order: four consecutive prefixes of one mode index are four
      // consecutive columns
      for (int e = 4 * tid; e < npg * ni * Rpad; e += 4 * kMergeThreads) {
        const int j = e / (npg * ni);
        const int r = e - j * npg * ni;
        const int pg = r % npg, ii = r / npg;
        const int64_t idx = lbase[pg] + (int64_t)(i0 + ii) * lsf;
        const f32x4 v = {packed(pg, ii, j), packed(pg + 1, ii, j), packed(pg + 2, ii, j), packed(pg + 3, ii, j)};
        store4<T>(outT + (int64_t)j * Nlong + idx, v, 4, true);
      }
    } else for (int e = tid; e < npg * ni * Rpad; e += kMergeThreads) {
      const int j = e / (npg * ni);
      const int r = e - j * npg * ni;
      const int pg = left ? r / ni : r % npg;
      const int ii = left ? r % ni : r / npg;
      const int b = j < reff ? live[j] : -1;
      const float val = b >= 0 ? ob[(pg * ci + ii) * rout + b] : 0.f;
      const E ev = (E)Mma<T>::from_f32(b >= 0 && !is_b ? dlive[j] * val : val);
      const int64_t idx = lbase[pg] + (int64_t)(i0 + ii) * lsf;
      outT[(int64_t)j * Nlong + idx] = ev;
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------
// shared helpers of the streaming kernels
// ------------------------------------------------------------------------------
// store 4 consecutive values of one row; `vec` says the 4-element group is
// aligned and fully in range
template <typename T>
__device__ __forceinline__ void store4(typename Elem<T>::type* p, f32x4 v, int valid, bool vec);

#ifndef TTC_NT_STORE
#define TTC_NT_STORE 0
#endif
template <>
__device__ __forceinline__ void store4<bf16_t>(unsigned short* p, f32x4 v, int valid, bool vec) {
  if (vec && valid >= 4) {
    const unsigned int lo = f32x2_to_bf16x2(v[0], v[1]), hi = f32x2_to_bf16x2(v[2], v[3]);
    const u16x4 o = __builtin_bit_cast(u16x4, (uint2){lo, hi});
#if TTC_NT_STORE
    __builtin_nontemporal_store(__builtin_bit_cast(unsigned long long, o), reinterpret_cast<unsigned long long*>(p));
#else
    *reinterpret_cast<u16x4*>(p) = o;
#endif
  } else {
    for (int e = 0; e < 4 && e < valid; ++e) p[e] = f32_to_bf16(v[e]);
  }
}
template <>
__device__ __forceinline__ void store4<fp8_t>(unsigned char* p, f32x4 v, int valid, bool vec) {
  (void)vec;
  for (int e = 0; e < 4 && e < valid; ++e) p[e] = Mma<fp8_t>::from_f32(v[e]);
}
template <>
__device__ __forceinline__ void store4<float>(float* p, f32x4 v, int valid, bool vec) {
  if (vec && valid >= 4) {
    *reinterpret_cast<f32x4*>(p) = v;
  } else {
    for (int e = 0; e < 4 && e < valid; ++e) p[e] = v[e];
  }
}

#ifndef TTC_SLAB_PAD
#define TTC_SLAB_PAD 16  // bytes of padding per LDS slab row
#endif
// four consecutive values of one row in the activation dtype, as one buffer
// store (a dead store at kNoOff is dropped)
template <typename T>
__device__ __forceinline__ void buf_store4(rsrc_t r, uint32_t off, f32x4 v) {
  if constexpr (sizeof(typename Elem<T>::type) == 2)
    buf_store8(r, off, uint2{f32x2_to_bf16x2(v[0], v[1]), f32x2_to_bf16x2(v[2], v[3])});
  else if constexpr (sizeof(typename Elem<T>::type) == 1)
    buf_store32(r, off, f32x4_to_fp8x4(v[0], v[1], v[2], v[3]));
  else
    buf_store_f32x4(r, off, v);
}

// fp32 partial sums: four consecutive columns of one row, one 16-byte store
// when the row is 16-byte aligned and the four are in range
__device__ __forceinline__ void store_partial4(float* p, f32x4 v, int64_t col, int64_t ncols, bool vec) {
  if (vec && col + 4 <= ncols) {
    *reinterpret_cast<f32x4*>(p) = v;
  } else {
    for (int e = 0; e < 4; ++e)
      if (col + e < ncols) p[e] = v[e];
  }
}

// Geometry shared by the two backward passes for activation type T and NR
// rank tiles of 16.
template <typename T, int NR>
struct Bwd {
  typedef typename Elem<T>::type E;
  static constexpr int ES = sizeof(E);
  static constexpr int EPV = Mma<T>::EPV;
  static constexpr int KSTEP = Mma<T>::KSTEP;
  static constexpr int Rpad = 16 * NR;
  // rank tile narrower than the k-step (e4m3 at 32): the rank-contracting
  // product takes one 32-wide k-step on the fragments' low halves
  static constexpr bool HALF = Rpad % KSTEP != 0;
  static constexpr int SW = 256 / ES;        // slab columns
  static constexpr int SLD = SW + TTC_SLAB_PAD / ES;  // slab row stride (elements), padded
  static constexpr int CTW = SW / 64;        // 16-column tiles per wave per slab
  static constexpr int ZLD = 64 + 16 / ES;   // row stride of a rank-major 64-token tile
  static constexpr int RLD = Rpad + 16 / ES; // row stride of a token-major rank tile
  // 2-byte activations: the token-contracting products read the Z / dZ tile's
  // columns with the transposing LDS read, so the tile is kept token-major
  // only; other types keep a rank-major copy and read its rows
  static constexpr bool ZT = ES == 2;
  static constexpr int ZTILE = ZT ? 64 * RLD : Rpad * ZLD;  // elements of that tile
  static constexpr int SLAB = 64 * SLD;      // elements of one slab buffer
  static constexpr int PER = 4;              // 16-byte slab groups per thread
  static constexpr int ZG = Rpad * ES / 16;  // 16-byte groups per row of a rank tile
  static constexpr int ZPER = (64 * ZG + 255) / 256;
};

// prefetch one 64 x SW slab of a row-major matrix into registers
template <typename T, int NR, bool VEC>
__device__ __forceinline__ void slab_fetch(typename Mma<T>::frag* r, const typename Elem<T>::type* src,
                                           int64_t t0, int64_t T_, int64_t c0, int64_t ncols) {
  typedef Bwd<T, NR> B;
#pragma unroll
  for (int q = 0; q < B::PER; ++q) {
    const int gi = threadIdx.x + 256 * q;
    const int row = gi >> 4, part = gi & 15;
    r[q] = ld_frag<T, VEC>(src, t0 + row, T_, c0 + part * B::EPV, ncols, ncols);
  }
}

template <typename T, int NR>
__device__ __forceinline__ void slab_store(typename Elem<T>::type* lds, const typename Mma<T>::frag* r) {
  typedef Bwd<T, NR> B;
#pragma unroll
  for (int q = 0; q < B::PER; ++q) {
    const int gi = threadIdx.x + 256 * q;
    const int row = gi >> 4, part = gi & 15;
    *reinterpret_cast<typename Mma<T>::frag*>(lds + row * B::SLD + part * B::EPV) = r[q];
  }
}

// prefetch a 64-token x Rpad tile (row-major, act dtype) into registers
template <typename T, int NR>
__device__ __forceinline__ void rank_fetch(typename Mma<T>::frag* r, const typename Elem<T>::type* src,
                                           int64_t t0, int64_t T_) {
  typedef Bwd<T, NR> B;
#pragma unroll
  for (int q = 0; q < B::ZPER; ++q) {
    const int gi = threadIdx.x + 256 * q;
    const int row = gi / B::ZG, part = gi % B::ZG;
    r[q] = load_frag_v<T>(src, gi < 64 * B::ZG ? t0 + row : T_, T_, part * B::EPV, B::Rpad, B::Rpad);
  }
}

// Buffer-load forms of the two prefetches (16-byte rows only).  `src` covers
// the work-group's token range from its first token; `row0` is the slab's
// first row in that range.  Rows past the last token lie beyond the resource
// and read as zero; a dead fetch (`live` false) issues the same loads at
// kNoOff, which return zero without touching memory.
template <typename T, int NR>
__device__ __forceinline__ void slab_fetch_b(typename Mma<T>::frag* r, rsrc_t src, int row0, int64_t c0,
                                             int64_t ncols, bool live) {
  typedef Bwd<T, NR> B;
#pragma unroll
  for (int q = 0; q < B::PER; ++q) {
    const int gi = threadIdx.x + 256 * q;
    const int row = gi >> 4, part = gi & 15;
    const int64_t col = c0 + part * B::EPV;
    const uint32_t o = (uint32_t)(((int64_t)(row0 + row) * ncols + col) * B::ES);
    r[q] = buf_frag_last<T>(src, (live & (col < ncols)) ? o : kNoOff);
  }
}

// Rank columns at or past r_eff are zero in the tile and are not read.
template <typename T, int NR>
__device__ __forceinline__ void rank_fetch_b(typename Mma<T>::frag* r, rsrc_t src, int row0, bool live, int reff) {
  typedef Bwd<T, NR> B;
#pragma unroll
  for (int q = 0; q < B::ZPER; ++q) {
    const int gi = threadIdx.x + 256 * q;
    const int row = gi / B::ZG, part = gi % B::ZG;
    const uint32_t o = (uint32_t)(((row0 + row) * B::Rpad + part * B::EPV) * B::ES);
    r[q] = buf_frag<T>(src, (live & (gi < 64 * B::ZG) & (part * B::EPV < reff)) ? o : kNoOff);
  }
}

// write a prefetched rank tile rank-major (transposed) and optionally token-major
template <typename T, int NR>
__device__ __forceinline__ void rank_store(typename Elem<T>::type* tr, typename Elem<T>::type* rm,
                                           const typename Mma<T>::frag* r) {
  typedef Bwd<T, NR> B;
#pragma unroll
  for (int q = 0; q < B::ZPER; ++q) {
    const int gi = threadIdx.x + 256 * q;
    if (gi < 64 * B::ZG) {
      const int row = gi / B::ZG, part = gi % B::ZG;
      if (tr) {
#pragma unroll
        for (int e = 0; e < B::EPV; ++e) tr[(part * B::EPV + e) * B::ZLD + row] = r[q][e];
      }
      if (rm) *reinterpret_cast<typename Mma<T>::frag*>(rm + row * B::RLD + part * B::EPV) = r[q];
    }
  }
}

// ------------------------------------------------------------------------------
// forward
// ------------------------------------------------------------------------------
// LDS of the forward: the Z reduction area (NW waves x 16*TT tokens x Rpad
// fp32) is dead once Z is summed; the Z tile (16*TT tokens, act dtype) then
// sits at offset 0 and two staged Y chunks of 16*TT rows x (at most) 256 columns
// follow it, overlaying the rest of the reduction area.
template <typename T, int NR, int TT>
constexpr int kFwdStageOff() {
  return ((16 * TT) * (16 * NR + 16 / (int)sizeof(typename Elem<T>::type)) * (int)sizeof(typename Elem<T>::type) +
          255) / 256 * 256;
}
// output tiles per wave and step of the forward's second product
constexpr int kFwdUO(int NR, int NW) { return NW == 8 ? 2 : (NR <= 2 ? 4 : 2); }
template <typename T, int NR, int TT, int NW>
constexpr size_t kFwdLdsBytes() {
  constexpr size_t red = (size_t)NW * 16 * TT * 16 * NR * 4;
  constexpr size_t stg = (size_t)kFwdStageOff<T, NR, TT>() + 2 * (size_t)(16 * TT) *
                                                                (256 + 16 / sizeof(typename Elem<T>::type)) *
                                                                sizeof(typename Elem<T>::type);
  // the x batch of the row-pattern loads: 16*TT rows of NW*UNR k-steps
  // (64 bytes each) plus a 16-byte pad
  constexpr size_t xs = (size_t)(16 * TT) * (NW * (NR <= 2 ? 2 : 1) * 64 + 16);
  return red > stg ? (red > xs ? red : xs) : (stg > xs ? stg : xs);
}

// NW waves per work-group split the input columns of the first product and
// the output tiles of the second.  Every work-group reads all of A and B, and
// those reads (L2 hits) count against the same per-CU load throughput as the
// reads of x, so the wide variant (NW = 8, 64 tokens, one work-group per CU)
// reads A and B half as often per token as two 32-token work-groups.
// Layers of one streaming launch: work-group i belongs to the layer q with
// first[q] <= i < first[q + 1] and runs as work-group i - first[q] of that
// layer's own grid (independent layers, e.g. the Q, K and V projections of an
// encoder, share one launch: one ramp-up and one tail instead of three).
constexpr int kMaxStream = 4;
template <typename T>
struct FwdArgs {
  const typename Elem<T>::type* x;
  const typename Elem<T>::type* Ac;
  const typename Elem<T>::type* Bc;
  typename Elem<T>::type* Z;
  typename Elem<T>::type* y;
  const int* meta;  // live-slice map of the split link (r_eff)
  int64_t T_, N_in, N_out;
  int vin, vout;
  int cg_n;  // column groups per token tile (>= 1, at most the tile's output steps)
};
template <typename A>
struct StreamBatch {
  A a[kMaxStream];
  int first[kMaxStream + 1];
  int n;
};
template <typename A>
__device__ __forceinline__ int batch_layer(const StreamBatch<A>& b, unsigned* local) {
  int q = 0;
  while (q < b.n - 1 && (int)blockIdx.x >= b.first[q + 1]) ++q;
  *local = blockIdx.x - (unsigned)b.first[q];
  return q;
}

#ifndef TTC_FWD_WIDE_UNR
#define TTC_FWD_WIDE_UNR 2
#endif
#ifndef TTC_FWD_WIDE_WPE
#define TTC_FWD_WIDE_WPE 1
#endif
// XR: x read in whole 256-byte row pieces (a wave instruction covers four
// rows) and staged through LDS, instead of straight into the fragment layout
// (a wave instruction there covers 16 rows x 64 bytes).  With the operand A
// read alongside from the L2, the row pieces stream at 5.2 against 3.7 TB/s
// (100 MB over 256 work-groups, a 3072-wide x); the launch takes this path
// for 2-byte rows of at least TTC_FWD_XROWS_BYTES (long k loops; with one
// or two batches per work-group the staging barriers cost more than the
// pattern gains: 768-wide inputs, Q+K+V 37.5 -> 42 us, FFN1 28.8 -> 30 us).
#ifndef TTC_FWD_XROWS
#define TTC_FWD_XROWS 1
#endif
#ifndef TTC_FWD_XROWS_BYTES
#define TTC_FWD_XROWS_BYTES 4096
#endif
// the row pieces with the streaming (non-temporal) hint.  Measured on the
// six-layer step: the dX pass of FFN2, which follows its forward, then reads
// its x from HBM (36.5 -> 43 us), but the passes after it gain more (O and
// FFN1 dX 15.5 -> 13.8 us, Q, K, V dX 33 -> 30.5 us): 0.3527 against
// 0.3452 ms per step without and with the hint
#ifndef TTC_FWD_XR_NT
#define TTC_FWD_XR_NT 1
#endif
#ifndef TTC_FWD_XR_NT_BYTES
#define TTC_FWD_XR_NT_BYTES 4096
#endif
// PS passes of 16*TT tokens per work-group (PS > 1 with 16-byte rows only):
// the first x batches of pass p + 1 and, with one rank tile pair, its first B
// fragments are requested before the stores of pass p, so that they arrive
// while pass p sums Z and writes Y.
template <typename T, int NR, bool VEC, int TT, int NW, int PS, int XRW>
__global__ __launch_bounds__(64 * NW, (NW == 8 ? TTC_FWD_WIDE_WPE : 1)) void k_fwd(StreamBatch<FwdArgs<T>> fb) {
  static_assert(PS == 1 || (VEC && NW == 8), "passes need 16-byte rows and one work-group per tile");
  typedef typename Elem<T>::type E;
  unsigned bid;
  const FwdArgs<T>& fa_ = fb.a[batch_layer(fb, &bid)];
  const E* __restrict__ x = fa_.x;
  const E* __restrict__ Ac = fa_.Ac;
  const E* __restrict__ Bc = fa_.Bc;
  E* __restrict__ Z = fa_.Z;
  E* __restrict__ y = fa_.y;
  const int64_t T_ = fa_.T_, N_in = fa_.N_in, N_out = fa_.N_out;
  const int vin = fa_.vin, vout = fa_.vout;
  // With few token tiles the output steps of a tile are split over cg_n
  // work-groups: work-group (tile, cg) computes the tile's Z and writes the
  // output steps cg, cg + cg_n, ...; only group 0 stores Z.  The wide
  // variant runs only with a tile for every CU and never splits.
  const int cg_n = NW == 8 ? 1 : fa_.cg_n;
  const int cg = (int)(bid % (unsigned)cg_n);
  bid /= (unsigned)cg_n;
  typedef typename Mma<T>::frag frag;
  constexpr int Rpad = 16 * NR;
  constexpr int EPV = Mma<T>::EPV, KSTEP = Mma<T>::KSTEP;
  constexpr int ZLD = Rpad + 16 / (int)sizeof(E);
  // k-steps per batch of loads and output tiles per wave and step: fewer for
  // the wider rank tiles, so that two batches in flight, the accumulators
  // and three batches of B fragments stay within about 128 registers
  constexpr int NT = 64 * NW;                           // threads
  constexpr int UNR = NW == 8 ? (NR <= 2 ? TTC_FWD_WIDE_UNR : 1) : (NR <= 2 ? 4 : 1);
  // a rank tile narrower than the k-step (e4m3 at 32): one 32-wide k-step
  // on the low halves of the fragments
  constexpr bool HALF = Rpad % KSTEP != 0;
  constexpr int KS = HALF ? 1 : Rpad / KSTEP;
  constexpr int UO = kFwdUO(NR, NW);
  constexpr int TPS = NW * UO;                           // output tiles per step (all waves)
  extern __shared__ __align__(16) char smem[];
  constexpr int TP = 16 * TT;                     // tokens per pass
  constexpr int TM = TP * PS;                     // tokens per work-group
  float* zred = reinterpret_cast<float*>(smem);  // [NW waves][TP tokens][Rpad]
  E* zl = reinterpret_cast<E*>(smem);            // [TP][ZLD], reuses zred after the sum

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int64_t t0 = (int64_t)bid * TM;

  f32x4 acc[TT][NR];
#pragma unroll
  for (int u = 0; u < TT; ++u)
#pragma unroll
    for (int n = 0; n < NR; ++n) acc[u][n] = zero4();

  // Loads and stores share one in-order completion counter, so a load issued
  // after a store cannot be waited for before that store completes.  Every
  // batch of operands is therefore requested one step ahead, before the
  // stores of the current step: the first B fragments at the very start,
  // the next x / A batch before the current batch's MFMAs.  With 16-byte
  // rows (VEC) every load and store is a buffer access and every batch and
  // output step runs, dead ones at kNoOff, so the count of memory operations
  // between a request and its use is the same on every path and each wait
  // leaves the later requests in flight.
  const int64_t nrows = std::min<int64_t>(TM, T_ - t0);
  const rsrc_t rx = make_rsrc(x + t0 * N_in, nrows * N_in * (int64_t)sizeof(E));
  const rsrc_t ra = make_rsrc(Ac, (int64_t)Rpad * N_in * (int64_t)sizeof(E));
  const rsrc_t rb = make_rsrc(Bc, N_out * Rpad * (int64_t)sizeof(E));
  const rsrc_t rz = make_rsrc(Z + t0 * Rpad, nrows * Rpad * (int64_t)sizeof(E));
  const rsrc_t ry = make_rsrc(y + t0 * N_out, nrows * N_out * (int64_t)sizeof(E));
  // rows of A and columns of B at or past the live rank r_eff are zero (the
  // merge compacts the live slices of the split link to the front)
  const int reff = fa_.meta[kMetaReff];
  const int not_ = (int)((N_out + 15) / 16);
  frag fo0[UO][KS], fo1[UO][KS], fo2[UO][KS];
  auto fetch_b = [&](frag (&f)[UO][KS], int ob, bool live) {
#pragma unroll
    for (int uo = 0; uo < UO; ++uo)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int64_t row = (int64_t)(ob + NW * uo) * 16 + c;
        if constexpr (HALF) {
          if constexpr (VEC)
            f[uo][0] = buf_frag_lo8<T>(rb, (live & (row < N_out) & (8 * g < reff))
                                               ? (uint32_t)((row * Rpad + 8 * g) * (int64_t)sizeof(E))
                                               : kNoOff);
          else
            f[uo][0] = load_frag_lo8<T>(Bc, row, N_out, 8 * g, Rpad);
        } else if constexpr (VEC) {
          const uint32_t o = (uint32_t)((row * Rpad + ks * KSTEP + g * EPV) * (int64_t)sizeof(E));
          // ranks at or past r_eff are zero in B: not read (a load at kNoOff is zero)
          f[uo][ks] = buf_frag<T>(rb, (live & (row < N_out) & (ks * KSTEP + g * EPV < reff)) ? o : kNoOff);
        } else {
          f[uo][ks] = load_frag_v<T>(Bc, row, N_out, ks * KSTEP + g * EPV, Rpad, Rpad);
        }
      }
  };
  // Likewise for B: work-group b visits its column group's output steps (TPS
  // tiles each) starting at its step b mod nsteps.
  const int nsteps = ((not_ + TPS - 1) / TPS - cg + cg_n - 1) / cg_n;  // this group's steps
  const int rot2 = (int)(bid % (unsigned)nsteps);
  auto ostep = [&](int sidx) { return (cg + cg_n * ((sidx + rot2) % nsteps)) * TPS; };
  // with one rank tile pair the first B batches are requested right away;
  // wider ranks wait for phase 2 (register budget)
  if constexpr (NR <= 2) {
    fetch_b(fo0, ostep(0) + w, true);
    fetch_b(fo1, ostep(1) + w, nsteps > 1);
  }

  // Z = x A^T: M = token, N = rank, K = input column; wave w takes the
  // k-steps w, w+NW, ... so the waves read adjacent 64-byte pieces.
  // Two register buffers, unrolled by two so that both stay in registers.
  const int nks = (int)((N_in + KSTEP - 1) / KSTEP);
  constexpr int KB = NW * UNR;
  frag fa0[UNR][TT], fb0[UNR][NR], fa1[UNR][TT], fb1[UNR][NR];
  auto fetch_x = [&](frag (&xa)[UNR][TT], frag (&xb)[UNR][NR], int p, int kb, bool live) {
    if (!VEC && !live) return;
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t col = (int64_t)(kb + NW * u + w) * KSTEP + g * EPV;
      if constexpr (VEC) {
        const bool ok = live & (col < N_in);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
          xa[u][tt] = buf_frag<T>(rx, ok ? (uint32_t)(((p * TP + 16 * tt + c) * N_in + col) * (int64_t)sizeof(E)) : kNoOff);
#pragma unroll
        for (int n = 0; n < NR; ++n)
          xb[u][n] = buf_frag<T>(ra, (ok & (16 * n + c < reff)) ? (uint32_t)(((16 * n + c) * N_in + col) * (int64_t)sizeof(E))
                                                               : kNoOff);
      } else {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) xa[u][tt] = ld_frag<T, VEC>(x, t0 + 16 * tt + c, T_, col, N_in, N_in);
#pragma unroll
        for (int n = 0; n < NR; ++n) xb[u][n] = ld_frag<T, VEC>(Ac, 16 * n + c, Rpad, col, N_in, N_in);
      }
    }
  };
  auto mma_x = [&](const frag (&xa)[UNR][TT], const frag (&xb)[UNR][NR]) {
#pragma unroll
    for (int u = 0; u < UNR; ++u)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int n = 0; n < NR; ++n) acc[tt][n] = Mma<T>::mma(xa[u][tt], xb[u][n], acc[tt][n]);
  };
  // Every work-group reads the same A; each starts at a different batch so
  // that concurrent requests for A spread over the L2 channels instead of
  // queueing on the same lines.
  const int nkb = (nks + KB - 1) / KB;
  const int rot1 = (int)(bid % (unsigned)nkb);
  auto kbat = [&](int j) { return ((j + rot1) % nkb) * KB; };
  // with several passes the batch stream runs on across them: both buffers
  // hold a batch in flight at every MFMA (the batch count of a pass rounded
  // up to even, the extra batch dead), the last two of pass p being the first
  // two of pass p + 1
  const int nkb2 = PS > 1 ? (nkb + 1) & ~1 : nkb;
  // the row-pattern path (16-byte rows, one pass, 64-token work-groups)
  constexpr bool XR = XRW > 0 && VEC && PS == 1 && NW == 8 && TT == 4;
  constexpr int RB = KB * 64;            // bytes of a row in one batch
  constexpr int CPR = RB / 256;          // 256-byte pieces per row and batch
  constexpr int XI = XR ? 16 * TT * CPR / 4 / NW : 1;  // wave instructions per batch
  constexpr int XLD = RB + 16;           // staged row stride (bytes)
  static_assert(!XR || (KSTEP * (int)sizeof(E) == 64 && RB % 256 == 0 && XI == UNR * TT), "row-pattern geometry");
  static_assert(!XR || (size_t)(16 * TT) * XLD <= kFwdLdsBytes<T, NR, TT, NW>(), "the staged batch fits");
  char* xs = smem;
  // (the row-piece path requests its first batches in its own loop)
  if constexpr (!XR && PS == 1) {
    fetch_x(fa0, fb0, 0, kbat(0), true);
  } else if constexpr (!XR) {
    fetch_x(fa0, fb0, 0, kbat(0), true);
    fetch_x(fa1, fb1, 0, kbat(1), 1 < nkb);
  }

  // Y^T = B Z^T: M = output column, N = token, K = rank.  The waves
  // cover TPS output tiles per step; the step's Y tile goes through LDS so
  // that it leaves as whole-row 16-byte stores.  Every out-step loop runs a
  // multiple of three steps (the B buffers rotate by three); with several
  // passes and one rank tile pair the fragment requests of the last two steps
  // of pass p are the first two steps of pass p + 1.
  constexpr int CW = 16 * TPS;                  // columns per step
  constexpr int YLD = CW + 16 / (int)sizeof(E);  // staged row stride
  E* ys0 = reinterpret_cast<E*>(smem + kFwdStageOff<T, NR, TT>());
  E* ys1 = ys0 + TP * YLD;
  constexpr int GPR = CW * (int)sizeof(E) / 16;  // 16-byte groups per staged row
  const int ns3 = (nsteps + 2) / 3 * 3;
  auto out_step = [&](const frag (&f)[UO][KS], frag (&fn)[UO][KS], int p, int sidx, E* ys) {
    const bool live = sidx < nsteps;
    const int ob0 = ostep(sidx);
#pragma unroll
    for (int uo = 0; uo < UO; ++uo) {
      const int lt = w + NW * uo;
#pragma unroll
      for (int u = 0; u < TT; ++u) {
        f32x4 a2 = zero4();
        if constexpr (HALF) {
          a2 = Mma<T>::mma_k32(f[uo][0], lds_frag_lo8<T>(zl + (16 * u + c) * ZLD + 8 * g), a2);
        } else {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            a2 = Mma<T>::mma(f[uo][ks], lds_frag<T>(zl + (16 * u + c) * ZLD + ks * KSTEP + g * EPV), a2);
        }
        E* d = ys + (16 * u + c) * YLD + lt * 16 + 4 * g;
        if constexpr (sizeof(E) == 2) {
          const uint2 pk = {f32x2_to_bf16x2(a2[0], a2[1]), f32x2_to_bf16x2(a2[2], a2[3])};
          *reinterpret_cast<uint2*>(d) = pk;
        } else if constexpr (sizeof(E) == 1) {
          *reinterpret_cast<unsigned*>(d) = f32x4_to_fp8x4(a2[0], a2[1], a2[2], a2[3]);
        } else {
#pragma unroll
          for (int vv = 0; vv < 4; ++vv) d[vv] = (E)Mma<T>::from_f32(a2[vv]);
        }
      }
    }
    if constexpr (PS > 1 && NR <= 2) {
      const int nx = sidx + 2;
      const bool wrap = nx >= ns3;
      fetch_b(fn, ostep(wrap ? nx - ns3 : nx) + w, wrap ? (p + 1 < PS) & (nx - ns3 < nsteps) : nx < nsteps);
    } else if (VEC || sidx + 2 < nsteps) {
      fetch_b(fn, ostep(sidx + 2) + w, sidx + 2 < nsteps);
    }
    lds_barrier();
    const int64_t c0 = (int64_t)ob0 * 16;
    const int64_t ncol = std::min<int64_t>(CW, N_out - c0);
    if constexpr (VEC) {
      constexpr int EPG = 16 / (int)sizeof(E);
      static_assert(TP * GPR % NT == 0, "whole 16-byte groups per thread");
#pragma unroll
      for (int k = 0; k < TP * GPR / NT; ++k) {
        const int idx = threadIdx.x + NT * k;
        const int row = idx / GPR, gr = idx - row * GPR;
        const int64_t col = c0 + gr * EPG;
        const uint32_t o = (uint32_t)(((p * TP + row) * N_out + col) * (int64_t)sizeof(E));
        buf_store16(ry, (live & (col < N_out)) ? o : kNoOff, *reinterpret_cast<const uint4*>(ys + row * YLD + gr * EPG));
      }
    } else if (vout && (ncol % (16 / (int)sizeof(E))) == 0) {
      const int ngr = (int)(ncol * (int64_t)sizeof(E) / 16);
      for (int idx = threadIdx.x; idx < TP * GPR; idx += NT) {
        const int row = idx / GPR, gr = idx - row * GPR;
        if (gr < ngr && t0 + row < T_)
          *reinterpret_cast<uint4*>(y + (t0 + row) * N_out + c0 + gr * (16 / (int)sizeof(E))) =
              *reinterpret_cast<const uint4*>(ys + row * YLD + gr * (16 / (int)sizeof(E)));
      }
    } else {
      for (int idx = threadIdx.x; idx < TP * CW; idx += NT) {
        const int row = idx / CW, col = idx - row * CW;
        if (col < ncol && t0 + row < T_) y[(t0 + row) * N_out + c0 + col] = ys[row * YLD + col];
      }
    }
  };

#pragma unroll
  for (int p = 0; p < PS; ++p) {
    if (p > 0) {
#pragma unroll
      for (int u = 0; u < TT; ++u)
#pragma unroll
        for (int n = 0; n < NR; ++n) acc[u][n] = zero4();
    }
    if constexpr (XR) {
      // batch kb: rows 0..TM-1, bytes [kb*64, kb*64 + RB) of each row; wave
      // instruction i = q*NW + w covers rows 4(i / CPR) .. +3, piece i % CPR
      frag xr0[XI], xr1[XI];
      auto fetch_xr = [&](frag (&r)[XI], int kb, bool live) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < XI; ++q) {
          const int i = q * NW + w;
          const int row = 4 * (i / CPR) + (lane >> 4);
          const int64_t cb = (int64_t)kb * 64 + (i % CPR) * 256 + (lane & 15) * 16;
          const uint32_t o = (live & (cb < N_in * (int64_t)sizeof(E))) ? (uint32_t)(row * N_in * (int64_t)sizeof(E) + cb)
                                                                       : kNoOff;
          r[q] = XRW == 2 ? buf_frag_last<T>(rx, o) : buf_frag<T>(rx, o);
        }
      };
      // every wave is done with the previous batch before the store, and the
      // batch is in LDS before any wave reads it
      auto stage = [&](const frag (&r)[XI]) __attribute__((always_inline)) {
        lds_barrier();
#pragma unroll
        for (int q = 0; q < XI; ++q) {
          const int i = q * NW + w;
          const int row = 4 * (i / CPR) + (lane >> 4);
          *reinterpret_cast<frag*>(xs + row * XLD + (i % CPR) * 256 + (lane & 15) * 16) = r[q];
        }
        lds_barrier();
      };
      // Z += x A^T over the wave's k-steps NW*u + w of the staged batch
      auto mma_s = [&](const frag (&xb)[UNR][NR]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < UNR; ++u)
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) {
            const frag xa = *reinterpret_cast<const frag*>(xs + (16 * tt + c) * XLD + (NW * u + w) * 64 + g * 16);
#pragma unroll
            for (int n = 0; n < NR; ++n) acc[tt][n] = Mma<T>::mma(xa, xb[u][n], acc[tt][n]);
          }
      };
      // the A fragments of a batch: rows 16n + c, the wave's k-steps
      auto fetch_a = [&](frag (&xb)[UNR][NR], int kb, bool live) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const int64_t col = (int64_t)(kb + NW * u + w) * KSTEP + g * EPV;
          const bool ok = live & (col < N_in);
#pragma unroll
          for (int n = 0; n < NR; ++n)
            xb[u][n] = buf_frag<T>(ra, (ok & (16 * n + c < reff)) ? (uint32_t)(((16 * n + c) * N_in + col) * (int64_t)sizeof(E))
                                                                 : kNoOff);
        }
      };
      // two batches in flight; the scheduling barriers keep every request
      // ahead of the products that do not need it
      // (in the order the loop's waits assume: x then A of batch 0, then of
      // batch 1; each wait then leaves the younger batch in flight)
      fetch_xr(xr0, kbat(0), true);
      __builtin_amdgcn_sched_barrier(0);
      fetch_a(fb0, kbat(0), true);
      __builtin_amdgcn_sched_barrier(0);
      fetch_xr(xr1, kbat(1), 1 < nkb);
      __builtin_amdgcn_sched_barrier(0);
      fetch_a(fb1, kbat(1), 1 < nkb);
      __builtin_amdgcn_sched_barrier(0);
      for (int j = 0; j < nkb; j += 2) {
        stage(xr0);
        __builtin_amdgcn_sched_barrier(0);
        fetch_xr(xr0, kbat(j + 2), j + 2 < nkb);
        __builtin_amdgcn_sched_barrier(0);
        mma_s(fb0);
        __builtin_amdgcn_sched_barrier(0);
        fetch_a(fb0, kbat(j + 2), j + 2 < nkb);
        __builtin_amdgcn_sched_barrier(0);
        stage(xr1);  // a dead batch is zeros and adds nothing
        __builtin_amdgcn_sched_barrier(0);
        fetch_xr(xr1, kbat(j + 3), j + 3 < nkb);
        __builtin_amdgcn_sched_barrier(0);
        mma_s(fb1);
        __builtin_amdgcn_sched_barrier(0);
        fetch_a(fb1, kbat(j + 3), j + 3 < nkb);
        __builtin_amdgcn_sched_barrier(0);
      }
      lds_barrier();  // the reduction area overlays the staged batch
    } else if constexpr (PS == 1) {
      for (int j = 0; j < nkb; j += 2) {
        fetch_x(fa1, fb1, 0, kbat(j + 1), j + 1 < nkb);
        mma_x(fa0, fb0);
        if (!VEC && j + 1 >= nkb) break;
        fetch_x(fa0, fb0, 0, kbat(j + 2), j + 2 < nkb);
        mma_x(fa1, fb1);  // a dead batch is zeros and adds nothing
      }
    } else {
      for (int j = 0; j < nkb2; j += 2) {
        mma_x(fa0, fb0);
        {
          const int k = j + 2;
          const bool nx = k >= nkb2;
          fetch_x(fa0, fb0, nx ? p + 1 : p, kbat(nx ? k - nkb2 : k), nx ? (p + 1 < PS) : k < nkb);
        }
        mma_x(fa1, fb1);  // a dead batch is zeros and adds nothing
        {
          const int k = j + 3;
          const bool nx = k >= nkb2;
          fetch_x(fa1, fb1, nx ? p + 1 : p, kbat(nx ? k - nkb2 : k), nx ? (p + 1 < PS) & (k - nkb2 < nkb) : k < nkb);
        }
      }
      // the previous pass's out steps are done with the Z tile and the
      // staging buffers that the reduction area overlays
      if (p > 0) lds_barrier();
    }
    // lane (g, c) holds Z rows 4g+v of token tile u, rank column 16n+c
#pragma unroll
    for (int u = 0; u < TT; ++u)
#pragma unroll
      for (int n = 0; n < NR; ++n)
#pragma unroll
        for (int vv = 0; vv < 4; ++vv) zred[(w * TP + 16 * u + 4 * g + vv) * Rpad + 16 * n + c] = acc[u][n][vv];
    lds_barrier();
    constexpr int PER = TP * Rpad / NT;
    float zs[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = threadIdx.x + NT * i;
      float z = zred[idx];
#pragma unroll
      for (int v = 1; v < NW; ++v) z += zred[v * TP * Rpad + idx];
      zs[i] = z;
    }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = threadIdx.x + NT * i;
      const int tt = idx / Rpad, j = idx % Rpad;
      const E e = (E)Mma<T>::from_f32(zs[i]);
      if constexpr (VEC)
        buf_store(rz, cg == 0 ? (uint32_t)(((p * TP + tt) * Rpad + j) * (int)sizeof(E)) : kNoOff, e);
      else if (cg == 0 && t0 + tt < T_)
        Z[(t0 + tt) * Rpad + j] = e;
      zl[tt * ZLD + j] = e;
    }
    lds_barrier();

    if constexpr (NR > 2) {
      fetch_b(fo0, ostep(0) + w, true);
      fetch_b(fo1, ostep(1) + w, nsteps > 1);
    }
    // three fragment buffers: the fragments of step s + 2 are requested in
    // step s, so waiting for them never waits for the stores of step s + 1
    // staging buffers alternate by step parity: a buffer is rewritten two
    // steps later, after the barrier of the step in between
    for (int sidx = 0; sidx < nsteps; sidx += 3) {
      out_step(fo0, fo2, p, sidx, (sidx & 1) ? ys1 : ys0);
      if (!VEC && sidx + 1 >= nsteps) break;
      out_step(fo1, fo0, p, sidx + 1, (sidx & 1) ? ys0 : ys1);
      if (!VEC && sidx + 2 >= nsteps) break;
      out_step(fo2, fo1, p, sidx + 2, (sidx & 1) ? ys1 : ys0);
    }
  }
}

// ------------------------------------------------------------------------------
// backward, dY pass
// ------------------------------------------------------------------------------
// Items (slabs) in flight per work-group in the two backward passes: one
// register set per item, the slab of item it + depth requested while item it
// is computed from LDS.
#ifndef TTC_BWD_DEPTH
#define TTC_BWD_DEPTH 2
#endif
constexpr int kBwdDepth = TTC_BWD_DEPTH;
static_assert(kBwdDepth == 2 || kBwdDepth == 3, "two or three items in flight");
template <typename T>
struct DyArgs {
  const typename Elem<T>::type* dy;
  const typename Elem<T>::type* BcT;  // Rpad x N_out
  const typename Elem<T>::type* Z;    // T x Rpad
  float* dZp;                         // gc x T x Rpad partials (gc > 1)
  typename Elem<T>::type* dZ;         // T x Rpad
  float* dBp;                         // gt x Rpad x N_out partials (rows < r_eff)
  const int* meta;
  int* gts;                           // [0] <- token groups of this launch (for the reduction)
  int64_t T_, N_out;
  int nsl, tpg, ntiles, gc_n, vec;
};

// calls f(integral_constant<int, I>) for I = B_ .. E_-1
template <int B_, int E_, typename Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
  if constexpr (B_ < E_) {
    f(std::integral_constant<int, B_>{});
    static_for<B_ + 1, E_>(f);
  }
}

// NSL > 0 (16-byte rows, two items in flight): the launch's work-groups own
// at most NSL slabs and the item loop is unrolled over them, so that every
// item's slab, and with it its dB^T accumulators, is known at compile time
// (a slab chosen at run time among NSM accumulator sets makes the compiler
// copy the sets at every item); a work-group with fewer slabs runs the
// missing ones on zeros (dead loads), and with NSL odd the tile count is
// rounded up to even the same way.  NSL = 0: the slab of an item at run time.
template <typename T, int NR, bool VEC, int NSL>
__global__ __launch_bounds__(256) void k_bwd_dy(StreamBatch<DyArgs<T>> bb) {
  unsigned bid;
  const DyArgs<T>& a = bb.a[batch_layer(bb, &bid)];
  typedef Bwd<T, NR> B;
  typedef typename B::E E;
  typedef typename Mma<T>::frag frag;
  static_assert(NSL == 0 || (VEC && kBwdDepth == 2), "static slabs need 16-byte rows and two items in flight");
  constexpr int NSM = NSL > 0 ? NSL : bwd_max_slabs(B::ES, NR);
  constexpr int BLD = NSM * B::SW + 16 / B::ES;
  extern __shared__ __align__(16) char smem[];
  E* btl = reinterpret_cast<E*>(smem);            // [Rpad][BLD]: B^T for the column range
  E* slab = btl + B::Rpad * BLD;                  // [2][64][SLD]
  E* ztl = slab + 2 * B::SLAB;  // Z of the current tile: [64][RLD] (ZT), else Z^T [Rpad][ZLD]

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int gc = (int)(bid % (unsigned)a.gc_n), gt = (int)(bid / (unsigned)a.gc_n);
  const int64_t c0 = (int64_t)gc * a.nsl * B::SW;
  const int nsl = (int)std::min<int64_t>(a.nsl, (a.N_out - c0 + B::SW - 1) / B::SW);
  const int reff = a.meta[kMetaReff];
  const int tt0 = gt * a.tpg;
  const int ntt = std::min(a.ntiles, tt0 + a.tpg) - tt0;
  const int nitems = ntt * nsl;
  const int64_t tb = (int64_t)tt0 * 64;
  const int64_t nrow = std::min<int64_t>(a.T_ - tb, (int64_t)ntt * 64);
  // items per tile and items run (static slabs: NSL per tile, an even tile
  // count when NSL is odd; the extra items are dead)
  const int ipt = NSL > 0 ? NSL : nsl;
  const int ntt_run = (NSL & 1) ? (ntt + 1) & ~1 : ntt;
  const int nit = NSL > 0 ? ntt_run * NSL : nitems;

  f32x4 accB[NSM][B::CTW][NR];
#pragma unroll
  for (int s = 0; s < NSM; ++s)
#pragma unroll
    for (int ct = 0; ct < B::CTW; ++ct)
#pragma unroll
      for (int n = 0; n < NR; ++n) accB[s][ct][n] = zero4();
  f32x4 accZ[NR];

  // one register set per item in flight: the slab (and, at a tile start,
  // the Z tile) of item it + depth is requested while item it is computed
  // from LDS
  frag srA[B::PER], srB[B::PER], srC[B::PER], zrA[B::ZPER], zrB[B::ZPER], zrC[B::ZPER];
  // With 16-byte rows every fetch, store and item is unconditional (buffer
  // accesses, dead ones at kNoOff), so the count of memory operations between
  // a fetch and its use is the same on every path and the wait before an item
  // leaves the later fetches in flight.
  const rsrc_t rsl = make_rsrc(a.dy + tb * a.N_out, nrow * a.N_out * B::ES);
  const rsrc_t rzt = make_rsrc(a.Z + tb * B::Rpad, nrow * B::Rpad * B::ES);
  const rsrc_t rdz = a.gc_n == 1 ? make_rsrc(a.dZ + tb * B::Rpad, nrow * B::Rpad * B::ES)
                                 : make_rsrc(a.dZp + ((int64_t)gc * a.T_ + tb) * B::Rpad, nrow * B::Rpad * 4);
  auto fetch = [&](int it, frag* sr, frag* zr) {
    if constexpr (VEC) {
      const int itc = it < nit ? it : 0;
      const int tn = itc / ipt, sn = itc - tn * ipt;
      const bool tile = (it < nit) & (tn < ntt);
      slab_fetch_b<T, NR>(sr, rsl, tn * 64, c0 + (int64_t)sn * B::SW, a.N_out, tile & (sn < nsl));
      rank_fetch_b<T, NR>(zr, rzt, tn * 64, tile & (sn == 0), reff);
    } else if (it < nitems) {
      const int tn = tt0 + it / nsl, sn = it % nsl;
      slab_fetch<T, NR, VEC>(sr, a.dy, (int64_t)tn * 64, a.T_, c0 + (int64_t)sn * B::SW, a.N_out);
      if (sn == 0) rank_fetch<T, NR>(zr, a.Z, (int64_t)tn * 64, a.T_);
    }
  };

  // B^T rows of this column range; with 16-byte rows a fixed number of loads
  // per thread, requested before the first two items so that the latencies
  // overlap
  {
    // (static slabs: all NSL slabs' columns, zero past the work-group's own)
    const int gpr = (NSL > 0 ? NSL : nsl) * B::SW / B::EPV;
    if constexpr (VEC) {
      constexpr int BPER = (B::Rpad * NSM * B::SW / B::EPV + 255) / 256;
      const rsrc_t rb = make_rsrc(a.BcT, (int64_t)B::Rpad * a.N_out * B::ES);
      frag bt[BPER];
#pragma unroll
      for (int q = 0; q < BPER; ++q) {
        const int gi = tid + 256 * q;
        const int j = gi / gpr, part = gi - j * gpr;
        const int64_t col = c0 + part * B::EPV;
        const uint32_t o = (uint32_t)(((int64_t)j * a.N_out + col) * B::ES);
        bt[q] = buf_frag<T>(rb, ((gi < B::Rpad * gpr) & (col < a.N_out) & (j < reff)) ? o : kNoOff);
      }
      fetch(0, srA, zrA);
      fetch(1, srB, zrB);
      if constexpr (kBwdDepth == 3) fetch(2, srC, zrC);
#pragma unroll
      for (int q = 0; q < BPER; ++q) {
        const int gi = tid + 256 * q;
        const int j = gi / gpr, part = gi - j * gpr;
        if (gi < B::Rpad * gpr) *reinterpret_cast<frag*>(btl + j * BLD + part * B::EPV) = bt[q];
      }
    } else {
      for (int gi = tid; gi < B::Rpad * gpr; gi += 256) {
        const int j = gi / gpr, part = gi % gpr;
        *reinterpret_cast<frag*>(btl + j * BLD + part * B::EPV) =
            ld_frag<T, VEC>(a.BcT, j, B::Rpad, c0 + part * B::EPV, a.N_out, a.N_out);
      }
      fetch(0, srA, zrA);
      fetch(1, srB, zrB);
      if constexpr (kBwdDepth == 3) fetch(2, srC, zrC);
    }
  }

  // sc: integral_constant of the item's slab (static slabs) or of -1
  auto body = [&](int it, frag* sr, frag* zr, int buf, auto sc) __attribute__((always_inline)) {
    constexpr int SS = decltype(sc)::value;
    const int tn = it / ipt;
    const int sb = SS >= 0 ? SS : it - tn * ipt;
    // static slabs: dead items hold zeros, so every item runs its products
    const bool live = SS >= 0 || it < nitems;
    if (sb == 0) {
      lds_barrier();  // readers of the previous tile's Z^T are done
      if constexpr (B::ZT)
        rank_store<T, NR>(nullptr, ztl, zr);
      else
        rank_store<T, NR>(ztl, nullptr, zr);
#pragma unroll
      for (int n = 0; n < NR; ++n) accZ[n] = zero4();
    }
    E* sl = slab + buf * B::SLAB;
    slab_store<T, NR>(sl, sr);
    fetch(it + kBwdDepth, sr, zr);
    lds_barrier();
    if (live) {
      // dZ^T: M = rank (tile n), N = token (16-row tile w), K = column of the
      // slab; a lane ends with four consecutive ranks of one token
#pragma unroll
      for (int ks = 0; ks < B::SW / B::KSTEP; ++ks) {
        const int kc = ks * B::KSTEP + g * B::EPV;
        const frag fy = lds_frag<T>(sl + (16 * w + c) * B::SLD + kc);
#pragma unroll
        for (int n = 0; n < NR; ++n)
          accZ[n] = Mma<T>::mma(lds_frag<T>(btl + (16 * n + c) * BLD + sb * B::SW + kc), fy, accZ[n]);
      }
      // dB: M = column (tiles ct*4+w of the slab), N = rank (tile n), K =
      // token; a lane ends with four consecutive columns of one rank
      auto dB_products = [&](f32x4 (&acc)[B::CTW][NR]) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < 64 / B::KSTEP; ++ks) {
          const int kt = ks * B::KSTEP + g * B::EPV;
          frag fb[B::CTW];
#pragma unroll
          for (int ct = 0; ct < B::CTW; ++ct)
            fb[ct] = lds_colT_frag<T>(sl + kt * B::SLD + (ct * 4 + w) * 16, B::SLD);
#pragma unroll
          for (int n = 0; n < NR; ++n) {
            const frag fz = B::ZT ? lds_colT_frag<T>(ztl + (ks * B::KSTEP + g * B::EPV) * B::RLD + 16 * n, B::RLD)
                                  : lds_frag<T>(ztl + (16 * n + c) * B::ZLD + kt);
#pragma unroll
            for (int ct = 0; ct < B::CTW; ++ct) acc[ct][n] = Mma<T>::mma(fb[ct], fz, acc[ct][n]);
          }
        }
      };
      if constexpr (SS >= 0) {
        dB_products(accB[SS]);
      } else {
#pragma unroll
        for (int s = 0; s < NSM; ++s)
          if (s == sb) dB_products(accB[s]);
      }
    }
    // dZ (or this column group's partial) once the tile's last slab is in:
    // token 64 tn + 16w + c of the group, ranks 16n + 4g .. 16n + 4g + 3
    if constexpr (VEC) {
      const bool st = live & (sb == ipt - 1) & (tn < ntt);
      const int row = 64 * tn + 16 * w + c;
#pragma unroll
      for (int n = 0; n < NR; ++n) {
        if (a.gc_n == 1)
          buf_store4<T>(rdz, st ? (uint32_t)((row * B::Rpad + 16 * n + 4 * g) * B::ES) : kNoOff, accZ[n]);
        else
          buf_store_f32x4(rdz, st ? (uint32_t)((row * B::Rpad + 16 * n + 4 * g) * 4) : kNoOff, accZ[n]);
      }
    } else if (live && sb == nsl - 1) {
      const int64_t t = tb + 64 * (int64_t)tn + 16 * w + c;
      if (t < a.T_) {
#pragma unroll
        for (int n = 0; n < NR; ++n)
#pragma unroll
          for (int vv = 0; vv < 4; ++vv) {
            const int j = 16 * n + 4 * g + vv;
            if (a.gc_n == 1)
              a.dZ[t * B::Rpad + j] = (E)Mma<T>::from_f32(accZ[n][vv]);
            else
              a.dZp[((int64_t)gc * a.T_ + t) * B::Rpad + j] = accZ[n][vv];
          }
      }
    }
  };
  if constexpr (NSL > 0) {
    // item it = tn * NSL + s; its register set and slab buffer follow the
    // parity of it, which each unrolled item knows
    for (int tn = 0; tn < ntt_run; tn += (NSL & 1) ? 2 : 1) {
      static_for<0, ((NSL & 1) ? 2 : 1) * NSL>([&](auto uc) __attribute__((always_inline)) {
        constexpr int u = decltype(uc)::value;
        constexpr int s = u % NSL;
        const int it = tn * NSL + u;
        if constexpr ((u & 1) == 0)
          body(it, srA, zrA, 0, std::integral_constant<int, s>{});
        else
          body(it, srB, zrB, 1, std::integral_constant<int, s>{});
      });
    }
  } else {
    for (int it = 0; it < nitems; it += kBwdDepth) {
      body(it, srA, zrA, it & 1, std::integral_constant<int, -1>{});
      if (VEC || it + 1 < nitems) body(it + 1, srB, zrB, (it + 1) & 1, std::integral_constant<int, -1>{});
      if constexpr (kBwdDepth == 3)
        if (VEC || it + 2 < nitems) body(it + 2, srC, zrC, (it + 2) & 1, std::integral_constant<int, -1>{});
    }
  }
  // dB^T partial of this token group: rank 16n + c, columns
  // c0 + s*SW + (ct*4+w)*16 + 4g .. + 3
  const bool pvec = (a.N_out & 3) == 0;
#pragma unroll
  for (int s = 0; s < NSM; ++s) {
    if (s < nsl) {
#pragma unroll
      for (int ct = 0; ct < B::CTW; ++ct) {
        const int64_t o = c0 + (int64_t)s * B::SW + (ct * 4 + w) * 16 + 4 * g;
#pragma unroll
        for (int n = 0; n < NR; ++n) {
          const int j = 16 * n + c;
          if (j < reff && o < a.N_out)
            store_partial4(a.dBp + ((int64_t)gt * B::Rpad + j) * a.N_out + o, accB[s][ct][n], o, a.N_out, pvec);
        }
      }
    }
  }
  // the token groups of this launch, for the reduction (one unconditional
  // store instruction, kept by work-group 0's first lane only)
  buf_store32(make_rsrc(a.gts, 8), (bid == 0 && tid == 0) ? 0u : kNoOff, (unsigned)((a.ntiles + a.tpg - 1) / a.tpg));
}

// dZ = sum of the column groups' partials, in group order (deterministic);
// every layer of the batch strides over its own range of work-groups
template <typename T>
struct DzArgs {
  const float* dZp;
  typename Elem<T>::type* dZ;
  int ngc;
  int64_t n4;
};
template <typename T>
__global__ __launch_bounds__(256) void k_dz_sum(StreamBatch<DzArgs<T>> zb) {
  typedef typename Elem<T>::type E;
  unsigned bid;
  const int q = batch_layer(zb, &bid);
  const DzArgs<T>& a = zb.a[q];
  const int64_t nb = zb.first[q + 1] - zb.first[q];
  for (int64_t i = (int64_t)bid * blockDim.x + threadIdx.x; i < a.n4; i += nb * blockDim.x) {
    f32x4 sum = zero4();
    for (int g = 0; g < a.ngc; ++g) sum += *reinterpret_cast<const f32x4*>(a.dZp + ((int64_t)g * a.n4 + i) * 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) a.dZ[i * 4 + e] = (E)Mma<T>::from_f32(sum[e]);
  }
}

// ------------------------------------------------------------------------------
// backward, dX pass
// ------------------------------------------------------------------------------
template <typename T>
struct DxArgs {
  const typename Elem<T>::type* x;
  const typename Elem<T>::type* AcT;  // N_in x Rpad
  const typename Elem<T>::type* dZ;   // T x Rpad
  const float* dZp;                   // ZS x T x Rpad partials of the dY pass (ZS > 0)
  float* dAp;                         // gt x Rpad x N_in partials (rows < r_eff)
  typename Elem<T>::type* dx;         // T x N_in or null
  const int* meta;
  int* gts;                           // [1] <- token groups of this launch (for the reduction)
  int64_t T_, N_in;
  int nsl, tpg, ntiles, vec, gcols;
};

// ZS > 0 (16-byte rows): dZ is the sum of the dY pass's ZS fp32 column-group
// partials, formed here per tile in group order and rounded to the activation
// type as the separate sum would (the same values bit for bit), so that
// layers whose dY pass splits its columns in two need no launch for the sum.
template <typename T, int NR, bool VEC, int ZS>
__global__ __launch_bounds__(256) void k_bwd_dx(StreamBatch<DxArgs<T>> bb) {
  unsigned bid;
  const DxArgs<T>& a = bb.a[batch_layer(bb, &bid)];
  typedef Bwd<T, NR> B;
  typedef typename B::E E;
  typedef typename Mma<T>::frag frag;
  constexpr int NSM = dx_max_slabs(B::ES, NR);
  extern __shared__ __align__(16) char smem[];
  E* atl = reinterpret_cast<E*>(smem);            // [NSM*SW][RLD]: A^T rows of the column range
  E* slab = atl + NSM * B::SW * B::RLD;           // [2][64][SLD]
  E* dzl = slab + 2 * B::SLAB;                    // [64][RLD]: dZ, token-major
  E* dztl = dzl + 64 * B::RLD;                    // [Rpad][ZLD]: dZ^T (not with ZT)

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int gc = (int)(bid % (unsigned)a.gcols), gt = (int)(bid / (unsigned)a.gcols);
  const int64_t c0 = (int64_t)gc * a.nsl * B::SW;
  const int nsl = (int)std::min<int64_t>(a.nsl, (a.N_in - c0 + B::SW - 1) / B::SW);
  const int reff = a.meta[kMetaReff];
  const int tt0 = gt * a.tpg;
  const int ntt = std::min(a.ntiles, tt0 + a.tpg) - tt0;
  const int nitems = ntt * nsl;
  const int64_t tb = (int64_t)tt0 * 64;
  const int64_t nrow = std::min<int64_t>(a.T_ - tb, (int64_t)ntt * 64);

  f32x4 accA[NSM][B::CTW][NR];
#pragma unroll
  for (int s = 0; s < NSM; ++s)
#pragma unroll
    for (int ct = 0; ct < B::CTW; ++ct)
#pragma unroll
      for (int n = 0; n < NR; ++n) accA[s][ct][n] = zero4();

  // one register set per item in flight; with 16-byte rows every fetch,
  // store and item is unconditional (buffer accesses, dead ones at kNoOff), so
  // the wait before an item leaves the later fetches in flight
  static_assert(ZS == 0 || VEC, "dZ partials with 16-byte rows only");
  constexpr int ZQ = B::EPV / 4;  // float4 per fragment of a partial
  frag srA[B::PER], srB[B::PER], srC[B::PER], zrA[B::ZPER], zrB[B::ZPER], zrC[B::ZPER];
  f32x4 zpA[ZS > 0 ? ZS * B::ZPER * ZQ : 1], zpB[ZS > 0 ? ZS * B::ZPER * ZQ : 1], zpC[ZS > 0 ? ZS * B::ZPER * ZQ : 1];
  const rsrc_t rsl = make_rsrc(a.x + tb * a.N_in, nrow * a.N_in * B::ES);
  const rsrc_t rzt = make_rsrc(a.dZ + tb * B::Rpad, nrow * B::Rpad * B::ES);
  const rsrc_t rdx = make_rsrc(a.dx ? a.dx + tb * a.N_in : a.x, a.dx ? nrow * a.N_in * B::ES : 0);
  rsrc_t rzp[ZS > 0 ? ZS : 1];
#pragma unroll
  for (int g2 = 0; g2 < ZS; ++g2) rzp[g2] = make_rsrc(a.dZp + ((int64_t)g2 * a.T_ + tb) * B::Rpad, nrow * B::Rpad * 4);
  auto fetch = [&](int it, frag* sr, frag* zr, f32x4* zp) {
    if constexpr (VEC) {
      const bool live = it < nitems;
      const int itc = live ? it : 0;
      const int tn = itc / nsl, sn = itc - tn * nsl;
      slab_fetch_b<T, NR>(sr, rsl, tn * 64, c0 + (int64_t)sn * B::SW, a.N_in, live);
      if constexpr (ZS == 0) {
        rank_fetch_b<T, NR>(zr, rzt, tn * 64, live & (sn == 0), reff);
      } else {
        // the rank tile's pieces of every partial (the layout of rank_fetch_b,
        // in fp32); rank columns at or past r_eff are zero and not read
#pragma unroll
        for (int q = 0; q < B::ZPER; ++q) {
          const int gi = tid + 256 * q;
          const int row = gi / B::ZG, part = gi % B::ZG;
          const bool ok = live & (sn == 0) & (gi < 64 * B::ZG) & (part * B::EPV < reff);
#pragma unroll
          for (int g2 = 0; g2 < ZS; ++g2)
#pragma unroll
            for (int e4 = 0; e4 < ZQ; ++e4)
              zp[(g2 * B::ZPER + q) * ZQ + e4] = __builtin_bit_cast(
                  f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                             rzp[g2], ok ? (int)(((tn * 64 + row) * B::Rpad + part * B::EPV + 4 * e4) * 4) : (int)kNoOff, 0,
                             0));
        }
      }
    } else if (it < nitems) {
      const int tn = tt0 + it / nsl, sn = it % nsl;
      slab_fetch<T, NR, VEC>(sr, a.x, (int64_t)tn * 64, a.T_, c0 + (int64_t)sn * B::SW, a.N_in);
      if (sn == 0) rank_fetch<T, NR>(zr, a.dZ, (int64_t)tn * 64, a.T_);
    }
  };

  // A^T rows of this column range (16-byte rows): a fixed number of loads per
  // thread, requested before the first two items so that the latencies overlap
  {
    constexpr int gpr = B::Rpad / B::EPV;
    constexpr int APER = (NSM * B::SW * gpr + 255) / 256;
    const rsrc_t ra = make_rsrc(a.AcT + c0 * B::Rpad, (std::min<int64_t>(a.N_in, c0 + (int64_t)nsl * B::SW) - c0) * B::Rpad * B::ES);
    frag at[APER];
#pragma unroll
    for (int q = 0; q < APER; ++q) {
      const int gi = tid + 256 * q;
      at[q] = buf_frag<T>(ra, ((gi < nsl * B::SW * gpr) & ((gi % gpr) * B::EPV < reff)) ? (uint32_t)(gi * B::EPV * B::ES)
                                                                                      : kNoOff);
    }
    fetch(0, srA, zrA, zpA);
    fetch(1, srB, zrB, zpB);
    if constexpr (kBwdDepth == 3) fetch(2, srC, zrC, zpC);
#pragma unroll
    for (int q = 0; q < APER; ++q) {
      const int gi = tid + 256 * q;
      const int i = gi / gpr, part = gi % gpr;
      if (gi < nsl * B::SW * gpr) *reinterpret_cast<frag*>(atl + i * B::RLD + part * B::EPV) = at[q];
    }
  }

  auto body = [&](int it, frag* sr, frag* zr, f32x4* zp, int buf) {
    const bool live = it < nitems;
    const int tn = it / nsl, sb = it - tn * nsl;
    const int64_t t0 = tb + 64 * (int64_t)tn;
    if (sb == 0) {
      lds_barrier();
      if constexpr (ZS == 0) {
        rank_store<T, NR>(B::ZT ? nullptr : dztl, dzl, zr);
      } else {
        // dZ = the partials summed in group order, rounded once
        frag zc[B::ZPER];
#pragma unroll
        for (int q = 0; q < B::ZPER; ++q)
#pragma unroll
          for (int e4 = 0; e4 < ZQ; ++e4) {
            f32x4 v = zero4();
#pragma unroll
            for (int g2 = 0; g2 < ZS; ++g2) v += zp[(g2 * B::ZPER + q) * ZQ + e4];
#pragma unroll
            for (int e = 0; e < 4; ++e) zc[q][4 * e4 + e] = Mma<T>::from_f32(v[e]);
          }
        rank_store<T, NR>(B::ZT ? nullptr : dztl, dzl, zc);
      }
    }
    E* sl = slab + buf * B::SLAB;
    slab_store<T, NR>(sl, sr);
    fetch(it + kBwdDepth, sr, zr, zp);
    lds_barrier();
    // (16-byte rows: a dead item's x slab holds zeros, so its products add
    // nothing and run unconditionally; a condition around the accumulators'
    // updates makes the compiler copy them)
    if (VEC || live) {
      // dA: M = input column, N = rank, K = token (reads the x slab first, so
      // that the slab buffer can then stage this slab's dX); a lane ends with
      // four consecutive columns of one rank
#pragma unroll
      for (int s = 0; s < NSM; ++s) {
        if (NSM == 1 || s == sb) {
#pragma unroll
          for (int ks = 0; ks < 64 / B::KSTEP; ++ks) {
            const int kt = ks * B::KSTEP + g * B::EPV;
            frag fb[B::CTW];
#pragma unroll
            for (int ct = 0; ct < B::CTW; ++ct)
              fb[ct] = lds_colT_frag<T>(sl + kt * B::SLD + (ct * 4 + w) * 16, B::SLD);
#pragma unroll
            for (int n = 0; n < NR; ++n) {
              const frag fz = B::ZT ? lds_colT_frag<T>(dzl + (ks * B::KSTEP + g * B::EPV) * B::RLD + 16 * n, B::RLD)
                                    : lds_frag<T>(dztl + (16 * n + c) * B::ZLD + kt);
#pragma unroll
              for (int ct = 0; ct < B::CTW; ++ct) accA[s][ct][n] = Mma<T>::mma(fb[ct], fz, accA[s][ct][n]);
            }
          }
        }
      }
    }
    // without dX (a null pointer) the 16-byte-row form still runs the stores,
    // all of them dropped by an empty resource, to keep the memory operations
    // the same on every path
    if (VEC || a.dx) {
      // dX^T = A^T dZ^T: M = input column (tiles ct*4+w of the slab), N = token, K = rank
      f32x4 accX[B::CTW][4];
#pragma unroll
      for (int ct = 0; ct < B::CTW; ++ct) {
        const int colt = (ct * 4 + w) * 16;
#pragma unroll
        for (int u = 0; u < 4; ++u) accX[ct][u] = zero4();
        if constexpr (B::HALF) {
          const frag fa = lds_frag_lo8<T>(atl + (sb * B::SW + colt + c) * B::RLD + 8 * g);
#pragma unroll
          for (int u = 0; u < 4; ++u)
            accX[ct][u] = Mma<T>::mma_k32(fa, lds_frag_lo8<T>(dzl + (16 * u + c) * B::RLD + 8 * g), accX[ct][u]);
        } else {
#pragma unroll
          for (int ks = 0; ks < B::Rpad / B::KSTEP; ++ks) {
            const int kc = ks * B::KSTEP + g * B::EPV;
            const frag fa = lds_frag<T>(atl + (sb * B::SW + colt + c) * B::RLD + kc);
#pragma unroll
            for (int u = 0; u < 4; ++u)
              accX[ct][u] = Mma<T>::mma(fa, lds_frag<T>(dzl + (16 * u + c) * B::RLD + kc), accX[ct][u]);
          }
        }
      }
      const int64_t cs0 = c0 + (int64_t)sb * B::SW;
      if constexpr (VEC) {
        // the slab's dX leaves through the slab buffer as whole 16-byte row
        // pieces: every wave is done reading the x slab, the tile is staged,
        // then stored row by row (dead rows, columns and items at kNoOff)
        lds_barrier();
#pragma unroll
        for (int ct = 0; ct < B::CTW; ++ct) {
          const int colt = (ct * 4 + w) * 16;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            E* d = sl + (16 * u + c) * B::SLD + colt + 4 * g;
            if constexpr (sizeof(E) == 2) {
              const uint2 pk = {f32x2_to_bf16x2(accX[ct][u][0], accX[ct][u][1]),
                                f32x2_to_bf16x2(accX[ct][u][2], accX[ct][u][3])};
              *reinterpret_cast<uint2*>(d) = pk;
            } else if constexpr (sizeof(E) == 1) {
              *reinterpret_cast<unsigned*>(d) =
                  f32x4_to_fp8x4(accX[ct][u][0], accX[ct][u][1], accX[ct][u][2], accX[ct][u][3]);
            } else {
              *reinterpret_cast<f32x4*>(d) = accX[ct][u];
            }
          }
        }
        lds_barrier();
        constexpr int GPR = B::SW * B::ES / 16;  // 16-byte groups per staged row
        constexpr int EPG = 16 / B::ES;
#pragma unroll
        for (int k = 0; k < 64 * GPR / 256; ++k) {
          const int idx = tid + 256 * k;
          const int row = idx / GPR, q = idx % GPR;
          const int64_t col = cs0 + q * EPG;
          const uint32_t o = (uint32_t)(((int64_t)(64 * tn + row) * a.N_in + col) * B::ES);
          buf_store16(rdx, (live & (col < a.N_in)) ? o : kNoOff,
                      *reinterpret_cast<const uint4*>(sl + row * B::SLD + q * EPG));
        }
      } else if (live) {
#pragma unroll
        for (int ct = 0; ct < B::CTW; ++ct) {
          const int64_t i0 = cs0 + (ct * 4 + w) * 16 + 4 * g;
          const int valid = (int)std::min<int64_t>(4, a.N_in - i0);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int64_t t = t0 + 16 * u + c;
            if (t < a.T_ && valid > 0) store4<T>(a.dx + t * a.N_in + i0, accX[ct][u], valid, false);
          }
        }
      }
    }
  };
  for (int it = 0; it < nitems; it += kBwdDepth) {
    body(it, srA, zrA, zpA, it & 1);
    if (VEC || it + 1 < nitems) body(it + 1, srB, zrB, zpB, (it + 1) & 1);
    if constexpr (kBwdDepth == 3)
      if (VEC || it + 2 < nitems) body(it + 2, srC, zrC, zpC, (it + 2) & 1);
  }
  // dA partial of this token group: rank 16n + c, columns
  // c0 + s*SW + (ct*4+w)*16 + 4g .. + 3
  const bool pvec = (a.N_in & 3) == 0;
#pragma unroll
  for (int s = 0; s < NSM; ++s) {
    if (s < nsl) {
#pragma unroll
      for (int ct = 0; ct < B::CTW; ++ct) {
        const int64_t i = c0 + (int64_t)s * B::SW + (ct * 4 + w) * 16 + 4 * g;
#pragma unroll
        for (int n = 0; n < NR; ++n) {
          const int j = 16 * n + c;
          if (j < reff && i < a.N_in)
            store_partial4(a.dAp + ((int64_t)gt * B::Rpad + j) * a.N_in + i, accA[s][ct][n], i, a.N_in, pvec);
        }
      }
    }
  }
  buf_store32(make_rsrc(a.gts, 8), (bid == 0 && tid == 0) ? 4u : kNoOff, (unsigned)((a.ntiles + a.tpg - 1) / a.tpg));
}

// ------------------------------------------------------------------------------
// partial sums -> gradients of the two half products (full rank, fp32)
// ------------------------------------------------------------------------------
struct ReduceArgs {
  const float* dBp;
  const float* dAp;
  const int* gts;  // token groups the data passes used (dY, dX)
  int gtB, gtA;    // most token groups the partial buffers hold
  const int* meta;
  const float* Ds;
  float* dL;
  float* dR;
  int64_t N_out, N_in;
  int rs, Rpad, in_first;
  // chain order inside the halves differing from the listed order: the
  // listed modes of each side and the chain stride of each (B: output, A: input)
  int perm, nmB, nmA;
  int szB[TTC_MAX_HALF_MODES], csB[TTC_MAX_HALF_MODES];
  int szA[TTC_MAX_HALF_MODES], csA[TTC_MAX_HALF_MODES];
};

// listed (mixed-radix) index -> index in the half's chain order
__device__ __forceinline__ int64_t listed_to_chain(int64_t li, int nm, const int* sz, const int* cs) {
  int64_t c = 0;
  for (int m = nm - 1; m >= 0; --m) {
    c += (li % sz[m]) * cs[m];
    li /= sz[m];
  }
  return c;
}

// Layers reduced by one launch.  A work-group owns 64 consecutive 4-column
// groups of one rank row of one side (B or A) of one layer; its four waves
// sum contiguous quarters of the token groups (float4 loads, eight in flight)
// and the quarters are added in wave order through LDS, so the order of every
// sum is fixed.  The result is scattered into the layout of the half
// product's gradient.
struct ReduceBatch {
  ReduceArgs r[kMaxBatch];
  int64_t first[kMaxBatch + 1];  // first work-group of each layer
  int n;
};

static_assert(sizeof(ReduceBatch) <= 2048, "ReduceBatch too large for a kernel argument");

__device__ __forceinline__ int64_t reduce_strips(int64_t N) { return ((N + 3) / 4 + 63) / 64; }

__global__ __launch_bounds__(256) void k_reduce(ReduceBatch rb) {
  __shared__ f32x4 part[3][64];
  int q = 0;
  while (q < rb.n - 1 && (int64_t)blockIdx.x >= rb.first[q + 1]) ++q;
  const ReduceArgs& a = rb.r[q];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int64_t item = (int64_t)blockIdx.x - rb.first[q];
  const int64_t sB = reduce_strips(a.N_out), sA = reduce_strips(a.N_in);
  const bool isB = item < (int64_t)a.rs * sB;
  if (!isB) item -= (int64_t)a.rs * sB;
  const int64_t ns = isB ? sB : sA;
  const int b = (int)(item / ns);
  const int64_t N = isB ? a.N_out : a.N_in;
  const int64_t r0 = ((item % ns) * 64 + lane) * 4;
  const int j = a.meta[kMetaPos + b];
  const float* src = isB ? a.dBp : a.dAp;
  const int gtn = max(0, min(a.gts[isB ? 0 : 1], isB ? a.gtB : a.gtA));
  const int per = (gtn + 3) / 4;
  const int qb = min(gtn, w * per), qe = min(gtn, qb + per);
  f32x4 acc = zero4();
  if (j >= 0 && r0 < N) {
    const float* col = src + (int64_t)j * N + r0;
    const int64_t qstride = (int64_t)a.Rpad * N;
    if ((N & 3) == 0) {
      f32x4 acc1 = zero4();
      int qq = qb;
      for (; qq + 8 <= qe; qq += 8) {
        f32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const f32x4*>(col + (int64_t)(qq + u) * qstride);
#pragma unroll
        for (int u = 0; u < 8; u += 2) {
          acc += v[u];
          acc1 += v[u + 1];
        }
      }
      for (; qq < qe; ++qq) acc += *reinterpret_cast<const f32x4*>(col + (int64_t)qq * qstride);
      acc += acc1;
    } else {
      for (int qq = qb; qq < qe; ++qq)
        for (int e = 0; e < 4; ++e)
          if (r0 + e < N) acc[e] += col[(int64_t)qq * qstride + e];
    }
  }
  if (w > 0) part[w - 1][lane] = acc;
  __syncthreads();
  auto row = [&](int64_t li) {
    return a.perm ? (isB ? listed_to_chain(li, a.nmB, a.szB, a.csB) : listed_to_chain(li, a.nmA, a.szA, a.csA)) : li;
  };
  if (w != 0 || j < 0 || r0 >= N) {
    // dead slice: its gradient rows / columns are exactly zero
    if (w == 0 && r0 < N) {
      const bool toL = isB != (a.in_first != 0);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (r0 + e < N) {
          if (toL)
            a.dL[row(r0 + e) * a.rs + b] = 0.f;
          else
            a.dR[(int64_t)b * N + row(r0 + e)] = 0.f;
        }
    }
    return;
  }
  acc = ((acc + part[0][lane]) + part[1][lane]) + part[2][lane];
  if (!isB) acc *= a.Ds[b];
  // B side feeds L (out first) or R (in first); A side the other one
  const bool toL = isB != (a.in_first != 0);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (r0 + e < N) {
      if (toL)
        a.dL[row(r0 + e) * a.rs + b] = acc[e];
      else
        a.dR[(int64_t)b * N + row(r0 + e)] = acc[e];
    }
  }
}

// ------------------------------------------------------------------------------
// reverse sweep for the core gradients as small GEMMs
// ------------------------------------------------------------------------------
// C(i, j) = rowscale(i) * colscale(j) * sum_k A(i, k) B(k, j) with
// A(i, k) = A[i*sAi + k*sAk], B(k, j) = B[k*sBk + j*sBj], C(i, j) at
// C[i*sCi + j*sCj]; scales are optional (null = 1).
struct Gemm {
  const float* A;
  int64_t sAi, sAk;
  const float* B;
  int64_t sBk, sBj;
  const float* rs_;
  const float* cs_;
  float* C;
  int64_t sCi, sCj;
  int M, N, K;
};

__host__ __device__ inline int gemm_tiles(const Gemm& g) { return ((g.M + 31) / 32) * ((g.N + 31) / 32); }

// One 32 x 32 output tile per work-group of kSweepWaves waves with fp32 MFMA
// 16x16x4.  These GEMMs are small (K up to a few hundred), so the time of a
// tile is the latency of its loads: wave w takes the 32-wide chunks of K w,
// w + 16, ... and requests a chunk's operands (all its loads for K <= 512)
// straight into registers before multiplying, so a tile costs about one
// memory round trip.  The waves' partial tiles are then added in wave order
// through LDS (fixed order, bitwise reproducible).
constexpr int kSweepWaves = 16;
constexpr int kSweepThreads = 64 * kSweepWaves;
constexpr int kSweepRedLd = 33;
constexpr size_t kSweepLds = (size_t)kSweepWaves * 32 * kSweepRedLd * 4;

__device__ void gemm_tile32(const Gemm& g, int tile, float* red) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int gq = lane >> 4, c = lane & 15;
  const int ntj = (g.N + 31) / 32;
  const int64_t i0 = (int64_t)(tile / ntj) * 32, j0 = (int64_t)(tile % ntj) * 32;
  f32x4 acc[2][2];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int q = 0; q < 2; ++q) acc[p][q] = zero4();
  // Wave w takes the 32-wide chunks of K w, w + 16, ...; within a chunk lane
  // group gq holds the 8 consecutive k = base + 8 gq + u (u = 0..7) and MFMA u
  // takes value u of every lane: any assignment of k to (lane group, MFMA)
  // gives the same sums as long as both operands use it.  An operand whose k
  // index is contiguous in memory then comes as two 16-byte loads per lane
  // (the lanes of one row share 64 contiguous bytes) instead of eight scalar
  // loads that each touch 16 rows; an operand contiguous along its other
  // index keeps the scalar loads, which are contiguous across the lanes.
  const bool va = g.sAk == 1 && (g.sAi & 3) == 0 && (g.K & 3) == 0 && ((uintptr_t)g.A & 15) == 0;
  const bool vb = g.sBk == 1 && (g.sBj & 3) == 0 && (g.K & 3) == 0 && ((uintptr_t)g.B & 15) == 0;
  for (int64_t kb = (int64_t)w * 32; kb < g.K; kb += (int64_t)kSweepWaves * 32) {
    const int64_t k0 = kb + 8 * gq;
    float fa[8][2], fb[8][2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int64_t i = i0 + 16 * p + c;
      const bool iok = i < g.M;
      if (va) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bool ok = iok && k0 + 4 * h < g.K;
          const f32x4 v = ok ? *reinterpret_cast<const f32x4*>(g.A + i * g.sAi + k0 + 4 * h) : zero4();
#pragma unroll
          for (int e = 0; e < 4; ++e) fa[4 * h + e][p] = v[e];
        }
      } else {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const bool ok = iok && k0 + u < g.K;
          const float v = g.A[ok ? i * g.sAi + (k0 + u) * g.sAk : 0];
          fa[u][p] = ok ? v : 0.f;
        }
      }
      const int64_t j = j0 + 16 * p + c;
      const bool jok = j < g.N;
      if (vb) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bool ok = jok && k0 + 4 * h < g.K;
          const f32x4 v = ok ? *reinterpret_cast<const f32x4*>(g.B + j * g.sBj + k0 + 4 * h) : zero4();
#pragma unroll
          for (int e = 0; e < 4; ++e) fb[4 * h + e][p] = v[e];
        }
      } else {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const bool ok = jok && k0 + u < g.K;
          const float v = g.B[ok ? (k0 + u) * g.sBk + j * g.sBj : 0];
          fb[u][p] = ok ? v : 0.f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int q = 0; q < 2; ++q) acc[p][q] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[u][p], fb[u][q], acc[p][q], 0, 0, 0);
  }
  // lane (gq, c) of sub-tile (p, q) holds rows 16p+4gq+v, column 16q+c
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[(w * 32 + 16 * p + 4 * gq + v) * kSweepRedLd + 16 * q + c] = acc[p][q][v];
  lds_barrier();
  {
    const int i = tid >> 5, j = tid & 31;
    const int64_t gi = i0 + i, gj = j0 + j;
    if (gi < g.M && gj < g.N) {
      float sum = red[i * kSweepRedLd + j];
#pragma unroll
      for (int v = 1; v < kSweepWaves; ++v) sum += red[(v * 32 + i) * kSweepRedLd + j];
      const float rsc = g.rs_ ? g.rs_[gi] : 1.f;
      const float csc = g.cs_ ? g.cs_[gj] : 1.f;
      g.C[gi * g.sCi + gj * g.sCj] = (sum * rsc) * csc;
    }
  }
}

// One level of the reverse sweep for one or more layers: up to kMaxGemm
// independent GEMMs (per half and layer, the core gradient and the gradient
// passed on to the next core), one 32 x 32 tile per work-group.
constexpr int kMaxGemm = 24;
struct SweepArgs {
  Gemm g[kMaxGemm];
  int tiles[kMaxGemm];
  int ng;
};

// kernel arguments stay inside the 4 KB argument segment
static_assert(sizeof(SweepArgs) <= 3072, "SweepArgs too large for a kernel argument");

__global__ __launch_bounds__(kSweepThreads) void k_sweep(SweepArgs a) {
  extern __shared__ __align__(16) char smem[];
  int t = blockIdx.x, q = 0;
  while (q < a.ng - 1 && t >= a.tiles[q]) {
    t -= a.tiles[q];
    ++q;
  }
  gemm_tile32(a.g[q], t, reinterpret_cast<float*>(smem));
}

// Left core k, gradient dM_k of the prefix M_k (rows prod_{j<=k} n_j, r_{k+1}
// cols), M_k[(alpha, m), c] = sum_a (M_{k-1} diag(D_{k-1}))[alpha, a] G_k[a, m, c]:
//   dG_k = P^T dM_k'         with P = M_{k-1} diag(D_{k-1}), dM_k' = dM_k as (alpha, (m, c))
//   dM_{k-1} = (dM_k' G_k'^T) diag(D_{k-1})
static Gemm left_dG(const LinearPlan& P, const float* chain, const float* const* D, float* dGk, int k,
                    const float* dMk, int64_t rows) {
  const int n = P.modes[k], r0 = P.ranks[k], r1 = P.ranks[k + 1];
  Gemm g;
  g.A = chain + P.chain_off[k - 1];
  g.sAi = 1;
  g.sAk = r0;
  g.rs_ = D[k - 1];
  g.B = dMk;
  g.sBk = (int64_t)n * r1;
  g.sBj = 1;
  g.cs_ = nullptr;
  g.C = dGk;
  g.sCi = (int64_t)n * r1;
  g.sCj = 1;
  g.M = r0;
  g.N = n * r1;
  g.K = (int)(rows / n);
  return g;
}
static Gemm left_dM(const LinearPlan& P, const float* const* G, const float* const* D, int k, const float* dMk,
                    int64_t rows, float* out) {
  const int n = P.modes[k], r0 = P.ranks[k], r1 = P.ranks[k + 1];
  Gemm g;
  g.A = dMk;
  g.sAi = (int64_t)n * r1;
  g.sAk = 1;
  g.rs_ = nullptr;
  g.B = G[k];
  g.sBk = 1;
  g.sBj = (int64_t)n * r1;
  g.cs_ = D[k - 1];
  g.C = out;
  g.sCi = r0;
  g.sCj = 1;
  g.M = (int)(rows / n);
  g.N = r0;
  g.K = n * r1;
  return g;
}
// Right core k, gradient dN_k of the suffix N_k (r_k rows, cols = prod_{j>=k}
// n_j), N_k[a, (m, beta)] = sum_c G_k[a, m, c] (diag(D_k) N_{k+1})[c, beta]:
//   dG_k = dN_k'' Q^T        with Q = diag(D_k) N_{k+1}, dN_k'' = dN_k as ((a, m), beta)
//   dN_{k+1} = diag(D_k) G_k''^T dN_k''
static Gemm right_dG(const LinearPlan& P, const float* chain, const float* const* D, float* dGk, int k,
                     const float* dNk, int64_t cols) {
  const int n = P.modes[k], r0 = P.ranks[k], r1 = P.ranks[k + 1];
  const int64_t be = cols / n;
  Gemm g;
  g.A = dNk;
  g.sAi = be;
  g.sAk = 1;
  g.rs_ = nullptr;
  g.B = chain + P.chain_off[k + 1];
  g.sBk = 1;
  g.sBj = be;
  g.cs_ = D[k];
  g.C = dGk;
  g.sCi = r1;
  g.sCj = 1;
  g.M = r0 * n;
  g.N = r1;
  g.K = (int)be;
  return g;
}
static Gemm right_dN(const LinearPlan& P, const float* const* G, const float* const* D, int k, const float* dNk,
                     int64_t cols, float* out) {
  const int n = P.modes[k], r0 = P.ranks[k], r1 = P.ranks[k + 1];
  const int64_t be = cols / n;
  Gemm g;
  g.A = G[k];
  g.sAi = 1;
  g.sAk = r1;
  g.rs_ = D[k];
  g.B = dNk;
  g.sBk = be;
  g.sBj = 1;
  g.cs_ = nullptr;
  g.C = out;
  g.sCi = be;
  g.sCj = 1;
  g.M = r1;
  g.N = (int)be;
  g.K = r0 * n;
  return g;
}

// ------------------------------------------------------------------------------
// gradients of the rank-control diagonals and the early-stage penalties
// ------------------------------------------------------------------------------
// Core k (chain position) carries the diagonal D_k of its right link as a
// factor of its slice b, so sum_{a,m} G_k[a,m,b] dG_k[a,m,b] = D_k[b] dL/dD_k[b]
// (project page, "Learn the ranks while training": a diagonal on every link).
// One work-group per core of a list (cores of one or more layers): thread t
// takes entry b = t mod r_k of row group t / r_k, so consecutive lanes read
// consecutive floats of a row (a, m); the row groups' sums are added in group
// order through LDS.  dD_k[b] = sum / D_k[b] + gamma sign(D_k[b]), and 0 for a
// pruned entry (D_k[b] == 0).  Then, after every read of dG_k, the work-group
// adds 2 beta G_k to dG_k.  The last core of a chain has no right link and
// only takes the penalty.
struct CoreJob {
  const float* G;
  const float* D;  // right link, or null
  float* dG;
  float* dD;       // right link, or null
  int rows;        // r_{k-1} n_k
  int r1;
};
constexpr int kMaxCoreJobs = 40;
struct RankGradArgs {
  CoreJob j[kMaxCoreJobs];
  int n;
  float gamma, beta;
};
static_assert(sizeof(RankGradArgs) <= 2048, "RankGradArgs too large for a kernel argument");

constexpr int kRankGradThreads = 1024;
__global__ __launch_bounds__(kRankGradThreads) void k_rank_grads(RankGradArgs a) {
  __shared__ float part[kRankGradThreads];
  const CoreJob& c = a.j[blockIdx.x];
  const int r1 = c.r1, rows = c.rows;
  if (c.D) {
    const int ng = (int)blockDim.x / r1;  // row groups (r1 <= 128)
    const int b = (int)threadIdx.x % r1, grp = (int)threadIdx.x / r1;
    if (grp < ng) {
      // eight rows in flight per thread, eight partial sums added in a fixed order
      float acc[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] = 0.f;
      int i = grp;
      for (; i + 7 * ng < rows; i += 8 * ng) {
        float gv[8], dv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          gv[u] = c.G[(int64_t)(i + u * ng) * r1 + b];
          dv[u] = c.dG[(int64_t)(i + u * ng) * r1 + b];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[u] = fmaf(gv[u], dv[u], acc[u]);
      }
      for (; i < rows; i += ng) acc[0] = fmaf(c.G[(int64_t)i * r1 + b], c.dG[(int64_t)i * r1 + b], acc[0]);
      part[threadIdx.x] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
    }
    __syncthreads();
    if ((int)threadIdx.x < r1) {
      float sum = 0.f;
      for (int g = 0; g < ng; ++g) sum += part[g * r1 + threadIdx.x];
      const float dv = c.D[threadIdx.x];
      c.dD[threadIdx.x] = dv != 0.f ? sum / dv + (dv > 0.f ? a.gamma : -a.gamma) : 0.f;
    }
  }
  if (a.beta != 0.f) {
    __syncthreads();
    const int64_t ne = (int64_t)rows * r1;
    const float tb = 2.f * a.beta;
    for (int64_t i = threadIdx.x; i < ne; i += blockDim.x) c.dG[i] = fmaf(tb, c.G[i], c.dG[i]);
  }
}

// ------------------------------------------------------------------------------
// sequential order (small batches)
// ------------------------------------------------------------------------------
// The core-by-core order of the project page's Proposition 4.1 comparison
// (section "Making small tensor operations fast on GPUs"): for few tokens it
// needs far fewer multiply-adds than merging the halves of the chain, whose
// cost does not shrink with the batch.  One work-group per token carries the
// token's state through the steps of the plan in LDS: the input modes are
// contracted one core at a time from the input half's chain end to the
// split, then the output modes are produced one core at a time.  The forward
// keeps the states between steps in `saved`; the backward walks the steps in
// reverse and writes, per token, the input gradient and one partial of every
// core gradient (fixed-order sums; the partials are added over the tokens by
// k_seq_reduce in token order).
struct SeqArgs {
  SeqStep st[kMaxCores];
  const float* G[kMaxCores];
  const float* D[kMaxCores];
  const void* x;
  const void* dy;
  void* y;
  void* dx;
  float* states;
  float* part;
  int64_t N_in, N_out, state_floats, part_floats, max_state, max_core;
  int d;
};
static_assert(sizeof(SeqArgs) <= 3072, "SeqArgs too large for a kernel argument");
constexpr int kSeqThreads = 1024;

// element (x, i, y) of a step's core in the core's own layout
__device__ __forceinline__ int seq_gidx(const SeqStep& st, int x, int i, int y) {
  return st.rightward ? (x * st.n + i) * st.rout + y : (y * st.n + i) * st.rin + x;
}

// the step's core and link diagonal into LDS (all of a thread's loads in flight
// at once: a core has at most 16384 entries)
__device__ __forceinline__ void seq_stage(const SeqArgs& a, const SeqStep& st, float* gsm, float* dv) {
  const float* G = a.G[st.core];
  const int csz = st.rin * st.n * st.rout;
  constexpr int U = 16;
  for (int e0 = threadIdx.x; e0 < csz; e0 += U * kSeqThreads) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = e0 + u * kSeqThreads < csz ? G[e0 + u * kSeqThreads] : 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (e0 + u * kSeqThreads < csz) gsm[e0 + u * kSeqThreads] = v[u];
  }
  for (int x = threadIdx.x; x < st.rin; x += kSeqThreads) dv[x] = st.dlink >= 0 ? a.D[st.dlink][x] : 1.0f;
}

// lanes per output when `outs` outputs share the work-group: a power of two
// up to 16, so that small steps still spread their sums over the threads
__device__ __forceinline__ int seq_group(int64_t outs) {
  int g = 1;
  while (g < 16 && (int64_t)(2 * g) * outs <= kSeqThreads) g *= 2;
  return g;
}

// sum_{k < K} term(k) by the G lanes of a group (lane j takes k = j, j+G, ...,
// four partial sums), then a fixed butterfly over the group; every lane of
// the group returns the total
template <typename F>
__device__ __forceinline__ float seq_group_sum(int K, int j, int G, F term) {
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  int k = j;
  for (; k + 3 * G < K; k += 4 * G) {
    a0 += term(k);
    a1 += term(k + G);
    a2 += term(k + 2 * G);
    a3 += term(k + 3 * G);
  }
  for (; k < K; k += G) a0 += term(k);
  float sum = (a0 + a1) + (a2 + a3);
  for (int o = G >> 1; o > 0; o >>= 1) sum += __shfl_xor(sum, o, G);
  return sum;
}

template <typename T>
__global__ __launch_bounds__(kSeqThreads) void k_seq_fwd(SeqArgs a) {
  typedef typename Elem<T>::type E;
  extern __shared__ __align__(16) float sm[];
  const int tid = threadIdx.x;
  const int64_t tok = blockIdx.x;
  float* in = sm;
  float* out = sm + a.max_state;
  float* gsm = sm + 2 * a.max_state;
  float* dv = gsm + a.max_core;
  const E* x = reinterpret_cast<const E*>(a.x) + tok * a.N_in;
  for (int i = tid; i < (int)a.N_in; i += kSeqThreads) in[i] = elem_to_f32<T>(x[i]);
  for (int t = 0; t < a.d; ++t) {
    const SeqStep& st = a.st[t];
    seq_stage(a, st, gsm, dv);
    __syncthreads();
    const int n = st.n, rin = st.rin, rout = st.rout;
    const int B = (int)st.B;
    const int outs = (int)st.out_size;
    const int G = seq_group(outs);
    const int j = tid % G;
    for (int e = tid / G; e < outs; e += kSeqThreads / G) {
      const int y = e % rout;
      float sum;
      if (!st.expand) {  // out[a][b][y] = sum_{i, x} in[a][i][b][x] dv[x] g(x, i, y)
        const int ab = e / rout;
        const int aa = ab / B, bb = ab - aa * B;
        const float* iv = in + (aa * n * B + bb) * rin;
        sum = seq_group_sum(n * rin, j, G, [&](int k) {
          const int i = k / rin, xx = k - i * rin;
          return iv[i * B * rin + xx] * dv[xx] * gsm[seq_gidx(st, xx, i, y)];
        });
      } else {  // out[a][i][b][y] = sum_x in[a][b][x] dv[x] g(x, i, y)
        const int r = e / rout;
        const int bb = r % B, ai = r / B;
        const int i = ai % n, aa = ai / n;
        const float* iv = in + (aa * B + bb) * rin;
        sum = seq_group_sum(rin, j, G, [&](int xx) { return iv[xx] * dv[xx] * gsm[seq_gidx(st, xx, i, y)]; });
      }
      if (j == 0) out[e] = sum;
    }
    __syncthreads();
    if (st.out_off >= 0) {
      float* sv = a.states + tok * a.state_floats + st.out_off;
      for (int e = tid; e < outs; e += kSeqThreads) sv[e] = out[e];
    } else {
      E* y = reinterpret_cast<E*>(a.y) + tok * a.N_out;
      for (int e = tid; e < (int)a.N_out; e += kSeqThreads) y[e] = (E)Mma<T>::from_f32(out[e]);
    }
    float* tmp = in;
    in = out;
    out = tmp;
  }
}

template <typename T>
__global__ __launch_bounds__(kSeqThreads) void k_seq_bwd(SeqArgs a) {
  typedef typename Elem<T>::type E;
  extern __shared__ __align__(16) float sm[];
  const int tid = threadIdx.x;
  const int64_t tok = blockIdx.x;
  float* sin = sm;
  float* gout = sm + a.max_state;
  float* gin = sm + 2 * a.max_state;
  float* gsm = sm + 3 * a.max_state;
  float* dv = gsm + a.max_core;
  const E* dy = reinterpret_cast<const E*>(a.dy) + tok * a.N_out;
  for (int i = tid; i < (int)a.N_out; i += kSeqThreads) gout[i] = elem_to_f32<T>(dy[i]);
  float* part = a.part + tok * a.part_floats;
  for (int t = a.d - 1; t >= 0; --t) {
    const SeqStep& st = a.st[t];
    if (st.in_off >= 0) {
      const float* sv = a.states + tok * a.state_floats + st.in_off;
      for (int e = tid; e < (int)st.in_size; e += kSeqThreads) sin[e] = sv[e];
    } else {
      const E* x = reinterpret_cast<const E*>(a.x) + tok * a.N_in;
      for (int e = tid; e < (int)a.N_in; e += kSeqThreads) sin[e] = elem_to_f32<T>(x[e]);
    }
    seq_stage(a, st, gsm, dv);
    __syncthreads();
    const int n = st.n, rin = st.rin, rout = st.rout;
    const int A = (int)st.A, B = (int)st.B;
    const int csz = rin * n * rout;
    // this token's share of the core gradient, in the core's own layout
    {
      const int G = seq_group(csz);
      const int j = tid % G;
      for (int ge = tid / G; ge < csz; ge += kSeqThreads / G) {
        int xx, i, y;
        if (st.rightward) {
          xx = ge / (n * rout);
          i = (ge / rout) % n;
          y = ge % rout;
        } else {
          y = ge / (n * rin);
          i = (ge / rin) % n;
          xx = ge % rin;
        }
        const float sum = seq_group_sum(A * B, j, G, [&](int k) {
          const int aa = k / B, bb = k - aa * B;
          return st.expand ? sin[(aa * B + bb) * rin + xx] * gout[((aa * n + i) * B + bb) * rout + y]
                           : sin[((aa * n + i) * B + bb) * rin + xx] * gout[(aa * B + bb) * rout + y];
        });
        if (j == 0) part[st.gp_off + ge] = sum * dv[xx];
      }
    }
    // gradient of the step's input state
    if (t > 0 || a.dx) {
      const int ins = (int)st.in_size;
      const int G = seq_group(ins);
      const int j = tid % G;
      for (int e = tid / G; e < ins; e += kSeqThreads / G) {
        const int xx = e % rin;
        float sum;
        if (!st.expand) {  // e = [a][i][b][x]
          const int r = e / rin;
          const int bb = r % B, ai = r / B;
          const int i = ai % n, aa = ai / n;
          const float* go = gout + (aa * B + bb) * rout;
          sum = seq_group_sum(rout, j, G, [&](int y) { return go[y] * gsm[seq_gidx(st, xx, i, y)]; });
        } else {  // e = [a][b][x]
          const int ab = e / rin;
          const int bb = ab % B, aa = ab / B;
          sum = seq_group_sum(n * rout, j, G, [&](int k) {
            const int i = k / rout, y = k - i * rout;
            return gout[((aa * n + i) * B + bb) * rout + y] * gsm[seq_gidx(st, xx, i, y)];
          });
        }
        if (j == 0) gin[e] = sum * dv[xx];
      }
    }
    __syncthreads();
    float* tmp = gout;
    gout = gin;
    gin = tmp;
  }
  if (a.dx) {
    E* dx = reinterpret_cast<E*>(a.dx) + tok * a.N_in;
    for (int e = tid; e < (int)a.N_in; e += kSeqThreads) dx[e] = (E)Mma<T>::from_f32(gout[e]);
  }
}

// dG_k = sum over the tokens of the partials, in token order
struct SeqRedArgs {
  const float* part;
  float* dG[kMaxCores];   // indexed by walk step
  int64_t off[kMaxCores + 1];
  int64_t T, part_floats;
  int d;
};
__global__ __launch_bounds__(256) void k_seq_reduce(SeqRedArgs a) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < a.part_floats;
       e += (int64_t)gridDim.x * blockDim.x) {
    int t = 0;
    while (t < a.d - 1 && e >= a.off[t + 1]) ++t;
    // eight tokens' partials requested together, added in token order
    const float* p = a.part + e;
    float acc = 0.f;
    int64_t k = 0;
    for (; k + 8 <= a.T; k += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = p[(k + u) * a.part_floats];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += v[u];
    }
    for (; k < a.T; ++k) acc += p[k * a.part_floats];
    a.dG[t][e - a.off[t]] = acc;
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

// dynamic LDS above 64 KB must be enabled per kernel; done once per kernel,
// before any graph capture can see it
static void allow_lds(const void* kern, size_t bytes) {
  if (bytes > 65536) (void)hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

// One layer's share of a streaming launch.
struct StreamJob {
  const LinearPlan* P;
  const void* x;
  const void* dy;
  char* sv;  // saved: the forward writes Z there, the backward reads it
  void* y;   // forward output
  void* dx;  // backward output, or null
  char* sc;  // backward scratch
};

#ifndef TTC_FWD_CUS
#define TTC_FWD_CUS 256  // compute units of an MI355X
#endif
constexpr int64_t kFwdCUs = TTC_FWD_CUS;
template <typename T, int NR, bool VEC, int TT, int NW, int PS, int XRW = 0>
static void launch_fwd_v(const StreamJob* jobs, int n, hipStream_t st) {
  typedef typename Elem<T>::type E;
  constexpr int TM = 16 * TT * PS;  // tokens per work-group
  const size_t lds = kFwdLdsBytes<T, NR, TT, NW>();
  auto kern = k_fwd<T, NR, VEC, TT, NW, PS, XRW>;
  static bool lds_set = false;
  if (!lds_set) {
    allow_lds((const void*)kern, lds);
    lds_set = true;
  }
  StreamBatch<FwdArgs<T>> b;
  memset(&b, 0, sizeof(b));
  // fewer token tiles than CUs: split each tile's output steps over column
  // groups so that the launch still covers the chip
  int64_t tiles_all = 0;
  for (int i = 0; i < n; ++i) tiles_all += (jobs[i].P->T + TM - 1) / TM;
  for (int i = 0; i < n; ++i) {
    const LinearPlan& P = *jobs[i].P;
    FwdArgs<T>& a = b.a[i];
    const int64_t tiles = (P.T + TM - 1) / TM;
    const int nst = (int)(((P.N_out + 15) / 16 + NW * kFwdUO(NR, NW) - 1) / (NW * kFwdUO(NR, NW)));
    a.cg_n = (NW == 8 || tiles_all == 0 || tiles_all >= kFwdCUs)
                 ? 1
                 : (int)std::min<int64_t>(nst, std::max<int64_t>(1, kFwdCUs / tiles_all));
    a.x = (const E*)jobs[i].x;
    a.Ac = (const E*)(jobs[i].sv + P.sv_Ac);
    a.Bc = (const E*)(jobs[i].sv + P.sv_Bc);
    a.Z = (E*)(jobs[i].sv + P.sv_Z);
    a.y = (E*)jobs[i].y;
    a.T_ = P.T;
    a.N_in = P.N_in;
    a.N_out = P.N_out;
    a.meta = (const int*)(jobs[i].sv + P.sv_meta);
    a.vin = (int)VEC;
    a.vout = (P.N_out % 4) == 0 && aligned16(jobs[i].y);
    b.first[i + 1] = b.first[i] + (int)(tiles * a.cg_n);
  }
  b.n = n;
  TraceScope ts("fwd", st);
  TTC_LAUNCH(kern, dim3((unsigned)b.first[n]), dim3(64 * NW), lds, st, b);
}

// 2-byte activations up to rank 64: 64-token work-groups of eight waves once
// there are enough tiles to give every CU one (with 16-byte rows in passes of
// 64 / TTC_FWD_PASSES tokens); otherwise 32-token work-groups of four waves.
#ifndef TTC_FWD_WIDE_TT
#define TTC_FWD_WIDE_TT 4
#endif
#ifndef TTC_FWD_PASSES
#define TTC_FWD_PASSES 1
#endif
static_assert(TTC_FWD_WIDE_TT % TTC_FWD_PASSES == 0, "whole 16-token tiles per pass");
#ifndef TTC_FWD_PASS_NIN
#define TTC_FWD_PASS_NIN 1024
#endif
#ifndef TTC_FWD_WIDE_TILES
#define TTC_FWD_WIDE_TILES 256
#endif
template <typename T>
static bool fwd_vec(const StreamJob& j) {
  const LinearPlan& P = *j.P;
  return (P.N_in % Mma<T>::EPV) == 0 && aligned16(j.x) && (P.N_out % Mma<T>::EPV) == 0 && aligned16(j.y);
}
template <typename T, int NR>
static void launch_fwd_group(const StreamJob* jobs, int n, bool vec, bool wide, hipStream_t st) {
  if constexpr (sizeof(typename Elem<T>::type) <= 2 && NR <= 4) {
    if (wide) {
      // passes for one layer per launch with a short input side (one round of
      // work-groups, little x per pass); otherwise one pass
      // (one-byte rows: at most two passes, so that a pass's Y chunk is a
      // whole number of 16-byte stores per thread)
      constexpr int PS = sizeof(typename Elem<T>::type) == 1 && TTC_FWD_PASSES > 2 ? 2 : TTC_FWD_PASSES;
      const bool passes = PS > 1 && n == 1 && jobs[0].P->N_in <= TTC_FWD_PASS_NIN;
      bool xr = TTC_FWD_XROWS && sizeof(typename Elem<T>::type) == 2 && TTC_FWD_WIDE_TT == 4, nt = TTC_FWD_XR_NT;
      for (int i = 0; i < n; ++i) {
        xr = xr && jobs[i].P->N_in * 2 >= TTC_FWD_XROWS_BYTES;
        nt = nt && jobs[i].P->N_in * 2 >= TTC_FWD_XR_NT_BYTES;
      }
      if (vec && passes) launch_fwd_v<T, NR, true, TTC_FWD_WIDE_TT / PS, 8, PS>(jobs, n, st);
      else if (vec && xr && nt) launch_fwd_v<T, NR, true, TTC_FWD_WIDE_TT, 8, 1, 2>(jobs, n, st);
      else if (vec && xr) launch_fwd_v<T, NR, true, TTC_FWD_WIDE_TT, 8, 1, 1>(jobs, n, st);
      else if (vec) launch_fwd_v<T, NR, true, TTC_FWD_WIDE_TT, 8, 1>(jobs, n, st);
      else launch_fwd_v<T, NR, false, TTC_FWD_WIDE_TT, 8, 1>(jobs, n, st);
      return;
    }
  }
  if (vec) launch_fwd_v<T, NR, true, 2, 4, 1>(jobs, n, st);
  else launch_fwd_v<T, NR, false, 2, 4, 1>(jobs, n, st);
}

// one dY-pass launch; NSL = 0: the slab of an item at run time, else the
// static-slab form for work-groups of at most NSL slabs
#ifndef TTC_DY_STATIC_SLABS
#define TTC_DY_STATIC_SLABS 1
#endif
template <typename T, int NR, bool VY, int NSL>
static void launch_dy(const StreamBatch<DyArgs<T>>& b, hipStream_t st) {
  typedef Bwd<T, NR> B;
  constexpr int NSM = NSL > 0 ? NSL : bwd_max_slabs(B::ES, NR);
  const size_t lds = size_t(B::Rpad) * (NSM * B::SW + 16 / B::ES) * B::ES + 2 * B::SLAB * B::ES +
                     size_t(B::ZTILE) * B::ES;
  static bool lds_set = false;
  if (!lds_set) {
    allow_lds((const void*)k_bwd_dy<T, NR, VY, NSL>, lds);
    lds_set = true;
  }
  TTC_LAUNCH((k_bwd_dy<T, NR, VY, NSL>), dim3((unsigned)b.first[b.n]), dim3(256), lds, st, b);
}
// the static-slab form for K = nsl (K <= MAX), else the run-time form
template <typename T, int NR, bool VY, int K, int MAX>
static void launch_dy_n(int nsl, const StreamBatch<DyArgs<T>>& b, hipStream_t st) {
  if constexpr (K > MAX)
    launch_dy<T, NR, VY, 0>(b, st);
  else if (nsl == K)
    launch_dy<T, NR, VY, K>(b, st);
  else
    launch_dy_n<T, NR, VY, K + 1, MAX>(nsl, b, st);
}

#ifndef TTC_DX_DZ_FOLD
#define TTC_DX_DZ_FOLD 1
#endif
template <typename T, int NR, bool VY, bool VX>
static void launch_bwd_v(const StreamJob* jobs, int n, hipStream_t st) {
  typedef Bwd<T, NR> B;
  typedef typename B::E E;
  // With several layers in one launch, each layer gets a share of the CUs by
  // its bytes and a grid shaped for that share (fewer, longer work-groups,
  // so fewer partial sums).  The partial buffers hold the plan's own grid,
  // which bounds the share's column groups (dY pass) and token groups.
  BwdGrid gy[kMaxStream], gx[kMaxStream];
  {
    double ty = 0.0, tx = 0.0;
    for (int i = 0; i < n; ++i) {
      ty += double(jobs[i].P->T) * double(jobs[i].P->N_out);
      tx += double(jobs[i].P->T) * double(jobs[i].P->N_in);
    }
    for (int i = 0; i < n; ++i) {
      const LinearPlan& P = *jobs[i].P;
      gy[i] = BwdGrid{P.dy_gc, P.dy_gt, P.dy_nsl, P.dy_tpg};
      gx[i] = BwdGrid{P.dx_gc, P.dx_gt, P.dx_nsl, P.dx_tpg};
      if (n > 1 && ty > 0.0 && tx > 0.0) {
        BwdGrid g;
        // (a batch's work-groups run long: shaped for two per CU; measured on
        // the batched Q, K, V passes: dY 27.6 -> 25.0 us, bf16 dX 35.4 -> 32.9
        // us; the e4m3 dX work-groups move half the bytes and lose, 24.2 ->
        // 31.8 us, so they stay at one per CU)
        const double cy = (TTC_BWD_TWO_PER_CU ? 2.0 : 1.0) * kPlanCUs;
        const double cx = (TTC_BWD_TWO_PER_CU && B::ES >= 2 ? 2.0 : 1.0) * kPlanCUs;
        if (plan_bwd_grid(P, true, std::max(1.0, cy * double(P.T) * double(P.N_out) / ty), P.dy_gc, P.dy_gt, &g))
          gy[i] = g;
        if (plan_bwd_grid(P, false, std::max(1.0, cx * double(P.T) * double(P.N_in) / tx), 0, P.dx_gt, &g))
          gx[i] = g;
      }
    }
  }
  {
    StreamBatch<DyArgs<T>> b;
    memset(&b, 0, sizeof(b));
    for (int i = 0; i < n; ++i) {
      const LinearPlan& P = *jobs[i].P;
      const char* saved = jobs[i].sv;
      char* scratch = jobs[i].sc;
      DyArgs<T>& a = b.a[i];
      a.dy = (const E*)jobs[i].dy;
      a.BcT = (const E*)(saved + P.sv_BcT);
      a.Z = (const E*)(saved + P.sv_Z);
      a.dZp = (float*)(scratch + P.sc_dZp);
      a.dZ = (E*)(scratch + P.sc_dZ);
      a.dBp = (float*)(scratch + P.sc_dBp);
      a.meta = (const int*)(saved + P.sv_meta);
      a.gts = (int*)(scratch + P.sc_gts);
      a.T_ = P.T;
      a.N_out = P.N_out;
      a.nsl = gy[i].nsl;
      a.tpg = gy[i].tpg;
      a.ntiles = P.ntiles;
      a.gc_n = gy[i].gc;
      a.vec = (P.N_out % B::EPV) == 0 && aligned16(jobs[i].dy);
      b.first[i + 1] = b.first[i] + gy[i].gc * gy[i].gt;
    }
    b.n = n;
    constexpr int NSM = bwd_max_slabs(B::ES, NR);
    int nsl_max = 1;
    for (int i = 0; i < n; ++i) nsl_max = std::max(nsl_max, gy[i].nsl);
    TraceScope ts("bwd_dy", st);
    if constexpr (VY && kBwdDepth == 2 && TTC_DY_STATIC_SLABS)
      launch_dy_n<T, NR, VY, 1, (NSM < 4 ? NSM : 4)>(nsl_max, b, st);
    else
      launch_dy<T, NR, VY, 0>(b, st);
  }
  // every layer's dY pass in two column groups and every dX work-group over
  // two slabs or more: the dX pass sums the two partials itself (one launch
  // fewer).  Measured: FFN2 (dX work-groups of two slabs) 4.2 us of sum
  // saved, its dX pass unchanged; the one-slab dX passes of O and Q, K, V
  // read four times the dZ bytes per slab and lose more than the sum costs
  // (O 14.5 -> 17.3 us, Q+K+V 29.7 -> 36.1 us)
  bool fold = VX && TTC_DX_DZ_FOLD;
  for (int i = 0; i < n; ++i) fold = fold && gy[i].gc == 2 && gx[i].nsl >= 2;
  if (!fold) {
    StreamBatch<DzArgs<T>> b;
    memset(&b, 0, sizeof(b));
    for (int i = 0; i < n; ++i) {
      const LinearPlan& P = *jobs[i].P;
      if (gy[i].gc <= 1) continue;
      const int64_t n4 = P.T * B::Rpad / 4;
      DzArgs<T>& a = b.a[b.n];
      a.dZp = (const float*)(jobs[i].sc + P.sc_dZp);
      a.dZ = (E*)(jobs[i].sc + P.sc_dZ);
      a.ngc = gy[i].gc;
      a.n4 = n4;
      b.first[b.n + 1] = b.first[b.n] + (int)std::min<int64_t>(4096, (n4 + 255) / 256);
      ++b.n;
    }
    if (b.n > 0) {
      TraceScope ts("dz_sum", st);
      TTC_LAUNCH(k_dz_sum<T>, dim3((unsigned)b.first[b.n]), dim3(256), 0, st, b);
    }
  }
  {
    StreamBatch<DxArgs<T>> b;
    memset(&b, 0, sizeof(b));
    for (int i = 0; i < n; ++i) {
      const LinearPlan& P = *jobs[i].P;
      const char* saved = jobs[i].sv;
      char* scratch = jobs[i].sc;
      DxArgs<T>& a = b.a[i];
      a.x = (const E*)jobs[i].x;
      a.AcT = (const E*)(saved + P.sv_AcT);
      a.dZ = (const E*)(scratch + P.sc_dZ);
      a.dZp = (const float*)(scratch + P.sc_dZp);
      a.dAp = (float*)(scratch + P.sc_dAp);
      a.dx = (E*)jobs[i].dx;
      a.meta = (const int*)(saved + P.sv_meta);
      a.gts = (int*)(scratch + P.sc_gts);
      a.T_ = P.T;
      a.N_in = P.N_in;
      a.nsl = gx[i].nsl;
      a.tpg = gx[i].tpg;
      a.ntiles = P.ntiles;
      a.vec = (P.N_in % B::EPV) == 0 && aligned16(jobs[i].x) && (jobs[i].dx == nullptr || aligned16(jobs[i].dx));
      a.gcols = gx[i].gc;
      b.first[i + 1] = b.first[i] + gx[i].gc * gx[i].gt;
    }
    b.n = n;
    constexpr int NSM = dx_max_slabs(B::ES, NR);
    const size_t lds = size_t(NSM) * B::SW * B::RLD * B::ES + 2 * B::SLAB * B::ES + size_t(64) * B::RLD * B::ES +
                       (B::ZT ? 0 : size_t(B::Rpad) * B::ZLD * B::ES);
    static bool lds_set = false;
    if (!lds_set) {
      allow_lds((const void*)k_bwd_dx<T, NR, VX, 0>, lds);
      if constexpr (VX) allow_lds((const void*)k_bwd_dx<T, NR, VX, 2>, lds);
      lds_set = true;
    }
    TraceScope ts("bwd_dx", st);
    if constexpr (VX) {
      if (fold) {
        TTC_LAUNCH((k_bwd_dx<T, NR, VX, 2>), dim3((unsigned)b.first[n]), dim3(256), lds, st, b);
        return;
      }
    }
    TTC_LAUNCH((k_bwd_dx<T, NR, VX, 0>), dim3((unsigned)b.first[n]), dim3(256), lds, st, b);
  }
}

template <typename T>
static bool bwd_vec(const StreamJob& j) {
  const LinearPlan& P = *j.P;
  const bool vy = (P.N_out % Mma<T>::EPV) == 0 && aligned16(j.dy);
  const bool vx = (P.N_in % Mma<T>::EPV) == 0 && aligned16(j.x) && (j.dx == nullptr || aligned16(j.dx));
  return vy && vx;
}
template <typename T, int NR>
static void launch_bwd_group(const StreamJob* jobs, int n, bool vec, hipStream_t st) {
  if (vec)
    launch_bwd_v<T, NR, true, true>(jobs, n, st);
  else
    launch_bwd_v<T, NR, false, false>(jobs, n, st);
}

static bool nr_supported(int NR) { return NR == 2 || NR == 4 || NR == 6 || NR == 8; }

// Streaming launches for a list of layers: layers that share a kernel
// instantiation (activation type, rank tile count, 16-byte form and, for the
// forward, the tile width) go into common launches of up to kMaxStream
// layers, in list order; the others get launches of their own.  The caller
// has checked nr_supported for every layer.
template <bool FWD, typename T>
static void launch_stream_group(const StreamJob* js, int m, int NR, bool vec, bool wide, hipStream_t st) {
  if constexpr (sizeof(typename Elem<T>::type) == 1) {
    // e4m3: rank tiles of 32 (one 32-wide k-step) and 64
    if constexpr (FWD) {
      if (NR == 2) launch_fwd_group<T, 2>(js, m, vec, wide, st);
      else launch_fwd_group<T, 4>(js, m, vec, wide, st);
    } else {
      if (NR == 2) launch_bwd_group<T, 2>(js, m, vec, st);
      else launch_bwd_group<T, 4>(js, m, vec, st);
    }
    return;
  }
  if constexpr (FWD) {
    switch (NR) {
      case 2: launch_fwd_group<T, 2>(js, m, vec, wide, st); break;
      case 4: launch_fwd_group<T, 4>(js, m, vec, wide, st); break;
      case 6: launch_fwd_group<T, 6>(js, m, vec, wide, st); break;
      case 8: launch_fwd_group<T, 8>(js, m, vec, wide, st); break;
    }
  } else {
    switch (NR) {
      case 2: launch_bwd_group<T, 2>(js, m, vec, st); break;
      case 4: launch_bwd_group<T, 4>(js, m, vec, st); break;
      case 6: launch_bwd_group<T, 6>(js, m, vec, st); break;
      case 8: launch_bwd_group<T, 8>(js, m, vec, st); break;
    }
  }
}

template <bool FWD>
static void launch_stream_jobs(const StreamJob* jobs, int n, hipStream_t st) {
  auto key = [&](const StreamJob& j) {
    const LinearPlan& P = *j.P;
    bool vec;
    if (P.act == TTC_BF16)
      vec = FWD ? fwd_vec<bf16_t>(j) : bwd_vec<bf16_t>(j);
    else if (P.act == TTC_FP8)
      vec = FWD ? fwd_vec<fp8_t>(j) : bwd_vec<fp8_t>(j);
    else
      vec = FWD ? fwd_vec<float>(j) : bwd_vec<float>(j);
    const bool wide = FWD && P.ntiles >= TTC_FWD_WIDE_TILES;
    return (P.act << 8) | (P.NR << 2) | ((int)vec << 1) | (int)wide;
  };
  std::vector<char> done(n, 0);
  std::vector<StreamJob> grp;
  for (int i = 0; i < n; ++i) {
    if (done[i]) continue;
    const int k = key(jobs[i]);
    grp.clear();
    for (int j = i; j < n; ++j)
      if (!done[j] && key(jobs[j]) == k) {
        grp.push_back(jobs[j]);
        done[j] = 1;
      }
    const int act = k >> 8;
    const int NR = (k >> 2) & 63;
    const bool vec = (k >> 1) & 1, wide = k & 1;
    for (size_t g0 = 0; g0 < grp.size(); g0 += kMaxStream) {
      const int m = (int)std::min<size_t>(kMaxStream, grp.size() - g0);
      const StreamJob* js = grp.data() + g0;
      if (act == TTC_BF16)
        launch_stream_group<FWD, bf16_t>(js, m, NR, vec, wide, st);
      else if (act == TTC_FP8)
        launch_stream_group<FWD, fp8_t>(js, m, NR, vec, wide, st);
      else
        launch_stream_group<FWD, float>(js, m, NR, vec, wide, st);
    }
  }
}

static SeqArgs seq_args(const LinearPlan& P, const float* const* G, const float* const* D, const void* x,
                        const void* dy, void* y, void* dx, const char* sv, char* sc) {
  SeqArgs a;
  memset(&a, 0, sizeof(a));
  for (int t = 0; t < P.d; ++t) a.st[t] = P.seq[t];
  for (int k = 0; k < P.d; ++k) a.G[k] = G[k];
  for (int k = 0; k < P.d - 1; ++k) a.D[k] = D[k];
  a.x = x;
  a.dy = dy;
  a.y = y;
  a.dx = dx;
  a.states = reinterpret_cast<float*>(const_cast<char*>(sv));
  a.part = reinterpret_cast<float*>(sc);
  a.N_in = P.N_in;
  a.N_out = P.N_out;
  a.state_floats = P.seq_state_floats;
  a.part_floats = P.seq_part_floats;
  a.max_state = P.seq_max_state;
  a.max_core = P.seq_max_core;
  a.d = P.d;
  return a;
}

// dynamic LDS above 64 KB for the sequential kernels, once per kernel
template <int WHICH>
static void seq_allow_lds(const void* kern) {
  static bool done = false;
  if (!done) {
    allow_lds(kern, kSeqMaxLds);
    done = true;
  }
}

static void launch_seq_fwd(const LinearPlan& P, const SeqArgs& a, hipStream_t st) {
  TraceScope ts("seq_fwd", st);
  if (P.act == TTC_BF16) {
    seq_allow_lds<0>((const void*)k_seq_fwd<bf16_t>);
    TTC_LAUNCH(k_seq_fwd<bf16_t>, dim3((unsigned)P.T), dim3(kSeqThreads), P.seq_lds_fwd, st, a);
  } else if (P.act == TTC_FP8) {
    seq_allow_lds<4>((const void*)k_seq_fwd<fp8_t>);
    TTC_LAUNCH(k_seq_fwd<fp8_t>, dim3((unsigned)P.T), dim3(kSeqThreads), P.seq_lds_fwd, st, a);
  } else {
    seq_allow_lds<1>((const void*)k_seq_fwd<float>);
    TTC_LAUNCH(k_seq_fwd<float>, dim3((unsigned)P.T), dim3(kSeqThreads), P.seq_lds_fwd, st, a);
  }
}

static void launch_seq_bwd(const LinearPlan& P, const SeqArgs& a, hipStream_t st) {
  TraceScope ts("seq_bwd", st);
  if (P.act == TTC_BF16) {
    seq_allow_lds<2>((const void*)k_seq_bwd<bf16_t>);
    TTC_LAUNCH(k_seq_bwd<bf16_t>, dim3((unsigned)P.T), dim3(kSeqThreads), P.seq_lds_bwd, st, a);
  } else if (P.act == TTC_FP8) {
    seq_allow_lds<5>((const void*)k_seq_bwd<fp8_t>);
    TTC_LAUNCH(k_seq_bwd<fp8_t>, dim3((unsigned)P.T), dim3(kSeqThreads), P.seq_lds_bwd, st, a);
  } else {
    seq_allow_lds<3>((const void*)k_seq_bwd<float>);
    TTC_LAUNCH(k_seq_bwd<float>, dim3((unsigned)P.T), dim3(kSeqThreads), P.seq_lds_bwd, st, a);
  }
}

static void launch_seq_reduce(const LinearPlan& P, const char* sc, float* const* dG, hipStream_t st) {
  SeqRedArgs r;
  memset(&r, 0, sizeof(r));
  r.part = reinterpret_cast<const float*>(sc);
  for (int t = 0; t < P.d; ++t) {
    r.dG[t] = dG[P.seq[t].core];
    r.off[t] = P.seq[t].gp_off;
  }
  r.off[P.d] = P.seq_part_floats;
  r.T = P.T;
  r.part_floats = P.seq_part_floats;
  r.d = P.d;
  TraceScope ts("seq_reduce", st);
  TTC_LAUNCH(k_seq_reduce, dim3((unsigned)std::max<int64_t>(1, std::min<int64_t>(1024, (P.seq_part_floats + 255) / 256))),
             dim3(256), 0, st, r);
}

static unsigned grid_for(int64_t n, int64_t per_block, int64_t cap) {
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(cap, (n + per_block - 1) / per_block));
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

namespace ttc {
// One layer of a batched merge or core-gradient launch.
struct LayerJob {
  LinearPlan P;
  ChainPtrs c;
  char* sv;
  char* sc;
  float* dG[kMaxCores];
};

// Independent GEMMs in launches of at most kMaxGemm.
static void launch_gemm_list(const Gemm* gs, int n, const char* name, hipStream_t s) {
  static bool lds_set = false;
  if (!lds_set) {
    allow_lds((const void*)k_sweep, kSweepLds);
    lds_set = true;
  }
  for (int i = 0; i < n; i += kMaxGemm) {
    SweepArgs a;
    memset(&a, 0, sizeof(a));
    int total = 0;
    for (int q = 0; q < std::min(kMaxGemm, n - i); ++q) {
      a.g[q] = gs[i + q];
      a.tiles[q] = gemm_tiles(gs[i + q]);
      total += a.tiles[q];
      ++a.ng;
    }
    TraceScope ts(name, s);
    TTC_LAUNCH(k_sweep, dim3(total), dim3(kSweepThreads), kSweepLds, s, a);
  }
}

// the FAST merge's limits (one layer): at most three cores per half, every
// rank at most kMergeX, each half's last core mode times the split rank at
// most one output per thread
static bool merge_fast_ok(const LinearPlan& P) {
  if (P.s > 3 || P.d - P.s > 3) return false;
  for (int k = 0; k <= P.d; ++k)
    if (P.ranks[k] > kMergeX) return false;
  return P.modes[P.s - 1] * P.rs <= kMergeThreads && P.modes[P.s] * P.rs <= kMergeThreads;
}

static MergeLayer merge_layer(const LayerJob& j) {
  const LinearPlan& P = j.P;
  char* sv = j.sv;
  MergeLayer m;
  memset(&m, 0, sizeof(m));
  for (int k = 0; k < P.d; ++k) {
    m.G[k] = j.c.G[k];
    m.modes[k] = P.modes[k];
    m.chain_off[k] = P.chain_off[k] < 0 ? 0 : (int)P.chain_off[k];
    m.lstride[k] = P.lstride[k];
  }
  for (int k = 0; k < P.d - 1; ++k) m.D[k] = j.c.D[k];
  for (int k = 0; k <= P.d; ++k) m.ranks[k] = P.ranks[k];
  m.chain = reinterpret_cast<float*>(sv + P.sv_chain);
  m.Ac = sv + P.sv_Ac;
  m.AcT = sv + P.sv_AcT;
  m.Bc = sv + P.sv_Bc;
  m.BcT = sv + P.sv_BcT;
  m.meta = reinterpret_cast<int*>(sv + P.sv_meta);
  m.N_in = P.N_in;
  m.N_out = P.N_out;
  m.npl = P.NL / P.modes[P.s - 1];
  m.npr = P.NRt / P.modes[P.s];
  m.wgl = (m.npl + kMergePG - 1) / kMergePG;
  m.d = P.d;
  m.s = P.s;
  m.in_first = P.in_first;
  m.rs = P.rs;
  m.Rpad = P.Rpad;
  return m;
}

// Merge of n layers: one launch per activation dtype and kMaxMerge layers.
#ifndef TTC_MERGE_FAST
#define TTC_MERGE_FAST 1
#endif
static void launch_merge_batch(const LayerJob* jobs, int n, hipStream_t s) {
  for (int act = 0; act < 3; ++act) {
    const int want = act == 0 ? TTC_BF16 : (act == 1 ? TTC_F32 : TTC_FP8);
    MergeBatch mb;
    memset(&mb, 0, sizeof(mb));
    bool fast = true;
    auto flush = [&]() {
      if (mb.n == 0) return;
      TraceScope ts("merge", s);
      const dim3 grid((unsigned)mb.first[mb.n]);
      if (want == TTC_BF16) {
        if (fast) TTC_LAUNCH((k_merge<bf16_t, true>), grid, dim3(kMergeThreads), 0, s, mb);
        else TTC_LAUNCH((k_merge<bf16_t, false>), grid, dim3(kMergeThreads), 0, s, mb);
      } else if (want == TTC_FP8) {
        if (fast) TTC_LAUNCH((k_merge<fp8_t, true>), grid, dim3(kMergeThreads), 0, s, mb);
        else TTC_LAUNCH((k_merge<fp8_t, false>), grid, dim3(kMergeThreads), 0, s, mb);
      } else {
        if (fast) TTC_LAUNCH((k_merge<float, true>), grid, dim3(kMergeThreads), 0, s, mb);
        else TTC_LAUNCH((k_merge<float, false>), grid, dim3(kMergeThreads), 0, s, mb);
      }
      memset(&mb, 0, sizeof(mb));
      fast = true;
    };
    for (int i = 0; i < n; ++i) {
      if (jobs[i].P.act != want) continue;
      MergeLayer& m = mb.l[mb.n];
      m = merge_layer(jobs[i]);
      fast = fast && TTC_MERGE_FAST && merge_fast_ok(jobs[i].P);
      mb.first[mb.n + 1] = mb.first[mb.n] + m.wgl + (m.npr + kMergePG - 1) / kMergePG;
      if (++mb.n == kMaxMerge) flush();
    }
    flush();
  }
}

static void launch_merge(const LinearPlan& P, const float* const* G, const float* const* D, char* sv, hipStream_t s) {
  LayerJob j;
  memset(&j, 0, sizeof(j));
  j.P = P;
  j.c = chain_ptrs(P, G, D);
  j.sv = sv;
  launch_merge_batch(&j, 1, s);
}

// one event orders the two streams of a split backward; a wait captures the
// event's state when it is enqueued, so the event can be recorded again
// right away
static hipEvent_t split_event() {
  static std::mutex mu;
  static hipEvent_t ev = nullptr;
  std::lock_guard<std::mutex> lk(mu);
  if (!ev && hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) ev = nullptr;
  return ev;
}
static std::mutex g_split_mu;
}  // namespace ttc

extern "C" ttc_status tt_linear_prepare(const tt_linear_desc* desc, int64_t T, const float* const* G,
                                        const float* const* D, void* saved, size_t saved_bytes,
                                        ttc_stream_t stream) {
  LinearPlan P;
  ttc_status st = make_linear_plan(desc, T, &P);
  if (st != TTC_OK) return st;
  if ((st = check_chain(P, G, D)) != TTC_OK) return st;
  if (!saved) return TTC_ERR_NULL;
  if (!aligned16(saved)) return TTC_ERR_ALIGN;
  if (saved_bytes < P.sv_total) return TTC_ERR_WORKSPACE;
  if (P.path == TTC_PATH_SEQUENTIAL) return TTC_OK;  // nothing to merge
  (void)hipGetLastError();
  launch_merge(P, G, D, static_cast<char*>(saved), reinterpret_cast<hipStream_t>(stream));
  return hip_status();
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
  if (P.path == TTC_PATH_SEQUENTIAL) {
    launch_seq_fwd(P, seq_args(P, G, D, x, nullptr, y, nullptr, sv, nullptr), s);
    return hip_status();
  }
  if (!nr_supported(P.NR)) return TTC_ERR_UNSUPPORTED;
  if (!(desc->flags & TTC_FLAG_PREPARED)) launch_merge(P, G, D, sv, s);
  StreamJob j{&P, x, nullptr, sv, y, nullptr, nullptr};
  launch_stream_jobs<true>(&j, 1, s);
  return hip_status();
}

namespace ttc {
// Partial sums left in scratch by the streaming passes -> gradients of the two
// half products (a half made of one core receives its gradient directly) ->
// reverse sweep through both halves; for n layers, the reductions in launches
// of kMaxBatch layers and one launch per sweep level for all of them.
static void launch_cores_batch(const LayerJob* jobs, int n, hipStream_t s) {
  struct Walk {
    const float* curL;
    const float* curR;
    int64_t rowsL, colsR;
  };
  std::vector<Walk> wk(n);
  ReduceBatch rb;
  memset(&rb, 0, sizeof(rb));
  auto flush = [&]() {
    if (rb.n == 0) return;
    TraceScope ts("reduce", s);
    TTC_LAUNCH(k_reduce, dim3((unsigned)rb.first[rb.n]), dim3(256), 0, s, rb);
    memset(&rb, 0, sizeof(rb));
  };
  for (int i = 0; i < n; ++i) {
    const LinearPlan& P = jobs[i].P;
    const char* sv = jobs[i].sv;
    char* sc = jobs[i].sc;
    float* const* dG = jobs[i].dG;
    float* dL = P.s == 1 ? dG[0] : (float*)(sc + P.sc_dL);
    float* dR = P.d - P.s == 1 ? dG[P.d - 1] : (float*)(sc + P.sc_dR);
    ReduceArgs& r = rb.r[rb.n];
    r.dBp = (const float*)(sc + P.sc_dBp);
    r.dAp = (const float*)(sc + P.sc_dAp);
    r.gts = (const int*)(sc + P.sc_gts);
    r.gtB = P.dy_gt;
    r.gtA = P.dx_gt;
    r.meta = (const int*)(sv + P.sv_meta);
    r.Ds = jobs[i].c.D[P.s - 1];
    r.dL = dL;
    r.dR = dR;
    r.N_out = P.N_out;
    r.N_in = P.N_in;
    r.rs = P.rs;
    r.Rpad = P.Rpad;
    r.in_first = P.in_first;
    r.perm = !P.perm_trivial;
    r.nmB = P.p;
    r.nmA = P.q;
    for (int k = 0; k < P.d; ++k) {
      if (P.is_in[k]) {
        r.szA[P.lidx[k]] = P.modes[k];
        r.csA[P.lidx[k]] = P.cstride[k];
      } else {
        r.szB[P.lidx[k]] = P.modes[k];
        r.csB[P.lidx[k]] = P.cstride[k];
      }
    }
    rb.first[rb.n + 1] =
        rb.first[rb.n] + (int64_t)P.rs * (((P.N_out + 3) / 4 + 63) / 64 + ((P.N_in + 3) / 4 + 63) / 64);
    if (++rb.n == kMaxBatch) flush();
    wk[i] = Walk{dL, dR, P.NL, P.NRt};
  }
  flush();
  std::vector<Gemm> gs;
  for (int lvl = 0;; ++lvl) {
    gs.clear();
    for (int i = 0; i < n; ++i) {
      const LinearPlan& P = jobs[i].P;
      const float* const* G = jobs[i].c.G;
      const float* const* D = jobs[i].c.D;
      float* const* dG = jobs[i].dG;
      char* sc = jobs[i].sc;
      const float* chain = reinterpret_cast<const float*>(jobs[i].sv + P.sv_chain);
      float* wL = (float*)(sc + ((lvl & 1) ? P.sc_w1 : P.sc_w0));
      float* wR = wL + P.wl_floats;
      const int kL = P.s - 1 - lvl, kR = P.s + lvl;
      const bool hasL = kL >= 1, hasR = kR <= P.d - 2;
      Walk& w = wk[i];
      if (hasL) {
        float* outL = kL - 1 == 0 ? dG[0] : wL;
        gs.push_back(left_dG(P, chain, D, dG[kL], kL, w.curL, w.rowsL));
        gs.push_back(left_dM(P, G, D, kL, w.curL, w.rowsL, outL));
        w.curL = outL;
        w.rowsL /= P.modes[kL];
      }
      if (hasR) {
        float* outR = kR + 1 == P.d - 1 ? dG[P.d - 1] : wR;
        gs.push_back(right_dG(P, chain, D, dG[kR], kR, w.curR, w.colsR));
        gs.push_back(right_dN(P, G, D, kR, w.curR, w.colsR, outR));
        w.curR = outR;
        w.colsR /= P.modes[kR];
      }
    }
    if (gs.empty()) break;
    launch_gemm_list(gs.data(), (int)gs.size(), "core", s);
  }
}

static void launch_bwd_cores(const LinearPlan& P, const float* const* G, const float* const* D, const char* sv,
                             char* sc, float* const* dG, hipStream_t s) {
  LayerJob j;
  memset(&j, 0, sizeof(j));
  j.P = P;
  j.c = chain_ptrs(P, G, D);
  j.sv = const_cast<char*>(sv);
  j.sc = sc;
  for (int k = 0; k < P.d; ++k) j.dG[k] = dG[k];
  launch_cores_batch(&j, 1, s);
}

static void launch_zero_grads(const LinearPlan& P, float* const* dG, hipStream_t s) {
  for (int k = 0; k < P.d; ++k) {
    const int64_t n = (int64_t)P.ranks[k] * P.modes[k] * P.ranks[k + 1];
    TraceScope ts("zero", s);
    TTC_LAUNCH(k_zero, dim3(grid_for(n, 256, 1024)), dim3(256), 0, s, dG[k], n);
  }
}

// argument checks shared by the backward entry points; *P is the plan
static ttc_status bwd_checks(const tt_linear_desc* desc, int64_t T, const float* const* G, const float* const* D,
                             LinearPlan* P) {
  ttc_status st = make_linear_plan(desc, T, P);
  if (st != TTC_OK) return st;
  return check_chain(*P, G, D);
}
static ttc_status grads_checks(const LinearPlan& P, float* const* dG) {
  if (!dG) return TTC_ERR_NULL;
  for (int k = 0; k < P.d; ++k)
    if (!dG[k]) return TTC_ERR_NULL;
  return TTC_OK;
}
// null pointers first, then alignment, then sizes; x and dy are checked
// when `data` is set (the streaming passes read them)
static ttc_status buffer_checks(const LinearPlan& P, bool data, const void* x, const void* dy, const void* dx,
                                const void* saved, size_t saved_bytes, const void* scratch, size_t scratch_bytes) {
  if ((data && (!x || !dy)) || !saved || !scratch) return TTC_ERR_NULL;
  if ((data && (!aligned16(x) || !aligned16(dy) || (dx && !aligned16(dx)))) || !aligned16(saved) ||
      !aligned16(scratch))
    return TTC_ERR_ALIGN;
  if (saved_bytes < P.sv_total || scratch_bytes < P.sc_total) return TTC_ERR_WORKSPACE;
  return TTC_OK;
}
}  // namespace ttc

extern "C" ttc_status tt_linear_bwd(const tt_linear_desc* desc, int64_t T, const void* x, const void* dy,
                                    const float* const* G, const float* const* D, const void* saved,
                                    size_t saved_bytes, void* dx, float* const* dG, void* scratch,
                                    size_t scratch_bytes, ttc_stream_t stream) {
  return tt_linear_bwd_split(desc, T, x, dy, G, D, saved, saved_bytes, dx, dG, scratch, scratch_bytes, stream,
                             stream);
}

extern "C" ttc_status tt_linear_bwd_split(const tt_linear_desc* desc, int64_t T, const void* x, const void* dy,
                                          const float* const* G, const float* const* D, const void* saved,
                                          size_t saved_bytes, void* dx, float* const* dG, void* scratch,
                                          size_t scratch_bytes, ttc_stream_t stream, ttc_stream_t grad_stream) {
  LinearPlan P;
  ttc_status st = bwd_checks(desc, T, G, D, &P);
  if (st != TTC_OK) return st;
  if ((st = grads_checks(P, dG)) != TTC_OK) return st;
  hipStream_t s_main = reinterpret_cast<hipStream_t>(stream);
  hipStream_t s = reinterpret_cast<hipStream_t>(grad_stream);  // the core-gradient tail
  (void)hipGetLastError();
  if (T == 0) {
    launch_zero_grads(P, dG, s);
    return hip_status();
  }
  if ((st = buffer_checks(P, true, x, dy, dx, saved, saved_bytes, scratch, scratch_bytes)) != TTC_OK) return st;
  const char* sv = static_cast<const char*>(saved);
  char* sc = static_cast<char*>(scratch);
  if (P.path == TTC_PATH_SEQUENTIAL) {
    launch_seq_bwd(P, seq_args(P, G, D, x, dy, nullptr, dx, sv, sc), s_main);
  } else {
    if (!nr_supported(P.NR)) return TTC_ERR_UNSUPPORTED;
    StreamJob job{&P, x, dy, const_cast<char*>(sv), nullptr, dx, sc};
    launch_stream_jobs<false>(&job, 1, s_main);
  }
  if (s != s_main) {
    hipEvent_t ev = split_event();
    if (!ev) return TTC_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_split_mu);
    if (hipEventRecord(ev, s_main) != hipSuccess || hipStreamWaitEvent(s, ev, 0) != hipSuccess) return TTC_ERR_HIP;
  }
  if (P.path == TTC_PATH_SEQUENTIAL)
    launch_seq_reduce(P, sc, dG, s);
  else
    launch_bwd_cores(P, G, D, sv, sc, dG, s);
  return hip_status();
}

// ------------------------------------------------------------------------------
// backward without a caller-provided scratch buffer
// ------------------------------------------------------------------------------
// For callers that cannot allocate device memory: the partial sums of the
// backward live in one file-scope device array.  Every GPU the library runs
// on holds its own copy until the process ends; calls on one GPU share it.
namespace ttc {
namespace noalloc {
static __device__ __align__(256) unsigned char scratch[TTC_NOALLOC_SCRATCH_BYTES];
}  // namespace noalloc

constexpr int kMaxDevices = 64;
static std::mutex g_noalloc_mu;
static void* g_noalloc_ptr[kMaxDevices];

// Device address of the current device's copy of noalloc::scratch, looked up
// once per device (with that device current).  In host code the array's name
// is only a stand-in: kernels get this address, never the name.
static ttc_status noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TTC_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_noalloc_mu);
  if (!g_noalloc_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc::scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return TTC_ERR_HIP;
    }
    g_noalloc_ptr[dev] = p;
  }
  *out = g_noalloc_ptr[dev];
  return TTC_OK;
}
}  // namespace ttc

extern "C" ttc_status tt_linear_bwd_noalloc(const tt_linear_desc* desc, int64_t T, const void* x, const void* dy,
                                            const float* const* G, const float* const* D, const void* saved,
                                            size_t saved_bytes, void* dx, float* const* dG, ttc_stream_t stream) {
  LinearPlan P;
  ttc_status st = bwd_checks(desc, T, G, D, &P);
  if (st != TTC_OK) return st;
  if ((st = grads_checks(P, dG)) != TTC_OK) return st;
  if (P.sc_total > (size_t)TTC_NOALLOC_SCRATCH_BYTES) return TTC_ERR_WORKSPACE;
  void* sc = nullptr;
  if ((st = noalloc_scratch(&sc)) != TTC_OK) return st;
  // every byte the backward reads from its scratch is written earlier in the
  // same call, so the array needs no clearing between calls
  return tt_linear_bwd(desc, T, x, dy, G, D, saved, saved_bytes, dx, dG, sc, TTC_NOALLOC_SCRATCH_BYTES, stream);
}

extern "C" ttc_status tt_linear_bwd_data(const tt_linear_desc* desc, int64_t T, const void* x, const void* dy,
                                         const float* const* G, const float* const* D, const void* saved,
                                         size_t saved_bytes, void* dx, void* scratch, size_t scratch_bytes,
                                         ttc_stream_t stream) {
  LinearPlan P;
  ttc_status st = bwd_checks(desc, T, G, D, &P);
  if (st != TTC_OK) return st;
  if (T == 0) return TTC_OK;
  if ((st = buffer_checks(P, true, x, dy, dx, saved, saved_bytes, scratch, scratch_bytes)) != TTC_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const char* sv = static_cast<const char*>(saved);
  char* sc = static_cast<char*>(scratch);
  if (P.path == TTC_PATH_SEQUENTIAL) {
    launch_seq_bwd(P, seq_args(P, G, D, x, dy, nullptr, dx, sv, sc), s);
    return hip_status();
  }
  if (!nr_supported(P.NR)) return TTC_ERR_UNSUPPORTED;
  StreamJob job{&P, x, dy, const_cast<char*>(sv), nullptr, dx, sc};
  launch_stream_jobs<false>(&job, 1, s);
  return hip_status();
}

extern "C" ttc_status tt_linear_bwd_cores(const tt_linear_desc* desc, int64_t T, const float* const* G,
                                          const float* const* D, const void* saved, size_t saved_bytes,
                                          float* const* dG, void* scratch, size_t scratch_bytes,
                                          ttc_stream_t stream) {
  LinearPlan P;
  ttc_status st = bwd_checks(desc, T, G, D, &P);
  if (st != TTC_OK) return st;
  if ((st = grads_checks(P, dG)) != TTC_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (T == 0) {
    launch_zero_grads(P, dG, s);
    return hip_status();
  }
  if ((st = buffer_checks(P, false, nullptr, nullptr, nullptr, saved, saved_bytes, scratch, scratch_bytes)) !=
      TTC_OK)
    return st;
  if (P.path == TTC_PATH_SEQUENTIAL)
    launch_seq_reduce(P, static_cast<const char*>(scratch), dG, s);
  else
    launch_bwd_cores(P, G, D, static_cast<const char*>(saved), static_cast<char*>(scratch), dG, s);
  return hip_status();
}

extern "C" ttc_status tt_linear_prepare_batch(int32_t n, const tt_linear_desc* const* descs, const int64_t* T,
                                              const float* const* const* G, const float* const* const* D,
                                              void* const* saved, const size_t* saved_bytes, ttc_stream_t stream) {
  if (n < 0) return TTC_ERR_SHAPE;
  if (n == 0) return TTC_OK;
  if (!descs || !T || !G || !D || !saved || !saved_bytes) return TTC_ERR_NULL;
  std::vector<LayerJob> jobs(n);
  for (int i = 0; i < n; ++i) {
    LayerJob& j = jobs[i];
    memset(&j, 0, sizeof(j));
    if (!descs[i]) return TTC_ERR_NULL;
    ttc_status st = make_linear_plan(descs[i], T[i], &j.P);
    if (st != TTC_OK) return st;
    if ((st = check_chain(j.P, G[i], D[i])) != TTC_OK) return st;
    if (!saved[i]) return TTC_ERR_NULL;
    if (!aligned16(saved[i])) return TTC_ERR_ALIGN;
    if (saved_bytes[i] < j.P.sv_total) return TTC_ERR_WORKSPACE;
    j.c = chain_ptrs(j.P, G[i], D[i]);
    j.sv = static_cast<char*>(saved[i]);
  }
  // layers on the sequential path have nothing to merge
  jobs.erase(std::remove_if(jobs.begin(), jobs.end(), [](const LayerJob& j) { return j.P.path == TTC_PATH_SEQUENTIAL; }),
             jobs.end());
  if (jobs.empty()) return TTC_OK;
  (void)hipGetLastError();
  if (!jobs.empty()) launch_merge_batch(jobs.data(), (int)jobs.size(), reinterpret_cast<hipStream_t>(stream));
  return hip_status();
}

extern "C" ttc_status tt_linear_bwd_cores_batch(int32_t n, const tt_linear_desc* const* descs, const int64_t* T,
                                                const float* const* const* G, const float* const* const* D,
                                                const void* const* saved, const size_t* saved_bytes,
                                                float* const* const* dG, void* const* scratch,
                                                const size_t* scratch_bytes, ttc_stream_t stream) {
  if (n < 0) return TTC_ERR_SHAPE;
  if (n == 0) return TTC_OK;
  if (!descs || !T || !G || !D || !saved || !saved_bytes || !dG || !scratch || !scratch_bytes) return TTC_ERR_NULL;
  std::vector<LayerJob> jobs;
  jobs.reserve(n);
  std::vector<int> empty;
  for (int i = 0; i < n; ++i) {
    LayerJob j;
    memset(&j, 0, sizeof(j));
    if (!descs[i]) return TTC_ERR_NULL;
    ttc_status st = bwd_checks(descs[i], T[i], G[i], D[i], &j.P);
    if (st != TTC_OK) return st;
    if ((st = grads_checks(j.P, dG[i])) != TTC_OK) return st;
    if (T[i] == 0) {
      empty.push_back(i);
      continue;
    }
    if ((st = buffer_checks(j.P, false, nullptr, nullptr, nullptr, saved[i], saved_bytes[i], scratch[i],
                            scratch_bytes[i])) != TTC_OK)
      return st;
    j.c = chain_ptrs(j.P, G[i], D[i]);
    j.sv = const_cast<char*>(static_cast<const char*>(saved[i]));
    j.sc = static_cast<char*>(scratch[i]);
    for (int k = 0; k < j.P.d; ++k) j.dG[k] = dG[i][k];
    jobs.push_back(j);
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  for (int i : empty) {
    LinearPlan P;
    make_linear_plan(descs[i], 0, &P);
    launch_zero_grads(P, dG[i], s);
  }
  std::vector<LayerJob> merged;
  for (const LayerJob& j : jobs) {
    if (j.P.path == TTC_PATH_SEQUENTIAL)
      launch_seq_reduce(j.P, j.sc, j.dG, s);
    else
      merged.push_back(j);
  }
  if (!merged.empty()) launch_cores_batch(merged.data(), (int)merged.size(), s);
  return hip_status();
}

extern "C" ttc_status tt_linear_fwd_batch(int32_t n, const tt_linear_desc* const* descs, const int64_t* T,
                                          const void* const* x, const float* const* const* G,
                                          const float* const* const* D, void* const* y, void* const* saved,
                                          const size_t* saved_bytes, ttc_stream_t stream) {
  if (n < 0) return TTC_ERR_SHAPE;
  if (n == 0) return TTC_OK;
  if (!descs || !T || !x || !G || !D || !y || !saved || !saved_bytes) return TTC_ERR_NULL;
  std::vector<LinearPlan> plans(n);
  std::vector<LayerJob> merges;
  std::vector<StreamJob> jobs;
  std::vector<SeqArgs> seqs;
  std::vector<const LinearPlan*> seq_plans;
  for (int i = 0; i < n; ++i) {
    if (!descs[i]) return TTC_ERR_NULL;
    LinearPlan& P = plans[i];
    ttc_status st = make_linear_plan(descs[i], T[i], &P);
    if (st != TTC_OK) return st;
    if ((st = check_chain(P, G[i], D[i])) != TTC_OK) return st;
    if (T[i] == 0) continue;
    if (!x[i] || !y[i] || !saved[i]) return TTC_ERR_NULL;
    if (!aligned16(x[i]) || !aligned16(y[i]) || !aligned16(saved[i])) return TTC_ERR_ALIGN;
    if (saved_bytes[i] < P.sv_total) return TTC_ERR_WORKSPACE;
    if (P.path == TTC_PATH_SEQUENTIAL) {
      seqs.push_back(seq_args(P, G[i], D[i], x[i], nullptr, y[i], nullptr, static_cast<char*>(saved[i]), nullptr));
      seq_plans.push_back(&P);
      continue;
    }
    if (!nr_supported(P.NR)) return TTC_ERR_UNSUPPORTED;
    if (!(descs[i]->flags & TTC_FLAG_PREPARED)) {
      LayerJob m;
      memset(&m, 0, sizeof(m));
      m.P = P;
      m.c = chain_ptrs(P, G[i], D[i]);
      m.sv = static_cast<char*>(saved[i]);
      merges.push_back(m);
    }
    jobs.push_back(StreamJob{&P, x[i], nullptr, static_cast<char*>(saved[i]), y[i], nullptr, nullptr});
  }
  if (jobs.empty() && seqs.empty()) return TTC_OK;  // every layer has T == 0
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  for (size_t i = 0; i < seqs.size(); ++i) launch_seq_fwd(*seq_plans[i], seqs[i], s);
  if (jobs.empty()) return hip_status();  // every layer is sequential or has T == 0
  if (!merges.empty()) launch_merge_batch(merges.data(), (int)merges.size(), s);
  launch_stream_jobs<true>(jobs.data(), (int)jobs.size(), s);
  return hip_status();
}

extern "C" ttc_status tt_linear_bwd_data_batch(int32_t n, const tt_linear_desc* const* descs, const int64_t* T,
                                               const void* const* x, const void* const* dy,
                                               const float* const* const* G, const float* const* const* D,
                                               const void* const* saved, const size_t* saved_bytes,
                                               void* const* dx, void* const* scratch, const size_t* scratch_bytes,
                                               ttc_stream_t stream) {
  if (n < 0) return TTC_ERR_SHAPE;
  if (n == 0) return TTC_OK;
  if (!descs || !T || !x || !dy || !G || !D || !saved || !saved_bytes || !scratch || !scratch_bytes)
    return TTC_ERR_NULL;
  std::vector<LinearPlan> plans(n);
  std::vector<StreamJob> jobs;
  std::vector<SeqArgs> seqs;
  std::vector<const LinearPlan*> seq_plans;
  for (int i = 0; i < n; ++i) {
    if (!descs[i]) return TTC_ERR_NULL;
    LinearPlan& P = plans[i];
    ttc_status st = bwd_checks(descs[i], T[i], G[i], D[i], &P);
    if (st != TTC_OK) return st;
    if (T[i] == 0) continue;
    void* dxi = dx ? dx[i] : nullptr;
    if ((st = buffer_checks(P, true, x[i], dy[i], dxi, saved[i], saved_bytes[i], scratch[i], scratch_bytes[i])) !=
        TTC_OK)
      return st;
    if (P.path == TTC_PATH_SEQUENTIAL) {
      seqs.push_back(seq_args(P, G[i], D[i], x[i], dy[i], nullptr, dxi, static_cast<const char*>(saved[i]),
                              static_cast<char*>(scratch[i])));
      seq_plans.push_back(&P);
      continue;
    }
    if (!nr_supported(P.NR)) return TTC_ERR_UNSUPPORTED;
    jobs.push_back(StreamJob{&P, x[i], dy[i], const_cast<char*>(static_cast<const char*>(saved[i])), nullptr, dxi,
                             static_cast<char*>(scratch[i])});
  }
  if (jobs.empty() && seqs.empty()) return TTC_OK;  // every layer has T == 0
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  for (size_t i = 0; i < seqs.size(); ++i) launch_seq_bwd(*seq_plans[i], seqs[i], s);
  if (jobs.empty()) return hip_status();  // every layer is sequential or has T == 0
  launch_stream_jobs<false>(jobs.data(), (int)jobs.size(), s);
  return hip_status();
}

namespace ttc {
static ttc_status rank_grads_checks(const tt_linear_desc* desc, const float* const* G, const float* const* D,
                                    float* const* dG, float* const* dD, LinearPlan* P) {
  ttc_status st = make_linear_plan(desc, 0, P);
  if (st != TTC_OK) return st;
  if ((st = check_chain(*P, G, D)) != TTC_OK) return st;
  if ((st = grads_checks(*P, dG)) != TTC_OK) return st;
  if (P->d > 1 && !dD) return TTC_ERR_NULL;
  for (int k = 0; k < P->d - 1; ++k)
    if (!dD[k]) return TTC_ERR_NULL;
  return TTC_OK;
}
}  // namespace ttc

extern "C" ttc_status tt_linear_rank_grads_batch(int32_t n, const tt_linear_desc* const* descs,
                                                 const float* const* const* G, const float* const* const* D,
                                                 float* const* const* dG, float* const* const* dD, float gamma,
                                                 float beta, ttc_stream_t stream) {
  if (n < 0) return TTC_ERR_SHAPE;
  if (!(gamma == gamma) || !(beta == beta)) return TTC_ERR_SHAPE;  // NaN penalty weights
  if (n == 0) return TTC_OK;
  if (!descs || !G || !D || !dG || !dD) return TTC_ERR_NULL;
  std::vector<CoreJob> jobs;
  for (int i = 0; i < n; ++i) {
    if (!descs[i]) return TTC_ERR_NULL;
    LinearPlan P;
    const ttc_status st = rank_grads_checks(descs[i], G[i], D[i], dG[i], dD[i], &P);
    if (st != TTC_OK) return st;
    for (int k = 0; k < P.d; ++k) {
      const bool link = k < P.d - 1;
      if (!link && beta == 0.f) continue;  // nothing to do for the last core
      CoreJob c;
      c.G = G[i][k];
      c.D = link ? D[i][k] : nullptr;
      c.dG = dG[i][k];
      c.dD = link ? dD[i][k] : nullptr;
      c.rows = P.ranks[k] * P.modes[k];
      c.r1 = P.ranks[k + 1];
      jobs.push_back(c);
    }
  }
  if (jobs.empty()) return TTC_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  for (size_t j0 = 0; j0 < jobs.size(); j0 += kMaxCoreJobs) {
    RankGradArgs a;
    memset(&a, 0, sizeof(a));
    a.n = (int)std::min<size_t>(kMaxCoreJobs, jobs.size() - j0);
    for (int q = 0; q < a.n; ++q) a.j[q] = jobs[j0 + q];
    a.gamma = gamma;
    a.beta = beta;
    TraceScope ts("rank_grads", s);
    TTC_LAUNCH(k_rank_grads, dim3((unsigned)a.n), dim3(kRankGradThreads), 0, s, a);
  }
  return hip_status();
}

extern "C" ttc_status tt_linear_rank_grads(const tt_linear_desc* desc, const float* const* G, const float* const* D,
                                           float* const* dG, float* const* dD, float gamma, float beta,
                                           ttc_stream_t stream) {
  return tt_linear_rank_grads_batch(1, &desc, &G, &D, &dG, &dD, gamma, beta, stream);
}

extern "C" ttc_status tt_linear_explain(const tt_linear_desc* desc, int64_t T, char* buf, size_t n) {
  if (!buf || n == 0) return TTC_ERR_NULL;
  LinearPlan P;
  const ttc_status st = make_linear_plan(desc, T, &P);
  if (st != TTC_OK) return st;
  double macs[4], bytes[4], usec[4];
  linear_path_costs(P, macs, bytes);
  linear_path_times(P, macs, bytes, usec);
  snprintf(buf, n,
           "path=%s split=%d rank=%d rpad=%d N_out=%lld N_in=%lld T=%lld "
           "merged_macs=%.6g merged_bytes=%.6g merged_us=%.4g sequential_macs=%.6g sequential_bytes=%.6g "
           "sequential_us=%.4g "
           "dense_macs=%.6g dense_bytes=%.6g dy_grid=%dx%d dy_slabs=%d dy_tiles=%d dx_grid=%dx%d dx_slabs=%d "
           "dx_tiles=%d saved=%zu scratch=%zu",
           P.path == TTC_PATH_SEQUENTIAL ? "sequential" : "merged", P.s, P.rs, P.Rpad, (long long)P.N_out,
           (long long)P.N_in, (long long)T, macs[1], bytes[1], usec[1], macs[2], bytes[2], usec[2], macs[3],
           bytes[3], P.dy_gc, P.dy_gt, P.dy_nsl, P.dy_tpg, P.dx_gc, P.dx_gt, P.dx_nsl, P.dx_tpg,
           P.sv_total, P.sc_total);
  return TTC_OK;
}

extern "C" ttc_status tt_linear_path_cost(const tt_linear_desc* desc, int64_t T, int32_t path, double* macs,
                                          double* bytes) {
  if (!macs || !bytes || !desc) return TTC_ERR_NULL;
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

extern "C" const char* ttc_version(void) { return "ttc 0.2 gfx950"; }
