// TTM embedding lookup and its backward for gfx950.
//
// A TTM table with vocabulary modes m_1..m_d, embedding modes n_1..n_d and
// cores F_k (r_{k-1}, m_k, n_k, r_k) has, for the id with digits
// (v_1..v_d), the row
//     E[v] = F_1[0, v_1] D_1 F_2[:, v_2] D_2 ... F_d[:, v_d]
// (NeurIPS 2024 poster page of CoMERA, figure on the TT and TTM structures;
// project page, "Learn the ranks while training").  The lookup follows the
// project page's section "Making small tensor operations fast on GPUs"
// (embedding lookup without repeated work): only distinct ids are
// evaluated, and neighbouring cores are contracted once per distinct prefix
// of digits and then shared by every id with that prefix.
//
// Data structure (built by one work-group, k_ttm_sort):
//   * the ids sorted by (id, position): `order`, the distinct ids `uids`
//     (ascending), `inverse` and the segment offsets `seg`;
//   * level l (0-based, l = 0..d-1) holds the distinct prefixes
//     (v_1..v_{l+1}) of the ids, ascending; level d-1 is the distinct ids.
//     Node j of level l knows its prefix value, its parent at level l-1 and
//     the range of its children at level l+1 (they are contiguous because
//     everything is sorted);
//   * "pieces": the sorted token positions are cut into chunks of kChunk
//     positions and every chunk into runs of equal id; a distinct id owns a
//     contiguous range of pieces;
//   * per level, the nodes sorted stably by their last digit, so that the
//     core gradient of one slice F_k[:, v] sums a fixed list in a fixed order.
//
// Forward: P_l[j] = (P_{l-1}[parent] D_l) F_{l+1}[:, v, :, :], one work-group
// per node, from level 1 to level d-1 (P_0 is a slice of F_1); the last level
// gives one row per distinct id, and a gather writes the token rows.
// Backward: per piece, the sum of its tokens' output gradients (the only
// pass over the T x N gradient); then, per node from level d-1 down to 1,
// the node's gradient G_j (sum of its pieces, or of its children's
// contributions), its share of dF (C_j) and its contribution to the
// parent's gradient (Q_j); finally every slice dF_k[a, v] sums the C's of
// its list.  No floating-point atomics: results are bitwise reproducible.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "../../include/ttc.h"
#include "ttc_trace.hpp"

namespace ttc {

constexpr int kTtmMaxT = 16384;     // ids per call (LDS-resident sort)
constexpr int kSortThreads = 1024;  // one work-group sorts
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kChunk = 32;          // sorted positions per piece chunk
constexpr int kHdrWords = 32;
constexpr int kTtmThreads = 256;
constexpr size_t kTtmMaxLds = 65536;

// header words of `saved`
constexpr int kHdrU = 0;       // distinct valid ids
constexpr int kHdrErr = 1;     // 1 if an id was out of range
constexpr int kHdrPieces = 2;  // number of pieces
constexpr int kHdrTv = 3;      // valid tokens
constexpr int kHdrUl = 4;      // 4 + l: nodes at level l

struct TtmPlan {
  int d;
  int m[TTC_TTM_MAX_MODES], n[TTC_TTM_MAX_MODES], r[TTC_TTM_MAX_MODES + 1];
  int64_t V, N, T, nch;
  int kbits;                        // bits of the sort key (ids and the out-of-range marker V)
  int dbits[TTC_TTM_MAX_MODES];     // bits of the last digit of level l
  uint32_t Mgt[TTC_TTM_MAX_MODES];  // prod m_{>l}: prefix of level l = id / Mgt[l]
  int64_t cap[TTC_TTM_MAX_MODES];   // max nodes at level l = min(T, prod m_{<=l})
  int64_t R[TTC_TTM_MAX_MODES];     // prod n_{<l}: rows of the parent product of level l
  int64_t psz[TTC_TTM_MAX_MODES];   // floats of P_l[j] = prod n_{<=l} * r_{l+1}
  // saved (bytes)
  size_t sv_order, sv_inverse, sv_uids, sv_seg, sv_piece_u, sv_piece_beg, sv_chunk_piece, sv_u_piece;
  size_t sv_pref[TTC_TTM_MAX_MODES], sv_parent[TTC_TTM_MAX_MODES], sv_child[TTC_TTM_MAX_MODES];
  size_t sv_list[TTC_TTM_MAX_MODES], sv_list_off[TTC_TTM_MAX_MODES], sv_P[TTC_TTM_MAX_MODES];
  size_t sv_total;
  // scratch (bytes)
  size_t sc_urow, sc_PS, sc_Q[TTC_TTM_MAX_MODES], sc_C[TTC_TTM_MAX_MODES], sc_fwd, sc_bwd, sc_total;
  size_t lds_fwd[TTC_TTM_MAX_MODES], lds_bwd[TTC_TTM_MAX_MODES];
};

// ------------------------------------------------------------------------------
// the sort work-group
// ------------------------------------------------------------------------------
struct SortArgs {
  const int64_t* ids;
  int n;
  uint32_t V;
  int kbits;
  int d;
  int m[TTC_TTM_MAX_MODES];
  uint32_t Mgt[TTC_TTM_MAX_MODES];
  int dbits[TTC_TTM_MAX_MODES];
  int nch;
  int32_t* hdr;
  int32_t* order;
  int32_t* inverse;
  int32_t* uids;
  int32_t* seg;
  int32_t* piece_u;
  int32_t* piece_beg;
  int32_t* chunk_piece;
  int32_t* u_piece;
  int32_t* pref[TTC_TTM_MAX_MODES];
  int32_t* parent[TTC_TTM_MAX_MODES];
  int32_t* child[TTC_TTM_MAX_MODES];
  int32_t* list[TTC_TTM_MAX_MODES];
  int32_t* list_off[TTC_TTM_MAX_MODES];
};

// Exclusive prefix sum of one value per thread over the work-group; *total
// receives the sum.  Contains barriers: every thread must call it.
__device__ uint32_t block_exscan(uint32_t v, uint32_t* s_red, uint32_t* total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_red[w] = x;
  __syncthreads();
  if (w == 0) {
    const uint32_t t0 = lane < kSortWaves ? s_red[lane] : 0u;
    uint32_t t = t0;
#pragma unroll
    for (int off = 1; off < kSortWaves; off <<= 1) {
      const uint32_t y = __shfl_up(t, off, 64);
      if (lane >= off) t += y;
    }
    if (lane < kSortWaves) s_red[lane] = t - t0;
    if (lane == kSortWaves - 1) s_red[kSortWaves] = t;
  }
  __syncthreads();
  const uint32_t r = s_red[w] + x - v;
  *total = s_red[kSortWaves];
  __syncthreads();
  return r;
}

// Stable LSD radix sort of keys[0..n) (with 16-bit payloads) in LDS, 8 bits
// per pass.  Wave w owns the contiguous range [w*L, (w+1)*L) and walks it in
// rounds of 64; lanes holding equal digits in one round are found with one
// ballot per digit bit, so each element's rank among equal digits of its
// wave is exact and in position order.  Counts are kept per (digit, wave),
// digit-major, so one exclusive scan over them gives every element's
// destination: the sort is stable.
__device__ void block_radix_sort(uint32_t* keys, uint16_t* vals, uint16_t* cnt, uint32_t* s_red, int n,
                                 int kbits) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int L = ((n + kSortWaves - 1) / kSortWaves + 63) & ~63;
  const int rounds = L >> 6;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int shift = 0; shift < kbits; shift += 8) {
    const int nb = kbits - shift < 8 ? kbits - shift : 8;
    const int nbins = 1 << nb;
    const uint32_t dmask = (uint32_t)nbins - 1u;
    for (int i = tid; i < nbins * kSortWaves; i += kSortThreads) cnt[i] = 0;
    __syncthreads();
    uint32_t k[16];
    uint16_t v[16];
    uint16_t rk[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (r < rounds) {
        const int i = w * L + r * 64 + lane;
        const bool valid = i < n;
        const uint32_t key = valid ? keys[i] : 0u;
        const uint32_t dg = (key >> shift) & dmask;
        uint64_t mask = __ballot(valid);
        for (int b = 0; b < nb; ++b) {
          const bool bit = (dg >> b) & 1u;
          const uint64_t bb = __ballot(valid && bit);
          mask &= bit ? bb : ~bb;
        }
        k[r] = key;
        v[r] = valid ? vals[i] : (uint16_t)0;
        if (valid) {
          const uint32_t pre = cnt[dg * kSortWaves + w];
          const uint32_t mine = (uint32_t)__popcll(mask & below);
          rk[r] = (uint16_t)(pre + mine);
          if (mine == 0) cnt[dg * kSortWaves + w] = (uint16_t)(pre + (uint32_t)__popcll(mask));
        }
      }
    }
    __syncthreads();
    // exclusive scan of the nbins * waves counters, 4 per thread
    const int tot = nbins * kSortWaves;
    uint32_t c4[4];
    uint32_t s = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = tid * 4 + e;
      c4[e] = i < tot ? cnt[i] : 0u;
      s += c4[e];
    }
    uint32_t total;
    uint32_t run = block_exscan(s, s_red, &total);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = tid * 4 + e;
      if (i < tot) cnt[i] = (uint16_t)run;
      run += c4[e];
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (r < rounds) {
        const int i = w * L + r * 64 + lane;
        if (i < n) {
          const uint32_t dg = (k[r] >> shift) & dmask;
          const int dest = (int)cnt[dg * kSortWaves + w] + (int)rk[r];
          keys[dest] = k[r];
          vals[dest] = v[r];
        }
      }
    }
    __syncthreads();
  }
}

// first index i in [0, n) with keys[i] >= x (keys ascending), n if none
__device__ int lower_bound_lds(const uint32_t* keys, int n, uint32_t x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (keys[mid] < x)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

constexpr int kPer = kTtmMaxT / kSortThreads;  // positions owned per thread in the scans

__global__ __launch_bounds__(kSortThreads) void k_ttm_sort(SortArgs a) {
  __shared__ uint32_t s_key[kTtmMaxT];
  __shared__ uint16_t s_val[kTtmMaxT];
  __shared__ uint16_t s_cnt[256 * kSortWaves];
  __shared__ uint32_t s_red[kSortWaves + 1];
  const int tid = threadIdx.x;
  const int n = a.n;

  // e0: keys; an id outside [0, V) becomes V and sorts after every valid id
  uint32_t bad = 0;
  for (int i = tid; i < n; i += kSortThreads) {
    const int64_t id = a.ids[i];
    const bool ok = id >= 0 && id < (int64_t)a.V;
    s_key[i] = ok ? (uint32_t)id : a.V;
    s_val[i] = (uint16_t)i;
    bad += ok ? 0u : 1u;
  }
  uint32_t nbad;
  (void)block_exscan(bad, s_red, &nbad);

  // e1: sort by (id, position)
  block_radix_sort(s_key, s_val, s_cnt, s_red, n, a.kbits);
  const int Tv = n - (int)nbad;

  // segment starts and piece starts over the positions owned by this thread
  const int i0 = tid * kPer;
  uint32_t kk[kPer];
  uint16_t vv[kPer];
  uint32_t nseg = 0, npc = 0;
  const uint32_t kprev0 = (i0 > 0 && i0 - 1 < n) ? s_key[i0 - 1] : 0xffffffffu;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int i = i0 + e;
    kk[e] = i < n ? s_key[i] : 0u;
    vv[e] = i < n ? s_val[i] : (uint16_t)0;
  }
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int i = i0 + e;
    const uint32_t kp = e == 0 ? kprev0 : kk[e - 1];
    const bool fs = i < Tv && (i == 0 || kk[e] != kp);
    const bool ps = i < Tv && (fs || (i % kChunk) == 0);
    nseg += fs;
    npc += ps;
  }
  uint32_t tot2;
  const uint32_t ex2 = block_exscan(nseg | (npc << 16), s_red, &tot2);
  const int U = (int)(tot2 & 0xffffu), P = (int)(tot2 >> 16);
  int u = (int)(ex2 & 0xffffu) - 1, p = (int)(ex2 >> 16) - 1;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int i = i0 + e;
    if (i >= n) break;
    const uint32_t kp = e == 0 ? kprev0 : kk[e - 1];
    const bool fs = i < Tv && (i == 0 || kk[e] != kp);
    const bool ps = i < Tv && (fs || (i % kChunk) == 0);
    u += fs;
    p += ps;
    a.order[i] = vv[e];
    if (vv[e] < n) a.inverse[vv[e]] = i < Tv ? u : -1;
    if (fs) {
      a.uids[u] = (int32_t)kk[e];
      a.seg[u] = i;
      a.u_piece[u] = p;
    }
    if (ps) {
      a.piece_u[p] = u;
      a.piece_beg[p] = i;
    }
    if (i < Tv && (i % kChunk) == 0) a.chunk_piece[i / kChunk] = p;
  }
  const int nchv = (Tv + kChunk - 1) / kChunk;
  for (int c = nchv + tid; c <= a.nch; c += kSortThreads) a.chunk_piece[c] = P;
  if (tid == 0) {
    a.seg[U] = Tv;
    a.u_piece[U] = P;
    a.piece_beg[P] = Tv;
    a.hdr[kHdrU] = U;
    a.hdr[kHdrErr] = nbad ? 1 : 0;
    a.hdr[kHdrPieces] = P;
    a.hdr[kHdrTv] = Tv;
    a.hdr[kHdrUl + a.d - 1] = U;
  }
  __syncthreads();
  // distinct ids into s_key[0..U), level d-1 node index of each into s_val
  {
    int uu = (int)(ex2 & 0xffffu) - 1;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int i = i0 + e;
      const uint32_t kp = e == 0 ? kprev0 : kk[e - 1];
      const bool fs = i < Tv && (i == 0 || kk[e] != kp);
      uu += fs;
      if (fs) {
        s_key[uu] = kk[e];
        s_val[uu] = (uint16_t)uu;
      }
    }
  }
  __syncthreads();

  // e1 (levels): distinct prefixes of every level, from level d-2 down to 0
  int Unext = U;
  for (int l = a.d - 2; l >= 0; --l) {
    const uint32_t M = a.Mgt[l];
    uint32_t cntl = 0;
    uint32_t pre[kPer];
    uint16_t nxt[kPer];
    const uint32_t pprev0 = (i0 > 0 && i0 - 1 < U) ? s_key[i0 - 1] / M : 0xffffffffu;
    const uint16_t nprev0 = (i0 > 0 && i0 - 1 < U) ? s_val[i0 - 1] : (uint16_t)0xffff;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int uu = i0 + e;
      pre[e] = uu < U ? s_key[uu] / M : 0u;
      nxt[e] = uu < U ? s_val[uu] : (uint16_t)0;
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int uu = i0 + e;
      const uint32_t pp = e == 0 ? pprev0 : pre[e - 1];
      cntl += (uu < U && (uu == 0 || pre[e] != pp)) ? 1u : 0u;
    }
    uint32_t Ul;
    int j = (int)block_exscan(cntl, s_red, &Ul) - 1;
    uint16_t mine[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int uu = i0 + e;
      const uint32_t pp = e == 0 ? pprev0 : pre[e - 1];
      const uint16_t np = e == 0 ? nprev0 : nxt[e - 1];
      const bool ns = uu < U && (uu == 0 || pre[e] != pp);
      const bool cs = uu < U && (uu == 0 || nxt[e] != np);  // a node of level l+1 starts here
      j += ns;
      mine[e] = (uint16_t)j;
      if (ns) {
        a.pref[l][j] = (int32_t)pre[e];
        a.child[l][j] = nxt[e];
      }
      if (cs) a.parent[l + 1][nxt[e]] = j;
    }
    if (tid == 0) {
      a.child[l][Ul] = Unext;
      a.hdr[kHdrUl + l] = (int32_t)Ul;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kPer; ++e)
      if (i0 + e < U) s_val[i0 + e] = mine[e];
    __syncthreads();
    Unext = (int)Ul;
  }
  // level 0 hangs off the single root
  for (int j = tid; j < Unext; j += kSortThreads) a.parent[0][j] = 0;
  __syncthreads();

  // lists: the nodes of each level sorted stably by their last digit
  for (int l = 0; l < a.d; ++l) {
    const int Ul = l == a.d - 1 ? U : a.hdr[kHdrUl + l];
    const int32_t* pref = l == a.d - 1 ? a.uids : a.pref[l];
    const uint32_t ml = (uint32_t)a.m[l];
    __syncthreads();
    for (int j = tid; j < Ul; j += kSortThreads) {
      s_key[j] = (uint32_t)pref[j] % ml;
      s_val[j] = (uint16_t)j;
    }
    __syncthreads();
    block_radix_sort(s_key, s_val, s_cnt, s_red, Ul, a.dbits[l]);
    for (int j = tid; j < Ul; j += kSortThreads) a.list[l][j] = s_val[j];
    for (int v = tid; v <= (int)ml; v += kSortThreads) a.list_off[l][v] = lower_bound_lds(s_key, Ul, (uint32_t)v);
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------
// forward: prefix products per node, rows per distinct id, token gather
// ------------------------------------------------------------------------------
struct LevelArgs {
  int l;                 // level (>= 1)
  int d;
  int m, nk, ra, rb;     // m_{l+1}, n_{l+1}, r_l, r_{l+1} (1-based core l+1)
  int64_t R;             // rows of the parent product
  const int32_t* hdr;
  const int32_t* pref;   // level l prefixes (digit = pref % m)
  const int32_t* parent; // level l parents
  const int32_t* ppref;  // level l-1 prefixes (for a parent that is a slice of F_1)
  const float* Fpar;     // F_1 when l == 1
  const float* Ppar;     // P_{l-1} when l >= 2
  const float* Dpar;     // D on the link into this level, NULL = identity
  const float* F;        // core F_{l+1}
  float* out;            // P_l, or the distinct-id rows at the last level
  int64_t osz;           // floats per node of `out`
  // backward only
  const float* src;      // gradient sources of a node: pieces or children's Q
  const int32_t* src_off;
  int64_t ssz;           // floats per source row (= osz)
  float* Cout;           // ra * nk * rb per node
  float* Qout;           // R * ra per node
};

// Stage the parent's product with D applied (R x ra) and the core slice
// F[:, v, :, :] (ra x nk*rb) into LDS.
__device__ __forceinline__ void stage_parent(const LevelArgs& a, int j, float* sPd, float* sW) {
  const int p = a.parent[j];
  const int v = (int)((uint32_t)a.pref[j] % (uint32_t)a.m);
  const float* Pp = a.l == 1 ? a.Fpar + (int64_t)((uint32_t)a.ppref[p]) * a.R * a.ra : a.Ppar + (int64_t)p * a.R * a.ra;
  const int64_t np = a.R * a.ra;
  for (int64_t e = threadIdx.x; e < np; e += blockDim.x) {
    const int aa = (int)(e % a.ra);
    sPd[e] = Pp[e] * (a.Dpar ? a.Dpar[aa] : 1.f);
  }
  const int64_t blk = (int64_t)a.nk * a.rb;
  const int64_t nw = (int64_t)a.ra * blk;
  for (int64_t e = threadIdx.x; e < nw; e += blockDim.x) {
    const int64_t aa = e / blk, cb = e - aa * blk;
    sW[e] = a.F[(aa * a.m + v) * blk + cb];
  }
}

__global__ __launch_bounds__(kTtmThreads) void k_ttm_level_fwd(LevelArgs a) {
  extern __shared__ float lds[];
  const int Ul = a.hdr[kHdrUl + a.l];
  const int64_t np = a.R * a.ra;
  float* sPd = lds;
  float* sW = lds + np;
  const int64_t blk = (int64_t)a.nk * a.rb;
  const int64_t nout = a.R * blk;
  for (int j = blockIdx.x; j < Ul; j += gridDim.x) {
    __syncthreads();
    stage_parent(a, j, sPd, sW);
    __syncthreads();
    float* o = a.out + (int64_t)j * a.osz;
    for (int64_t e = threadIdx.x; e < nout; e += blockDim.x) {
      const int64_t c = e / blk, cb = e - c * blk;
      const float* pr = sPd + c * a.ra;
      const float* wc = sW + cb;
      float acc = 0.f;
      for (int aa = 0; aa < a.ra; ++aa) acc = fmaf(pr[aa], wc[aa * blk], acc);
      o[e] = acc;
    }
  }
}

// out[t] = row of inverse[t] (through `map` when given: the row index of a
// distinct id); zero for an id that was out of range
template <bool VEC>
__global__ __launch_bounds__(kTtmThreads) void k_ttm_gather(const int32_t* __restrict__ inverse,
                                                            const int32_t* __restrict__ map,
                                                            const float* __restrict__ rows, float* __restrict__ out,
                                                            int64_t T, int64_t N) {
  const int64_t nv = VEC ? N / 4 : N;
  const int64_t total = T * nv;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total; g += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = g / nv, c = g - t * nv;
    int u = inverse[t];
    if (map && u >= 0) u = map[u];
    if constexpr (VEC) {
      float4 val = make_float4(0.f, 0.f, 0.f, 0.f);
      if (u >= 0) val = reinterpret_cast<const float4*>(rows + (int64_t)u * N)[c];
      reinterpret_cast<float4*>(out + t * N)[c] = val;
    } else {
      out[t * N + c] = u >= 0 ? rows[(int64_t)u * N + c] : 0.f;
    }
  }
}

// ------------------------------------------------------------------------------
// backward
// ------------------------------------------------------------------------------
// e5: per chunk of sorted positions, the sum of the output gradients of each
// piece's tokens, in position order.
template <bool VEC>
__global__ __launch_bounds__(kTtmThreads) void k_ttm_seg(const int32_t* __restrict__ order,
                                                         const int32_t* __restrict__ piece_beg,
                                                         const int32_t* __restrict__ chunk_piece,
                                                         const float* __restrict__ dout, float* __restrict__ PS,
                                                         int64_t N) {
  const int c = blockIdx.x;
  const int p0 = chunk_piece[c], p1 = chunk_piece[c + 1];
  const int64_t nv = VEC ? N / 4 : N;
  for (int p = p0; p < p1; ++p) {
    const int b = piece_beg[p], e = piece_beg[p + 1];
    for (int64_t col = threadIdx.x; col < nv; col += blockDim.x) {
      if constexpr (VEC) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        int i = b;
        for (; i + 4 <= e; i += 4) {
          float4 x[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) x[q] = reinterpret_cast<const float4*>(dout + (int64_t)order[i + q] * N)[col];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc.x += x[q].x;
            acc.y += x[q].y;
            acc.z += x[q].z;
            acc.w += x[q].w;
          }
        }
        for (; i < e; ++i) {
          const float4 x = reinterpret_cast<const float4*>(dout + (int64_t)order[i] * N)[col];
          acc.x += x.x;
          acc.y += x.y;
          acc.z += x.z;
          acc.w += x.w;
        }
        reinterpret_cast<float4*>(PS + (int64_t)p * N)[col] = acc;
      } else {
        float acc = 0.f;
        for (int i = b; i < e; ++i) acc += dout[(int64_t)order[i] * N + col];
        PS[(int64_t)p * N + col] = acc;
      }
    }
  }
}

// e6, one level: per node j, G_j = sum of its sources, then
//   C_j[a, c_k, b] = sum_c Pd[c, a] G_j[(c, c_k), b]          (its share of dF)
//   Q_j[c, a]      = D[a] sum_{c_k, b} G_j[(c, c_k), b] F[a, v, c_k, b]
// (the gradient of the parent's product).
__global__ __launch_bounds__(kTtmThreads) void k_ttm_level_bwd(LevelArgs a) {
  extern __shared__ float lds[];
  const int Ul = a.hdr[kHdrUl + a.l];
  const int64_t np = a.R * a.ra;
  const int64_t blk = (int64_t)a.nk * a.rb;
  const int64_t nw = (int64_t)a.ra * blk;
  const int64_t ng = a.R * blk;
  float* sPd = lds;
  float* sW = sPd + np;
  float* sG = sW + nw;
  for (int j = blockIdx.x; j < Ul; j += gridDim.x) {
    __syncthreads();
    stage_parent(a, j, sPd, sW);
    const int s0 = a.src_off[j], s1 = a.src_off[j + 1];
    for (int64_t e = threadIdx.x; e < ng; e += blockDim.x) {
      float acc = 0.f;
      for (int s = s0; s < s1; ++s) acc += a.src[(int64_t)s * a.ssz + e];
      sG[e] = acc;
    }
    __syncthreads();
    float* C = a.Cout + (int64_t)j * nw;
    for (int64_t e = threadIdx.x; e < nw; e += blockDim.x) {
      const int64_t aa = e / blk, cb = e - aa * blk;
      float acc = 0.f;
      for (int64_t c = 0; c < a.R; ++c) acc = fmaf(sPd[c * a.ra + aa], sG[c * blk + cb], acc);
      C[e] = acc;
    }
    float* Q = a.Qout + (int64_t)j * np;
    for (int64_t e = threadIdx.x; e < np; e += blockDim.x) {
      const int64_t c = e / a.ra, aa = e - c * a.ra;
      const float* g = sG + c * blk;
      const float* wv = sW + aa * blk;
      float acc = 0.f;
      for (int64_t q = 0; q < blk; ++q) acc = fmaf(g[q], wv[q], acc);
      Q[e] = acc * (a.Dpar ? a.Dpar[aa] : 1.f);
    }
  }
}

// Final step: every slice dF_{l+1}[a, v, :, :] is the sum, over the level-l
// nodes whose last digit is v (in node order), of their C; at level 0 a
// node's C is its gradient G itself, the sum of its sources.
struct ReduceArgs {
  int d;
  int m[TTC_TTM_MAX_MODES], nk[TTC_TTM_MAX_MODES], ra[TTC_TTM_MAX_MODES], rb[TTC_TTM_MAX_MODES];
  int item_off[TTC_TTM_MAX_MODES + 1];  // first work item (v) of each level
  const int32_t* hdr;
  const int32_t* list[TTC_TTM_MAX_MODES];
  const int32_t* list_off[TTC_TTM_MAX_MODES];
  const float* C[TTC_TTM_MAX_MODES];    // levels >= 1
  const float* src0;                    // level 0: sources (pieces or level-1 Q)
  const int32_t* src0_off;
  float* dF[TTC_TTM_MAX_MODES];
  int accumulate;
};

__global__ __launch_bounds__(kTtmThreads) void k_ttm_reduce(ReduceArgs a) {
  const int it = blockIdx.x;
  int l = 0;
  while (l + 1 < a.d && it >= a.item_off[l + 1]) ++l;
  const int v = it - a.item_off[l];
  const int m = a.m[l];
  const int64_t blk = (int64_t)a.nk[l] * a.rb[l];
  const int64_t nw = (int64_t)a.ra[l] * blk;
  const int b0 = a.list_off[l][v], b1 = a.list_off[l][v + 1];
  const int32_t* lst = a.list[l];
  float* dF = a.dF[l];
  for (int64_t e = threadIdx.x; e < nw; e += blockDim.x) {
    const int64_t aa = e / blk, cb = e - aa * blk;
    float acc = 0.f;
    if (l == 0) {
      // ra == 1: e indexes the node's gradient directly
      for (int q = b0; q < b1; ++q) {
        const int j = lst[q];
        const int s0 = a.src0_off[j], s1 = a.src0_off[j + 1];
        for (int s = s0; s < s1; ++s) acc += a.src0[(int64_t)s * nw + e];
      }
    } else {
      const float* C = a.C[l];
      for (int q = b0; q < b1; ++q) acc += C[(int64_t)lst[q] * nw + e];
    }
    float* o = dF + (aa * m + v) * blk + cb;
    *o = a.accumulate ? *o + acc : acc;
  }
}

__global__ void k_ttm_zero(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

// ------------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------------
static bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
static size_t up256(size_t x) { return (x + 255) & ~size_t(255); }
static int bit_length(uint64_t x) {
  int b = 0;
  while (x) {
    ++b;
    x >>= 1;
  }
  return b;
}

static ttc_status make_ttm_plan(const ttm_embed_desc* desc, int64_t T, TtmPlan* P) {
  if (!desc || !P) return TTC_ERR_NULL;
  memset(P, 0, sizeof(*P));
  const int d = desc->d;
  if (d < 1 || d > TTC_TTM_MAX_MODES) return TTC_ERR_SHAPE;
  if (T < 0) return TTC_ERR_SHAPE;
  if (T > kTtmMaxT) return TTC_ERR_UNSUPPORTED;
  P->d = d;
  P->T = T;
  int64_t V = 1, N = 1;
  for (int k = 0; k < d; ++k) {
    if (desc->vocab_modes[k] < 1 || desc->dim_modes[k] < 1) return TTC_ERR_SHAPE;
    P->m[k] = desc->vocab_modes[k];
    P->n[k] = desc->dim_modes[k];
    V *= P->m[k];
    N *= P->n[k];
    if (V >= (int64_t(1) << 31) || N > (int64_t(1) << 24)) return TTC_ERR_SHAPE;
  }
  for (int k = 0; k <= d; ++k) {
    const int r = desc->ranks[k];
    if (r < 1 || r > TTC_MAX_RANK) return TTC_ERR_RANK;
    P->r[k] = r;
  }
  if (P->r[0] != 1 || P->r[d] != 1) return TTC_ERR_RANK;
  P->V = V;
  P->N = N;
  P->kbits = bit_length((uint64_t)V);
  P->nch = (T + kChunk - 1) / kChunk;
  {
    uint64_t g = 1;
    for (int l = d - 1; l >= 0; --l) {
      P->Mgt[l] = (uint32_t)g;
      g *= (uint64_t)P->m[l];
    }
  }
  int64_t mprod = 1, nprod = 1;
  for (int l = 0; l < d; ++l) {
    P->dbits[l] = bit_length((uint64_t)(P->m[l] - 1));
    P->R[l] = nprod;
    mprod *= P->m[l];
    nprod *= P->n[l];
    P->cap[l] = mprod < T ? mprod : T;
    P->psz[l] = nprod * P->r[l + 1];
    const size_t blk = (size_t)P->n[l] * P->r[l + 1];
    P->lds_fwd[l] = 4 * ((size_t)P->R[l] * P->r[l] + (size_t)P->r[l] * blk);
    P->lds_bwd[l] = P->lds_fwd[l] + 4 * ((size_t)P->R[l] * blk);
    if (l >= 1 && (P->lds_fwd[l] > kTtmMaxLds || P->lds_bwd[l] > kTtmMaxLds)) return TTC_ERR_UNSUPPORTED;
  }
  // saved
  size_t o = 4 * kHdrWords;
  auto take = [&](int64_t words) {
    const size_t at = o;
    o += up256(4 * (size_t)(words > 0 ? words : 0));
    return at;
  };
  P->sv_order = take(T);
  P->sv_inverse = take(T);
  P->sv_uids = take(T);
  P->sv_seg = take(T + 1);
  P->sv_piece_u = take(T);
  P->sv_piece_beg = take(T + 1);
  P->sv_chunk_piece = take(P->nch + 1);
  P->sv_u_piece = take(T + 1);
  for (int l = 0; l < d; ++l) {
    const int64_t c = P->cap[l];
    P->sv_pref[l] = l == d - 1 ? P->sv_uids : take(c);
    P->sv_parent[l] = take(c);
    P->sv_child[l] = l == d - 1 ? P->sv_u_piece : take(c + 1);
    P->sv_list[l] = take(c);
    P->sv_list_off[l] = take((int64_t)P->m[l] + 1);
  }
  for (int l = 1; l + 1 < d; ++l) P->sv_P[l] = take(P->cap[l] * P->psz[l]);
  P->sv_total = o;
  // scratch: the forward needs the distinct-id rows, the backward the piece
  // sums and per-level Q and C
  P->sc_urow = 0;
  P->sc_fwd = d >= 2 ? up256(4 * (size_t)(P->cap[d - 1] * N)) : 0;
  size_t s = 0;
  P->sc_PS = s;
  s += up256(4 * (size_t)(T * N));
  for (int l = 1; l < d; ++l) {
    P->sc_Q[l] = s;
    s += up256(4 * (size_t)(P->cap[l] * P->R[l] * P->r[l]));
    P->sc_C[l] = s;
    s += up256(4 * (size_t)(P->cap[l] * P->r[l] * P->n[l] * P->r[l + 1]));
  }
  P->sc_bwd = s;
  P->sc_total = P->sc_fwd > P->sc_bwd ? P->sc_fwd : P->sc_bwd;
  if (P->sc_total == 0) P->sc_total = 256;
  return TTC_OK;
}

static ttc_status hip_ok() { return hipGetLastError() == hipSuccess ? TTC_OK : TTC_ERR_HIP; }

static unsigned grid_nodes(int64_t cap) { return (unsigned)(cap < 1 ? 1 : (cap > 4096 ? 4096 : cap)); }

template <typename Ptr>
static Ptr at(void* base, size_t off) {
  return reinterpret_cast<Ptr>(static_cast<char*>(base) + off);
}
template <typename Ptr>
static Ptr atc(const void* base, size_t off) {
  return reinterpret_cast<Ptr>(static_cast<const char*>(base) + off);
}

static void fill_level(const TtmPlan& P, int l, const void* saved, const float* const* F, const float* const* D,
                       LevelArgs* a) {
  memset(a, 0, sizeof(*a));
  a->l = l;
  a->d = P.d;
  a->m = P.m[l];
  a->nk = P.n[l];
  a->ra = P.r[l];
  a->rb = P.r[l + 1];
  a->R = P.R[l];
  a->hdr = atc<const int32_t*>(saved, 0);
  a->pref = atc<const int32_t*>(saved, P.sv_pref[l]);
  a->parent = atc<const int32_t*>(saved, P.sv_parent[l]);
  a->ppref = atc<const int32_t*>(saved, P.sv_pref[l - 1]);
  a->Fpar = F[0];
  a->Ppar = l >= 2 ? atc<const float*>(saved, P.sv_P[l - 1]) : nullptr;
  a->Dpar = D ? D[l - 1] : nullptr;
  a->F = F[l];
}

static ttc_status check_cores(const TtmPlan& P, const float* const* F, const float* const* D) {
  if (!F) return TTC_ERR_NULL;
  for (int k = 0; k < P.d; ++k)
    if (!F[k]) return TTC_ERR_NULL;
  if (D)
    for (int k = 0; k < P.d - 1; ++k)
      if (!D[k]) return TTC_ERR_NULL;
  return TTC_OK;
}

}  // namespace ttc

using namespace ttc;

extern "C" ttc_status ttm_embed_workspace(const ttm_embed_desc* desc, int64_t T, size_t* saved_bytes,
                                          size_t* scratch_bytes) {
  if (!saved_bytes || !scratch_bytes) return TTC_ERR_NULL;
  TtmPlan P;
  const ttc_status st = make_ttm_plan(desc, T, &P);
  if (st != TTC_OK) return st;
  *saved_bytes = P.sv_total;
  *scratch_bytes = P.sc_total;
  return TTC_OK;
}

extern "C" ttc_status ttm_embed_fwd(const ttm_embed_desc* desc, int64_t T, const int64_t* ids,
                                    const float* const* F, const float* const* D, float* out, void* saved,
                                    size_t saved_bytes, void* scratch, size_t scratch_bytes, ttc_stream_t stream) {
  TtmPlan P;
  ttc_status st = make_ttm_plan(desc, T, &P);
  if (st != TTC_OK) return st;
  if ((st = check_cores(P, F, D)) != TTC_OK) return st;
  if (T == 0) return TTC_OK;
  if (!ids || !out || !saved || (P.d >= 2 && !scratch)) return TTC_ERR_NULL;
  if (!al16(out) || !al16(saved) || (scratch && !al16(scratch))) return TTC_ERR_ALIGN;
  if (saved_bytes < P.sv_total || (P.d >= 2 && scratch_bytes < P.sc_fwd)) return TTC_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();

  SortArgs sa;
  memset(&sa, 0, sizeof(sa));
  sa.ids = ids;
  sa.n = (int)T;
  sa.V = (uint32_t)P.V;
  sa.kbits = P.kbits;
  sa.d = P.d;
  sa.nch = (int)P.nch;
  for (int l = 0; l < P.d; ++l) {
    sa.m[l] = P.m[l];
    sa.Mgt[l] = P.Mgt[l];
    sa.dbits[l] = P.dbits[l];
    sa.pref[l] = at<int32_t*>(saved, P.sv_pref[l]);
    sa.parent[l] = at<int32_t*>(saved, P.sv_parent[l]);
    sa.child[l] = at<int32_t*>(saved, P.sv_child[l]);
    sa.list[l] = at<int32_t*>(saved, P.sv_list[l]);
    sa.list_off[l] = at<int32_t*>(saved, P.sv_list_off[l]);
  }
  sa.hdr = at<int32_t*>(saved, 0);
  sa.order = at<int32_t*>(saved, P.sv_order);
  sa.inverse = at<int32_t*>(saved, P.sv_inverse);
  sa.uids = at<int32_t*>(saved, P.sv_uids);
  sa.seg = at<int32_t*>(saved, P.sv_seg);
  sa.piece_u = at<int32_t*>(saved, P.sv_piece_u);
  sa.piece_beg = at<int32_t*>(saved, P.sv_piece_beg);
  sa.chunk_piece = at<int32_t*>(saved, P.sv_chunk_piece);
  sa.u_piece = at<int32_t*>(saved, P.sv_u_piece);
  {
    TraceScope ts("ttm_sort", s);
    hipLaunchKernelGGL(k_ttm_sort, dim3(1), dim3(kSortThreads), 0, s, sa);
  }
  // prefix products, level 1 .. d-1 (level 0 is a slice of F_1)
  for (int l = 1; l < P.d; ++l) {
    LevelArgs a;
    fill_level(P, l, saved, F, D, &a);
    a.out = l == P.d - 1 ? at<float*>(scratch, P.sc_urow) : at<float*>(saved, P.sv_P[l]);
    a.osz = P.psz[l];
    TraceScope ts("ttm_level", s);
    hipLaunchKernelGGL(k_ttm_level_fwd, dim3(grid_nodes(P.cap[l])), dim3(kTtmThreads), P.lds_fwd[l], s, a);
  }
  // with one core the rows are those of F_1 itself, indexed by the id
  const float* rows = P.d >= 2 ? at<const float*>(scratch, P.sc_urow) : F[0];
  const int32_t* map = P.d >= 2 ? nullptr : at<const int32_t*>(saved, P.sv_uids);
  const int32_t* inv = at<const int32_t*>(saved, P.sv_inverse);
  {
    const bool vec = (P.N % 4) == 0 && al16(rows);
    const int64_t blocks = (T * (vec ? P.N / 4 : P.N) + kTtmThreads - 1) / kTtmThreads;
    const unsigned grid = (unsigned)(blocks < 8192 ? blocks : 8192);
    TraceScope ts("ttm_gather", s);
    if (vec)
      hipLaunchKernelGGL(k_ttm_gather<true>, dim3(grid), dim3(kTtmThreads), 0, s, inv, map, rows, out, T, P.N);
    else
      hipLaunchKernelGGL(k_ttm_gather<false>, dim3(grid), dim3(kTtmThreads), 0, s, inv, map, rows, out, T, P.N);
  }
  return hip_ok();
}

extern "C" ttc_status ttm_embed_bwd(const ttm_embed_desc* desc, int64_t T, const int64_t* ids, const float* dout,
                                    const float* const* F, const float* const* D, const void* saved,
                                    size_t saved_bytes, float* const* dF, void* scratch, size_t scratch_bytes,
                                    ttc_stream_t stream) {
  TtmPlan P;
  ttc_status st = make_ttm_plan(desc, T, &P);
  if (st != TTC_OK) return st;
  if ((st = check_cores(P, F, D)) != TTC_OK) return st;
  if (!dF) return TTC_ERR_NULL;
  for (int k = 0; k < P.d; ++k)
    if (!dF[k]) return TTC_ERR_NULL;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  if (T == 0) {
    if (!desc->accumulate) {
      for (int k = 0; k < P.d; ++k) {
        const int64_t n = (int64_t)P.r[k] * P.m[k] * P.n[k] * P.r[k + 1];
        TraceScope ts("zero", s);
        hipLaunchKernelGGL(k_ttm_zero, dim3((unsigned)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024)), dim3(256),
                           0, s, dF[k], n);
      }
    }
    return hip_ok();
  }
  (void)ids;
  if (!dout || !saved || !scratch) return TTC_ERR_NULL;
  if (!al16(dout) || !al16(saved) || !al16(scratch)) return TTC_ERR_ALIGN;
  if (saved_bytes < P.sv_total || scratch_bytes < P.sc_bwd) return TTC_ERR_WORKSPACE;

  float* PS = at<float*>(scratch, P.sc_PS);
  {
    const bool vec = (P.N % 4) == 0;
    TraceScope ts("ttm_seg", s);
    if (vec)
      hipLaunchKernelGGL(k_ttm_seg<true>, dim3((unsigned)P.nch), dim3(kTtmThreads), 0, s,
                         atc<const int32_t*>(saved, P.sv_order), atc<const int32_t*>(saved, P.sv_piece_beg),
                         atc<const int32_t*>(saved, P.sv_chunk_piece), dout, PS, P.N);
    else
      hipLaunchKernelGGL(k_ttm_seg<false>, dim3((unsigned)P.nch), dim3(kTtmThreads), 0, s,
                         atc<const int32_t*>(saved, P.sv_order), atc<const int32_t*>(saved, P.sv_piece_beg),
                         atc<const int32_t*>(saved, P.sv_chunk_piece), dout, PS, P.N);
  }
  for (int l = P.d - 1; l >= 1; --l) {
    LevelArgs a;
    fill_level(P, l, saved, F, D, &a);
    a.src = l == P.d - 1 ? PS : at<const float*>(scratch, P.sc_Q[l + 1]);
    a.src_off = atc<const int32_t*>(saved, P.sv_child[l]);
    a.ssz = P.psz[l];
    a.Cout = at<float*>(scratch, P.sc_C[l]);
    a.Qout = at<float*>(scratch, P.sc_Q[l]);
    TraceScope ts("ttm_bwd_level", s);
    hipLaunchKernelGGL(k_ttm_level_bwd, dim3(grid_nodes(P.cap[l])), dim3(kTtmThreads), P.lds_bwd[l], s, a);
  }
  ReduceArgs ra;
  memset(&ra, 0, sizeof(ra));
  ra.d = P.d;
  int items = 0;
  for (int l = 0; l < P.d; ++l) {
    ra.m[l] = P.m[l];
    ra.nk[l] = P.n[l];
    ra.ra[l] = P.r[l];
    ra.rb[l] = P.r[l + 1];
    ra.item_off[l] = items;
    items += P.m[l];
    ra.list[l] = atc<const int32_t*>(saved, P.sv_list[l]);
    ra.list_off[l] = atc<const int32_t*>(saved, P.sv_list_off[l]);
    ra.C[l] = l >= 1 ? at<const float*>(scratch, P.sc_C[l]) : nullptr;
    ra.dF[l] = dF[l];
  }
  ra.item_off[P.d] = items;
  ra.hdr = atc<const int32_t*>(saved, 0);
  ra.src0 = P.d == 1 ? PS : at<const float*>(scratch, P.sc_Q[1]);
  ra.src0_off = atc<const int32_t*>(saved, P.sv_child[0]);
  ra.accumulate = desc->accumulate ? 1 : 0;
  {
    TraceScope ts("ttm_reduce", s);
    hipLaunchKernelGGL(k_ttm_reduce, dim3((unsigned)items), dim3(kTtmThreads), 0, s, ra);
  }
  return hip_ok();
}
