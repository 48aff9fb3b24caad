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
#include "ttc_device.hpp"
#include "ttc_trace.hpp"

namespace ttc {

constexpr int kTtmMaxT = 16384;     // ids per call (LDS-resident sort)
constexpr int kSortThreads = 1024;  // one work-group sorts
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kChunk = 32;          // sorted positions per piece chunk
constexpr int kHdrWords = 32;
constexpr int kTtmThreads = 256;
constexpr int kLevelThreads = 128;  // per-node work-groups: many resident per CU
// backward per-node work-groups (measured: 256 threads beat 128 and 512)
#ifndef TTC_TTM_BWD_THREADS
#define TTC_TTM_BWD_THREADS 256
#endif
constexpr int kLevelBwdThreads = TTC_TTM_BWD_THREADS;
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
  int mode;                         // TTC_TTM_DEDUP / _UNIQUE / _PLAIN
  int dbits[TTC_TTM_MAX_MODES];     // bits of the last digit of level l
  uint32_t Mgt[TTC_TTM_MAX_MODES];  // prod m_{>l}: prefix of level l = id / Mgt[l]
  int64_t cap[TTC_TTM_MAX_MODES];   // max nodes at level l = min(T, prod m_{<=l})
  int64_t R[TTC_TTM_MAX_MODES];     // prod n_{<l}: rows of the parent product of level l
  int64_t psz[TTC_TTM_MAX_MODES];   // floats of P_l[j] = prod n_{<=l} * r_{l+1}
  // saved (bytes)
  size_t sv_order, sv_inverse, sv_uids, sv_seg, sv_piece_beg, sv_chunk_piece, sv_u_piece;
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
// x / M for x < 2^31 by one 64-bit multiply: (x * magic) >> shift, with
// shift = 32 + ceil(log2 M) and magic = ceil(2^shift / M); the error term is
// below 1/(2M), so the floor is exact.
struct FastDiv {
  uint64_t magic;
  int shift;
};
__device__ __forceinline__ uint32_t fdiv(uint32_t x, FastDiv f) {
  return (uint32_t)(((uint64_t)x * f.magic) >> f.shift);
}

struct SortArgs {
  const int64_t* ids;
  int n;
  int mode;  // TTC_TTM_DEDUP / _UNIQUE / _PLAIN
  uint32_t V;
  int kbits;
  int d;
  int m[TTC_TTM_MAX_MODES];
  FastDiv div_pre[TTC_TTM_MAX_MODES];  // x / prod m_{>l}
  FastDiv div_m[TTC_TTM_MAX_MODES];    // x / m_l
  int dbits[TTC_TTM_MAX_MODES];
  int nch;
  int32_t* hdr;
  int32_t* order;
  int32_t* inverse;
  int32_t* uids;
  int32_t* seg;
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
  lds_barrier();
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
  lds_barrier();
  const uint32_t r = s_red[w] + x - v;
  *total = s_red[kSortWaves];
  lds_barrier();
  return r;
}

// LDS layout of the sort arrays: one pad word after every 16 keys and two
// pad halves after every 16 payloads, so that a thread reading its 16
// consecutive elements and 64 lanes reading 64 consecutive ones both hit
// distinct banks.
__device__ __forceinline__ int KI(int i) { return i + (i >> 4); }
__device__ __forceinline__ int VI(int i) { return i + 2 * (i >> 4); }
constexpr int kKeyWords = kTtmMaxT + kTtmMaxT / 16;
constexpr int kValHalves = kTtmMaxT + kTtmMaxT / 8;

// Stable LSD radix sort of keys[0..n) (with 16-bit payloads) in LDS, 4 bits
// per pass.  Thread t owns the contiguous elements [16 t, 16 t + 16) and
// counts their digits in two packed 64-bit
// registers (8 bits per digit), which also gives each element its rank among
// the thread's equal digits.  The (digit, thread) counts go to LDS
// digit-major; one exclusive scan over them gives every element's
// destination, so the sort is stable.
constexpr int kRadixE = kTtmMaxT / kSortThreads;

__device__ void block_radix_sort(uint32_t* keys, uint16_t* vals, uint16_t* cnt, uint32_t* s_red, int n,
                                 int kbits) {
  const int tid = threadIdx.x;
  const int i0 = tid * kRadixE;
  // padded addresses of the thread's elements and of its counters (linear in
  // the unrolled index, so they become instruction offsets)
  const int kt = KI(i0), vt = VI(i0), ct = VI(tid), cs = VI(tid * 16);
  for (int shift = 0; shift < kbits; shift += 4) {
    // payloads two per register, ranks four per register
    uint32_t k[kRadixE], vp[kRadixE / 2], rp[kRadixE / 4];
    uint64_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < kRadixE / 2; ++e) vp[e] = 0;
#pragma unroll
    for (int e = 0; e < kRadixE / 4; ++e) rp[e] = 0;
#pragma unroll
    for (int e = 0; e < kRadixE; ++e) {
      k[e] = 0;
      if (i0 + e < n) {
        k[e] = keys[kt + e];
        vp[e >> 1] |= (uint32_t)vals[vt + e] << (16 * (e & 1));
        const uint32_t dg = (k[e] >> shift) & 15u;
        const int sh = (int)(dg & 7u) * 8;
        rp[e >> 2] |= (uint32_t)(((dg < 8 ? lo : hi) >> sh) & 0xffu) << (8 * (e & 3));
        if (dg < 8)
          lo += 1ull << sh;
        else
          hi += 1ull << sh;
      }
    }
#pragma unroll
    for (int dg = 0; dg < 16; ++dg)
      cnt[ct + dg * (kSortThreads + kSortThreads / 8)] = (uint16_t)(((dg < 8 ? lo : hi) >> ((dg & 7) * 8)) & 0xffu);
    lds_barrier();
    uint32_t sum = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) sum += cnt[cs + q];
    uint32_t total;
    uint32_t run = block_exscan(sum, s_red, &total);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const uint32_t c = cnt[cs + q];
      cnt[cs + q] = (uint16_t)run;
      run += c;
    }
    lds_barrier();
#pragma unroll
    for (int e = 0; e < kRadixE; ++e) {
      if (i0 + e < n) {
        const uint32_t dg = (k[e] >> shift) & 15u;
        const int dest = (int)cnt[ct + dg * (kSortThreads + kSortThreads / 8)] + (int)((rp[e >> 2] >> (8 * (e & 3))) & 0xffu);
        keys[KI(dest)] = k[e];
        vals[VI(dest)] = (uint16_t)(vp[e >> 1] >> (16 * (e & 1)));
      }
    }
    lds_barrier();
  }
}

// One stable counting-sort pass over the digit (key >> shift) mod 2^nb,
// nb <= 8.  Wave w owns the contiguous range [w*L, (w+1)*L) and walks it in
// rounds of 64 lanes; lanes holding equal digits in a round are found with
// one ballot per digit bit, which ranks each element among equal digits of
// its wave in position order.  Counts per (digit, wave), digit-major, are
// scanned once for the destinations.
__device__ void block_multisplit(uint32_t* keys, uint16_t* vals, uint16_t* cnt, uint32_t* s_red, int n, int nb,
                                 int shift = 0) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int L = ((n + kSortWaves - 1) / kSortWaves + 63) & ~63;
  const int rounds = L >> 6;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int nbins = 1 << nb;
  for (int i = tid; i < nbins * kSortWaves; i += kSortThreads) cnt[i] = 0;
  lds_barrier();
  const int kw = KI(w * L + lane), vw = VI(w * L + lane);
  uint32_t k[16], vp[8], rp[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    vp[r] = 0;
    rp[r] = 0;
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    k[r] = 0;
    if (r < rounds) {
      const int i = w * L + r * 64 + lane;
      const bool valid = i < n;
      const uint32_t key = valid ? keys[kw + 68 * r] : 0u;
      const uint32_t dg = (key >> shift) & ((1u << nb) - 1u);
      uint64_t mask = __ballot(valid);
      for (int b = 0; b < nb; ++b) {
        const bool bit = (dg >> b) & 1u;
        const uint64_t bb = __ballot(valid && bit);
        mask &= bit ? bb : ~bb;
      }
      k[r] = key;
      if (valid) {
        vp[r >> 1] |= (uint32_t)vals[vw + 72 * r] << (16 * (r & 1));
        const uint32_t pre = cnt[dg * kSortWaves + w];
        const uint32_t mine = (uint32_t)__popcll(mask & below);
        rp[r >> 1] |= (pre + mine) << (16 * (r & 1));
        if (mine == 0) cnt[dg * kSortWaves + w] = (uint16_t)(pre + (uint32_t)__popcll(mask));
      }
    }
  }
  lds_barrier();
  const int tot = nbins * kSortWaves;
  uint32_t c4[4];
  uint32_t sum = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = tid * 4 + e;
    c4[e] = i < tot ? cnt[i] : 0u;
    sum += c4[e];
  }
  uint32_t total;
  uint32_t run = block_exscan(sum, s_red, &total);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = tid * 4 + e;
    if (i < tot) cnt[i] = (uint16_t)run;
    run += c4[e];
  }
  lds_barrier();
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (r < rounds && w * L + r * 64 + lane < n) {
      const uint32_t dg = (k[r] >> shift) & ((1u << nb) - 1u);
      const int dest = (int)cnt[dg * kSortWaves + w] + (int)((rp[r >> 1] >> (16 * (r & 1))) & 0xffffu);
      keys[KI(dest)] = k[r];
      vals[VI(dest)] = (uint16_t)(vp[r >> 1] >> (16 * (r & 1)));
    }
  }
  lds_barrier();
}

// Stable LSD radix sort of keys[0..n) < 2^kbits (16-bit payloads) in LDS:
// passes of block_multisplit over 8-bit digits, lowest digit first (one
// pass for the last digits of a level, which have at most 8 bits for
// vocabulary modes up to 256).
__device__ void block_radix_sort8(uint32_t* keys, uint16_t* vals, uint16_t* cnt, uint32_t* s_red, int n, int kbits) {
  for (int shift = 0; shift < kbits; shift += 8)
    block_multisplit(keys, vals, cnt, s_red, n, kbits - shift < 8 ? kbits - shift : 8, shift);
}

// first index i in [0, n) with keys[i] >= x (keys ascending), n if none
__device__ int lower_bound_lds(const uint32_t* keys, int n, uint32_t x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (keys[KI(mid)] < x)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

// Wave w owns positions [w * kPer * 64, (w + 1) * kPer * 64), visited in
// rows of 64 consecutive positions; a position's rank among the flagged ones
// is the popcount of the flag ballot below its lane plus the counts of the
// rows and waves before it.
constexpr int kPer = kTtmMaxT / kSortThreads;

__global__ __launch_bounds__(kSortThreads) void k_ttm_sort(SortArgs a) {
  __shared__ uint32_t s_key[kKeyWords];
  __shared__ uint16_t s_val[kValHalves];
  __shared__ uint16_t s_cnt[16 * kSortThreads + 16 * kSortThreads / 8];
  __shared__ uint32_t s_red[kSortWaves + 1];
  __shared__ uint32_t s_w[2 * kSortWaves];
  __shared__ int32_t s_ul[TTC_TTM_MAX_MODES];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const uint64_t upto = below | (1ull << lane);
  const int n = a.n;
  const int base = w * kPer * 64;
  // padded addresses of row 0 of this lane and of the element before it;
  // row e adds 68 (keys) or 72 (payloads)
  const int kb = KI(base + lane), kbm = kb - 1 - ((lane & 15) == 0 ? 1 : 0);
  const int vb = VI(base + lane), vbm = vb - 1 - ((lane & 15) == 0 ? 2 : 0);

  // e0: keys; an id outside [0, V) becomes V and sorts after every valid id
  {
    int64_t idv[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int i = base + e * 64 + lane;
      idv[e] = i < n ? a.ids[i] : 0;
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int i = base + e * 64 + lane;
      if (i < n) {
        const bool ok = idv[e] >= 0 && idv[e] < (int64_t)a.V;
        s_key[kb + 68 * e] = ok ? (uint32_t)idv[e] : a.V;
        s_val[vb + 72 * e] = (uint16_t)i;
      }
    }
    lds_barrier();
  }
  // e1: sort by (id, position)
  block_radix_sort(s_key, s_val, s_cnt, s_red, n, a.kbits);
  // the valid ids are the keys below V
  int Tv;
  {
    uint32_t ok = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int i = base + e * 64 + lane;
      ok += (i < n && s_key[kb + 68 * e] < a.V) ? 1u : 0u;
    }
    uint32_t tot;
    (void)block_exscan(ok, s_red, &tot);
    Tv = (int)tot;
  }

  // segment starts (fs) and piece starts (ps): counts per wave
  uint32_t key[kPer];
  uint16_t val[kPer];
  uint32_t fsm = 0, psm = 0, cf = 0, cp = 0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int i = base + e * 64 + lane;
    key[e] = i < n ? s_key[kb + 68 * e] : 0u;
    val[e] = i < n ? s_val[vb + 72 * e] : (uint16_t)0;
    const uint32_t kp = (i > 0 && i - 1 < n) ? s_key[kbm + 68 * e] : 0xffffffffu;
    // a segment per distinct id, or (PLAIN) per valid token
    const bool fs = i < Tv && (i == 0 || key[e] != kp || a.mode == TTC_TTM_PLAIN);
    const bool ps = i < Tv && (fs || (i & (kChunk - 1)) == 0);
    fsm |= (uint32_t)fs << e;
    psm |= (uint32_t)ps << e;
    cf += (uint32_t)__popcll(__ballot(fs));
    cp += (uint32_t)__popcll(__ballot(ps));
  }
  if (lane == 0) {
    s_w[w] = cf;
    s_w[kSortWaves + w] = cp;
  }
  lds_barrier();
  int U = 0, P = 0, uu = 0, pp = 0;
  for (int w2 = 0; w2 < kSortWaves; ++w2) {
    const int x = (int)s_w[w2], y = (int)s_w[kSortWaves + w2];
    if (w2 < w) {
      uu += x;
      pp += y;
    }
    U += x;
    P += y;
  }
  --uu;
  --pp;
  // indices, outputs, and the distinct ids compacted into s_key[0..U)
  // (every read of s_key above happened before the barrier)
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int i = base + e * 64 + lane;
    const bool fs = (fsm >> e) & 1u;
    const bool ps = (psm >> e) & 1u;
    const uint64_t mf = __ballot(fs), mp = __ballot(ps);
    const int ui = uu + __popcll(mf & upto);
    const int pi = pp + __popcll(mp & upto);
    uu += __popcll(mf);
    pp += __popcll(mp);
    if (i < n) {
      a.order[i] = val[e];
      // inverse staged in LDS (free after the sort), stored in token order below
      if (val[e] < n) s_cnt[val[e]] = i < Tv ? (uint16_t)ui : (uint16_t)0xffffu;
    }
    if (fs) {
      a.uids[ui] = (int32_t)key[e];
      a.seg[ui] = i;
      a.u_piece[ui] = pi;
      s_key[KI(ui)] = key[e];
      s_val[VI(ui)] = (uint16_t)ui;
    }
    if (ps) a.piece_beg[pi] = i;
    if (i < Tv && (i & (kChunk - 1)) == 0) a.chunk_piece[i / kChunk] = pi;
  }
  const int nchv = (Tv + kChunk - 1) / kChunk;
  for (int c = nchv + tid; c <= a.nch; c += kSortThreads) a.chunk_piece[c] = P;
  if (tid == 0) {
    a.seg[U] = Tv;
    a.u_piece[U] = P;
    a.piece_beg[P] = Tv;
    s_ul[a.d - 1] = U;
  }
  lds_barrier();
  for (int t = tid; t < n; t += kSortThreads) a.inverse[t] = s_cnt[t] == 0xffffu ? -1 : (int32_t)s_cnt[t];

  // e1 (levels): distinct prefixes of every level, from level d-2 down to 0;
  // s_val[u] holds the level-(l+1) node of distinct id u
  int Unext = U;
  for (int l = a.d - 2; l >= 0; --l) {
    const FastDiv M = a.div_pre[l];
    uint32_t pre[kPer];
    uint16_t nx[kPer];
    uint32_t nsm = 0, csm = 0, cnt = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int u = base + e * 64 + lane;
      const bool in = u < U;
      pre[e] = in ? fdiv(s_key[kb + 68 * e], M) : 0u;
      nx[e] = in ? s_val[vb + 72 * e] : (uint16_t)0;
      const bool prev = u > 0 && u - 1 < U;
      const uint32_t pp2 = prev ? fdiv(s_key[kbm + 68 * e], M) : 0xffffffffu;
      const uint32_t nxp = prev ? (uint32_t)s_val[vbm + 72 * e] : 0xffffffffu;
      // a new node per distinct prefix; without prefix sharing, a node per
      // node of the level below
      const bool share = a.mode == TTC_TTM_DEDUP;
      const bool ns = in && (u == 0 || pre[e] != pp2 || !share);
      const bool cs = in && (u == 0 || (uint32_t)nx[e] != nxp || !share);
      nsm |= (uint32_t)ns << e;
      csm |= (uint32_t)cs << e;
      cnt += (uint32_t)__popcll(__ballot(ns));
    }
    if (lane == 0) s_w[w] = cnt;
    lds_barrier();
    int Ul = 0, jj = 0;
    for (int w2 = 0; w2 < kSortWaves; ++w2) {
      const int x = (int)s_w[w2];
      if (w2 < w) jj += x;
      Ul += x;
    }
    --jj;
    uint16_t jx[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const bool ns = (nsm >> e) & 1u;
      const bool cs = (csm >> e) & 1u;
      const uint64_t m1 = __ballot(ns);
      const int j = jj + __popcll(m1 & upto);
      jj += __popcll(m1);
      jx[e] = (uint16_t)j;
      if (ns) {
        a.pref[l][j] = (int32_t)pre[e];
        a.child[l][j] = nx[e];
      }
      if (cs) a.parent[l + 1][nx[e]] = j;
    }
    if (tid == 0) {
      a.child[l][Ul] = Unext;
      s_ul[l] = Ul;
    }
    lds_barrier();
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int u = base + e * 64 + lane;
      if (u < U) s_val[vb + 72 * e] = jx[e];
    }
    lds_barrier();
    Unext = Ul;
  }
  // level 0 hangs off the single root
  for (int j = tid; j < Unext; j += kSortThreads) a.parent[0][j] = 0;
  if (tid == 0) {
    a.hdr[kHdrU] = U;
    a.hdr[kHdrErr] = Tv < n ? 1 : 0;
    a.hdr[kHdrPieces] = P;
    a.hdr[kHdrTv] = Tv;
    for (int l = 0; l < a.d; ++l) a.hdr[kHdrUl + l] = s_ul[l];
  }
}

// Digit lists: the nodes of level l (blockIdx.x) sorted stably by their last
// digit, so that every slice of a core gradient sums a fixed list in node
// order.  One work-group per level, all levels at once.
__global__ __launch_bounds__(kSortThreads) void k_ttm_lists(SortArgs a) {
  __shared__ uint32_t s_key[kKeyWords];
  __shared__ uint16_t s_val[kValHalves];
  __shared__ uint16_t s_cnt[16 * kSortThreads + 16 * kSortThreads / 8];
  __shared__ uint32_t s_red[kSortWaves + 1];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int base = w * kPer * 64;
  const int kb = KI(base + lane), vb = VI(base + lane);
  const int l = blockIdx.x;
  const int Ul = a.hdr[kHdrUl + l];
  const uint32_t ml = (uint32_t)a.m[l];
  const FastDiv dm = a.div_m[l];
  const int32_t* pref = l == a.d - 1 ? a.uids : a.pref[l];
  uint32_t pv[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int j = base + e * 64 + lane;
    pv[e] = j < Ul ? (uint32_t)pref[j] : 0u;
  }
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int j = base + e * 64 + lane;
    if (j < Ul) {
      s_key[kb + 68 * e] = pv[e] - fdiv(pv[e], dm) * ml;
      s_val[vb + 72 * e] = (uint16_t)j;
    }
  }
  lds_barrier();
  block_radix_sort8(s_key, s_val, s_cnt, s_red, Ul, a.dbits[l]);
  for (int j = tid; j < Ul; j += kSortThreads) a.list[l][j] = s_val[VI(j)];
  for (int v = tid; v <= (int)ml; v += kSortThreads) a.list_off[l][v] = lower_bound_lds(s_key, Ul, (uint32_t)v);
}

// ------------------------------------------------------------------------------
// per-node products
// ------------------------------------------------------------------------------
// Flat index e = q * div + r walked with a fixed stride, without divisions.
struct Walk {
  int q, r, dq, dr, div;
  __device__ __forceinline__ Walk(int start, int step, int d) : div(d) {
    q = start / d;
    r = start - q * d;
    dq = step / d;
    dr = step - dq * d;
  }
  __device__ __forceinline__ void next() {
    r += dr;
    q += dq;
    if (r >= div) {
      r -= div;
      ++q;
    }
  }
};

// A node's gradient is the sum of a range of source rows (off != NULL:
// rows off[j] .. off[j+1]-1) or a single row j (off == NULL).
struct Src {
  const float* p;
  const int32_t* off;
  int64_t ld;
};

struct LevelArgs {
  int l;                  // level (>= 1)
  int m, nk, ra, rb, R;   // m_{l+1}, n_{l+1}, r_l, r_{l+1}; R = prod n_{<=l-1}
  int blk;                // nk * rb
  const int32_t* hdr;
  const int32_t* pref;    // level l prefixes (digit = pref % m)
  const int32_t* parent;  // level l parents
  const int32_t* ppref;   // level l-1 prefixes (a level-0 product is the slice F_1[0, v])
  const float* F0;        // F_1
  const float* Ppar;      // products of level l-1 (l >= 2)
  const float* Dpar;      // D on the link into level l, NULL = identity
  const float* F;         // core l+1 (1-based)
  float* out;             // forward: P_l (or the distinct-id rows at the last level)
  Src src;                // backward: gradient sources of the level-l nodes
  float* C;               // backward: ra * blk per level-l node
  float* Q;               // backward: R * ra per level-l node
};

// the parent's product with D applied, R x ra (16-byte loads when ra is a
// multiple of 4 and the product is aligned)
__device__ __forceinline__ void stage_pd(const LevelArgs& a, int p, float* sPd) {
  const int np = a.R * a.ra;
  const float* Pp = a.l == 1 ? a.F0 + (int64_t)((uint32_t)a.ppref[p]) * np : a.Ppar + (int64_t)p * np;
  if ((a.ra & 3) == 0 && ((uintptr_t)Pp & 15) == 0) {
    Walk wk(4 * threadIdx.x, 4 * blockDim.x, a.ra);
#pragma unroll 4
    for (int e = 4 * threadIdx.x; e < np; e += 4 * blockDim.x) {
      f32x4 v = *reinterpret_cast<const f32x4*>(Pp + e);
      if (a.Dpar) {
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] *= a.Dpar[wk.r + u];
      }
      *reinterpret_cast<f32x4*>(sPd + e) = v;
      wk.next();
    }
    return;
  }
  Walk wk(threadIdx.x, blockDim.x, a.ra);
#pragma unroll 4
  for (int e = threadIdx.x; e < np; e += blockDim.x) {
    sPd[e] = Pp[e] * (a.Dpar ? a.Dpar[wk.r] : 1.f);
    wk.next();
  }
}

// the core slice F[:, v, :, :] of node j, ra x blk, rows padded to blk + 1
// floats so that lanes reading one column of different rows do not collide
// (16-byte loads when blk is a multiple of 4 and the core is aligned)
__device__ __forceinline__ void stage_w(const LevelArgs& a, int j, float* sW) {
  const int v = (int)((uint32_t)a.pref[j] % (uint32_t)a.m);
  const int nw = a.ra * a.blk;
  if ((a.blk & 3) == 0 && ((uintptr_t)a.F & 15) == 0) {
    Walk wk(4 * threadIdx.x, 4 * blockDim.x, a.blk);
#pragma unroll 4
    for (int e = 4 * threadIdx.x; e < nw; e += 4 * blockDim.x) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(a.F + ((int64_t)wk.q * a.m + v) * a.blk + wk.r);
#pragma unroll
      for (int u = 0; u < 4; ++u) sW[wk.q * (a.blk + 1) + wk.r + u] = x[u];
      wk.next();
    }
    return;
  }
  Walk wk(threadIdx.x, blockDim.x, a.blk);
#pragma unroll 4
  for (int e = threadIdx.x; e < nw; e += blockDim.x) {
    sW[wk.q * (a.blk + 1) + wk.r] = a.F[((int64_t)wk.q * a.m + v) * a.blk + wk.r];
    wk.next();
  }
}

// ranks a forward thread keeps its core column of in registers
constexpr int kTtmRegRank = 32;

// dot product of n terms x[i * sx] * y[i * sy] in order, loads issued 8 ahead
__device__ __forceinline__ float dot_lds(const float* x, int sx, const float* y, int sy, int n) {
  float acc = 0.f;
  int i = 0;
  for (; i + 8 <= n; i += 8) {
    float xv[8], yv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      xv[k] = x[(i + k) * sx];
      yv[k] = y[(i + k) * sy];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) acc = fmaf(xv[k], yv[k], acc);
  }
  for (; i < n; ++i) acc = fmaf(x[i * sx], y[i * sy], acc);
  return acc;
}

__device__ __forceinline__ void add4(float4& acc, const float4& x) {
  acc.x += x.x;
  acc.y += x.y;
  acc.z += x.z;
  acc.w += x.w;
}

// Sum of a node's source rows, elements [e, e + 4) of each row (float4-aligned
// rows).  Rows are added one at a time in increasing order (one accumulator), in
// batches of kRowBatch loads with the next batch requested before the current
// one is added, so a long run of rows costs about one memory latency per
// kRowBatch rows.  (Measured on the 32x32x32 table's backward levels: 4 beats
// 8, 86 -> 54 registers, five -> eight waves per SIMD, the last level 28.5 ->
// 25.7 us, since most nodes have one or two rows and the launch runs in rounds
// of resident work-groups; 16 costs more registers than it saves.)
#ifndef TTC_TTM_ROW_BATCH
#define TTC_TTM_ROW_BATCH 4
#endif
constexpr int kRowBatch = TTC_TTM_ROW_BATCH;
__device__ __forceinline__ float4 sum_rows4(const float* p, int64_t ld, int s0, int s1, int e) {
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  auto row = [&](int q) { return *reinterpret_cast<const float4*>(p + (int64_t)q * ld + e); };
  int q = s0;
  if (q + kRowBatch <= s1) {
    float4 x0[kRowBatch], x1[kRowBatch];
#pragma unroll
    for (int k = 0; k < kRowBatch; ++k) x0[k] = row(q + k);
    q += kRowBatch;
    while (true) {
      const bool more1 = q + kRowBatch <= s1;
      if (more1) {
#pragma unroll
        for (int k = 0; k < kRowBatch; ++k) x1[k] = row(q + k);
      }
#pragma unroll
      for (int k = 0; k < kRowBatch; ++k) add4(acc, x0[k]);
      if (!more1) break;
      q += kRowBatch;
      const bool more0 = q + kRowBatch <= s1;
      if (more0) {
#pragma unroll
        for (int k = 0; k < kRowBatch; ++k) x0[k] = row(q + k);
      }
#pragma unroll
      for (int k = 0; k < kRowBatch; ++k) add4(acc, x1[k]);
      if (!more0) break;
      q += kRowBatch;
    }
  }
  for (; q < s1; ++q) add4(acc, row(q));
  return acc;
}

__device__ __forceinline__ float sum_rows1(const float* p, int64_t ld, int s0, int s1, int e) {
  float acc = 0.f;
  int q = s0;
  for (; q + 8 <= s1; q += 8) {
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = p[(int64_t)(q + k) * ld + e];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc += x[k];
  }
  for (; q < s1; ++q) acc += p[(int64_t)q * ld + e];
  return acc;
}

// the node's gradient, R x blk (ng floats)
__device__ __forceinline__ void stage_g(const Src& s, int j, int ng, float* sG) {
  const int s0 = s.off ? s.off[j] : j, s1 = s.off ? s.off[j + 1] : j + 1;
  if ((ng & 3) == 0 && (s.ld & 3) == 0) {
    for (int e = 4 * threadIdx.x; e < ng; e += 4 * blockDim.x)
      *reinterpret_cast<float4*>(sG + e) = sum_rows4(s.p, s.ld, s0, s1, e);
  } else {
    for (int e = threadIdx.x; e < ng; e += blockDim.x) sG[e] = sum_rows1(s.p, s.ld, s0, s1, e);
  }
}

// forward, one work-group per level-l node:
//   P_l[j][(c, c_k), b] = sum_a Pd[c, a] F[a, v, c_k, b]
__global__ __launch_bounds__(kLevelThreads) void k_ttm_level_fwd(LevelArgs a) {
  extern __shared__ float lds[];
  const int Ul = a.hdr[kHdrUl + a.l];
  const int np = a.R * a.ra;
  const int ldw = a.blk + 1;
  float* sPd = lds;
  float* sW = lds + np;
  const int nout = a.R * a.blk;
  for (int j = blockIdx.x; j < Ul; j += gridDim.x) {
    stage_pd(a, a.parent[j], sPd);
    stage_w(a, j, sW);
    lds_barrier();
    float* o = a.out + (int64_t)j * nout;
    if (kLevelThreads % a.blk == 0 && (a.ra & 3) == 0 && a.ra <= kTtmRegRank) {
      // blk divides the work-group: every output of this thread is in column
      // r of the slice, which it keeps in registers; the rows of Pd come as
      // 16-byte LDS reads (same terms, same order as the general form)
      const int r = (int)threadIdx.x % a.blk;
      float w[kTtmRegRank];
#pragma unroll
      for (int x = 0; x < kTtmRegRank; ++x) w[x] = x < a.ra ? sW[x * ldw + r] : 0.f;
      for (int q = (int)threadIdx.x / a.blk; q < a.R; q += kLevelThreads / a.blk) {
        const float* pr = sPd + q * a.ra;
        float acc = 0.f;
#pragma unroll
        for (int x = 0; x < kTtmRegRank; x += 4) {
          if (x < a.ra) {
            const f32x4 pv = *reinterpret_cast<const f32x4*>(pr + x);
#pragma unroll
            for (int u = 0; u < 4; ++u) acc = fmaf(pv[u], w[x + u], acc);
          }
        }
        o[q * a.blk + r] = acc;
      }
    } else {
      Walk wk(threadIdx.x, blockDim.x, a.blk);
      for (int e = threadIdx.x; e < nout; e += blockDim.x) {
        o[e] = dot_lds(sPd + wk.q * a.ra, 1, sW + wk.r, ldw, a.ra);
        wk.next();
      }
    }
    lds_barrier();
  }
}

// backward, one work-group per level-l node j: its share of dF,
//   C_j[a, c_k, b] = sum_c Pd[c, a] G_j[(c, c_k), b],
// and its contribution to the parent's gradient,
//   Q_j[c, a] = D[a] sum_{c_k, b} G_j[(c, c_k), b] F[a, v, c_k, b].
// C4: the grouped form of C (host's choice per level, a separate instance so
// that the other form keeps its smaller register count)
template <bool C4>
__global__ __launch_bounds__(kLevelBwdThreads) void k_ttm_level_bwd(LevelArgs a) {
  extern __shared__ float lds[];
  const int np = a.R * a.ra;
  const int nw = a.ra * a.blk;
  const int ng = a.R * a.blk;
  const int ldw = a.blk + 1;
  float* sPd = lds;
  float* sW = sPd + np;
  float* sG = sW + a.ra * ldw;
  const int Ul = a.hdr[kHdrUl + a.l];
  for (int j = blockIdx.x; j < Ul; j += gridDim.x) {
    stage_pd(a, a.parent[j], sPd);
    stage_w(a, j, sW);
    stage_g(a.src, j, ng, sG);
    lds_barrier();
    float* C = a.C + (int64_t)j * nw;
    if (C4 && ((uintptr_t)sG & 15) == 0) {
      // four adjacent outputs C[a][r..r+3] per thread: one read of Pd[c][a]
      // and one 16-byte read of G[c][r..r+3] per term (each output sums its
      // terms in the same order as the general form)
      const int nb4 = a.blk / 4;
      Walk wk(threadIdx.x, blockDim.x, nb4);
      for (int e = threadIdx.x; e < a.ra * nb4; e += blockDim.x) {
        const int x = wk.q, r = 4 * wk.r;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        int c = 0;
        for (; c + 8 <= a.R; c += 8) {  // eight terms' reads issued together
          float p[8];
          f32x4 g[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            p[k] = sPd[(c + k) * a.ra + x];
            g[k] = *reinterpret_cast<const f32x4*>(sG + (c + k) * a.blk + r);
          }
#pragma unroll
          for (int k = 0; k < 8; ++k)
#pragma unroll
            for (int u = 0; u < 4; ++u) acc[u] = fmaf(p[k], g[k][u], acc[u]);
        }
        for (; c < a.R; ++c) {
          const float p = sPd[c * a.ra + x];
          const f32x4 g = *reinterpret_cast<const f32x4*>(sG + c * a.blk + r);
#pragma unroll
          for (int u = 0; u < 4; ++u) acc[u] = fmaf(p, g[u], acc[u]);
        }
        *reinterpret_cast<f32x4*>(C + x * a.blk + r) = acc;
        wk.next();
      }
    } else {
      Walk wk(threadIdx.x, blockDim.x, a.blk);
      for (int e = threadIdx.x; e < nw; e += blockDim.x) {
        C[e] = dot_lds(sPd + wk.q, a.ra, sG + wk.r, a.blk, a.R);
        wk.next();
      }
    }
    float* Q = a.Q + (int64_t)j * np;
    Walk wk(threadIdx.x, blockDim.x, a.ra);
    for (int e = threadIdx.x; e < np; e += blockDim.x) {
      const float acc = dot_lds(sG + wk.q * a.blk, 1, sW + wk.r * ldw, 1, a.blk);
      Q[e] = acc * (a.Dpar ? a.Dpar[wk.r] : 1.f);
      wk.next();
    }
    lds_barrier();
  }
}

// 16-byte accesses of data the step touches once (the token rows written by the
// gather, the row gradients read by the segment sums): non-temporal, so that
// they do not displace the cores, products and partial sums that are re-read.
typedef float stream_f4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld_stream4(const float* p) {
  const stream_f4 t = __builtin_nontemporal_load(reinterpret_cast<const stream_f4*>(p));
  return make_float4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ void st_stream4(float* p, float4 v) {
  const stream_f4 t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, reinterpret_cast<stream_f4*>(p));
}

// out[t] = row of inverse[t] (through `map` when given: the row index of a
// distinct id); zero for an id that was out of range.  Each wave copies
// kRowsPerWave rows, loading all of them before storing.
constexpr int kRowsPerWave = 4;

template <bool VEC>
__global__ __launch_bounds__(kTtmThreads) void k_ttm_gather(const int32_t* __restrict__ inverse,
                                                            const int32_t* __restrict__ map,
                                                            const float* __restrict__ rows, float* __restrict__ out,
                                                            int64_t T, int64_t N) {
  const int lane = threadIdx.x & 63;
  const int64_t t0 = ((int64_t)blockIdx.x * (kTtmThreads / 64) + (threadIdx.x >> 6)) * kRowsPerWave;
  int u[kRowsPerWave];
#pragma unroll
  for (int k = 0; k < kRowsPerWave; ++k) {
    const int64_t t = t0 + k;
    int x = t < T ? inverse[t] : -1;
    if (map && x >= 0) x = map[x];
    u[k] = x;
  }
  if constexpr (VEC) {
    const int64_t nv = N / 4;
    for (int64_t c = lane; c < nv; c += 64) {
      float4 v[kRowsPerWave];
#pragma unroll
      for (int k = 0; k < kRowsPerWave; ++k)
        v[k] = u[k] >= 0 ? reinterpret_cast<const float4*>(rows + (int64_t)u[k] * N)[c]
                         : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int k = 0; k < kRowsPerWave; ++k)
        if (t0 + k < T) st_stream4(out + (t0 + k) * N + 4 * (int64_t)c, v[k]);
    }
  } else {
    for (int64_t c = lane; c < N; c += 64) {
      float v[kRowsPerWave];
#pragma unroll
      for (int k = 0; k < kRowsPerWave; ++k) v[k] = u[k] >= 0 ? rows[(int64_t)u[k] * N + c] : 0.f;
#pragma unroll
      for (int k = 0; k < kRowsPerWave; ++k)
        if (t0 + k < T) out[(t0 + k) * N + c] = v[k];
    }
  }
}

// ------------------------------------------------------------------------------
// backward
// ------------------------------------------------------------------------------
// e5: per chunk of kChunk sorted positions, the sum of the output gradients
// of each piece's tokens, in position order.  All rows of the chunk are loaded
// ahead of the (piece-ordered) accumulation.
template <bool VEC>
__global__ __launch_bounds__(kTtmThreads) void k_ttm_seg(const int32_t* __restrict__ hdr,
                                                         const int32_t* __restrict__ order,
                                                         const int32_t* __restrict__ piece_beg,
                                                         const int32_t* __restrict__ chunk_piece,
                                                         const float* __restrict__ dout, float* __restrict__ PS,
                                                         int64_t N) {
  __shared__ int32_t s_ord[kChunk];
  __shared__ int32_t s_pb[kChunk + 1];
  const int c = blockIdx.x;
  const int p0 = chunk_piece[c], p1 = chunk_piece[c + 1];
  if (p0 == p1) return;
  const int Tv = hdr[kHdrTv];
  const int i0 = c * kChunk;
  const int i1 = (i0 + kChunk < Tv) ? i0 + kChunk : Tv;
  if (threadIdx.x < kChunk) s_ord[threadIdx.x] = i0 + (int)threadIdx.x < i1 ? order[i0 + threadIdx.x] : 0;
  if ((int)threadIdx.x <= p1 - p0) s_pb[threadIdx.x] = piece_beg[p0 + threadIdx.x];
  lds_barrier();
  constexpr int B = kChunk;  // the whole chunk's rows in flight at once
  const int64_t nv = VEC ? N / 4 : N;
  for (int64_t col = threadIdx.x; col < nv; col += blockDim.x) {
    int pi = 0;
    int pend = s_pb[1];
    if constexpr (VEC) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int ib = i0; ib < i1; ib += B) {
        float4 x[B];
#pragma unroll
        for (int q = 0; q < B; ++q)
          x[q] = ib + q < i1 ? ld_stream4(dout + (int64_t)s_ord[ib + q - i0] * N + 4 * (int64_t)col)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int q = 0; q < B; ++q) {
          if (ib + q < i1) {
            acc.x += x[q].x;
            acc.y += x[q].y;
            acc.z += x[q].z;
            acc.w += x[q].w;
            if (ib + q + 1 == pend) {
              reinterpret_cast<float4*>(PS + (int64_t)(p0 + pi) * N)[col] = acc;
              acc = make_float4(0.f, 0.f, 0.f, 0.f);
              ++pi;
              pend = pi < p1 - p0 ? s_pb[pi + 1] : 0x7fffffff;
            }
          }
        }
      }
    } else {
      float acc = 0.f;
      for (int ib = i0; ib < i1; ib += B) {
        float x[B];
#pragma unroll
        for (int q = 0; q < B; ++q) x[q] = ib + q < i1 ? dout[(int64_t)s_ord[ib + q - i0] * N + col] : 0.f;
#pragma unroll
        for (int q = 0; q < B; ++q) {
          if (ib + q < i1) {
            acc += x[q];
            if (ib + q + 1 == pend) {
              PS[(int64_t)(p0 + pi) * N + col] = acc;
              acc = 0.f;
              ++pi;
              pend = pi < p1 - p0 ? s_pb[pi + 1] : 0x7fffffff;
            }
          }
        }
      }
    }
  }
}

// Final step: dF_{l+1}[a, v, :, :] is the sum, over the level-l nodes whose
// last digit is v (in node order), of their C[a, :, :]; at level 0 a node's C
// is its gradient itself (the sum of its sources).  One work-group per
// (level, v, a); the list is split over QL lanes, each summing every QL-th
// entry in order, and the QL partial sums are added by a fixed tree.
struct ReduceArgs {
  int d;
  int m[TTC_TTM_MAX_MODES], blk[TTC_TTM_MAX_MODES], ra[TTC_TTM_MAX_MODES];
  int item_off[TTC_TTM_MAX_MODES + 1];
  const int32_t* list[TTC_TTM_MAX_MODES];
  const int32_t* list_off[TTC_TTM_MAX_MODES];
  const float* C[TTC_TTM_MAX_MODES];
  Src src0;
  float* dF[TTC_TTM_MAX_MODES];
  int accumulate;
};

__global__ __launch_bounds__(kTtmThreads) void k_ttm_reduce(ReduceArgs a) {
  __shared__ float s_red[kTtmThreads];
  const int it = blockIdx.x;
  int l = 0;
  while (l + 1 < a.d && it >= a.item_off[l + 1]) ++l;
  const int rem = it - a.item_off[l];
  const int ra = a.ra[l], blk = a.blk[l], m = a.m[l];
  const int v = rem / ra, aa = rem - v * ra;
  const int b0 = a.list_off[l][v], b1 = a.list_off[l][v + 1];
  const int32_t* lst = a.list[l];
  int BW = 1;
  while (BW < blk && BW < kTtmThreads) BW <<= 1;
  const int QL = kTtmThreads / BW;
  const int ql = threadIdx.x / BW, cb0 = threadIdx.x - ql * BW;
  const int nw = ra * blk;
  float* dF = a.dF[l];
  for (int cbase = 0; cbase < blk; cbase += BW) {
    const int cb = cbase + cb0;
    float acc = 0.f;
    if (cb < blk) {
      const int e = aa * blk + cb;
      if (l == 0) {
        for (int q = b0 + ql; q < b1; q += QL) {
          const int j = lst[q];
          acc += sum_rows1(a.src0.p, a.src0.ld, a.src0.off[j], a.src0.off[j + 1], e);
        }
      } else {
        const float* C = a.C[l];
        int q = b0 + ql;
        for (; q + 3 * QL < b1; q += 4 * QL) {
          const float x0 = C[(int64_t)lst[q] * nw + e];
          const float x1 = C[(int64_t)lst[q + QL] * nw + e];
          const float x2 = C[(int64_t)lst[q + 2 * QL] * nw + e];
          const float x3 = C[(int64_t)lst[q + 3 * QL] * nw + e];
          acc += x0;
          acc += x1;
          acc += x2;
          acc += x3;
        }
        for (; q < b1; q += QL) acc += C[(int64_t)lst[q] * nw + e];
      }
    }
    if (QL > 1) {
      s_red[threadIdx.x] = acc;
      lds_barrier();
      for (int sft = QL / 2; sft >= 1; sft >>= 1) {
        if (ql < sft) s_red[threadIdx.x] += s_red[threadIdx.x + sft * BW];
        lds_barrier();
      }
      acc = s_red[threadIdx.x];
    }
    if (ql == 0 && cb < blk) {
      float* o = dF + ((int64_t)aa * m + v) * blk + cb;
      *o = a.accumulate ? *o + acc : acc;
    }
    lds_barrier();
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

static FastDiv make_fastdiv(uint32_t M) {
  int lg = 0;
  while ((uint64_t(1) << lg) < M) ++lg;
  FastDiv f;
  f.shift = 32 + lg;
  const unsigned __int128 num = (unsigned __int128)1 << f.shift;
  f.magic = (uint64_t)((num + M - 1) / M);
  return f;
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
  if (desc->mode < TTC_TTM_DEDUP || desc->mode > TTC_TTM_PLAIN) return TTC_ERR_SHAPE;
  P->mode = desc->mode;
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
    // most nodes of level l: distinct prefixes (DEDUP), distinct ids (UNIQUE)
    // or tokens (PLAIN)
    const int64_t lim = P->mode == TTC_TTM_DEDUP ? mprod : (P->mode == TTC_TTM_UNIQUE ? V : T);
    P->cap[l] = lim < T ? lim : T;
    P->psz[l] = nprod * P->r[l + 1];
    const size_t blk = (size_t)P->n[l] * P->r[l + 1];
    P->lds_fwd[l] = 4 * ((size_t)P->R[l] * P->r[l] + (size_t)P->r[l] * (blk + 1));
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

// work-groups of a per-node level launch: the node count is known only on
// the device, so the grid is capped and each work-group strides over nodes
// (measured: a cap of 4096 beats launching one work-group per possible node)
#ifndef TTC_TTM_NODE_GRID
#define TTC_TTM_NODE_GRID 4096
#endif
static unsigned grid_nodes(int64_t cap) {
  return (unsigned)(cap < 1 ? 1 : (cap > TTC_TTM_NODE_GRID ? TTC_TTM_NODE_GRID : cap));
}

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
  a->m = P.m[l];
  a->nk = P.n[l];
  a->ra = P.r[l];
  a->rb = P.r[l + 1];
  a->R = (int)P.R[l];
  a->blk = P.n[l] * P.r[l + 1];
  a->hdr = atc<const int32_t*>(saved, 0);
  a->pref = atc<const int32_t*>(saved, P.sv_pref[l]);
  a->parent = atc<const int32_t*>(saved, P.sv_parent[l]);
  a->ppref = atc<const int32_t*>(saved, P.sv_pref[l - 1]);
  a->F0 = F[0];
  a->Ppar = l >= 2 ? atc<const float*>(saved, P.sv_P[l - 1]) : nullptr;
  a->Dpar = D ? D[l - 1] : nullptr;
  a->F = F[l];
}

// where the gradient of each level-l node comes from
static Src level_src(const TtmPlan& P, int l, const void* saved, void* scratch) {
  Src s;
  if (l == P.d - 1) {
    s.p = at<const float*>(scratch, P.sc_PS);
    s.off = atc<const int32_t*>(saved, P.sv_u_piece);
    s.ld = P.N;
  } else {
    s.p = at<const float*>(scratch, P.sc_Q[l + 1]);
    s.off = atc<const int32_t*>(saved, P.sv_child[l]);
    s.ld = P.psz[l];
  }
  return s;
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

extern "C" ttc_status ttc_device_error(const void* saved, ttc_stream_t stream, int32_t* code) {
  if (!saved || !code) return TTC_ERR_NULL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int32_t word = 0;
  (void)hipGetLastError();
  if (hipMemcpyAsync(&word, static_cast<const char*>(saved) + 4, sizeof(word), hipMemcpyDeviceToHost, s) !=
          hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return TTC_ERR_HIP;
  *code = word;
  return TTC_OK;
}

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

namespace ttc {
// The index of a lookup (depends on the ids only): sort, distinct ids,
// segments, pieces, distinct digit prefixes per level and the digit lists.
static void launch_index(const TtmPlan& P, int64_t T, const int64_t* ids, void* saved, hipStream_t s) {
  SortArgs sa;
  memset(&sa, 0, sizeof(sa));
  sa.ids = ids;
  sa.n = (int)T;
  sa.V = (uint32_t)P.V;
  sa.kbits = P.kbits;
  sa.mode = P.mode;
  sa.d = P.d;
  sa.nch = (int)P.nch;
  for (int l = 0; l < P.d; ++l) {
    sa.m[l] = P.m[l];
    sa.div_pre[l] = make_fastdiv(P.Mgt[l]);
    sa.div_m[l] = make_fastdiv((uint32_t)P.m[l]);
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
  sa.piece_beg = at<int32_t*>(saved, P.sv_piece_beg);
  sa.chunk_piece = at<int32_t*>(saved, P.sv_chunk_piece);
  sa.u_piece = at<int32_t*>(saved, P.sv_u_piece);
  {
    TraceScope ts("ttm_sort", s);
    TTC_LAUNCH(k_ttm_sort, dim3(1), dim3(kSortThreads), 0, s, sa);
  }
  {
    TraceScope ts("ttm_lists", s);
    TTC_LAUNCH(k_ttm_lists, dim3((unsigned)P.d), dim3(kSortThreads), 0, s, sa);
  }
}

// The rows of a lookup from its index: prefix products level by level, the
// distinct-id rows, and the token gather.
static void launch_lookup(const TtmPlan& P, int64_t T, const float* const* F, const float* const* D, float* out,
                          void* saved, void* scratch, hipStream_t s) {
  // prefix products, level 1 .. d-1 (level 0 is a slice of F_1)
  for (int l = 1; l < P.d; ++l) {
    LevelArgs a;
    fill_level(P, l, saved, F, D, &a);
    a.out = l == P.d - 1 ? at<float*>(scratch, P.sc_urow) : at<float*>(saved, P.sv_P[l]);
    TraceScope ts("ttm_level", s);
    TTC_LAUNCH(k_ttm_level_fwd, dim3(grid_nodes(P.cap[l])), dim3(kLevelThreads), P.lds_fwd[l], s, a);
  }
  // with one core the rows are those of F_1 itself, indexed by the id
  const float* rows = P.d >= 2 ? at<const float*>(scratch, P.sc_urow) : F[0];
  const int32_t* map = P.d >= 2 ? nullptr : at<const int32_t*>(saved, P.sv_uids);
  const int32_t* inv = at<const int32_t*>(saved, P.sv_inverse);
  const bool vec = (P.N % 4) == 0 && al16(rows);
  const int64_t per_block = (kTtmThreads / 64) * kRowsPerWave;
  const unsigned grid = (unsigned)((T + per_block - 1) / per_block);
  TraceScope ts("ttm_gather", s);
  if (vec)
    TTC_LAUNCH(k_ttm_gather<true>, dim3(grid), dim3(kTtmThreads), 0, s, inv, map, rows, out, T, P.N);
  else
    TTC_LAUNCH(k_ttm_gather<false>, dim3(grid), dim3(kTtmThreads), 0, s, inv, map, rows, out, T, P.N);
}
}  // namespace ttc

extern "C" ttc_status ttm_embed_index(const ttm_embed_desc* desc, int64_t T, const int64_t* ids, void* saved,
                                      size_t saved_bytes, ttc_stream_t stream) {
  TtmPlan P;
  ttc_status st = make_ttm_plan(desc, T, &P);
  if (st != TTC_OK) return st;
  if (T == 0) return TTC_OK;
  if (!ids || !saved) return TTC_ERR_NULL;
  if (!al16(saved)) return TTC_ERR_ALIGN;
  if (saved_bytes < P.sv_total) return TTC_ERR_WORKSPACE;
  (void)hipGetLastError();
  launch_index(P, T, ids, saved, (hipStream_t)stream);
  return hip_ok();
}

extern "C" ttc_status ttm_embed_lookup(const ttm_embed_desc* desc, int64_t T, const float* const* F,
                                       const float* const* D, float* out, void* saved, size_t saved_bytes,
                                       void* scratch, size_t scratch_bytes, ttc_stream_t stream) {
  TtmPlan P;
  ttc_status st = make_ttm_plan(desc, T, &P);
  if (st != TTC_OK) return st;
  if ((st = check_cores(P, F, D)) != TTC_OK) return st;
  if (T == 0) return TTC_OK;
  if (!out || !saved || (P.d >= 2 && !scratch)) return TTC_ERR_NULL;
  if (!al16(out) || !al16(saved) || (scratch && !al16(scratch))) return TTC_ERR_ALIGN;
  if (saved_bytes < P.sv_total || (P.d >= 2 && scratch_bytes < P.sc_fwd)) return TTC_ERR_WORKSPACE;
  (void)hipGetLastError();
  launch_lookup(P, T, F, D, out, saved, scratch, (hipStream_t)stream);
  return hip_ok();
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
  launch_index(P, T, ids, saved, s);
  launch_lookup(P, T, F, D, out, saved, scratch, s);
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
        TTC_LAUNCH(k_ttm_zero, dim3((unsigned)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024)), dim3(256),
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
    const int32_t* hdr = atc<const int32_t*>(saved, 0);
    if (vec)
      TTC_LAUNCH(k_ttm_seg<true>, dim3((unsigned)P.nch), dim3(kTtmThreads), 0, s, hdr,
                         atc<const int32_t*>(saved, P.sv_order), atc<const int32_t*>(saved, P.sv_piece_beg),
                         atc<const int32_t*>(saved, P.sv_chunk_piece), dout, PS, P.N);
    else
      TTC_LAUNCH(k_ttm_seg<false>, dim3((unsigned)P.nch), dim3(kTtmThreads), 0, s, hdr,
                         atc<const int32_t*>(saved, P.sv_order), atc<const int32_t*>(saved, P.sv_piece_beg),
                         atc<const int32_t*>(saved, P.sv_chunk_piece), dout, PS, P.N);
  }
  for (int l = P.d - 1; l >= 1; --l) {
    LevelArgs a;
    fill_level(P, l, saved, F, D, &a);
    a.src = level_src(P, l, saved, scratch);
    a.C = at<float*>(scratch, P.sc_C[l]);
    a.Q = at<float*>(scratch, P.sc_Q[l]);
    TraceScope ts("ttm_bwd_level", s);
    // the grouped C form only with a group of four outputs for every thread
    // (fewer, longer sums measured slower: the last level of a 32x32x32
    // vocabulary has 16 x 2 groups of 96 terms)
    const bool c4 = (a.blk & 3) == 0 && a.ra * (a.blk / 4) >= kLevelBwdThreads;
    if (c4)
      TTC_LAUNCH(k_ttm_level_bwd<true>, dim3(grid_nodes(P.cap[l])), dim3(kLevelBwdThreads), P.lds_bwd[l], s, a);
    else
      TTC_LAUNCH(k_ttm_level_bwd<false>, dim3(grid_nodes(P.cap[l])), dim3(kLevelBwdThreads), P.lds_bwd[l], s, a);
  }
  ReduceArgs ra;
  memset(&ra, 0, sizeof(ra));
  ra.d = P.d;
  int items = 0;
  for (int l = 0; l < P.d; ++l) {
    ra.m[l] = P.m[l];
    ra.blk[l] = P.n[l] * P.r[l + 1];
    ra.ra[l] = P.r[l];
    ra.item_off[l] = items;
    items += P.m[l] * P.r[l];
    ra.list[l] = atc<const int32_t*>(saved, P.sv_list[l]);
    ra.list_off[l] = atc<const int32_t*>(saved, P.sv_list_off[l]);
    ra.C[l] = l >= 1 ? at<const float*>(scratch, P.sc_C[l]) : nullptr;
    ra.dF[l] = dF[l];
  }
  ra.item_off[P.d] = items;
  ra.src0 = level_src(P, 0, saved, scratch);
  ra.accumulate = desc->accumulate ? 1 : 0;
  {
    TraceScope ts("ttm_reduce", s);
    TTC_LAUNCH(k_ttm_reduce, dim3((unsigned)items), dim3(kTtmThreads), 0, s, ra);
  }
  return hip_ok();
}
