// Validation, contraction-path cost model and buffer layout of a TT-linear call.
//
// The merged path is the contraction order of the CoMERA project page, section
// "Making small tensor operations fast on GPUs" (Proposition 4.1): both halves
// of the chain are multiplied out first, the tokens then pass through two
// skinny products, and the rank-sized intermediate is kept for the backward.
// The page argues that this order costs close to the minimum once the batch is
// large; the model below prices it next to a core-by-core sweep and the dense
// weight, so the crossover can be computed for any shape, batch and rank.
#include "tt_plan.hpp"

#include <string.h>

#include <algorithm>
#include <cmath>

namespace ttc {

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// largest extent of one buffer resource of the streaming kernels
constexpr int64_t kRsrcMax = 0x7fffffff;
static bool fits_rsrc(int64_t bytes) { return bytes <= kRsrcMax; }

// Launch shape of a backward streaming pass.  A work-group owns a range of
// columns (whole 256-byte slabs) and a range of token tiles.  Splitting the
// columns of the dY pass costs partial sums of the T x r intermediate dZ (and
// the dX pass re-reads dZ once per column group); splitting the tokens costs
// partial sums of the r x N weight-side gradients.  The passes are bound by
// each CU's share of the memory traffic, so the time of a shape is the bytes
// of the busiest CU: the work-groups per CU (rounded up) times the bytes of
// one work-group.  The partials that the reductions read back later run
// beside the streaming passes and weigh half.
#ifndef TTC_LATER_WEIGHT
#define TTC_LATER_WEIGHT 0.5
#endif
bool plan_bwd_grid(const LinearPlan& P, bool dy, double ncu, int gc_max, int gt_max, BwdGrid* out) {
  const double kLaterWeight = TTC_LATER_WEIGHT;
  const int64_t ncols = dy ? P.N_out : P.N_in;
  const int maxs = dy ? bwd_max_slabs(P.es, P.NR) : dx_max_slabs(P.es, P.NR);
  const int nt = std::max(1, P.ntiles);
  const int chunks = (int)std::max<int64_t>(1, (ncols + P.sw - 1) / P.sw);
  const int gc_min = (chunks + maxs - 1) / maxs;
  double best = 1e300;
  int bsl = 0, bper = 0;
  for (int g = gc_min; g <= chunks; ++g) {
    const int sl = (chunks + g - 1) / g;
    if ((chunks + sl - 1) / sl != g) continue;  // same shape as a smaller g
    if (gc_max > 0 && g > gc_max) continue;
    for (int per = 1; per <= nt; ++per) {
      const int tg = (nt + per - 1) / per;
      if ((nt + tg - 1) / tg != per) continue;
      if (gt_max > 0 && tg > gt_max) continue;
      // a work-group's token range of the streamed activation, of its rank
      // tile and of the fp32 dZ partials are each one buffer resource
      const int64_t toks64 = int64_t(per) * kTileT;
      if (!fits_rsrc(toks64 * ncols * P.es) || !fits_rsrc(toks64 * P.Rpad * 4)) break;
      const double cols = double(sl) * P.sw, toks = double(per) * kTileT;
      double wg = toks * cols * P.es * (dy ? 1.0 : 2.0);  // streamed activations
      wg += 4.0 * P.rs * cols;                           // weight-side partial
      if (dy)
        wg += (g > 1 ? 4.0 : 0.0) * toks * P.Rpad + toks * P.Rpad * P.es;  // dZ partial, Z tile
      else
        wg += toks * P.Rpad * P.es;  // dZ tile
      const double later = 4.0 * tg * P.rs * double(ncols) + (dy && g > 1 ? 4.0 * g * double(P.T) * P.Rpad : 0.0);
      const double cost = std::ceil(double(g) * tg / ncu) * wg + kLaterWeight * later / ncu;
      if (cost < best * (1 - 1e-9)) {
        best = cost;
        bsl = sl;
        bper = per;
      }
    }
  }
  if (bsl == 0) return false;
  out->nsl = bsl;
  out->gc = (chunks + bsl - 1) / bsl;
  out->tpg = bper;
  out->gt = (nt + bper - 1) / bper;
  return true;
}

ttc_status make_linear_plan(const tt_linear_desc* desc, int64_t T, LinearPlan* P) {
  if (!desc || !P) return TTC_ERR_NULL;
  memset(P, 0, sizeof(*P));
  const int p = desc->p, q = desc->q;
  if (p < 1 || q < 1 || p > TTC_MAX_HALF_MODES || q > TTC_MAX_HALF_MODES) return TTC_ERR_SHAPE;
  if (T < 0 || T > (int64_t(1) << 31) - 1) return TTC_ERR_SHAPE;
  if (desc->act_dtype != TTC_F32 && desc->act_dtype != TTC_BF16 && desc->act_dtype != TTC_FP8) return TTC_ERR_DTYPE;
  if (desc->in_first != 0 && desc->in_first != 1) return TTC_ERR_SHAPE;
  int in_first = desc->in_first;
  if (desc->path < TTC_PATH_AUTO || desc->path > TTC_PATH_DENSE) return TTC_ERR_UNSUPPORTED;
  if (desc->path == TTC_PATH_DENSE) return TTC_ERR_UNSUPPORTED;
  if (desc->flags & ~TTC_FLAG_PREPARED) return TTC_ERR_UNSUPPORTED;
  const int d = p + q;
  // chain position of each listed mode (output modes, then input modes)
  int pos_of[kMaxCores];
  {
    bool all_m1 = true, all_0 = true;
    for (int m = 0; m < d; ++m) {
      all_m1 = all_m1 && desc->chain_perm[m] == -1;
      all_0 = all_0 && desc->chain_perm[m] == 0;
    }
    if (all_m1 || all_0) {
      for (int m = 0; m < d; ++m) pos_of[m] = in_first ? (m < p ? q + m : m - p) : m;
    } else {
      bool seen[kMaxCores] = {};
      for (int m = 0; m < d; ++m) {
        const int k = desc->chain_perm[m];
        if (k < 0 || k >= d || seen[k]) return TTC_ERR_SHAPE;
        seen[k] = true;
        pos_of[m] = k;
      }
      // one link between the kinds: the output modes fill one end of the chain
      int lo = d;
      for (int m = 0; m < p; ++m) lo = std::min(lo, pos_of[m]);
      if (lo != 0 && lo != q) return TTC_ERR_UNSUPPORTED;
      for (int m = 0; m < p; ++m)
        if (pos_of[m] >= lo + p) return TTC_ERR_UNSUPPORTED;
      in_first = lo == q;
    }
  }
  P->p = p;
  P->q = q;
  P->d = d;
  P->in_first = in_first;
  P->act = desc->act_dtype;
  int64_t nout = 1, nin = 1;
  for (int k = 0; k < p; ++k) {
    if (desc->out_modes[k] < 1 || desc->out_modes[k] > 65536) return TTC_ERR_SHAPE;
    nout *= desc->out_modes[k];
  }
  for (int k = 0; k < q; ++k) {
    if (desc->in_modes[k] < 1 || desc->in_modes[k] > 65536) return TTC_ERR_SHAPE;
    nin *= desc->in_modes[k];
  }
  if (nout > (1 << 24) || nin > (1 << 24)) return TTC_ERR_SHAPE;
  P->N_out = nout;
  P->N_in = nin;
  for (int m = 0; m < d; ++m) {
    const int k = pos_of[m];
    P->is_in[k] = m >= p;
    P->lidx[k] = m < p ? m : m - p;
    P->modes[k] = m < p ? desc->out_modes[m] : desc->in_modes[m - p];
  }
  // strides of each position: in its kind's listed index, in its half's chain index
  {
    const int sp = in_first ? q : p;
    for (int k = 0; k < d; ++k) {
      const int* md = P->is_in[k] ? desc->in_modes : desc->out_modes;
      const int nk = P->is_in[k] ? q : p;
      int64_t ls = 1;
      for (int u = P->lidx[k] + 1; u < nk; ++u) ls *= md[u];
      int64_t cs = 1;
      for (int u = k + 1; u < (k < sp ? sp : d); ++u) cs *= P->modes[u];
      P->lstride[k] = (int)ls;
      P->cstride[k] = (int)cs;
    }
    P->perm_trivial = 1;
    for (int k = 0; k < d; ++k) P->perm_trivial &= P->lstride[k] == P->cstride[k];
  }
  if (desc->ranks[0] != 1 || desc->ranks[d] != 1) return TTC_ERR_RANK;
  for (int k = 0; k <= d; ++k) {
    if (desc->ranks[k] < 1 || desc->ranks[k] > TTC_MAX_RANK) return TTC_ERR_RANK;
    P->ranks[k] = desc->ranks[k];
  }
  P->s = in_first ? q : p;
  if (desc->split != -1 && desc->split != P->s) return TTC_ERR_UNSUPPORTED;
  P->rs = P->ranks[P->s];
  // rank tile: a multiple of 32 (the k-step of the rank-contracting products:
  // one MFMA k-step for bf16, two for fp32, and for e4m3 either one 32-wide
  // step on half fragments or whole 64-wide steps)
  const int rstep = 32;
  P->Rpad = ((P->rs + rstep - 1) / rstep) * rstep;
  P->NR = P->Rpad / 16;
  P->NL = in_first ? nin : nout;
  P->NRt = in_first ? nout : nin;
  P->T = T;
  P->es = desc->act_dtype == TTC_BF16 ? 2 : (desc->act_dtype == TTC_FP8 ? 1 : 4);
  // The streaming kernels address their operands through buffer resources of
  // at most 2^31 - 1 bytes with 32-bit offsets: the merged operands
  // (Rpad x N activation elements each) and a 64-token slab of any activation
  // must fit, or the call is refused instead of reading zeros past the range.
  if (!fits_rsrc(int64_t(P->Rpad) * nin * P->es) || !fits_rsrc(int64_t(P->Rpad) * nout * P->es) ||
      !fits_rsrc(int64_t(kTileT) * nin * P->es) || !fits_rsrc(int64_t(kTileT) * nout * P->es))
    return TTC_ERR_UNSUPPORTED;
  P->max_rank = 1;
  for (int k = 0; k <= d; ++k) P->max_rank = std::max(P->max_rank, P->ranks[k]);

  // chain area: M_k (rows prod_{j<=k} n_j, r_{k+1} cols) for k < s-1 and
  // N_k (r_k rows, prod_{j>=k} n_j cols) for k > s
  int64_t off = 0;
  for (int k = 0; k < d; ++k) P->chain_off[k] = -1;
  int64_t rows = 1;
  for (int k = 0; k < P->s - 1; ++k) {
    rows *= P->modes[k];
    P->chain_off[k] = off;
    off += rows * P->ranks[k + 1];
  }
  int64_t cols = 1;
  for (int k = d - 1; k > P->s; --k) {
    cols *= P->modes[k];
    P->chain_off[k] = off;
    off += cols * P->ranks[k];
  }
  P->chain_floats = off;
  if (off > 0x7fffffff) return TTC_ERR_UNSUPPORTED;  // offsets are 32-bit in the merge kernel
  // merge work items: one per row of every left prefix M_k (k < s) and one per
  // column of every right suffix N_k (k >= s)
  int64_t items = 0;
  rows = 1;
  for (int k = 0; k < P->s; ++k) {
    rows *= P->modes[k];
    P->item_off[k] = items;
    items += rows;
  }
  cols = 1;
  for (int k = d - 1; k >= P->s; --k) {
    cols *= P->modes[k];
    P->item_off[k] = items;
    items += cols;
  }
  P->item_off[d] = items;

  // ---- the sequential order's steps ---------------------------------------------------
  {
    const int* lidx = P->lidx;
    const int s = P->s;
    const bool in_left = in_first != 0;  // the input half is left of the split
    int order[kMaxCores], nst = 0;
    if (in_left)
      for (int k = 0; k < s; ++k) order[nst++] = k;
    else
      for (int k = d - 1; k >= s; --k) order[nst++] = k;
    if (in_left)
      for (int k = s; k < d; ++k) order[nst++] = k;
    else
      for (int k = s - 1; k >= 0; --k) order[nst++] = k;
    bool remaining[TTC_MAX_HALF_MODES], produced[TTC_MAX_HALF_MODES];
    for (int m = 0; m < TTC_MAX_HALF_MODES; ++m) {
      remaining[m] = m < q;
      produced[m] = false;
    }
    int64_t soff = 0, goff = 0, prev_size = nin;
    P->seq_max_state = std::max(nin, nout);
    P->seq_max_core = 0;
    for (int t = 0; t < d; ++t) {
      SeqStep& st = P->seq[t];
      const int k = order[t];
      // both halves are walked leftwards when the input half is on the
      // right (its chain end first, then the output half from the split to
      // its end) and rightwards otherwise
      const bool rightward = in_left;
      st.core = k;
      st.n = P->modes[k];
      st.rightward = rightward;
      st.rin = rightward ? P->ranks[k] : P->ranks[k + 1];
      st.rout = rightward ? P->ranks[k + 1] : P->ranks[k];
      st.expand = t >= q;
      // link between this core and the previous one of the walk (the split
      // link for the first output step); none at the input half's chain end
      st.dlink = t == 0 ? -1 : (rightward ? k - 1 : k);
      const int m = lidx[k];
      const int* md = st.expand ? desc->out_modes : desc->in_modes;
      bool* set = st.expand ? produced : remaining;
      int64_t A = 1, B = 1;
      for (int u = 0; u < (st.expand ? p : q); ++u) {
        if (!set[u] || u == m) continue;
        if (u < m) A *= md[u];
        else B *= md[u];
      }
      st.A = A;
      st.B = B;
      if (st.expand) produced[m] = true;
      else remaining[m] = false;
      st.in_size = prev_size;
      st.out_size = st.expand ? A * st.n * B * st.rout : A * B * st.rout;
      st.in_off = t == 0 ? -1 : soff - prev_size;
      st.out_off = t == d - 1 ? -1 : soff;
      if (t < d - 1) soff += st.out_size;
      prev_size = st.out_size;
      st.gp_off = goff;
      goff += (int64_t)st.rin * st.n * st.rout;
      P->seq_max_state = std::max(P->seq_max_state, st.out_size);
      P->seq_max_core = std::max<int64_t>(P->seq_max_core, (int64_t)st.rin * st.n * st.rout);
    }
    P->seq_state_floats = soff;
    P->seq_part_floats = goff;
    P->seq_lds_fwd = size_t(2 * P->seq_max_state + P->seq_max_core + TTC_MAX_RANK) * 4;
    P->seq_lds_bwd = size_t(3 * P->seq_max_state + P->seq_max_core + TTC_MAX_RANK) * 4;
    P->seq_ok = P->seq_lds_bwd <= kSeqMaxLds && T <= kSeqMaxTokens;
  }
  {
    double macs[4], bytes[4], usec[4];
    linear_path_costs(*P, macs, bytes);
    linear_path_times(*P, macs, bytes, usec);
    // the e4m3 merged kernels are built for rank tiles of 32 and 64
    const bool merged_ok = !(desc->act_dtype == TTC_FP8 && P->Rpad > 64);
    if (desc->path == TTC_PATH_SEQUENTIAL) {
      if (!P->seq_ok) return TTC_ERR_UNSUPPORTED;
      P->path = TTC_PATH_SEQUENTIAL;
    } else if (desc->path == TTC_PATH_MERGED) {
      if (!merged_ok) return TTC_ERR_UNSUPPORTED;
      P->path = TTC_PATH_MERGED;
    } else if (!merged_ok) {
      if (!P->seq_ok) return TTC_ERR_UNSUPPORTED;
      P->path = TTC_PATH_SEQUENTIAL;
    } else {
      P->path = (P->seq_ok && usec[2] < usec[1]) ? TTC_PATH_SEQUENTIAL : TTC_PATH_MERGED;
    }
  }

  // ---- launch shapes of the two backward streaming passes ---------------------
  P->ntiles = (int)((T + kTileT - 1) / kTileT);
  P->sw = slab_cols(P->es);
  BwdGrid gy, gx;
  plan_bwd_grid(*P, true, kPlanCUs, 0, 0, &gy);
  plan_bwd_grid(*P, false, kPlanCUs, 0, 0, &gx);
  P->dy_gc = gy.gc;
  P->dy_gt = gy.gt;
  P->dy_nsl = gy.nsl;
  P->dy_tpg = gy.tpg;
  P->dx_gc = gx.gc;
  P->dx_gt = gx.gt;
  P->dx_nsl = gx.nsl;
  P->dx_tpg = gx.tpg;

  // ---- saved layout -----------------------------------------------------------
  const size_t es = P->es;
  size_t o = 0;
  P->sv_meta = o;
  o = align256(o + kMetaBytes);
  P->sv_Ac = o;
  o = align256(o + size_t(P->Rpad) * nin * es);
  P->sv_AcT = o;
  o = align256(o + size_t(P->Rpad) * nin * es);
  P->sv_Bc = o;
  o = align256(o + size_t(P->Rpad) * nout * es);
  P->sv_BcT = o;
  o = align256(o + size_t(P->Rpad) * nout * es);
  P->sv_chain = o;
  o = align256(o + size_t(P->chain_floats) * 4);
  P->sv_Z = o;
  o = align256(o + size_t(T) * P->Rpad * es);
  P->sv_total = o;

  // ---- scratch layout -------------------------------------------------------------
  // ping-pong buffers for the gradients passed between levels of the sweep:
  // left dM_k for 1 <= k <= s-2, right dN_k for s+1 <= k <= d-2
  int64_t wl = 0, wr = 0;
  rows = 1;
  for (int k = 0; k < P->s - 1; ++k) {
    rows *= P->modes[k];
    if (k >= 1) wl = std::max(wl, rows * (int64_t)P->ranks[k + 1]);
  }
  cols = 1;
  for (int k = d - 1; k > P->s; --k) {
    cols *= P->modes[k];
    if (k <= d - 2) wr = std::max(wr, cols * (int64_t)P->ranks[k]);
  }
  P->wl_floats = wl;
  P->wr_floats = wr;
  o = 0;
  P->sc_gts = o;  // token groups the last data pass used: dY pass, dX pass (int32)
  o = align256(o + 2 * 4);
  P->sc_dZp = o;
  o = align256(o + (P->dy_gc > 1 ? size_t(P->dy_gc) * T * P->Rpad * 4 : 0));
  P->sc_dZ = o;
  o = align256(o + size_t(T) * P->Rpad * es);
  P->sc_dBp = o;
  o = align256(o + size_t(P->dy_gt) * P->Rpad * nout * 4);
  P->sc_dAp = o;
  o = align256(o + size_t(P->dx_gt) * P->Rpad * nin * 4);
  P->sc_dL = o;
  o = align256(o + size_t(P->NL) * P->rs * 4);
  P->sc_dR = o;
  o = align256(o + size_t(P->NRt) * P->rs * 4);
  P->sc_w0 = o;
  o = align256(o + size_t(wl + wr) * 4);
  P->sc_w1 = o;
  o = align256(o + size_t(wl + wr) * 4);
  P->sc_total = o;
  if (P->path == TTC_PATH_SEQUENTIAL) {
    // saved: every token's states between the steps; scratch: every token's
    // core-gradient partials
    P->sv_total = align256(size_t(T) * P->seq_state_floats * 4);
    P->sc_total = align256(size_t(T) * P->seq_part_floats * 4);
  }
  return TTC_OK;
}

// Multiply-adds and bytes of one forward+backward for T tokens.
//   [1] merged: merge both halves, x -> Z = x A^T -> Y = Z B^T; backward
//       dZ = dY B, dB = dY^T Z, dX = dZ A, dA = dZ^T x, then back through
//       each half's chain for the core gradients.
//   [2] sequential: contract x through one core at a time (input side, then
//       output side), every intermediate T x (modes) x r kept for backward.
//   [3] dense: W = B A, Y = x W^T, dX = dY W, dW = dY^T x, core gradients
//       from dW.
void linear_path_costs(const LinearPlan& P, double macs[4], double bytes[4]) {
  const double T = double(P.T);
  const double es = P.act == TTC_BF16 ? 2.0 : (P.act == TTC_FP8 ? 1.0 : 4.0);
  const int d = P.d, s = P.s;
  const double r = P.rs;
  // chain products of the two halves (prefix rows built left to right,
  // suffix columns right to left, each step a (rows x r) x (r x n r) product)
  double merge = 0.0;
  double rows = P.modes[0];
  for (int k = 1; k < s; ++k) {
    merge += rows * P.ranks[k] * double(P.modes[k]) * P.ranks[k + 1];
    rows *= P.modes[k];
  }
  double cols = P.modes[d - 1];
  for (int k = d - 2; k >= s; --k) {
    merge += cols * P.ranks[k + 1] * double(P.modes[k]) * P.ranks[k];
    cols *= P.modes[k];
  }
  double core_elems = 0.0;
  for (int k = 0; k < d; ++k) core_elems += double(P.ranks[k]) * P.modes[k] * P.ranks[k + 1];
  const double act_bytes = T * (3.0 * P.N_in + 2.0 * P.N_out) * es;
  macs[0] = -1.0;
  bytes[0] = -1.0;
  // merged: 3 skinny GEMM pairs plus merge and its reverse sweep (about 2x)
  macs[1] = 3.0 * T * r * double(P.N_in + P.N_out) + 3.0 * merge;
  bytes[1] = act_bytes + 2.0 * T * r * 4.0 + 2.0 * core_elems * 4.0;
  // sequential: the steps of the core-by-core order; each step costs
  // (state entries around its mode) x rin x rout per token; the backward
  // (input and core gradients) about twice the forward
  {
    double f = 0.0, inter = 0.0;
    for (int t = 0; t < d; ++t) {
      const SeqStep& st = P.seq[t];
      const double around = double(st.A) * st.n * double(st.B);
      f += T * around * st.rin * st.rout;
      if (t < d - 1) inter += T * double(st.out_size);
    }
    macs[2] = 3.0 * f;
    bytes[2] = act_bytes + 4.0 * 3.0 * inter + 2.0 * core_elems * 4.0;
  }
  // dense
  const double w = double(P.N_out) * double(P.N_in);
  macs[3] = 3.0 * T * w + 3.0 * w * r + 3.0 * merge;
  bytes[3] = act_bytes + 3.0 * w * 4.0 + 2.0 * core_elems * 4.0;
}

// Modelled time of one forward+backward.  At the sizes where the two orders
// compete (a few tokens) both are bound by latency, not by multiply-adds:
// the time is a count of dependent launches and in-kernel steps, each about
// one memory round trip plus its barrier, with the multiply-adds and bytes
// at the MI355X's fp32 MFMA and HBM rates on top.  Constants measured on one
// MI355X with the six config-2 layer shapes at 1 to 128 tokens:
//   a dependent launch of the merged order      ~7 us (six layers at one
//                                                 token: 158 us per step)
//   one step of the sequential kernels           ~14 us forward, ~23 us backward
//                                                 (86 and 136 us per six-core layer)
// so the sequential order, d dependent steps in each pass, is slower there
// even where it needs fewer multiply-adds (below ~10 tokens).
void linear_path_times(const LinearPlan& P, const double macs[4], const double bytes[4], double usec[4]) {
  constexpr double kLaunch = 7.0, kSeqFwdStep = 14.0, kSeqBwdStep = 23.0;
  constexpr double kMacPerUs = 157.3e6 / 2, kBytePerUs = 8.0e6;  // fp32 MFMA, HBM
  const int levels = std::max(P.s - 1, P.d - 1 - P.s);
  usec[0] = usec[3] = -1.0;
  // merge, forward, dY pass, dZ sum, dX pass, reduction, one launch per sweep level
  usec[1] = kLaunch * (6 + levels) + macs[1] / kMacPerUs + bytes[1] / kBytePerUs;
  // forward, backward and reduction launches; one token per work-group, so
  // more tokens than CUs add rounds of steps
  const double rounds = std::ceil(double(std::max<int64_t>(1, P.T)) / 256.0);
  usec[2] = P.seq_ok ? kLaunch * 3 + rounds * P.d * (kSeqFwdStep + kSeqBwdStep) + macs[2] / kMacPerUs +
                           bytes[2] / kBytePerUs
                     : -1.0;
}

}  // namespace ttc
