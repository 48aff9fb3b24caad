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

ttc_status make_linear_plan(const tt_linear_desc* desc, int64_t T, LinearPlan* P) {
  if (!desc || !P) return TTC_ERR_NULL;
  memset(P, 0, sizeof(*P));
  const int p = desc->p, q = desc->q;
  if (p < 1 || q < 1 || p > TTC_MAX_HALF_MODES || q > TTC_MAX_HALF_MODES) return TTC_ERR_SHAPE;
  if (T < 0 || T > (int64_t(1) << 31) - 1) return TTC_ERR_SHAPE;
  if (desc->act_dtype != TTC_F32 && desc->act_dtype != TTC_BF16) return TTC_ERR_DTYPE;
  if (desc->in_first != 0 && desc->in_first != 1) return TTC_ERR_SHAPE;
  if (desc->path < TTC_PATH_AUTO || desc->path > TTC_PATH_DENSE) return TTC_ERR_UNSUPPORTED;
  if (desc->path == TTC_PATH_SEQUENTIAL || desc->path == TTC_PATH_DENSE) return TTC_ERR_UNSUPPORTED;
  if (desc->flags & ~TTC_FLAG_PREPARED) return TTC_ERR_UNSUPPORTED;
  const int d = p + q;
  P->p = p;
  P->q = q;
  P->d = d;
  P->in_first = desc->in_first;
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
  for (int k = 0; k < d; ++k) {
    if (!desc->in_first)
      P->modes[k] = k < p ? desc->out_modes[k] : desc->in_modes[k - p];
    else
      P->modes[k] = k < q ? desc->in_modes[k] : desc->out_modes[k - q];
  }
  if (desc->ranks[0] != 1 || desc->ranks[d] != 1) return TTC_ERR_RANK;
  for (int k = 0; k <= d; ++k) {
    if (desc->ranks[k] < 1 || desc->ranks[k] > TTC_MAX_RANK) return TTC_ERR_RANK;
    P->ranks[k] = desc->ranks[k];
  }
  P->s = desc->in_first ? q : p;
  P->rs = P->ranks[P->s];
  P->Rpad = ((P->rs + 31) / 32) * 32;
  P->NR = P->Rpad / 16;
  P->NL = desc->in_first ? nin : nout;
  P->NRt = desc->in_first ? nout : nin;
  P->T = T;
  P->es = desc->act_dtype == TTC_BF16 ? 2 : 4;
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

  // ---- launch shapes of the two backward streaming passes ---------------------
  // A work-group owns a range of columns (whole 256-byte slabs) and a range of
  // token tiles.  Splitting the columns of the dY pass costs partial sums of
  // the T x r intermediate dZ (and the dX pass re-reads dZ once per column
  // group); splitting the tokens costs partial sums of the r x N weight-side
  // gradients.  The passes are bound by each CU's share of the memory
  // traffic, so the time of a shape is the bytes of the busiest CU: the
  // work-groups per CU (rounded up) times the bytes of one work-group.  The
  // partials that the reductions read back later run beside the streaming
  // passes and weigh half.
  P->ntiles = (int)((T + kTileT - 1) / kTileT);
  const int nt = std::max(1, P->ntiles);
  P->sw = slab_cols(P->es);
#ifndef TTC_BWD_CUS
#define TTC_BWD_CUS 256  // compute units of an MI355X
#endif
  const double ncu = TTC_BWD_CUS;
#ifndef TTC_LATER_WEIGHT
#define TTC_LATER_WEIGHT 0.5
#endif
  const double kLaterWeight = TTC_LATER_WEIGHT;
  auto choose = [&](int64_t ncols, int maxs, bool dy, int* gc, int* gt, int* nsl, int* tpg) {
    const int chunks = (int)std::max<int64_t>(1, (ncols + P->sw - 1) / P->sw);
    const int gc_min = (chunks + maxs - 1) / maxs;
    double best = 1e300;
    int bsl = (chunks + gc_min - 1) / gc_min, bper = 1;
    for (int g = gc_min; g <= chunks; ++g) {
      const int sl = (chunks + g - 1) / g;
      if ((chunks + sl - 1) / sl != g) continue;  // same shape as a smaller g
      for (int per = 1; per <= nt; ++per) {
        const int tg = (nt + per - 1) / per;
        if ((nt + tg - 1) / tg != per) continue;
        // a work-group's token range of the streamed activation, of its rank
        // tile and of the fp32 dZ partials are each one buffer resource
        const int64_t toks64 = int64_t(per) * kTileT;
        if (!fits_rsrc(toks64 * ncols * P->es) || !fits_rsrc(toks64 * P->Rpad * 4)) break;
        const double cols = double(sl) * P->sw, toks = double(per) * kTileT;
        double wg = toks * cols * P->es * (dy ? 1.0 : 2.0);  // streamed activations
        wg += 4.0 * P->rs * cols;                             // weight-side partial
        if (dy)
          wg += (g > 1 ? 4.0 : 0.0) * toks * P->Rpad + toks * P->Rpad * P->es;  // dZ partial, Z tile
        else
          wg += toks * P->Rpad * P->es;  // dZ tile
        const double later = 4.0 * tg * P->rs * double(ncols) + (dy && g > 1 ? 4.0 * g * double(T) * P->Rpad : 0.0);
        const double cost = std::ceil(double(g) * tg / ncu) * wg + kLaterWeight * later / ncu;
        if (cost < best * (1 - 1e-9)) {
          best = cost;
          bsl = sl;
          bper = per;
        }
      }
    }
    *nsl = bsl;
    *gc = (chunks + bsl - 1) / bsl;
    *tpg = bper;
    *gt = (nt + bper - 1) / bper;
  };
  choose(nout, bwd_max_slabs(P->es, P->NR), true, &P->dy_gc, &P->dy_gt, &P->dy_nsl, &P->dy_tpg);
  choose(nin, dx_max_slabs(P->es, P->NR), false, &P->dx_gc, &P->dx_gt, &P->dx_nsl, &P->dx_tpg);

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
  const double es = P.act == TTC_BF16 ? 2.0 : 4.0;
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
  // sequential: sweep the input-side cores from the far end of the chain
  // towards the split over x, then the output-side cores from the split
  // outwards; forward cost f, backward about 2 f
  {
    const int p = P.p, q = P.q;
    int in_pos[kMaxCores], out_pos[kMaxCores];
    for (int k = 0; k < q; ++k) in_pos[k] = P.in_first ? k : d - 1 - k;   // far end first
    for (int k = 0; k < p; ++k) out_pos[k] = P.in_first ? q + k : p - 1 - k;  // split first
    double f = 0.0, inter = 0.0;
    double lead = double(P.N_in);
    for (int k = 0; k < q; ++k) {
      const int c = in_pos[k];
      const double far = P.in_first ? P.ranks[c] : P.ranks[c + 1];
      const double near = P.in_first ? P.ranks[c + 1] : P.ranks[c];
      f += T * lead * far * near;  // lead still includes this core's mode
      lead /= P.modes[c];
      inter += T * lead * near;
    }
    double trail = 1.0;
    for (int k = 0; k < p; ++k) {
      const int c = out_pos[k];
      const double near = P.in_first ? P.ranks[c] : P.ranks[c + 1];
      const double far = P.in_first ? P.ranks[c + 1] : P.ranks[c];
      trail *= P.modes[c];
      f += T * trail * near * far;
      inter += T * trail * far;
    }
    macs[2] = 3.0 * f;
    bytes[2] = act_bytes + 4.0 * 3.0 * inter + 2.0 * core_elems * 4.0;
  }
  // dense
  const double w = double(P.N_out) * double(P.N_in);
  macs[3] = 3.0 * T * w + 3.0 * w * r + 3.0 * merge;
  bytes[3] = act_bytes + 3.0 * w * 4.0 + 2.0 * core_elems * 4.0;
}

}  // namespace ttc
