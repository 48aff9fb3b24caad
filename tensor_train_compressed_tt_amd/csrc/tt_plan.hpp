// Host-side plan of one TT-linear call: validated shapes, the split of the
// chain into its output-side and input-side halves, launch shapes and the
// byte layout of the caller's `saved` and `scratch` buffers.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/ttc.h"

namespace ttc {

constexpr int kMaxCores = 2 * TTC_MAX_HALF_MODES;
// most dynamic LDS the sequential kernels may use (one work-group per CU)
constexpr size_t kSeqMaxLds = 152 * 1024;
// most tokens of a sequential-path call (one work-group per token; meant for
// small batches, where it needs fewer multiply-adds than the merged order)
constexpr int64_t kSeqMaxTokens = 65536;
constexpr int kTileT = 64;  // tokens per tile of the streaming kernels

// Streaming kernels move 64-token x 256-byte slabs: 128 bf16 or 64 fp32 columns.
constexpr int slab_cols(int act_bytes) { return 256 / act_bytes; }
// Most 256-byte slabs one work-group of a backward pass keeps accumulators
// for: bounded so that the per-lane accumulators stay within 64 registers
// and the work-group's LDS within ~80 KB (two work-groups per CU).
constexpr int bwd_max_slabs(int act_bytes, int NR) {
  // one-byte activations: a 256-column slab already needs 4 column tiles per
  // wave, i.e. 64 accumulator registers at a rank tile of 64
  return act_bytes == 1 ? 1 : (2048 / (NR * act_bytes)) / slab_cols(act_bytes) < 1
             ? 1
             : ((2048 / (NR * act_bytes)) / slab_cols(act_bytes) > 8 ? 8
                                                                     : (2048 / (NR * act_bytes)) / slab_cols(act_bytes));
}
constexpr int dx_max_slabs(int act_bytes, int NR) {
  return bwd_max_slabs(act_bytes, NR) / 2 < 1 ? 1 : bwd_max_slabs(act_bytes, NR) / 2;
}

// One step of the core-by-core (sequential) contraction order: the input
// modes are contracted one core at a time from the input half's chain end
// towards the split, then the output modes are produced one core at a time
// from the split outwards.  A token's state before and after the step is a
// row-major array [A][n][B][rank] around the step's mode (the mode is absent
// from the contracted / not yet produced side).
struct SeqStep {
  int core;        // chain position of the core
  int n, rin, rout;
  int rightward;   // walk direction: element (x, i, y) of the core at
                   // (x n + i) rout + y when rightward, else (y n + i) rin + x
  int expand;      // 0: contracts an input mode, 1: produces an output mode
  int64_t A, B;
  int dlink;       // index of the link diagonal applied to the input state's rank, -1: none
  int64_t in_off, out_off;    // state offsets in a token's state area (floats), -1: x / y
  int64_t in_size, out_size;  // state sizes (floats)
  int64_t gp_off;  // offset of this core's gradient partial in a token's partial area (floats)
};

struct LinearPlan {
  // ---- shape, chain order -------------------------------------------------
  int p, q, d;
  int in_first;
  int act;                 // TTC_F32 / TTC_BF16
  int es;                  // bytes per activation element
  int modes[kMaxCores];    // n_k in chain order
  int ranks[kMaxCores + 1];
  int lidx[kMaxCores];     // listed index (within its kind) of the mode at each chain position
  int is_in[kMaxCores];    // the mode at each chain position is an input mode
  int lstride[kMaxCores];  // stride of that mode in the listed index of its kind
  int cstride[kMaxCores];  // stride of that position in its half's chain-order index
  int perm_trivial;        // each half's chain order is its kind's listed order
  int s;                   // cores in the left half of the chain
  int rs;                  // rank of the link between the halves
  int Rpad;                // rs rounded up to 32 (MFMA tile multiple)
  int NR;                  // Rpad / 16
  int64_t NL, NRt;         // prod of the left / right half's modes
  int64_t N_out, N_in;
  int64_t T;
  // prefix products M_k (k < s-1) and suffix products N_k (k > s), fp32,
  // offsets in floats inside the chain area of `saved`
  int64_t chain_off[kMaxCores];
  int64_t chain_floats;
  // merge work items: left rows of M_k (k < s) and right columns of N_k (k >= s)
  int64_t item_off[kMaxCores + 1];  // per core k: first item; item_off[d] = total
  int max_rank;
  // ---- launch shapes ---------------------------------------------------------
  int ntiles;              // ceil(T / kTileT)
  int sw;                  // slab width in elements
  int dy_gc, dy_gt, dy_nsl, dy_tpg;  // dY pass: column groups, token groups, slabs/group, tiles/group
  int dx_gc, dx_gt, dx_nsl, dx_tpg;  // dX pass
  // ---- path ------------------------------------------------------------------------
  int path;                // resolved: TTC_PATH_MERGED or TTC_PATH_SEQUENTIAL
  int seq_ok;              // the sequential path fits the device limits
  SeqStep seq[kMaxCores];  // d steps: q contractions, then p expansions
  int64_t seq_state_floats;  // per token: states 1 .. d-1
  int64_t seq_part_floats;   // per token: one gradient partial per core
  int64_t seq_max_state, seq_max_core;
  size_t seq_lds_fwd, seq_lds_bwd;  // dynamic LDS bytes of the two sequential kernels
  // ---- saved layout (bytes) ----------------------------------------------------
  size_t sv_meta, sv_Ac, sv_AcT, sv_Bc, sv_BcT, sv_chain, sv_Z, sv_total;
  // ---- scratch layout (bytes) ----------------------------------------------------
  size_t sc_gts, sc_dZp, sc_dZ, sc_dBp, sc_dAp, sc_dL, sc_dR, sc_w0, sc_w1, sc_total;
  int64_t wl_floats, wr_floats;  // size of one left / right ping-pong buffer
};

// saved meta block (int32 words)
constexpr int kMetaLive = 0;    // live[j]: link index of the j-th nonzero D entry, -1 past r_eff
constexpr int kMetaPos = 128;   // pos[b]: compact index of link entry b, -1 when D[b] == 0
constexpr int kMetaReff = 256;  // r_eff
constexpr size_t kMetaBytes = 1088;

ttc_status make_linear_plan(const tt_linear_desc* desc, int64_t T, LinearPlan* P);

// compute units the plan's own backward grids are shaped for
#ifndef TTC_BWD_CUS
#define TTC_BWD_CUS 256  // compute units of an MI355X
#endif
constexpr double kPlanCUs = TTC_BWD_CUS;
// the backward passes of a batched launch (long work-groups) shaped for two
// work-groups per CU
#ifndef TTC_BWD_TWO_PER_CU
#define TTC_BWD_TWO_PER_CU 1
#endif

// Launch shape of one backward streaming pass (dY pass when dy, else dX) for
// `ncu` compute units, with at most gc_max column groups and gt_max token
// groups (0: no limit).  False when no shape qualifies.  make_linear_plan
// takes it for all the CUs; a batched launch takes it for each layer's share.
struct BwdGrid {
  int gc, gt, nsl, tpg;
};
bool plan_bwd_grid(const LinearPlan& P, bool dy, double ncu, int gc_max, int gt_max, BwdGrid* out);



// multiply-adds and bytes of one forward+backward for each path (planner model)
void linear_path_costs(const LinearPlan& P, double macs[4], double bytes[4]);
// modelled time (microseconds) of one forward+backward per path on an
// MI355X, -1 where the path does not apply (see tt_plan.cpp)
void linear_path_times(const LinearPlan& P, const double macs[4], const double bytes[4], double usec[4]);

}  // namespace ttc
