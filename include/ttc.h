/*
 * ttc.h - C ABI of the tensor-train compressed layer library (HIP, gfx950).
 *
 * The library computes the data-parallel hot path of rank-adaptive
 * tensor-compressed training as described for CoMERA ("CoMERA: Computing- and
 * Memory-Efficient Training via Rank-Adaptive Tensor Optimization", NeurIPS
 * 2024, project page):
 *
 *   - a linear layer whose weight W (N_out x N_in) is stored as a tensor train:
 *     cores G_k of shape (r_{k-1}, n_k, r_k), r_0 = r_d = 1, with a diagonal
 *     D_k on every link (section "Learn the ranks while training"); the
 *     forward Y = x W^T, the input gradient dX = dY W and the core gradients
 *     dG_k, evaluated in the contraction order of section "Making small tensor
 *     operations fast on GPUs" (multiply the output-side cores together and the
 *     input-side cores together, contract the input through them, keep the
 *     intermediate for the backward pass);
 *   - an embedding table in tensor-train-matrix (TTM) format, cores F_k of
 *     shape (r_{k-1}, m_k, n_k, r_k) (same section; NeurIPS poster page, figure
 *     on the TT and TTM structures), looked up for a batch of ids with
 *     deduplication and pairwise core contraction (section "Making small tensor
 *     operations fast on GPUs", embedding lookup without repeated work), and
 *     its backward into the core gradients.
 *
 * Conventions shared by every entry point
 *   - Every tensor argument is a DEVICE pointer to caller-owned, contiguous,
 *     row-major memory, unless the comment says "host".  The library never
 *     allocates or frees device memory in these calls and never synchronises
 *     the stream; all work is enqueued on `stream` (0 = the null stream), so
 *     the calls may be captured into a HIP graph.
 *   - Arrays of per-core pointers (G, D, dG, F, dF) are HOST arrays holding
 *     device pointers.
 *   - Row and column indices of W and of the TTM table are mixed-radix over
 *     their modes, first mode most significant.
 *   - The tensor train's chain lists the output modes first, then the input
 *     modes (in_first = 0), or the input modes first (in_first = 1); W is the
 *     chain tensor reshaped to (N_out, N_in), or the transpose of its
 *     (N_in, N_out) reshape.
 *   - D_k is a real-valued scale (fp32) on link k; an entry that is exactly 0
 *     removes the matching slice of both neighbouring cores, and the results
 *     are then exactly those of the smaller chain (dead-slice core gradients
 *     are exactly 0).  D is read on the device at every call.
 *   - Errors are returned synchronously, before anything is enqueued; on a
 *     non-zero status nothing was launched.  T = 0 is valid: the forward does
 *     nothing and the backward writes zero core gradients.
 */
#ifndef TTC_H
#define TTC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* ttc_stream_t; /* a hipStream_t */

typedef enum {
  TTC_OK = 0,
  TTC_ERR_NULL = 1,        /* a required pointer is NULL                         */
  TTC_ERR_SHAPE = 2,       /* mode counts / modes / T out of range                */
  TTC_ERR_RANK = 3,        /* ranks inconsistent (r_0, r_d != 1, r_k < 1)          */
  TTC_ERR_DTYPE = 4,       /* unknown dtype                                        */
  TTC_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned                     */
  TTC_ERR_WORKSPACE = 6,   /* saved / scratch buffer smaller than required         */
  TTC_ERR_UNSUPPORTED = 7, /* valid but not implemented (path, size limits)        */
  TTC_ERR_HIP = 8          /* a HIP runtime call failed                            */
} ttc_status;

/* Activation dtypes.  TTC_FP8 (FP8 mixed precision; CoMERA poster page,
 * tables and figures on FP8-mix products and FP8/FP32 training): x, y, dy, dx
 * stored as OCP e4m3 bytes (largest finite 448), every MFMA operand of the
 * merged order in e4m3 (the packed rank-side operands and the kept
 * intermediates too), fp32 accumulation, cores, D and dG in fp32; ranks up
 * to 64 on the merged order (the rank tile is padded to 64). */
typedef enum { TTC_F32 = 0, TTC_BF16 = 1, TTC_FP8 = 2 } ttc_dtype;

typedef enum {
  TTC_PATH_AUTO = 0,       /* planner picks                                        */
  TTC_PATH_MERGED = 1,     /* merge each half of the chain, two skinny GEMMs       */
  TTC_PATH_SEQUENTIAL = 2, /* core-by-core sweep, one work-group per token         */
  TTC_PATH_DENSE = 3       /* materialise W (costed by the planner only)           */
} ttc_path;

#define TTC_MAX_HALF_MODES 8 /* at most 8 output and 8 input modes */
#define TTC_MAX_RANK 128     /* every r_k <= 128 */

/* TT-linear layer descriptor (host memory). */
typedef struct {
  int32_t p;                              /* number of output modes, >= 1          */
  int32_t q;                              /* number of input modes, >= 1           */
  int32_t out_modes[TTC_MAX_HALF_MODES];  /* n of each output mode, >= 1           */
  int32_t in_modes[TTC_MAX_HALF_MODES];   /* n of each input mode, >= 1            */
  int32_t ranks[2 * TTC_MAX_HALF_MODES + 1]; /* r_0..r_{p+q} in chain order      */
  int32_t in_first;                       /* 0: chain = out modes, in modes; 1: in, out */
  int32_t act_dtype;                      /* ttc_dtype of x, y, dy, dx              */
  int32_t path;                           /* ttc_path                               */
  int32_t flags;                          /* TTC_FLAG_* bits, 0 by default          */
  /* Chain order of the modes.  Listing the modes as the p output modes, then
   * the q input modes (mode m < p is out_modes[m], mode p + j is in_modes[j]),
   * chain_perm[m] is the chain position (0 .. p+q-1) of mode m, i.e. core m'
   * with chain_perm[m] == m' carries that mode; the cores, ranks and diagonals
   * are given in chain order.  The row and column indices of W stay the
   * listed mixed-radix indices whatever the chain order.  All entries -1 (or
   * all 0) for the first p+q: the default order set by in_first, which is
   * then ignored otherwise.  The output modes must fill one end of the chain
   * and the input modes the other (any order inside each block), so that
   * one link joins the two kinds (TTC_ERR_UNSUPPORTED otherwise: the weight
   * is still defined, but neither contraction order here takes it);
   * TTC_ERR_SHAPE when the entries are not a permutation.  Example: the
   * mirrored layout whose end cores carry the largest modes (project page,
   * results, rank table of the compressed encoder: ranks (12,30,30,30,12) for
   * modes (12,8,8) x (12,8,8)) is out (12,8,8), in (12,8,8) with
   * chain_perm = {0,1,2,5,4,3}. */
  int32_t chain_perm[2 * TTC_MAX_HALF_MODES];
  /* The link at which the merged order cuts the chain into the two products
   * it multiplies out (project page, "Making small tensor operations fast on
   * GPUs"): -1 for the link between the output and the input modes, the only
   * link where each product holds modes of one kind, which the skinny
   * token products need; that link's index (s = number of modes in the first
   * block) is accepted too, any other value gives TTC_ERR_UNSUPPORTED. */
  int32_t split;
} tt_linear_desc;

/* tt_linear_fwd: `saved` already holds the merged halves written by
 * tt_linear_prepare for these cores and D; skip the merge. */
#define TTC_FLAG_PREPARED 1

/*
 * Bytes of the two caller-provided device buffers for T tokens.
 *   saved   - written by tt_linear_fwd, read by tt_linear_bwd: the merged halves
 *             of the chain and the T x r intermediate Z = x A^T kept from the
 *             forward pass.  Must outlive the fwd -> bwd pair, with the same
 *             cores, D and x.
 *   scratch - temporary space of one call (partial reductions).
 * Host-only; launches nothing.
 */
ttc_status tt_linear_workspace(const tt_linear_desc* desc, int64_t T,
                               size_t* saved_bytes, size_t* scratch_bytes);

/*
 * Forward: y = x W^T.
 *   x  - T x N_in  (act_dtype)
 *   G  - host array of p+q device pointers, core k is fp32 (r_{k-1}, n_k, r_k)
 *   D  - host array of p+q-1 device pointers, fp32 vectors of length r_k
 *   y  - T x N_out (act_dtype), overwritten
 *   saved / scratch - device buffers of at least tt_linear_workspace() bytes,
 *        16-byte aligned.
 * fp32 activations are computed with fp32 MFMA; bf16 activations with bf16
 * MFMA operands and fp32 accumulation (y rounded to nearest-even).
 */
ttc_status tt_linear_fwd(const tt_linear_desc* desc, int64_t T, const void* x,
                         const float* const* G, const float* const* D, void* y,
                         void* saved, size_t saved_bytes, void* scratch,
                         size_t scratch_bytes, ttc_stream_t stream);

/*
 * Merge step of the forward pass alone: multiplies each half of the chain
 * (with its link diagonals, the zero entries of the split link's diagonal
 * dropped) into `saved`.  It depends only on G and D, so it can run on a
 * stream of its own, ahead of the forward pass; tt_linear_fwd called with
 * desc->flags & TTC_FLAG_PREPARED then launches only the streaming kernel.
 * The caller orders the two (e.g. an event).  T sizes `saved` as for
 * tt_linear_workspace.
 */
ttc_status tt_linear_prepare(const tt_linear_desc* desc, int64_t T,
                             const float* const* G, const float* const* D,
                             void* saved, size_t saved_bytes,
                             ttc_stream_t stream);

/*
 * Backward: dX = dY W (skipped when dx == NULL) and dG_k = d<dY, x W^T>/dG_k.
 *   x, G, D, saved - exactly as passed to the matching tt_linear_fwd
 *   dy - T x N_out (act_dtype)
 *   dx - T x N_in  (act_dtype), overwritten, or NULL
 *   dG - host array of p+q device pointers, fp32, shapes of the cores,
 *        overwritten
 * Every reduction runs in a fixed order: results are bitwise reproducible.
 */
ttc_status tt_linear_bwd(const tt_linear_desc* desc, int64_t T, const void* x,
                         const void* dy, const float* const* G,
                         const float* const* D, const void* saved,
                         size_t saved_bytes, void* dx, float* const* dG,
                         void* scratch, size_t scratch_bytes,
                         ttc_stream_t stream);

/*
 * tt_linear_bwd with the core-gradient tail moved to a second stream.  The
 * passes over dY and x (which produce dX) run on `stream`; the reduction of
 * their partial sums and the reverse sweep through the chain (which produce
 * only dG) are enqueued on `grad_stream` behind an event recorded on `stream`,
 * so they overlap whatever the caller enqueues on `stream` next.  dX is
 * complete when `stream` passes the call, dG when `grad_stream` does; scratch
 * stays in use until then.  grad_stream == stream is exactly tt_linear_bwd.
 * Works under HIP graph capture (the event becomes a graph edge).
 */
ttc_status tt_linear_bwd_split(const tt_linear_desc* desc, int64_t T,
                               const void* x, const void* dy,
                               const float* const* G, const float* const* D,
                               const void* saved, size_t saved_bytes, void* dx,
                               float* const* dG, void* scratch,
                               size_t scratch_bytes, ttc_stream_t stream,
                               ttc_stream_t grad_stream);

/*
 * tt_linear_bwd for callers that cannot allocate device memory (code under
 * HIP graph capture that may not call hipMalloc, tight serving loops,
 * harnesses that forbid allocation): the same computation, bitwise the same
 * results, with the scratch buffer taken from a device array the library
 * holds in each GPU's memory from its load to the end of the process, of
 * TTC_NOALLOC_SCRATCH_BYTES bytes per GPU.  The caller still passes every
 * input and output.  A shape whose scratch (tt_linear_workspace) is larger
 * gives TTC_ERR_WORKSPACE before anything is enqueued; a failure to look the
 * array up on the current device gives TTC_ERR_HIP.  Calls on one GPU share
 * that array: two calls whose work overlaps on the device (different
 * streams, or one call's stream not ordered after the other's) race and give
 * wrong gradients; order them on one stream or with events.  This call itself
 * allocates nothing and enqueues no memset; its first call on a device looks
 * up the array's address (a host-side query, outside any stream).
 */
#define TTC_NOALLOC_SCRATCH_BYTES (64u << 20)
ttc_status tt_linear_bwd_noalloc(const tt_linear_desc* desc, int64_t T,
                                 const void* x, const void* dy,
                                 const float* const* G, const float* const* D,
                                 const void* saved, size_t saved_bytes,
                                 void* dx, float* const* dG,
                                 ttc_stream_t stream);

/*
 * The backward in two calls, for callers that schedule the core-gradient
 * work themselves (e.g. the tails of many layers together, after every
 * layer's dX is done).  The split follows the merged contraction order of the
 * project page (section "Making small tensor operations fast on GPUs"): the
 * passes over the T-sized activations, then the T-independent sweep back
 * through the two half products of the chain.
 *
 * tt_linear_bwd_data: the passes over dY and x on `stream`.  Writes dX
 *   (skipped when dx == NULL) and leaves the partial sums of the half-product
 *   gradients in `scratch`.  Arguments as for tt_linear_bwd.
 * tt_linear_bwd_cores: reduces those partial sums and sweeps back through
 *   the chain on `stream`; writes dG (fp32, shapes of the cores, overwritten).
 *   It must run after the tt_linear_bwd_data call with the same desc, T,
 *   saved and scratch has completed on the device (same stream, or an event);
 *   scratch must not be reused in between.  x and dy are not read.
 * Results are bitwise identical to tt_linear_bwd.  T == 0: bwd_data does
 * nothing, bwd_cores zeroes dG.  Errors are returned before any launch.
 */
ttc_status tt_linear_bwd_data(const tt_linear_desc* desc, int64_t T,
                              const void* x, const void* dy,
                              const float* const* G, const float* const* D,
                              const void* saved, size_t saved_bytes, void* dx,
                              void* scratch, size_t scratch_bytes,
                              ttc_stream_t stream);
ttc_status tt_linear_bwd_cores(const tt_linear_desc* desc, int64_t T,
                               const float* const* G, const float* const* D,
                               const void* saved, size_t saved_bytes,
                               float* const* dG, void* scratch,
                               size_t scratch_bytes, ttc_stream_t stream);

/*
 * Batched forms of tt_linear_prepare and tt_linear_bwd_cores for n layers
 * (arrays of n entries, entry i exactly the arguments of the single-layer
 * call).  Every layer's merge level (or sweep level) goes into one launch
 * with the other layers', so n layers cost about as many launches as one;
 * these T-independent steps are small and bound by launch latency.  Results
 * are bitwise those of the single-layer calls.  All arguments of all layers
 * are checked before anything is launched; n == 0 does nothing; n < 0 gives
 * TTC_ERR_SHAPE.  The layers must not share saved or scratch buffers.
 *   descs[i]  - descriptor of layer i
 *   T[i]      - tokens of layer i (sizes its buffers)
 *   G[i], D[i] - host arrays of layer i's core / diagonal device pointers
 *   dG[i]     - host array of layer i's core-gradient device pointers
 */
ttc_status tt_linear_prepare_batch(int32_t n, const tt_linear_desc* const* descs,
                                   const int64_t* T,
                                   const float* const* const* G,
                                   const float* const* const* D,
                                   void* const* saved, const size_t* saved_bytes,
                                   ttc_stream_t stream);
ttc_status tt_linear_bwd_cores_batch(int32_t n, const tt_linear_desc* const* descs,
                                     const int64_t* T,
                                     const float* const* const* G,
                                     const float* const* const* D,
                                     const void* const* saved,
                                     const size_t* saved_bytes,
                                     float* const* const* dG,
                                     void* const* scratch,
                                     const size_t* scratch_bytes,
                                     ttc_stream_t stream);

/*
 * Batched forms of tt_linear_fwd and tt_linear_bwd_data for n independent
 * layers (arrays of n entries, entry i exactly the arguments of the
 * single-layer call; dx may be NULL as a whole or per entry).  Layers that
 * share a kernel form (activation type, rank tile count, 16-byte rows and,
 * for the forward, the token tile) run in common launches of up to four
 * layers: each streaming pass then has one ramp-up and one tail for all of
 * them, which matters for passes of a few tens of MB such as the Q, K and V
 * projections of one encoder (project page, section "Making small tensor
 * operations fast on GPUs": many small contractions cost more than their
 * arithmetic).  The forward merges the cores of every layer whose descriptor
 * lacks TTC_FLAG_PREPARED (batched as tt_linear_prepare_batch).  Results are
 * bitwise those of the single-layer calls.  All arguments of all layers are
 * checked before anything is launched; n == 0 does nothing; n < 0 gives
 * TTC_ERR_SHAPE.  The layers must not share output, saved or scratch buffers.
 */
ttc_status tt_linear_fwd_batch(int32_t n, const tt_linear_desc* const* descs,
                               const int64_t* T, const void* const* x,
                               const float* const* const* G,
                               const float* const* const* D, void* const* y,
                               void* const* saved, const size_t* saved_bytes,
                               ttc_stream_t stream);
ttc_status tt_linear_bwd_data_batch(int32_t n, const tt_linear_desc* const* descs,
                                    const int64_t* T, const void* const* x,
                                    const void* const* dy,
                                    const float* const* const* G,
                                    const float* const* const* D,
                                    const void* const* saved,
                                    const size_t* saved_bytes, void* const* dx,
                                    void* const* scratch,
                                    const size_t* scratch_bytes,
                                    ttc_stream_t stream);

/*
 * Gradients of the early-stage objective of the project page (section "Learn
 * the ranks while training"): L(G, D) + gamma * S(D) + beta * ||G||^2, read as
 * S(D) = sum over the layer's links of |D_k|_1 (the l1 stand-in for the link
 * ranks) and ||G||^2 = sum_k ||G_k||_F^2.
 *   G, D - as for tt_linear_fwd (chain order)
 *   dG   - in: dL/dG_k as written by tt_linear_bwd / tt_linear_bwd_cores for
 *          these G and D; out: dL/dG_k + 2 beta G_k (in place)
 *   dD   - host array of d-1 device pointers, fp32 vectors of length r_k,
 *          overwritten: dL/dD_k[b] + gamma sign(D_k[b]); an entry with
 *          D_k[b] == 0 is a pruned slice and gets exactly 0
 * dL/dD_k[b] comes from dG_k: core k carries D_k[b] as a factor of its slice
 * b, so sum_{a,m} G_k[a,m,b] dG_k[a,m,b] = D_k[b] dL/dD_k[b].  One small
 * launch; fixed-order sums (bitwise reproducible).  Must run after the
 * backward that wrote dG has completed on the device (same stream, or an
 * event).  NaN gamma or beta gives TTC_ERR_SHAPE; errors are returned before
 * any launch.
 */
ttc_status tt_linear_rank_grads(const tt_linear_desc* desc, const float* const* G,
                                const float* const* D, float* const* dG,
                                float* const* dD, float gamma, float beta,
                                ttc_stream_t stream);
/* The same for n layers in one launch (arrays of n entries, entry i the
 * arguments of the single-layer call; same gamma and beta for all).  n == 0
 * does nothing, n < 0 gives TTC_ERR_SHAPE; every layer is checked first. */
ttc_status tt_linear_rank_grads_batch(int32_t n, const tt_linear_desc* const* descs,
                                      const float* const* const* G,
                                      const float* const* const* D,
                                      float* const* const* dG,
                                      float* const* const* dD, float gamma,
                                      float beta, ttc_stream_t stream);

/*
 * Planner report (host-only): writes a NUL-terminated text into buf (at most
 * n bytes) with the chosen path and the modelled flops / bytes of the merged,
 * sequential and dense paths for T tokens.
 */
ttc_status tt_linear_explain(const tt_linear_desc* desc, int64_t T, char* buf,
                             size_t n);

/* Modelled multiply-adds of one path for T tokens (forward + backward),
 * host-only; *out is set to -1 when the path does not apply. */
ttc_status tt_linear_path_cost(const tt_linear_desc* desc, int64_t T,
                               int32_t path, double* macs, double* bytes);

/* TTM embedding descriptor (host memory). */
#define TTC_TTM_MAX_MODES 8
#define TTC_TTM_MAX_IDS 16384 /* ids per call (the sort runs in one work-group) */
typedef struct {
  int32_t d;                              /* number of cores, 1..8                   */
  int32_t vocab_modes[TTC_TTM_MAX_MODES]; /* m_k; vocabulary = prod m_k < 2^31       */
  int32_t dim_modes[TTC_TTM_MAX_MODES];   /* n_k; embedding dim = prod n_k <= 2^24   */
  int32_t ranks[TTC_TTM_MAX_MODES + 1];   /* r_0..r_d, r_0 = r_d = 1, r_k <= 128     */
  int32_t accumulate;                     /* bwd: 1 = add into dF, 0 = overwrite     */
  int32_t mode;                           /* TTC_TTM_DEDUP (0), _UNIQUE or _PLAIN    */
} ttm_embed_desc;

/* Lookup modes (project page, section "Making small tensor operations fast on
 * GPUs", and its figure comparing lookup variants): DEDUP evaluates every
 * distinct id once and every distinct digit prefix once, shared by the ids
 * that carry it (the proposed lookup); UNIQUE evaluates every distinct id
 * once but shares no prefixes; PLAIN evaluates every token's row on its own.
 * All three give bitwise the same rows and, within rounding, the same core
 * gradients; they differ in work, in saved / scratch bytes (workspace query)
 * and in speed.  The mode must be the same for the workspace query, the
 * forward and the backward of one lookup.  Any other value: TTC_ERR_SHAPE. */
#define TTC_TTM_DEDUP 0
#define TTC_TTM_UNIQUE 1
#define TTC_TTM_PLAIN 2

/*
 * Bytes of the saved / scratch buffers for a lookup of T ids (host-only).
 * `saved` is written by ttm_embed_fwd and read by ttm_embed_bwd; `scratch`
 * is only used during a call.  TTC_ERR_UNSUPPORTED when T > TTC_TTM_MAX_IDS
 * or when one level's prefix product and core slice exceed 64 KB of LDS.
 *
 * The head of `saved` has a fixed layout, so that the integer results of the
 * deduplication can be read back (all int32; U = number of distinct valid
 * ids; Tv = number of valid ids):
 *   word 0            U
 *   word 1            1 if some id was outside [0, prod m_k), else 0
 *   word 2            number of pieces (private)
 *   word 3            Tv
 *   words 4 .. 4+d    number of distinct digit prefixes (v_1..v_l), l = 1..d
 *   at byte 128                 order[T]: token positions sorted by (id, position);
 *                               the Tv valid ones first
 *   at byte 128 + A             inverse[T]: index of each token's id in the
 *                               distinct list, -1 for an invalid id
 *   at byte 128 + 2A            uids[T]: the distinct valid ids, ascending (U used)
 *   at byte 128 + 3A            seg[T+1]: segment offsets into order (U+1 used)
 * where A = 4*T rounded up to a multiple of 256.  The rest is private.
 */
ttc_status ttm_embed_workspace(const ttm_embed_desc* desc, int64_t T,
                               size_t* saved_bytes, size_t* scratch_bytes);

/*
 * Forward lookup: out[t] = E[ids[t]] for t < T, where
 *   E[(v_1..v_d), (c_1..c_d)] = F_1[0,v_1,c_1,:] D_1 F_2[:,v_2,c_2,:] ... F_d[:,v_d,c_d,0]
 * (NeurIPS 2024 poster page of CoMERA, figure on the TT and TTM structures).
 * Each distinct id is evaluated once and each distinct digit prefix once
 * (project page, "Making small tensor operations fast on GPUs", embedding
 * lookup without repeated work); repeated ids get bitwise-identical rows.
 *   ids - T int64 ids; an id outside [0, prod m_k) gives a zero row and sets
 *         word 1 of `saved`
 *   F   - host array of d device pointers, fp32 cores (r_{k-1}, m_k, n_k, r_k)
 *   D   - host array of d-1 device pointers (fp32 length r_k), or NULL for the
 *         identity on every link
 *   out - T x prod n_k fp32, overwritten
 * out, saved and scratch must be 16-byte aligned (TTC_ERR_ALIGN).
 */
ttc_status ttm_embed_fwd(const ttm_embed_desc* desc, int64_t T,
                         const int64_t* ids, const float* const* F,
                         const float* const* D, float* out, void* saved,
                         size_t saved_bytes, void* scratch, size_t scratch_bytes,
                         ttc_stream_t stream);

/*
 * The forward in two calls, for callers that build the index of a batch
 * ahead of its lookup (e.g. the next batch's ids beside the current step's
 * work, since the index depends on the ids only).  The split follows the
 * lookup of the project page (section "Making small tensor operations fast on
 * GPUs"): first find the distinct ids and shared digit prefixes, then
 * contract the cores once per distinct prefix and assemble the rows.
 * ttm_embed_index: sort, distinct ids, segments and the per-level prefix
 *   tree into `saved` (the head documented above and the private index
 *   arrays).  Reads only ids.
 * ttm_embed_lookup: from an index built in `saved` for the same desc and T,
 *   the prefix products (into the rest of `saved`) and out.  The index stays
 *   valid, so the same saved then serves ttm_embed_bwd.
 * ttm_embed_fwd is exactly index then lookup.  The caller orders the two
 * (same stream or an event); two batches in flight need two saved buffers.
 * Errors are returned before any launch.
 */
ttc_status ttm_embed_index(const ttm_embed_desc* desc, int64_t T,
                           const int64_t* ids, void* saved, size_t saved_bytes,
                           ttc_stream_t stream);
ttc_status ttm_embed_lookup(const ttm_embed_desc* desc, int64_t T,
                            const float* const* F, const float* const* D,
                            float* out, void* saved, size_t saved_bytes,
                            void* scratch, size_t scratch_bytes,
                            ttc_stream_t stream);

/*
 * Backward: dF_k = d( sum_t <dout[t], E[ids[t]]> ) / dF_k, D held fixed.
 * The output gradients of equal ids are summed along their sorted segment
 * (no floating-point atomics; the result is bitwise reproducible).
 *   ids  - not read (the sorted structure comes from `saved`); may be NULL
 *   F, D, saved - as passed to the matching ttm_embed_fwd; saved unchanged
 *   dout - T x prod n_k fp32, 16-byte aligned
 *   dF   - host array of d device pointers, fp32, shapes of the cores;
 *          overwritten, or added to when desc->accumulate
 * Invalid ids contribute nothing.  T = 0 zeroes dF (unless accumulate).
 */
ttc_status ttm_embed_bwd(const ttm_embed_desc* desc, int64_t T,
                         const int64_t* ids, const float* dout,
                         const float* const* F, const float* const* D,
                         const void* saved, size_t saved_bytes,
                         float* const* dF, void* scratch, size_t scratch_bytes,
                         ttc_stream_t stream);

/*
 * Device-side error of a TTM lookup, for tests and diagnostics: waits for
 * `stream` (a host synchronisation: not for use under graph capture), then
 * sets *code to the flag the lookup keeps in word 1 of its `saved` buffer:
 * 1 if some id of the batch was outside [0, prod m_k) (such ids give zero
 * rows and no gradient), 0 otherwise.  `saved` is the buffer passed to
 * ttm_embed_fwd / ttm_embed_index.  The TT-linear entry points check every
 * argument on the host before enqueuing anything, so they have no
 * device-side error to report.  TTC_ERR_NULL for a NULL pointer,
 * TTC_ERR_HIP if the copy or the wait fails.
 */
ttc_status ttc_device_error(const void* saved, ttc_stream_t stream, int32_t* code);

/* Human-readable name of a status code (static storage). */
const char* ttc_status_str(ttc_status s);

/* Library version string (static storage). */
const char* ttc_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TTC_H */
