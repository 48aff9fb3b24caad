"""Plain fp64 CPU oracle for the tensor-train (TT) linear layer and the
tensor-train-matrix (TTM) embedding lookup.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this package.  The GPU library never calls it
and shares no code with it: the two meet only in the seeded input generators of
``synth``, which hold none of the method's arithmetic.

Every function computes the plain mathematical definition of its result in
float64, with numpy primitives (``@``, ``einsum``, ``np.add.at``) as single
steps and no blocking or reordering of its own.  The definitions follow

* the CoMERA project page ("CoMERA: Computing- and Memory-Efficient Training
  via Rank-Adaptive Tensor Optimization", NeurIPS 2024), section
  "Learn the ranks while training": a weight matrix reshaped into a high-order
  tensor stored as a chain of cores linked by ranks; embedding tables in the
  related tensor-train-matrix format; a diagonal D on every link whose nonzero
  count is the link rank, a zero entry dropping the matching slice of both
  neighbouring cores;
* the same page, section "Making small tensor operations fast on GPUs": the
  deduplicated embedding lookup and the merged contraction order reach the
  plain result exactly (up to rounding order), so the oracle is that plain
  result;
* the NeurIPS 2024 poster summary page of CoMERA, figure caption on the TT and
  TTM tensor-network structures (cores G_k of shape r_{k-1} x n_k x r_k;
  TTM cores F_k with an extra mode m_k).

Every function is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py`` (brute-force index sums, Kronecker closed forms,
TT-SVD round trips, exact linear finite differences, slice-deletion
invariants).
"""

from .tt_linear import (  # noqa: F401
    chain_layout,
    chain_link_grads,
    early_stage_grads,
    tt_linear_link_grads,
    chain_tensor,
    chain_prefix,
    chain_suffix,
    dense_weight,
    tt_linear_forward,
    tt_linear_backward,
    tt_linear_core_grads,
    chain_core_grads,
)
from .ttm_embed import (  # noqa: F401
    ttm_table,
    ttm_forward,
    ttm_backward,
    decode_digits,
    sort_segments,
)
from .tt_svd import tt_svd  # noqa: F401
