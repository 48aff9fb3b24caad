"""TT-SVD: sequential truncated SVDs that turn a dense tensor into TT cores.

TEST INFRASTRUCTURE ONLY (see the package docstring).

This is the textbook decomposition (I. V. Oseledets, "Tensor-Train
Decomposition", SIAM J. Sci. Comput. 33(5), 2011, algorithm TT-SVD), used to
pin the chain reconstruction: decomposing a random dense tensor at full ranks
and rebuilding it with the oracle must return the tensor.  It does not appear
on the CoMERA pages, which start from cores (project page, "Learn the ranks
while training"); it is an independent check, not part of the method.
"""

from __future__ import annotations

import numpy as np


def tt_svd(A, modes, max_rank: int | None = None, rtol: float = 0.0) -> list:
    """Cores G_k (r_{k-1}, n_k, r_k) whose chain product is ``A`` (row-major).

    Each unfolding C (r_{k-1} n_k x rest) is split by an SVD C = U S V^T;
    U's leading columns become core k and S V^T carries on to the next mode.
    Singular values below ``rtol`` times the largest, and any beyond
    ``max_rank``, are dropped.
    """
    modes = [int(n) for n in modes]
    C = np.asarray(A, dtype=np.float64).reshape(-1)
    if C.size != int(np.prod(modes)):
        raise ValueError("size of A does not match the modes")
    cores = []
    r_prev = 1
    for n in modes[:-1]:
        C = C.reshape(r_prev * n, -1)
        U, S, Vt = np.linalg.svd(C, full_matrices=False)
        keep = int(np.sum(S > rtol * (S[0] if S.size else 0.0))) if rtol > 0 else S.size
        if max_rank is not None:
            keep = min(keep, int(max_rank))
        keep = max(keep, 1)
        cores.append(U[:, :keep].reshape(r_prev, n, keep))
        C = S[:keep, None] * Vt[:keep]
        r_prev = keep
    cores.append(C.reshape(r_prev, modes[-1], 1))
    return cores
