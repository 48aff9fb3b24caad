"""fp64 oracle for the TT-linear layer with rank-control diagonals.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Notation (CoMERA project page, "Learn the ranks while training"; NeurIPS 2024
poster page, figure caption on the TT / TTM network structures):

* ``cores[k]`` is G_{k+1} with shape (r_k, n_{k+1}, r_{k+1}); r_0 = r_d = 1.
* ``D[k]`` is the diagonal on the link between ``cores[k]`` and ``cores[k+1]``
  (length r_{k+1}); there are d-1 of them, none at the chain ends.
* The full chain tensor T[j_1, ..., j_d] = G_1[0, j_1, :] D_1 G_2[:, j_2, :]
  ... D_{d-1} G_d[:, j_d, 0], flattened row-major (first mode most
  significant).
* A weight W (N_out x N_in) is that tensor reshaped: with the output modes
  first in the chain, W = T.reshape(N_out, N_in); with the input modes first,
  W = T.reshape(N_in, N_out)^T.  Y = x W^T (no bias).

Readings where the pages are silent: the order
of the modes in the chain is a parameter (``in_first``); index linearisation
is row-major mixed radix; D is a real-valued scale, not only a 0/1 mask.
"""

from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _check_chain(cores, D):
    d = len(cores)
    if d < 1:
        raise ValueError("a chain needs at least one core")
    if len(D) != d - 1:
        raise ValueError("a chain of d cores has d-1 link diagonals")
    if _f64(cores[0]).shape[0] != 1 or _f64(cores[-1]).shape[2] != 1:
        raise ValueError("boundary ranks must be 1")
    for k in range(d - 1):
        rk = _f64(cores[k]).shape[2]
        if _f64(cores[k + 1]).shape[0] != rk or _f64(D[k]).shape != (rk,):
            raise ValueError(f"rank mismatch on link {k + 1}")


def chain_prefix(cores, D, k: int) -> np.ndarray:
    """Product of the cores left of core ``k`` with their links' diagonals.

    Returns P of shape (prod(n_1..n_k), r_k): P = G_1 D_1 G_2 ... G_k D_k with
    the mode indices flattened row-major, i.e. the part of the chain product
    (project page, "Learn the ranks while training") to the left of G_{k+1}.
    For k = 0 it is the 1x1 identity.
    """
    M = np.ones((1, 1))
    for j in range(k):
        G = _f64(cores[j])
        r0, n, r1 = G.shape
        M = (M @ G.reshape(r0, n * r1)).reshape(-1, r1)
        M = M * _f64(D[j])[None, :]
    return M


def chain_suffix(cores, D, k: int) -> np.ndarray:
    """Product of the cores right of core ``k`` with their links' diagonals.

    Returns S of shape (r_{k+1}, prod(n_{k+2}..n_d)): S = D_{k+1} G_{k+2} ...
    D_{d-1} G_d, mode indices flattened row-major.  For the last core it is
    the 1x1 identity.
    """
    d = len(cores)
    M = np.ones((1, 1))
    for j in range(d - 1, k, -1):
        G = _f64(cores[j])
        r0, n, r1 = G.shape
        M = (G.reshape(r0 * n, r1) @ M).reshape(r0, -1)
        M = _f64(D[j - 1])[:, None] * M
    return M


def chain_tensor(cores, D) -> np.ndarray:
    """The full chain tensor, flattened row-major (length prod(n_k)).

    Definition of the TT format with a rank-control diagonal on every link
    (project page, "Learn the ranks while training", figure of the tensor-train
    layer with rank-control diagonals).
    """
    _check_chain(cores, D)
    d = len(cores)
    M = chain_prefix(cores, D, d - 1)          # (prod n_<d, r_{d-1})
    G = _f64(cores[d - 1])
    r0, n, _ = G.shape
    return (M @ G.reshape(r0, n)).reshape(-1)


def chain_layout(out_modes, in_modes, in_first: bool = False, chain_perm=None):
    """Where each mode sits in the chain.

    Modes are listed output modes first, then input modes (mode m < p is
    output mode m, mode p + j is input mode j).  ``chain_perm[m]`` is the
    chain position of mode m; without it the chain holds the output modes
    then the input modes in listed order, or the input modes first when
    ``in_first``.  Returns (perm, chain_modes) with chain_modes[k] the size of
    the mode at position k.  Any permutation is a valid chain order for the
    weight itself (the pages leave the order of the modes in the chain open).
    """
    p, q = len(out_modes), len(in_modes)
    listed = list(out_modes) + list(in_modes)
    if chain_perm is None:
        perm = [q + m for m in range(p)] + list(range(q)) if in_first else list(range(p + q))
    else:
        perm = [int(k) for k in chain_perm]
    if sorted(perm) != list(range(p + q)):
        raise ValueError(f"chain_perm {perm} is not a permutation of 0..{p + q - 1}")
    chain_modes = [0] * (p + q)
    for m, k in enumerate(perm):
        chain_modes[k] = int(listed[m])
    return perm, chain_modes


def dense_weight(out_modes, in_modes, cores, D, in_first: bool = False, chain_perm=None) -> np.ndarray:
    """Dense W (N_out x N_in) reconstructed from the cores in fp64: the chain
    tensor with its axes put in listed mode order (output modes, then input
    modes) and reshaped row-major."""
    n_out = int(np.prod(out_modes))
    n_in = int(np.prod(in_modes))
    perm, modes = chain_layout(out_modes, in_modes, in_first, chain_perm)
    got = [int(_f64(c).shape[1]) for c in cores]
    if got != modes:
        raise ValueError(f"core modes {got} do not match the chain {modes}")
    T = chain_tensor(cores, D).reshape(modes)
    return np.transpose(T, perm).reshape(n_out, n_in)


def _dW_to_chain(dW, out_modes, in_modes, in_first, chain_perm):
    """A gradient with respect to W, laid out as the chain tensor (flat)."""
    perm, _ = chain_layout(out_modes, in_modes, in_first, chain_perm)
    listed = list(out_modes) + list(in_modes)
    inv = [0] * len(perm)
    for m, k in enumerate(perm):
        inv[k] = m
    return np.transpose(_f64(dW).reshape(listed), inv).reshape(-1)


def chain_core_grads(dT, cores, D) -> list:
    """Gradient of <dT, T(G, D)> with respect to every core (D held fixed).

    T is linear in each core: T = P_k . G_k . S_k with P_k the prefix and S_k
    the suffix of core k, so
        dG_k[a, m, b] = sum_{alpha, beta} P_k[alpha, a] dT[alpha, m, beta] S_k[b, beta]
    where dT is viewed as (prod n_<k, n_k, prod n_>k).
    """
    _check_chain(cores, D)
    dT = _f64(dT).reshape(-1)
    d = len(cores)
    grads = []
    for k in range(d):
        G = _f64(cores[k])
        P = chain_prefix(cores, D, k)
        S = chain_suffix(cores, D, k)
        dTk = dT.reshape(P.shape[0], G.shape[1], S.shape[1])
        # one sum over alpha and beta; numpy picks the pairwise order
        # (P^T dT first, then S^T), which changes nothing but the rounding order
        grads.append(np.einsum("xa,xmy,by->amb", P, dTk, S, optimize=True))
    return grads


def tt_linear_forward(x, out_modes, in_modes, cores, D, in_first: bool = False, chain_perm=None) -> np.ndarray:
    """Y = x W^T for a batch of tokens x (T x N_in)."""
    W = dense_weight(out_modes, in_modes, cores, D, in_first, chain_perm)
    return _f64(x) @ W.T


def tt_linear_backward(x, dy, out_modes, in_modes, cores, D, in_first: bool = False, chain_perm=None):
    """Input gradient and core gradients of the TT-linear layer.

    dX = dY W, dW = dY^T x, and dG_k = d<dW, W>/dG_k, i.e. the gradient of
    <dY, x W^T> with respect to each core with D fixed.  Returns (dX, [dG_k]).
    """
    W = dense_weight(out_modes, in_modes, cores, D, in_first, chain_perm)
    dX = _f64(dy) @ W
    return dX, tt_linear_core_grads(x, dy, cores, D, in_first, chain_perm, out_modes, in_modes)


def _modes_of(cores, in_first, chain_perm, out_modes, in_modes):
    if out_modes is not None:
        return out_modes, in_modes
    if chain_perm is not None:
        raise ValueError("a chain_perm needs out_modes and in_modes")
    return None, None


def tt_linear_core_grads(x, dy, cores, D, in_first: bool = False, chain_perm=None, out_modes=None,
                         in_modes=None) -> list:
    """The core gradients alone: dW = dY^T x, then dG_k = d<dW, W>/dG_k."""
    dW = _f64(dy).T @ _f64(x)
    out_modes, in_modes = _modes_of(cores, in_first, chain_perm, out_modes, in_modes)
    if out_modes is None:
        dT = dW.T if in_first else dW           # back to the chain's own layout
        return chain_core_grads(dT.reshape(-1), cores, D)
    return chain_core_grads(_dW_to_chain(dW, out_modes, in_modes, in_first, chain_perm), cores, D)


def chain_link_grads(dT, cores, D) -> list:
    """Gradient of <dT, T(G, D)> with respect to every link diagonal D_k.

    T is linear in each diagonal: T = P_k' diag(D_k) S_k' with P_k' the chain
    product up to and including core k (its own left diagonals applied) and
    S_k' the product from core k+1 on (its own right diagonals applied), so
        dD_k[b] = sum_{alpha, beta} P_k'[alpha, b] dT[alpha, beta] S_k'[b, beta]
    with dT viewed as (prod n_<=k, prod n_>k).  This is the exact gradient for
    every entry, zero entries included.
    """
    _check_chain(cores, D)
    dT = _f64(dT).reshape(-1)
    d = len(cores)
    grads = []
    for k in range(d - 1):
        G = _f64(cores[k])
        r0, n, r1 = G.shape
        P = (chain_prefix(cores, D, k) @ G.reshape(r0, n * r1)).reshape(-1, r1)
        Gn = _f64(cores[k + 1])
        q0, m, q1 = Gn.shape
        S = (Gn.reshape(q0 * m, q1) @ chain_suffix(cores, D, k + 1)).reshape(q0, -1)
        dTk = dT.reshape(P.shape[0], S.shape[1])
        grads.append(np.einsum("xb,xy,by->b", P, dTk, S))
    return grads


def tt_linear_link_grads(x, dy, cores, D, in_first: bool = False, chain_perm=None, out_modes=None,
                         in_modes=None) -> list:
    """dL/dD_k for L = <dY, x W^T>: dW = dY^T x, then chain_link_grads."""
    dW = _f64(dy).T @ _f64(x)
    out_modes, in_modes = _modes_of(cores, in_first, chain_perm, out_modes, in_modes)
    if out_modes is None:
        dT = dW.T if in_first else dW
        return chain_link_grads(dT.reshape(-1), cores, D)
    return chain_link_grads(_dW_to_chain(dW, out_modes, in_modes, in_first, chain_perm), cores, D)


def early_stage_grads(x, dy, cores, D, gamma: float, beta: float, in_first: bool = False):
    """Gradients of the early-stage objective L + gamma * S^(D) + beta * ||G||^2
    (project page, section "Learn the ranks while training").

    Readings: S^(D) is the l1 norm of all link diagonals,
    sum_k |D_k|_1, and ||G||^2 the squared Frobenius norm of all cores.  An
    entry with D_k[b] == 0 is a pruned slice: its diagonal gradient is reported
    as 0 (the l1 subgradient at 0 is taken as 0 as well).  Returns
    (dG_k + 2 beta G_k for every core, dD_k for every link).
    """
    dG = tt_linear_core_grads(x, dy, cores, D, in_first)
    dD = tt_linear_link_grads(x, dy, cores, D, in_first)
    dG = [g + 2.0 * beta * _f64(c) for g, c in zip(dG, cores)]
    out = []
    for g, v in zip(dD, D):
        v = _f64(v)
        out.append(np.where(v != 0.0, g + gamma * np.sign(v), 0.0))
    return dG, out
