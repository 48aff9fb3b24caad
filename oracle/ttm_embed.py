"""fp64 oracle for the TT-matrix (TTM) embedding lookup and its backward.

TEST INFRASTRUCTURE ONLY (see the package docstring).

A TTM table with vocabulary modes (m_1..m_d) and embedding modes (n_1..n_d)
has cores F_k of shape (r_{k-1}, m_k, n_k, r_k), r_0 = r_d = 1 (NeurIPS 2024
poster page of CoMERA, figure caption on the TT and TTM structures; project
page, "Learn the ranks while training", for the TTM format of embedding
tables).  Entry

    E[(v_1..v_d), (c_1..c_d)] = F_1[0, v_1, c_1, :] D_1 F_2[:, v_2, c_2, :] ... F_d[:, v_d, c_d, 0]

with the row index v = (v_1 .. v_d) and the column index c = (c_1 .. c_d)
both row-major mixed radix, first mode most significant.  The optimised
lookup of the project page ("Making small tensor operations fast on GPUs",
embedding lookup without repeated work) returns exactly these rows, so the
oracle builds the whole table and gathers.

``D`` may be None: the identity on every link (no rank-control diagonal).
"""

from __future__ import annotations

import numpy as np

from .tt_linear import chain_core_grads, chain_tensor


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _as_tt(cores):
    """View each TTM core (r, m, n, r') as a TT core over the merged mode (m, n)."""
    out = []
    for F in cores:
        F = _f64(F)
        r0, m, n, r1 = F.shape
        out.append(F.reshape(r0, m * n, r1))
    return out


def _links(cores, D):
    if D is not None:
        return [_f64(v) for v in D]
    return [np.ones(_f64(F).shape[3]) for F in cores[:-1]]


def ttm_table(cores, D=None) -> np.ndarray:
    """The full table E (prod m_k x prod n_k) in fp64."""
    d = len(cores)
    ms = [int(_f64(F).shape[1]) for F in cores]
    ns = [int(_f64(F).shape[2]) for F in cores]
    T = chain_tensor(_as_tt(cores), _links(cores, D))
    inter = []
    for m, n in zip(ms, ns):
        inter += [m, n]
    T = T.reshape(inter)
    T = T.transpose([2 * k for k in range(d)] + [2 * k + 1 for k in range(d)])
    return T.reshape(int(np.prod(ms)), int(np.prod(ns)))


def ttm_forward(ids, cores, D=None) -> np.ndarray:
    """out[t] = E[ids[t]] for every token t."""
    E = ttm_table(cores, D)
    ids = np.asarray(ids, dtype=np.int64)
    if ids.size and (ids.min() < 0 or ids.max() >= E.shape[0]):
        raise ValueError("id out of range")
    return E[ids]


def ttm_backward(ids, dout, cores, D=None) -> list:
    """Core gradients of sum_t <dout[t], E[ids[t]]> (D fixed).

    dE is the scatter-add of the row gradients onto their table rows
    (``np.add.at``); each dF_k is the gradient of <dE, E> with respect to F_k,
    taken through the TT view of the table over merged (m_k, n_k) modes.
    """
    d = len(cores)
    ms = [int(_f64(F).shape[1]) for F in cores]
    ns = [int(_f64(F).shape[2]) for F in cores]
    dE = np.zeros((int(np.prod(ms)), int(np.prod(ns))))
    np.add.at(dE, np.asarray(ids, dtype=np.int64), _f64(dout))
    # back to the chain layout (m_1, n_1, m_2, n_2, ...)
    dT = dE.reshape(ms + ns)
    perm = []
    for k in range(d):
        perm += [k, d + k]
    dT = dT.transpose(perm).reshape(-1)
    grads = chain_core_grads(dT, _as_tt(cores), _links(cores, D))
    return [g.reshape(_f64(F).shape) for g, F in zip(grads, cores)]


def decode_digits(ids, vocab_modes) -> np.ndarray:
    """Mixed-radix digits of each id, first mode most significant.

    Returns an int64 array (len(ids), d) with ids = sum_k digit_k * prod(m_{>k}).
    Integer arithmetic only (div / mod), so the result is bit-exact.
    """
    ids = np.asarray(ids, dtype=np.int64)
    d = len(vocab_modes)
    out = np.zeros((ids.size, d), dtype=np.int64)
    rem = ids.copy()
    for k in range(d - 1, -1, -1):
        out[:, k] = rem % int(vocab_modes[k])
        rem //= int(vocab_modes[k])
    return out


def sort_segments(ids):
    """Sorted unique ids, the stable sorting permutation and segment offsets.

    Returns (uniques ascending, order, offsets, inverse) where ``order`` lists
    the token positions sorted by id (ties by position), ``offsets`` has
    len(uniques)+1 entries so that ids[order[offsets[u]:offsets[u+1]]] are all
    equal to uniques[u], and ``inverse[t]`` is the index of ids[t] in uniques.
    This is the deduplication step of the optimised lookup (project page,
    embedding lookup without repeated work: only unique rows are kept).
    """
    ids = np.asarray(ids, dtype=np.int64)
    order = np.argsort(ids, kind="stable")
    uniques, inverse, counts = np.unique(ids, return_inverse=True, return_counts=True)
    offsets = np.zeros(uniques.size + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    return uniques, order, offsets, inverse.reshape(-1)
