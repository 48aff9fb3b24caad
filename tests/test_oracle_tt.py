"""Pins for the fp64 TT-linear oracle, each independent of the oracle's own code.

* brute-force index sums over every rank index (the TT definition written as
  explicit nested sums);
* closed forms: all ranks 1 gives a Kronecker product; two cores give the
  textbook low-rank product G_1 diag(D) G_2;
* TT-SVD (Oseledets 2011) of a random dense W at full ranks rebuilds W;
* the loss <dY, x W^T> is linear in each core, so probing it with unit
  tensors gives every gradient entry exactly;
* a zero D entry is the same as deleting the matching slices of both
  neighbouring cores (project page, "Learn the ranks while training");
* a hand-worked two-core example under tests/golden/;
* a chain whose modes sit in any order (chain_perm): the brute-force sum
  with each listed digit placed at its chain position.
"""

import itertools
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_chain(rng, modes, ranks, zero_frac=0.0):
    cores = [rng.standard_normal((ranks[k], modes[k], ranks[k + 1])) for k in range(len(modes))]
    D = []
    for k in range(1, len(modes)):
        v = rng.uniform(0.5, 1.5, ranks[k])
        nz = int(np.floor(zero_frac * ranks[k]))
        v[rng.permutation(ranks[k])[:nz]] = 0.0
        D.append(v)
    return cores, D


def _digits(idx, modes):
    out = []
    for n in reversed(modes):
        out.append(idx % n)
        idx //= n
    return out[::-1]


def _brute_entry(cores, D, js):
    """Sum over every tuple of rank indices of the product of core entries and D."""
    d = len(cores)
    ranks = [c.shape[0] for c in cores] + [1]
    total = 0.0
    for a in itertools.product(*[range(r) for r in ranks[1:d]]):
        a = (0,) + a + (0,)
        term = 1.0
        for k in range(d):
            term *= cores[k][a[k], js[k], a[k + 1]]
            if k < d - 1:
                term *= D[k][a[k + 1]]
        total += term
    return total


def _brute_W(out_modes, in_modes, cores, D, in_first=False):
    n_out, n_in = int(np.prod(out_modes)), int(np.prod(in_modes))
    W = np.zeros((n_out, n_in))
    for i in range(n_out):
        for j in range(n_in):
            di, dj = _digits(i, out_modes), _digits(j, in_modes)
            js = dj + di if in_first else di + dj
            W[i, j] = _brute_entry(cores, D, js)
    return W


@pytest.mark.parametrize("in_first", [False, True])
def test_W_matches_brute_force(in_first):
    rng = np.random.default_rng(1)
    out_modes, in_modes = (2, 3), (3, 2)
    ranks = [1, 2, 3, 2, 1]
    modes = list(in_modes) + list(out_modes) if in_first else list(out_modes) + list(in_modes)
    cores, D = _rand_chain(rng, modes, ranks, zero_frac=0.34)
    W = oracle.dense_weight(out_modes, in_modes, cores, D, in_first)
    Wb = _brute_W(out_modes, in_modes, cores, D, in_first)
    assert np.max(np.abs(W - Wb)) <= 1e-13 * max(1.0, np.max(np.abs(Wb)))


def test_W_matches_brute_force_six_cores():
    rng = np.random.default_rng(2)
    out_modes, in_modes = (2, 3, 2), (3, 2, 2)
    ranks = [1, 2, 3, 4, 3, 2, 1]
    cores, D = _rand_chain(rng, list(out_modes) + list(in_modes), ranks, zero_frac=0.3)
    W = oracle.dense_weight(out_modes, in_modes, cores, D)
    Wb = _brute_W(out_modes, in_modes, cores, D)
    assert np.max(np.abs(W - Wb)) <= 1e-13 * max(1.0, np.max(np.abs(Wb)))


@pytest.mark.parametrize("in_first", [False, True])
def test_rank_one_is_kronecker(in_first):
    rng = np.random.default_rng(3)
    out_modes, in_modes = (3, 4, 2), (2, 5)
    modes = list(in_modes) + list(out_modes) if in_first else list(out_modes) + list(in_modes)
    vecs = [rng.standard_normal(n) for n in modes]
    cores = [v.reshape(1, -1, 1) for v in vecs]
    D = [np.array([s]) for s in rng.uniform(0.5, 1.5, len(modes) - 1)]
    scale = np.prod([v[0] for v in D])
    if in_first:
        kin = np.kron(vecs[0], vecs[1])
        kout = np.kron(np.kron(vecs[2], vecs[3]), vecs[4])
    else:
        kout = np.kron(np.kron(vecs[0], vecs[1]), vecs[2])
        kin = np.kron(vecs[3], vecs[4])
    want = np.outer(kout, kin) * scale
    W = oracle.dense_weight(out_modes, in_modes, cores, D, in_first)
    np.testing.assert_allclose(W, want, rtol=1e-14, atol=1e-14)


def test_two_cores_is_low_rank_product():
    rng = np.random.default_rng(4)
    n1, n2, r = 7, 5, 4
    G1 = rng.standard_normal((1, n1, r))
    G2 = rng.standard_normal((r, n2, 1))
    Dv = rng.uniform(0.5, 1.5, r)
    Dv[1] = 0.0
    want = G1[0] @ np.diag(Dv) @ G2[:, :, 0]
    W = oracle.dense_weight((n1,), (n2,), [G1, G2], [Dv])
    np.testing.assert_allclose(W, want, rtol=1e-14, atol=1e-14)


def test_tt_svd_full_rank_round_trip():
    rng = np.random.default_rng(5)
    out_modes, in_modes = (3, 4), (2, 5)
    W = rng.standard_normal((12, 10))
    cores = oracle.tt_svd(W, list(out_modes) + list(in_modes))
    D = [np.ones(c.shape[2]) for c in cores[:-1]]
    W2 = oracle.dense_weight(out_modes, in_modes, cores, D)
    assert np.max(np.abs(W2 - W)) <= 1e-12


def test_forward_and_input_grad_against_loops():
    rng = np.random.default_rng(6)
    out_modes, in_modes = (2, 3), (3, 2)
    cores, D = _rand_chain(rng, [2, 3, 3, 2], [1, 3, 2, 3, 1], zero_frac=0.34)
    Wb = _brute_W(out_modes, in_modes, cores, D)
    x = rng.standard_normal((5, 6))
    dy = rng.standard_normal((5, 6))
    Y = oracle.tt_linear_forward(x, out_modes, in_modes, cores, D)
    dX, _ = oracle.tt_linear_backward(x, dy, out_modes, in_modes, cores, D)
    Yb = np.zeros((5, 6))
    dXb = np.zeros((5, 6))
    for t in range(5):
        for i in range(6):
            for j in range(6):
                Yb[t, i] += x[t, j] * Wb[i, j]
                dXb[t, j] += dy[t, i] * Wb[i, j]
    np.testing.assert_allclose(Y, Yb, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dX, dXb, rtol=1e-13, atol=1e-13)
    # adjoint identity <dY, x W^T> = <dY W, x>
    assert abs(np.sum(dy * Y) - np.sum(dX * x)) <= 1e-12 * np.sum(np.abs(dy * Y))


def _loss(x, dy, out_modes, in_modes, cores, D, in_first=False):
    Wb = _brute_W(out_modes, in_modes, cores, D, in_first)
    return float(np.sum(dy * (x @ Wb.T)))


@pytest.mark.parametrize("in_first", [False, True])
def test_core_grads_by_unit_probes(in_first):
    """f(G) = <dY, x W(G)^T> is linear in each core: f(G_k = e_amb) = dG_k[a,m,b]."""
    rng = np.random.default_rng(7)
    out_modes, in_modes = (2, 3), (2, 2)
    modes = list(in_modes) + list(out_modes) if in_first else list(out_modes) + list(in_modes)
    ranks = [1, 2, 3, 2, 1]
    cores, D = _rand_chain(rng, modes, ranks, zero_frac=0.34)
    x = rng.standard_normal((4, 4))
    dy = rng.standard_normal((4, 6))
    _, dG = oracle.tt_linear_backward(x, dy, out_modes, in_modes, cores, D, in_first)
    for k in range(len(cores)):
        probe = np.zeros_like(cores[k])
        for idx in np.ndindex(*cores[k].shape):
            probe[...] = 0.0
            probe[idx] = 1.0
            trial = list(cores)
            trial[k] = probe
            want = _loss(x, dy, out_modes, in_modes, trial, D, in_first)
            assert abs(dG[k][idx] - want) <= 1e-12 * (1.0 + abs(want)), (k, idx)


def test_core_grads_finite_difference_random_direction():
    rng = np.random.default_rng(8)
    out_modes, in_modes = (3, 2, 2), (2, 3, 2)
    ranks = [1, 3, 4, 3, 4, 3, 1]
    cores, D = _rand_chain(rng, list(out_modes) + list(in_modes), ranks, zero_frac=0.25)
    x = rng.standard_normal((6, 12))
    dy = rng.standard_normal((6, 12))
    _, dG = oracle.tt_linear_backward(x, dy, out_modes, in_modes, cores, D)
    f0 = _loss(x, dy, out_modes, in_modes, cores, D)
    for k in range(len(cores)):
        E = rng.standard_normal(cores[k].shape)
        trial = list(cores)
        trial[k] = cores[k] + E
        df = _loss(x, dy, out_modes, in_modes, trial, D) - f0
        assert abs(df - np.sum(dG[k] * E)) <= 1e-10 * (1.0 + abs(df))


def test_zero_D_entry_equals_deleting_slices():
    rng = np.random.default_rng(9)
    out_modes, in_modes = (3, 4), (2, 5)
    ranks = [1, 4, 5, 3, 1]
    cores, D = _rand_chain(rng, [3, 4, 2, 5], ranks)
    link, b = 2, 3  # zero D_2[3]: drop slice 3 of G_2's last axis and G_3's first axis
    D[link - 1][b] = 0.0
    x = rng.standard_normal((7, 10))
    dy = rng.standard_normal((7, 12))
    W = oracle.dense_weight(out_modes, in_modes, cores, D)
    keep = [i for i in range(ranks[link]) if i != b]
    cores_s = list(cores)
    cores_s[link - 1] = cores[link - 1][:, :, keep]
    cores_s[link] = cores[link][keep, :, :]
    D_s = list(D)
    D_s[link - 1] = D[link - 1][keep]
    W_s = oracle.dense_weight(out_modes, in_modes, cores_s, D_s)
    assert np.max(np.abs(W - W_s)) <= 1e-15 * np.max(np.abs(W)) * 10
    _, dG = oracle.tt_linear_backward(x, dy, out_modes, in_modes, cores, D)
    assert np.all(dG[link - 1][:, :, b] == 0.0)
    assert np.all(dG[link][b, :, :] == 0.0)


def test_all_zero_link_removes_layer():
    rng = np.random.default_rng(10)
    out_modes, in_modes = (2, 3), (3, 2)
    cores, D = _rand_chain(rng, [2, 3, 3, 2], [1, 3, 3, 3, 1])
    D[1][:] = 0.0
    x = rng.standard_normal((4, 6))
    dy = rng.standard_normal((4, 6))
    Y = oracle.tt_linear_forward(x, out_modes, in_modes, cores, D)
    dX, dG = oracle.tt_linear_backward(x, dy, out_modes, in_modes, cores, D)
    assert np.all(Y == 0.0) and np.all(dX == 0.0)
    # cores adjacent to the dead link see an exactly-zero D factor in every term
    assert np.all(dG[1] == 0.0) and np.all(dG[2] == 0.0)


def test_hand_worked_golden():
    with open(os.path.join(GOLDEN, "tt_two_core_worked.json")) as f:
        g = json.load(f)
    cores = [np.array(c, dtype=np.float64) for c in g["cores"]]
    D = [np.array(v, dtype=np.float64) for v in g["D"]]
    x = np.array(g["x"], dtype=np.float64)
    dy = np.array(g["dy"], dtype=np.float64)
    W = oracle.dense_weight(g["out_modes"], g["in_modes"], cores, D)
    Y = oracle.tt_linear_forward(x, g["out_modes"], g["in_modes"], cores, D)
    dX, dG = oracle.tt_linear_backward(x, dy, g["out_modes"], g["in_modes"], cores, D)
    assert np.array_equal(W, np.array(g["W"]))
    assert np.array_equal(Y, np.array(g["Y"]))
    assert np.array_equal(dX, np.array(g["dX"]))
    for k in range(2):
        assert np.array_equal(dG[k], np.array(g["dG"][k]))


# ---- link diagonals: dL/dD_k and the early-stage objective ---------------------

@pytest.mark.parametrize("in_first", [False, True])
def test_link_grads_by_unit_probes(in_first):
    """f(D) = <dY, x W(G, D)^T> is linear in each diagonal: setting D_k to the
    unit vector e_b (the other diagonals fixed) gives dL/dD_k[b] exactly, for
    zero entries of D_k as well (the brute-force W is independent code)."""
    rng = np.random.default_rng(17)
    out_modes, in_modes = (2, 3), (3, 2)
    modes = list(in_modes) + list(out_modes) if in_first else list(out_modes) + list(in_modes)
    ranks = [1, 2, 4, 2, 1]
    cores, D = _rand_chain(rng, modes, ranks, zero_frac=0.34)
    x = rng.standard_normal((5, 6))
    dy = rng.standard_normal((5, 6))
    dD = oracle.tt_linear_link_grads(x, dy, cores, D, in_first)
    assert len(dD) == len(D)
    for k in range(len(D)):
        for b in range(len(D[k])):
            probe = [v.copy() for v in D]
            probe[k][:] = 0.0
            probe[k][b] = 1.0
            want = _loss(x, dy, out_modes, in_modes, cores, probe, in_first)
            assert abs(dD[k][b] - want) <= 1e-12 * (1.0 + abs(want)), (k, b)


def test_link_grads_finite_difference_and_core_identity():
    """Exact linear finite differences along a random direction, and the
    identity sum_{a,m} G_k[a,m,b] dG_k[a,m,b] = D_k[b] dL/dD_k[b]: the core
    gradient of core k carries D_k[b] as a factor of its slice b."""
    rng = np.random.default_rng(18)
    out_modes, in_modes = (3, 2, 2), (2, 3, 2)
    ranks = [1, 3, 4, 3, 4, 3, 1]
    cores, D = _rand_chain(rng, list(out_modes) + list(in_modes), ranks, zero_frac=0.25)
    x = rng.standard_normal((6, 12))
    dy = rng.standard_normal((6, 12))
    _, dG = oracle.tt_linear_backward(x, dy, out_modes, in_modes, cores, D)
    dD = oracle.tt_linear_link_grads(x, dy, cores, D)
    f0 = _loss(x, dy, out_modes, in_modes, cores, D)
    for k in range(len(D)):
        E = rng.standard_normal(D[k].shape)
        trial = [v.copy() for v in D]
        trial[k] = D[k] + E
        df = _loss(x, dy, out_modes, in_modes, cores, trial) - f0
        assert abs(df - np.sum(dD[k] * E)) <= 1e-10 * (1.0 + abs(df))
        lhs = np.einsum("amb,amb->b", cores[k], dG[k])
        assert np.allclose(lhs, D[k] * dD[k], rtol=1e-12, atol=1e-12 * np.abs(lhs).max())


def test_early_stage_grads_central_differences():
    """Gradients of J = L + gamma * sum_k |D_k|_1 + beta * sum_k ||G_k||^2 by
    central differences, which are exact here: L is linear in each core and
    diagonal, the penalty on the cores is quadratic, and the l1 term is linear
    as long as the step keeps every live entry's sign.  Dead entries (D = 0,
    pruned slices) report 0."""
    rng = np.random.default_rng(19)
    out_modes, in_modes = (2, 3), (3, 2)
    ranks = [1, 3, 2, 3, 1]
    cores, D = _rand_chain(rng, list(out_modes) + list(in_modes), ranks, zero_frac=0.34)
    x = rng.standard_normal((4, 6))
    dy = rng.standard_normal((4, 6))
    gamma, beta = 0.3, 0.05

    def J(cs, ds):
        return (_loss(x, dy, out_modes, in_modes, cs, ds) + gamma * sum(np.abs(v).sum() for v in ds)
                + beta * sum((c * c).sum() for c in cs))

    dG, dD = oracle.early_stage_grads(x, dy, cores, D, gamma, beta)
    h = 1e-3
    for k in range(len(cores)):
        E = rng.standard_normal(cores[k].shape)
        cp, cm = list(cores), list(cores)
        cp[k] = cores[k] + h * E
        cm[k] = cores[k] - h * E
        df = (J(cp, D) - J(cm, D)) / (2 * h)
        assert abs(df - np.sum(dG[k] * E)) <= 1e-8 * (1.0 + abs(df)), k
    for k in range(len(D)):
        live = D[k] != 0.0
        E = rng.standard_normal(D[k].shape) * live  # dead entries stay at 0
        dp, dm = [v.copy() for v in D], [v.copy() for v in D]
        dp[k] = D[k] + h * E
        dm[k] = D[k] - h * E
        df = (J(cores, dp) - J(cores, dm)) / (2 * h)
        assert abs(df - np.sum(dD[k] * E)) <= 1e-8 * (1.0 + abs(df)), k
        assert np.all(dD[k][~live] == 0.0)


# ---- modes in any chain order ----------------------------------------------------

def _brute_W_perm(out_modes, in_modes, cores, D, perm):
    """W[i, j]: the listed digits of (i, j), each put at its chain position."""
    p = len(out_modes)
    n_out, n_in = int(np.prod(out_modes)), int(np.prod(in_modes))
    W = np.zeros((n_out, n_in))
    for i in range(n_out):
        for j in range(n_in):
            listed = _digits(i, out_modes) + _digits(j, in_modes)
            js = [0] * len(perm)
            for m, k in enumerate(perm):
                js[k] = listed[m]
            W[i, j] = _brute_entry(cores, D, js)
    return W


PERMS = [
    # out (2,3) in (3,2): mirrored input block, output block first
    [0, 1, 3, 2],
    # input block first, both blocks permuted
    [3, 2, 1, 0],
    # interleaved (the weight is still defined; the GPU's orders need blocks)
    [0, 2, 1, 3],
]


@pytest.mark.parametrize("perm", PERMS)
def test_W_chain_perm_matches_brute_force(perm):
    rng = np.random.default_rng(11)
    out_modes, in_modes = (2, 3), (3, 2)
    listed = list(out_modes) + list(in_modes)
    modes = [0] * 4
    for m, k in enumerate(perm):
        modes[k] = listed[m]
    cores, D = _rand_chain(rng, modes, [1, 2, 3, 2, 1], zero_frac=0.34)
    W = oracle.dense_weight(out_modes, in_modes, cores, D, chain_perm=perm)
    Wb = _brute_W_perm(out_modes, in_modes, cores, D, perm)
    assert np.max(np.abs(W - Wb)) <= 1e-13 * max(1.0, np.max(np.abs(Wb)))


@pytest.mark.parametrize("in_first", [False, True])
def test_default_chain_perm_is_the_listed_order(in_first):
    rng = np.random.default_rng(12)
    out_modes, in_modes = (2, 3, 2), (3, 2)
    perm, modes = oracle.chain_layout(out_modes, in_modes, in_first)
    assert perm == ([2, 3, 4, 0, 1] if in_first else [0, 1, 2, 3, 4])
    cores, D = _rand_chain(rng, modes, [1, 2, 3, 2, 3, 1], zero_frac=0.3)
    W1 = oracle.dense_weight(out_modes, in_modes, cores, D, in_first)
    W2 = oracle.dense_weight(out_modes, in_modes, cores, D, chain_perm=perm)
    assert np.array_equal(W1, W2)
    np.testing.assert_allclose(W1, _brute_W(out_modes, in_modes, cores, D, in_first), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("perm", PERMS)
def test_core_and_link_grads_chain_perm_by_unit_probes(perm):
    """The loss is linear in each core and in each diagonal: unit probes give
    every gradient entry, for modes in any chain order."""
    rng = np.random.default_rng(13)
    out_modes, in_modes = (2, 3), (3, 2)
    listed = list(out_modes) + list(in_modes)
    modes = [0] * 4
    for m, k in enumerate(perm):
        modes[k] = listed[m]
    cores, D = _rand_chain(rng, modes, [1, 2, 3, 2, 1], zero_frac=0.0)
    x = rng.standard_normal((3, 6))
    dy = rng.standard_normal((3, 6))

    def loss(cs, Ds):
        return float(np.sum(dy * (x @ _brute_W_perm(out_modes, in_modes, cs, Ds, perm).T)))

    _, dG = oracle.tt_linear_backward(x, dy, out_modes, in_modes, cores, D, chain_perm=perm)
    for k in range(len(cores)):
        for idx in np.ndindex(*cores[k].shape):
            probe = np.zeros_like(cores[k])
            probe[idx] = 1.0
            trial = list(cores)
            trial[k] = probe
            want = loss(trial, D)
            assert abs(dG[k][idx] - want) <= 1e-12 * (1.0 + abs(want)), (k, idx)
    dD = oracle.tt_linear_link_grads(x, dy, cores, D, chain_perm=perm, out_modes=out_modes, in_modes=in_modes)
    for k in range(len(D)):
        for b in range(len(D[k])):
            probe = [v.copy() for v in D]
            probe[k][:] = 0.0
            probe[k][b] = 1.0
            want = loss(cores, probe)
            assert abs(dD[k][b] - want) <= 1e-12 * (1.0 + abs(want)), (k, b)
