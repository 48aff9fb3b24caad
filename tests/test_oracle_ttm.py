"""Pins for the fp64 TTM-embedding oracle, independent of the oracle's own code.

* all ranks 1: the table is the Kronecker product of the core slices, which
  fixes the digit order of the row index and the column index;
* brute-force index sums on a tiny table;
* the backward's scatter-add against an explicit per-token loop, and the core
  gradients by unit probes of the (linear) loss sum_t <dout[t], E[ids[t]]>;
* integer decoding and segmenting against plain Python loops (bit-exact).
"""

import itertools

import numpy as np
import pytest

import oracle


def _rand_ttm(rng, vocab, dims, ranks, with_D=True):
    cores = [rng.standard_normal((ranks[k], vocab[k], dims[k], ranks[k + 1])) for k in range(len(vocab))]
    D = None
    if with_D:
        D = []
        for k in range(1, len(vocab)):
            v = rng.uniform(0.5, 1.5, ranks[k])
            v[rng.integers(ranks[k])] = 0.0
            D.append(v)
    return cores, D


def _digits(idx, modes):
    out = []
    for n in reversed(modes):
        out.append(idx % n)
        idx //= n
    return out[::-1]


def _brute_table(cores, D, vocab, dims):
    d = len(cores)
    ranks = [c.shape[0] for c in cores] + [1]
    V, N = int(np.prod(vocab)), int(np.prod(dims))
    E = np.zeros((V, N))
    for v in range(V):
        dv = _digits(v, vocab)
        for c in range(N):
            dc = _digits(c, dims)
            total = 0.0
            for a in itertools.product(*[range(r) for r in ranks[1:d]]):
                a = (0,) + a + (0,)
                term = 1.0
                for k in range(d):
                    term *= cores[k][a[k], dv[k], dc[k], a[k + 1]]
                    if k < d - 1 and D is not None:
                        term *= D[k][a[k + 1]]
                total += term
            E[v, c] = total
    return E


def test_rank_one_table_is_kronecker():
    rng = np.random.default_rng(11)
    vocab, dims = (3, 4, 2), (2, 3, 2)
    mats = [rng.standard_normal((m, n)) for m, n in zip(vocab, dims)]
    cores = [M.reshape(1, M.shape[0], M.shape[1], 1) for M in mats]
    D = [np.array([1.25]), np.array([0.5])]
    want = np.kron(np.kron(mats[0], mats[1]), mats[2]) * 1.25 * 0.5
    E = oracle.ttm_table(cores, D)
    np.testing.assert_allclose(E, want, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("with_D", [False, True])
def test_table_matches_brute_force(with_D):
    rng = np.random.default_rng(12)
    vocab, dims, ranks = (2, 3, 2), (2, 2, 3), [1, 3, 2, 1]
    cores, D = _rand_ttm(rng, vocab, dims, ranks, with_D)
    E = oracle.ttm_table(cores, D)
    Eb = _brute_table(cores, D, vocab, dims)
    assert np.max(np.abs(E - Eb)) <= 1e-13 * max(1.0, np.max(np.abs(Eb)))


def test_forward_gathers_rows():
    rng = np.random.default_rng(13)
    vocab, dims, ranks = (2, 3, 2), (2, 2, 3), [1, 3, 2, 1]
    cores, D = _rand_ttm(rng, vocab, dims, ranks)
    Eb = _brute_table(cores, D, vocab, dims)
    ids = rng.integers(0, 12, 20)
    out = oracle.ttm_forward(ids, cores, D)
    for t in range(20):
        np.testing.assert_allclose(out[t], Eb[ids[t]], rtol=1e-13, atol=1e-13)
    with pytest.raises(ValueError):
        oracle.ttm_forward(np.array([12]), cores, D)


def _loss(ids, dout, cores, D, vocab, dims):
    Eb = _brute_table(cores, D, vocab, dims)
    total = 0.0
    for t in range(len(ids)):
        total += float(np.dot(dout[t], Eb[ids[t]]))
    return total


def test_backward_by_unit_probes():
    rng = np.random.default_rng(14)
    vocab, dims, ranks = (2, 3, 2), (2, 1, 2), [1, 2, 2, 1]
    cores, D = _rand_ttm(rng, vocab, dims, ranks)
    ids = np.array([0, 5, 5, 11, 3, 5, 0])
    dout = rng.standard_normal((7, 4))
    dF = oracle.ttm_backward(ids, dout, cores, D)
    for k in range(3):
        probe = np.zeros_like(cores[k])
        for idx in np.ndindex(*cores[k].shape):
            probe[...] = 0.0
            probe[idx] = 1.0
            trial = list(cores)
            trial[k] = probe
            want = _loss(ids, dout, trial, D, vocab, dims)
            assert abs(dF[k][idx] - want) <= 1e-12 * (1.0 + abs(want)), (k, idx)


def test_backward_finite_difference_random_direction():
    rng = np.random.default_rng(15)
    vocab, dims, ranks = (3, 2, 2), (2, 2, 2), [1, 3, 3, 1]
    cores, D = _rand_ttm(rng, vocab, dims, ranks)
    ids = rng.integers(0, 12, 30)
    dout = rng.standard_normal((30, 8))
    dF = oracle.ttm_backward(ids, dout, cores, D)
    f0 = _loss(ids, dout, cores, D, vocab, dims)
    for k in range(3):
        E = rng.standard_normal(cores[k].shape)
        trial = list(cores)
        trial[k] = cores[k] + E
        df = _loss(ids, dout, trial, D, vocab, dims) - f0
        assert abs(df - np.sum(dF[k] * E)) <= 1e-10 * (1.0 + abs(df))


def test_decode_digits_bit_exact():
    rng = np.random.default_rng(16)
    vocab = (32, 32, 32)
    ids = rng.integers(0, 32768, 500)
    got = oracle.decode_digits(ids, vocab)
    for t, v in enumerate(ids.tolist()):
        v1, rest = divmod(v, 32 * 32)
        v2, v3 = divmod(rest, 32)
        assert got[t].tolist() == [v1, v2, v3]


def test_sort_segments_bit_exact():
    rng = np.random.default_rng(17)
    ids = rng.integers(0, 40, 300)
    uniq, order, offsets, inverse = oracle.sort_segments(ids)
    want_uniq = sorted(set(ids.tolist()))
    assert uniq.tolist() == want_uniq
    want_order = [t for _, t in sorted((v, t) for t, v in enumerate(ids.tolist()))]
    assert order.tolist() == want_order
    pos = 0
    for u, v in enumerate(want_uniq):
        cnt = ids.tolist().count(v)
        assert offsets[u] == pos and offsets[u + 1] == pos + cnt
        pos += cnt
    assert [want_uniq[i] for i in inverse.tolist()] == ids.tolist()
