"""Host-only checks of the C ABI: the library loads, exports every symbol the
header declares, validates descriptors and sizes buffers, and its planner's
cost model agrees with an independent operation count.  No GPU needed: none
of these calls launches work."""

import ctypes
import os
import re

import pytest

import tensor_train_compressed_tt_amd as ttc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = "".join(open(os.path.join(ROOT, "include", h)).read() for h in sorted(os.listdir(os.path.join(ROOT, "include"))))
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(?:ttc_status|const char\s*\*)\s+(\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = ttc.lib()
    names = _header_functions()
    assert set(names) == set(ttc.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n
    assert ttc.version().startswith("ttc")


def _desc(**kw):
    base = dict(out_modes=(12, 8, 8), in_modes=(12, 8, 8), ranks=[1, 30, 30, 30, 30, 30, 1], act_dtype=ttc.TTC_BF16)
    base.update(kw)
    return ttc.make_linear_desc(**base)


def test_workspace_sizes_scale_with_tokens():
    d = _desc()
    s0, c0 = ttc.tt_linear_workspace(d, 0)
    s1, c1 = ttc.tt_linear_workspace(d, 16384)
    # the kept intermediate Z is T x 32 in the activation dtype (bf16 here)
    assert s1 - s0 >= 16384 * 32 * 2
    assert c1 > c0


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(ranks=[2, 30, 30, 30, 30, 30, 1]), 3),
        (dict(ranks=[1, 30, 30, 0, 30, 30, 1]), 3),
        (dict(ranks=[1, 30, 30, 129, 30, 30, 1]), 3),
        (dict(act_dtype=7), 4),
        (dict(out_modes=(12, 0, 8)), 2),
        (dict(path=ttc.TTC_PATH_DENSE), 7),
    ],
)
def test_bad_descriptors_are_rejected(kw, code):
    d = _desc(**kw)
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_workspace(d, 64)
    assert e.value.code == code


def test_too_many_modes_rejected():
    d = _desc()
    d.p = 9
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_workspace(d, 64)
    assert e.value.code == 2


def test_negative_tokens_rejected():
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_workspace(_desc(), -1)
    assert e.value.code == 2


def test_fwd_errors_before_launch():
    """Argument errors come back synchronously and nothing is launched."""
    d = _desc()
    sb, cb = ttc.tt_linear_workspace(d, 64)
    G = [16] * 6  # never dereferenced: validation fails first
    D = [16] * 5
    # null x
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_fwd(d, 64, None, G, D, 16, 16, sb, None, 0)
    assert e.value.code == 1
    # misaligned x
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_fwd(d, 64, 18, G, D, 16, 16, sb, None, 0)
    assert e.value.code == 5
    # saved too small
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_fwd(d, 64, 16, G, D, 16, 16, sb - 1, None, 0)
    assert e.value.code == 6
    # null core pointer
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_fwd(d, 64, 16, [16, 16, 0, 16, 16, 16], D, 16, 16, sb, None, 0)
    assert e.value.code == 1
    # T = 0 is a no-op that succeeds without touching anything
    ttc.tt_linear_fwd(d, 0, None, G, D, None, None, 0, None, 0)


def test_bwd_errors_before_launch():
    d = _desc()
    sb, cb = ttc.tt_linear_workspace(d, 64)
    G = [16] * 6
    D = [16] * 5
    dG = [16] * 6
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_bwd(d, 64, 16, 16, G, D, 16, sb, 16, dG, 16, cb - 1)
    assert e.value.code == 6
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_bwd(d, 64, 16, 16, G, D, 16, sb, 16, [16] * 5 + [0], 16, cb)
    assert e.value.code == 1



def test_bwd_data_and_cores_errors_before_launch():
    d = _desc()
    sb, cb = ttc.tt_linear_workspace(d, 64)
    G = [16] * 6
    D = [16] * 5
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_bwd_data(d, 64, 16, 16, G, D, 16, sb, 16, 16, cb - 1)
    assert e.value.code == 6
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_bwd_data(d, 64, None, 16, G, D, 16, sb, 16, 16, cb)
    assert e.value.code == 1
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_bwd_data(d, 64, 16, 24, G, D, 16, sb, 16, 16, cb)
    assert e.value.code == 5
    # T = 0: the data pass has nothing to do and touches nothing
    ttc.tt_linear_bwd_data(d, 0, None, None, G, D, None, 0, None, None, 0)
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_bwd_cores(d, 64, G, D, 16, sb - 1, [16] * 6, 16, cb)
    assert e.value.code == 6
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_bwd_cores(d, 64, G, D, 16, sb, [16] * 5 + [0], 16, cb)
    assert e.value.code == 1
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_bwd_cores(d, 64, G, D, None, sb, [16] * 6, 16, cb)
    assert e.value.code == 1


def test_batch_calls_check_every_layer_before_launch():
    d = _desc()
    d2 = _desc(out_modes=(12, 16, 16))
    sb, cb = ttc.tt_linear_workspace(d, 64)
    sb2, cb2 = ttc.tt_linear_workspace(d2, 64)
    G = [[16] * 6, [16] * 6]
    D = [[16] * 5, [16] * 5]
    # the second layer's saved buffer is too small (sized for the first layer)
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_prepare_batch([d, d2], [64, 64], G, D, [16, 32], [sb, sb])
    assert e.value.code == 6
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_prepare_batch([d, d2], [64, 64], G, D, [16, None], [sb, sb2])
    assert e.value.code == 1
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_prepare_batch([d, d2], [64, 64], G, [[16] * 5, [16] * 4 + [0]], [16, 32], [sb, sb2])
    assert e.value.code == 1
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_bwd_cores_batch([d, d2], [64, 64], G, D, [16, 32], [sb, sb2], [[16] * 6, [16] * 6],
                                      [16, 32], [cb, cb2 - 1])
    assert e.value.code == 6
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_bwd_cores_batch([d, d2], [64, 64], G, D, [16, 32], [sb, sb2], [[16] * 6, [16] * 5 + [0]],
                                      [16, 32], [cb, cb2])
    assert e.value.code == 1
    # nothing to do
    ttc.tt_linear_prepare_batch([], [], [], [], [], [])
    ttc.tt_linear_bwd_cores_batch([], [], [], [], [], [], [], [], [])
    code = ttc.lib().tt_linear_prepare_batch(-1, None, None, None, None, None, None, None)
    assert code == 2


def test_batched_streaming_calls_check_every_layer_before_launch():
    d = _desc()
    d2 = _desc(out_modes=(12, 16, 16))
    sb, cb = ttc.tt_linear_workspace(d, 64)
    sb2, cb2 = ttc.tt_linear_workspace(d2, 64)
    G = [[16] * 6, [16] * 6]
    D = [[16] * 5, [16] * 5]
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_fwd_batch([d, d2], [64, 64], [16, 32], G, D, [48, 64], [80, 96], [sb, sb])
    assert e.value.code == 6
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_fwd_batch([d, d2], [64, 64], [16, 32], G, D, [48, 72], [80, 96], [sb, sb2])
    assert e.value.code == 5
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_fwd_batch([d, d2], [64, 64], [16, None], G, D, [48, 64], [80, 96], [sb, sb2])
    assert e.value.code == 1
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_bwd_data_batch([d, d2], [64, 64], [16, 32], [48, 64], G, D, [80, 96], [sb, sb2], None,
                                     [112, 128], [cb, cb2 - 1])
    assert e.value.code == 6
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_bwd_data_batch([d, d2], [64, 64], [16, 32], [48, None], G, D, [80, 96], [sb, sb2], None,
                                     [112, 128], [cb, cb2])
    assert e.value.code == 1
    # T = 0 layers are skipped; nothing to do
    ttc.tt_linear_fwd_batch([d], [0], [None], [[16] * 6], [[16] * 5], [None], [None], [0])
    ttc.tt_linear_bwd_data_batch([], [], [], [], [], [], [], [], None, [], [])
    assert ttc.lib().tt_linear_fwd_batch(-1, None, None, None, None, None, None, None, None, None) == 2


def test_rank_grads_errors_before_launch():
    d = _desc()
    G = [16] * 6
    D = [16] * 5
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_rank_grads(d, G, D, [16] * 6, [16] * 4 + [0], 0.1, 0.0)
    assert e.value.code == 1
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_rank_grads(d, G, D, [16] * 5 + [0], [16] * 5, 0.1, 0.0)
    assert e.value.code == 1
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_rank_grads(d, G, D, [16] * 6, [16] * 5, float("nan"), 0.0)
    assert e.value.code == 2

# ---- planner: contraction orders ----------------------------------------------------
#
# The forward pass is the tensor network {x, G_1, ..., G_d} contracted down to
# Y (project page, "Making small tensor operations fast on GPUs": the order of
# the pairwise contractions decides the cost; Proposition 4.1 compares the
# merged order with the core-by-core one).  Contracting two tensors costs the
# product of the sizes of all indices they carry.  These helpers count that
# for every order of a small chain, independently of the library.


def _network(out_modes, in_modes, ranks, in_first, T):
    p, q = len(out_modes), len(in_modes)
    d = p + q
    chain = ([("i", m) for m in range(q)] + [("o", m) for m in range(p)]) if in_first else \
        ([("o", m) for m in range(p)] + [("i", m) for m in range(q)])
    dims = {"T": T}
    for m in range(p):
        dims[f"o{m}"] = out_modes[m]
    for m in range(q):
        dims[f"i{m}"] = in_modes[m]
    for k in range(1, d):
        dims[f"r{k}"] = ranks[k]
    tensors = [frozenset(["T"] + [f"i{m}" for m in range(q)])]  # x
    for k, (side, m) in enumerate(chain):
        idx = {f"{side}{m}"}
        if k > 0:
            idx.add(f"r{k}")
        if k < d - 1:
            idx.add(f"r{k + 1}")
        tensors.append(frozenset(idx))
    out = frozenset(["T"] + [f"o{m}" for m in range(p)])
    return tensors, dims, out, chain


def _free(tensors, sub, out):
    """Indices a group of tensors still carries after contracting it."""
    inside = set().union(*(tensors[i] for i in sub))
    outside = set().union(*(tensors[i] for i in range(len(tensors)) if i not in sub)) if len(sub) < len(tensors) else set()
    return frozenset(i for i in inside if i in outside or i in out)


def _pair_cost(a, b, dims):
    c = 1
    for i in a | b:
        c *= dims[i]
    return c


def _optimal_cost(tensors, dims, out):
    """Fewest multiply-adds over every pairwise contraction order (exhaustive)."""
    n = len(tensors)
    full = (1 << n) - 1
    best = {}
    for mask in range(1, full + 1):
        sub = [i for i in range(n) if mask >> i & 1]
        if len(sub) == 1:
            best[mask] = 0
            continue
        b = None
        part = (mask - 1) & mask
        while part:
            rest = mask ^ part
            if part < rest:  # each split once
                fa = _free(tensors, [i for i in range(n) if part >> i & 1], out)
                fb = _free(tensors, [i for i in range(n) if rest >> i & 1], out)
                c = best[part] + best[rest] + _pair_cost(fa, fb, dims)
                b = c if b is None else min(b, c)
            part = (part - 1) & mask
        best[mask] = b
    return best[full]


def _order_cost(tensors, dims, out, steps):
    """Cost of one given order: `steps` is a list of (group, group) pairs of
    tensor-index tuples, each group already contracted."""
    tot = 0
    for ga, gb in steps:
        tot += _pair_cost(_free(tensors, list(ga), out), _free(tensors, list(gb), out), dims)
    return tot


def _merged_order(d, s):
    """Each half of the chain multiplied out from its end, then x through the
    input half, then the output half (tensor 0 is x, core k is k + 1)."""
    return s, d - s


def _chain_orders(out_modes, in_modes, in_first, T, ranks):
    tensors, dims, out, chain = _network(out_modes, in_modes, ranks, in_first, T)
    p, q = len(out_modes), len(in_modes)
    d = p + q
    s = q if in_first else p
    left = list(range(1, s + 1))          # cores of the left half (tensor ids)
    right = list(range(s + 1, d + 1))
    steps = []
    # merged: left half from core 1 rightwards, right half from core d leftwards
    g = (left[0],)
    for c in left[1:]:
        steps.append((g, (c,)))
        g = g + (c,)
    Lg = g
    g = (right[-1],)
    for c in reversed(right[:-1]):
        steps.append(((c,), g))
        g = (c,) + g
    Rg = g
    inp, outp = (Lg, Rg) if in_first else (Rg, Lg)
    steps.append(((0,), inp))
    steps.append(((0,) + inp, outp))
    merged = _order_cost(tensors, dims, out, steps)
    # sequential: x through the input half from its chain end, then the
    # output half from the split outwards
    walk = (left + right) if in_first else (right[::-1] + left[::-1])
    g, steps = (0,), []
    for c in walk:
        steps.append((g, (c,)))
        g = g + (c,)
    sequential = _order_cost(tensors, dims, out, steps)
    return merged, sequential, _optimal_cost(tensors, dims, out)


CHAINS = [
    ((2, 3), (3, 2), [1, 2, 3, 4, 1]),
    ((2, 3), (3, 2), [1, 3, 2, 3, 1]),
    ((2, 3, 2), (2, 2, 3), [1, 2, 3, 4, 3, 2, 1]),
    ((4,), (2, 3, 2), [1, 3, 4, 2, 1]),
    ((2, 2, 3), (5,), [1, 2, 3, 2, 1]),
    ((3, 4), (4, 3), [1, 5, 5, 5, 1]),
]


@pytest.mark.parametrize("in_first", [False, True])
@pytest.mark.parametrize("chain", CHAINS)
@pytest.mark.parametrize("T", [1, 4, 64, 4096])
def test_planner_costs_match_exhaustive_contraction_orders(chain, in_first, T):
    """The planner's multiply-add counts of the merged and the core-by-core
    orders equal the counts of those two orders in the network (forward;
    the planner's totals are forward + backward = 3x), no order of the network
    beats the merged order at a large batch, and AUTO picks the order with the
    smaller modelled time."""
    out_modes, in_modes, ranks = chain
    d = ttc.make_linear_desc(out_modes, in_modes, ranks, ttc.TTC_F32, in_first)
    merged, sequential, best = _chain_orders(out_modes, in_modes, in_first, T, ranks)
    m1, _ = ttc.tt_linear_path_cost(d, T, ttc.TTC_PATH_MERGED)
    m2, _ = ttc.tt_linear_path_cost(d, T, ttc.TTC_PATH_SEQUENTIAL)
    assert m1 == 3 * merged
    assert m2 == 3 * sequential
    assert best <= min(merged, sequential)
    if T >= 4096:
        assert best >= 0.99 * merged  # Proposition 4.1: near the fewest operations for large batches
    f = _explain_fields(d, T)
    assert f["path"] == ("sequential" if float(f["sequential_us"]) < float(f["merged_us"]) else "merged")


def test_merged_order_wins_at_large_batch_and_loses_at_batch_one():
    """Project page, one contraction order for both passes: close to the fewest
    operations for large batches (Proposition 4.1); at batch 1 the core-by-core
    sweep needs fewer multiply-adds, so a crossover exists.  On this GPU both
    orders are latency-bound at a few tokens and the modelled time of the
    merged one is lower, so AUTO keeps it there too."""
    d = ttc.make_linear_desc((12, 8, 8), (12, 8, 8), [1, 30, 30, 30, 30, 30, 1], ttc.TTC_F32)
    for T in (64, 4096, 16384):
        assert ttc.tt_linear_path_cost(d, T, ttc.TTC_PATH_MERGED)[0] < ttc.tt_linear_path_cost(d, T, ttc.TTC_PATH_SEQUENTIAL)[0]
        assert ttc.tt_linear_explain(d, T).startswith("path=merged")
    assert ttc.tt_linear_path_cost(d, 1, ttc.TTC_PATH_SEQUENTIAL)[0] < ttc.tt_linear_path_cost(d, 1, ttc.TTC_PATH_MERGED)[0]
    f = _explain_fields(d, 1)
    assert float(f["merged_us"]) < float(f["sequential_us"]) and f["path"] == "merged"


def test_forced_paths():
    d = _desc(path=ttc.TTC_PATH_MERGED)
    assert ttc.tt_linear_explain(d, 1).startswith("path=merged")
    d = _desc(path=ttc.TTC_PATH_SEQUENTIAL)
    assert ttc.tt_linear_explain(d, 4096).startswith("path=sequential")
    # the sequential kernels keep a token's states and one core in LDS: a
    # rank-64 core of mode 16 (256 KB) does not fit, so forcing it is refused
    big = ttc.make_linear_desc((16, 16, 16), (16, 8, 8), [1] + [64] * 5 + [1], ttc.TTC_BF16, False,
                               ttc.TTC_PATH_SEQUENTIAL)
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_workspace(big, 8)
    assert e.value.code == 7
    auto = ttc.make_linear_desc((16, 16, 16), (16, 8, 8), [1] + [64] * 5 + [1], ttc.TTC_BF16)
    assert ttc.tt_linear_explain(auto, 1).startswith("path=merged")


# ---- TTM embedding -------------------------------------------------------------

def _ttm(vocab=(32, 32, 32), dims=(12, 8, 8), ranks=(1, 16, 16, 1), accumulate=False):
    return ttc.make_ttm_desc(vocab, dims, ranks, accumulate)


def test_ttm_workspace_holds_documented_head_and_products():
    T = 16384
    sb, cb = ttc.ttm_embed_workspace(_ttm(), T)
    A = ((4 * T + 255) // 256) * 256
    # header, order, inverse, distinct ids, segment offsets come first
    assert sb >= 128 + 3 * A + 4 * (T + 1)
    # the level-1 prefix products: at most 32*32 prefixes of 96 x 16 floats
    assert sb >= 1024 * 96 * 16 * 4
    # scratch: the backward's piece sums are at most T rows of 768 floats
    assert cb >= T * 768 * 4
    s1, c1 = ttc.ttm_embed_workspace(_ttm(), 1000)
    assert s1 < sb and c1 < cb


@pytest.mark.parametrize("kw,code", [
    (dict(ranks=(2, 16, 16, 1)), 3),          # r_0 != 1
    (dict(ranks=(1, 0, 16, 1)), 3),           # r_k < 1
    (dict(ranks=(1, 200, 16, 1)), 3),         # r_k > 128
    (dict(vocab=(32, 0, 32)), 2),             # empty mode
    (dict(vocab=(2048, 2048, 2048), dims=(2, 2, 2)), 2),  # vocabulary >= 2^31
])
def test_ttm_bad_descriptors(kw, code):
    with pytest.raises(ttc.TTCError) as e:
        ttc.ttm_embed_workspace(_ttm(**kw), 64)
    assert e.value.code == code


def test_ttm_limits():
    with pytest.raises(ttc.TTCError) as e:
        ttc.ttm_embed_workspace(_ttm(), 16385)
    assert e.value.code == 7
    # one level's product and core slice must fit 64 KB of LDS
    with pytest.raises(ttc.TTCError) as e:
        ttc.ttm_embed_workspace(_ttm(vocab=(4, 4), dims=(64, 64), ranks=(1, 128, 1)), 64)
    assert e.value.code == 7


def test_ttm_lookup_modes_size_their_workspace():
    """Without shared prefixes every level can hold as many nodes as there are
    distinct ids (UNIQUE) or tokens (PLAIN): the saved buffer grows; an
    unknown mode is rejected."""
    sizes = []
    for mode in (0, 1, 2):
        d = ttc.make_ttm_desc((32, 32, 32), (12, 8, 8), (1, 16, 16, 1), mode=mode)
        sizes.append(ttc.ttm_embed_workspace(d, 16384))
    assert sizes[0][0] < sizes[1][0] <= sizes[2][0]
    with pytest.raises(ttc.TTCError) as e:
        ttc.ttm_embed_workspace(ttc.make_ttm_desc((32, 32, 32), (12, 8, 8), (1, 16, 16, 1), mode=3), 64)
    assert e.value.code == 2

def test_ttm_index_and_lookup_errors_before_launch():
    d = ttc.make_ttm_desc((32, 32, 32), (12, 8, 8), (1, 16, 16, 1))
    sb, cb = ttc.ttm_embed_workspace(d, 64)
    with pytest.raises(ttc.TTCError) as e:
        ttc.ttm_embed_index(d, 64, None, 16, sb)
    assert e.value.code == 1
    with pytest.raises(ttc.TTCError) as e:
        ttc.ttm_embed_index(d, 64, 16, 16, sb - 1)
    assert e.value.code == 6
    with pytest.raises(ttc.TTCError) as e:
        ttc.ttm_embed_lookup(d, 64, [16, 16, 16], None, 16, 16, sb, 16, 16)  # scratch far too small
    assert e.value.code == 6
    with pytest.raises(ttc.TTCError) as e:
        ttc.ttm_embed_lookup(d, 64, [16, 16, 0], None, 16, 16, sb, 16, cb)
    assert e.value.code == 1
    # T = 0: nothing to do
    ttc.ttm_embed_index(d, 0, None, None, 0)
    ttc.ttm_embed_lookup(d, 0, [16, 16, 16], None, None, None, 0, None, 0)

def test_ttm_errors_before_launch():
    d = _ttm()
    sb, cb = ttc.ttm_embed_workspace(d, 64)
    F = [16] * 3
    with pytest.raises(ttc.TTCError) as e:
        ttc.ttm_embed_fwd(d, 64, None, F, None, 16, 16, sb, 16, cb)
    assert e.value.code == 1
    with pytest.raises(ttc.TTCError) as e:
        ttc.ttm_embed_fwd(d, 64, 16, F, None, 24, 16, sb, 16, cb)
    assert e.value.code == 5
    with pytest.raises(ttc.TTCError) as e:
        ttc.ttm_embed_fwd(d, 64, 16, F, None, 16, 16, sb - 1, 16, cb)
    assert e.value.code == 6
    with pytest.raises(ttc.TTCError) as e:
        ttc.ttm_embed_fwd(d, 64, 16, [16, 0, 16], None, 16, 16, sb, 16, cb)
    assert e.value.code == 1
    with pytest.raises(ttc.TTCError) as e:
        ttc.ttm_embed_bwd(d, 64, None, 16, F, None, 16, sb, [16] * 3, 16, cb - 1)
    assert e.value.code == 6
    # T = 0 forward is a no-op
    ttc.ttm_embed_fwd(d, 0, None, F, None, None, None, 0, None, 0)


def _explain_fields(d, T):
    return dict(kv.split("=", 1) for kv in ttc.tt_linear_explain(d, T).split())


@pytest.mark.parametrize("act,rank,in_modes,ok", [
    (ttc.TTC_F32, 128, (2048, 2048), False),   # fp32 A operand: 128 x 2^22 x 4 B = 2^31 B
    (ttc.TTC_BF16, 128, (2048, 2048), True),   # the same in bf16: 2^30 B
    (ttc.TTC_F32, 32, (4096, 4096), False),    # fp32 A operand 32 x 2^24 x 4 B = 2^31 B
    (ttc.TTC_BF16, 32, (4096, 4096), False),   # a 64-token bf16 slab of 2^24 columns = 2^31 B
    (ttc.TTC_BF16, 32, (4096, 2048), True),
])
def test_buffer_resource_extents_are_bounded(act, rank, in_modes, ok):
    """Every operand a streaming kernel reaches through a buffer resource is at
    most 2^31 - 1 bytes: shapes beyond that are refused before any launch
    instead of reading zeros past the resource's end."""
    d = ttc.make_linear_desc((4,), in_modes, [1, rank, rank, 1], act)
    if not ok:
        with pytest.raises(ttc.TTCError) as e:
            ttc.tt_linear_workspace(d, 64)
        assert e.value.code == 7
        return
    ttc.tt_linear_workspace(d, 64)
    # many tokens: the planner's token groups keep each work-group's slab of
    # x, dY, its rank tile and the fp32 dZ partials within one resource
    es = 2 if act == ttc.TTC_BF16 else 4
    n_in = in_modes[0] * in_modes[1]
    for T in (1 << 16, 1 << 20):
        f = _explain_fields(d, T)
        rpad = int(f["rpad"])
        for pas, ncols in (("dy", 4), ("dx", n_in)):
            toks = int(f[f"{pas}_tiles"]) * 64
            assert toks * ncols * es <= 2**31 - 1, (pas, T, toks)
            assert toks * rpad * 4 <= 2**31 - 1, (pas, T, toks)


# ---- chain order (chain_perm) and split ----------------------------------------------

def test_chain_perm_and_split_validation():
    base = dict(out_modes=(12, 8, 8), in_modes=(12, 8, 8), ranks=[1, 30, 30, 30, 30, 30, 1], act_dtype=ttc.TTC_BF16)

    def desc(**kw):
        b = dict(base)
        b.update(kw)
        return ttc.make_linear_desc(**b)

    def code(d):
        try:
            ttc.tt_linear_workspace(d, 64)
            return 0
        except ttc.TTCError as e:
            return e.code

    assert code(desc(chain_perm=(0, 1, 2, 5, 4, 3))) == 0           # mirrored input block
    assert code(desc(chain_perm=(5, 4, 3, 0, 1, 2))) == 0           # inputs first, outputs reversed
    assert code(desc(chain_perm=(0, 1, 2, 3, 4, 4))) == 2           # not a permutation
    assert code(desc(chain_perm=(0, 1, 2, 3, 4, 6))) == 2           # out of range
    assert code(desc(chain_perm=(0, 3, 1, 2, 4, 5))) == 7           # interleaved kinds: two links between them
    assert code(desc(split=3)) == 0 and code(desc(split=-1)) == 0
    assert code(desc(split=2)) == 7 and code(desc(split=4)) == 7
    assert code(desc(chain_perm=(3, 4, 5, 0, 1, 2), split=3)) == 0  # inputs first: s = 3 as well
    # the explicit identity and all-zero entries both mean the default order
    for perm in ((0, 1, 2, 3, 4, 5), None):
        assert ttc.tt_linear_explain(desc(chain_perm=perm), 64) == ttc.tt_linear_explain(desc(), 64)
    d0 = desc()
    for i in range(16):
        d0.chain_perm[i] = 0
    assert ttc.tt_linear_explain(d0, 64) == ttc.tt_linear_explain(desc(), 64)
    # inputs-first permutation ignores in_first
    assert ttc.tt_linear_explain(desc(chain_perm=(3, 4, 5, 0, 1, 2), in_first=False), 64) == \
        ttc.tt_linear_explain(desc(in_first=True), 64)


def test_fp8_descriptor_limits():
    # e4m3 rank tiles are 32 (one 32-wide k-step) or 64; wider ones take the
    # sequential order
    d = ttc.make_linear_desc((12, 8, 8), (12, 8, 8), [1] + [30] * 5 + [1], ttc.TTC_FP8)
    f = _explain_fields(d, 16384)
    assert f["path"] == "merged" and f["rpad"] == "32"
    d64 = ttc.make_linear_desc((12, 8, 8), (12, 8, 8), [1] + [40] * 5 + [1], ttc.TTC_FP8)
    f = _explain_fields(d64, 16384)
    assert f["path"] == "merged" and f["rpad"] == "64"
    big = ttc.make_linear_desc((12, 8, 8), (12, 8, 8), [1] + [65] * 5 + [1], ttc.TTC_FP8, False, ttc.TTC_PATH_MERGED)
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_workspace(big, 64)
    assert e.value.code == 7
    # activations take one byte each: Z is T x 32 bytes
    s0, _ = ttc.tt_linear_workspace(d, 0)
    s1, _ = ttc.tt_linear_workspace(d, 16384)
    assert s1 - s0 == 16384 * 32
