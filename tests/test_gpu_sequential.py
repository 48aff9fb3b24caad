"""GPU parity of the core-by-core (sequential) contraction order against the
fp64 oracle, and of the planner's automatic choice.

The sequential order (project page, "Making small tensor operations fast on
GPUs", Proposition 4.1 comparison) contracts a token's input modes one core
at a time and then produces its output modes one core at a time; for a few
tokens it needs far fewer multiply-adds than merging the two halves of the
chain.  Same bounds as the merged order: rel-L2 <= 1e-5 (fp32), <= 2e-2 (bf16
storage, fp32 accumulation) per output tensor, dead-slice gradients exactly 0.
"""

import numpy as np
import pytest
import torch

import synth
from test_gpu_tt_linear import MERGED, SEQUENTIAL, _check, _run, _to_dev

pytestmark = pytest.mark.gpu

AUTO = 0


def _ttc():
    import tensor_train_compressed_tt_amd as ttc
    return ttc


@pytest.mark.parametrize("T", [1, 8, 63])
@pytest.mark.parametrize("li", range(6))
def test_config2_layers_small_batches(li, T):
    spec = synth.config_layers(2, 30)[li]
    layer = synth.make_tt_layer(2, 600 + li, spec, T, 0.40, "bf16")
    _check(spec, layer, "bf16", path=SEQUENTIAL)


@pytest.mark.parametrize("T", [1, 8, 63])
@pytest.mark.parametrize("li", [0, 4, 5])
def test_config1_layers_small_batches_fp32(li, T):
    spec = synth.config_layers(1)[li]
    layer = synth.make_tt_layer(1, 610 + li, spec, T, 0.25, "f32")
    _check(spec, layer, "f32", path=SEQUENTIAL)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("in_first", [False, True])
@pytest.mark.parametrize("T", [1, 70])
def test_tiny_odd_shapes(dtype, in_first, T):
    spec = synth.LayerSpec("tiny", (2, 3), (3, 2), 3, in_first)
    layer = synth.make_tt_layer(620, T, spec, T, 0.34, dtype)
    _check(spec, layer, dtype, path=SEQUENTIAL)


@pytest.mark.parametrize("in_first", [False, True])
@pytest.mark.parametrize("modes", [((5,), (7,)), ((2, 2, 2, 2), (3,)), ((4,), (2, 3, 2, 2, 1)),
                                   ((1, 3), (2, 1, 2))])
def test_chain_lengths(modes, in_first):
    spec = synth.LayerSpec("chain", modes[0], modes[1], 5, in_first)
    layer = synth.make_tt_layer(621, len(modes[0]) * 10 + len(modes[1]), spec, 9, 0.2, "f32")
    _check(spec, layer, "f32", path=SEQUENTIAL)


@pytest.mark.parametrize("rank", [1, 8, 16, 33, 64])
def test_rank_range(rank):
    spec = synth.LayerSpec("r", (4, 6), (6, 4), rank)
    layer = synth.make_tt_layer(622, rank, spec, 5, 0.3, "f32")
    _check(spec, layer, "f32", path=SEQUENTIAL)


def test_all_zero_link_and_skip_dx():
    spec = synth.LayerSpec("dead", (4, 6), (6, 4), 8)
    layer = synth.make_tt_layer(623, 0, spec, 7, 0.0, "f32")
    layer["D"][1][:] = 0.0
    y, dx, dG = _run(spec, layer, "f32", path=SEQUENTIAL)
    assert np.all(y == 0.0) and np.all(dx == 0.0)
    assert np.all(dG[1] == 0.0) and np.all(dG[2] == 0.0)
    layer = synth.make_tt_layer(623, 1, spec, 7, 0.25, "f32")
    _check(spec, layer, "f32", want_dx=False, path=SEQUENTIAL)


def test_auto_order_and_both_orders_agree():
    """AUTO runs the order the planner reports (the one with the smaller
    modelled time); both forced orders match the oracle and each other."""
    ttc = _ttc()
    spec = synth.config_layers(2, 30)[0]
    d = ttc.make_linear_desc(spec.out_modes, spec.in_modes, spec.ranks, ttc.TTC_BF16)
    pick = SEQUENTIAL if ttc.tt_linear_explain(d, 1).startswith("path=sequential") else MERGED
    layer = synth.make_tt_layer(2, 630, spec, 1, 0.40, "bf16")
    _check(spec, layer, "bf16", path=AUTO)
    a = _run(spec, layer, "bf16", path=SEQUENTIAL)
    m = _run(spec, layer, "bf16", path=MERGED)
    b = _run(spec, layer, "bf16", path=AUTO)
    want = a if pick == SEQUENTIAL else m
    assert np.array_equal(want[0], b[0]) and np.array_equal(want[1], b[1])
    assert np.linalg.norm(a[0] - m[0]) <= 2e-2 * np.linalg.norm(m[0])


def test_deterministic_and_split_calls_match():
    """Bitwise reproducible; the backward as data + cores calls and with a
    separate grad stream equals the single call."""
    ttc = _ttc()
    spec = synth.config_layers(2, 30)[4]
    T = 11
    layer = synth.make_tt_layer(2, 640, spec, T, 0.40, "bf16")
    a = _run(spec, layer, "bf16", path=SEQUENTIAL)
    b = _run(spec, layer, "bf16", path=SEQUENTIAL)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    for g1, g2 in zip(a[2], b[2]):
        assert np.array_equal(g1, g2)
    mod = ttc.TTLinear(spec.out_modes, spec.in_modes, spec.ranks, torch.bfloat16, spec.in_first, SEQUENTIAL)
    cores, D, x, dy = _to_dev(layer, "bf16")
    saved = mod.prepare(T, cores, D)  # nothing to merge on this order
    y, _ = mod.forward(x, cores, D, saved=saved, prepared=True)
    _, cb = mod.workspace(T)
    scratch = torch.empty(cb, dtype=torch.uint8, device="cuda")
    dx = mod.backward_data(x, dy, cores, D, saved, scratch)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dG = mod.backward_cores(T, cores, D, saved, scratch)
    torch.cuda.current_stream().wait_stream(side)
    dx2, dG2 = mod.backward(x, dy, cores, D, saved, grad_stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy()
    assert np.array_equal(f(y), a[0]) and np.array_equal(f(dx), a[1]) and np.array_equal(f(dx2), a[1])
    for g, g2, r in zip(dG, dG2, a[2]):
        assert np.array_equal(f(g), r) and np.array_equal(f(g2), r)


def test_batched_calls_mix_both_orders():
    """The batched entry points take layers of either order in one call and
    give bitwise the single-layer results."""
    ttc = _ttc()
    specs = synth.config_layers(2, 30)
    items = [(specs[0], 3, SEQUENTIAL), (specs[4], 200, MERGED), (specs[5], 5, AUTO)]
    mods, xs, dys, cores, Ds, ys, saved, scratch, dxs, dGs, refs, Ts = [], [], [], [], [], [], [], [], [], [], [], []
    for k, (spec, T, path) in enumerate(items):
        layer = synth.make_tt_layer(2, 650 + k, spec, T, 0.40, "bf16")
        refs.append(_run(spec, layer, "bf16", path=path))
        mod = ttc.TTLinear(spec.out_modes, spec.in_modes, spec.ranks, torch.bfloat16, spec.in_first, path)
        c, D, x, dy = _to_dev(layer, "bf16")
        sb, cb = mod.workspace(T)
        mods.append(mod), xs.append(x), dys.append(dy), cores.append(c), Ds.append(D), Ts.append(T)
        ys.append(torch.empty((T, spec.n_out), dtype=torch.bfloat16, device="cuda"))
        saved.append(torch.empty(max(sb, 256), dtype=torch.uint8, device="cuda"))
        scratch.append(torch.empty(max(cb, 256), dtype=torch.uint8, device="cuda"))
        dxs.append(torch.empty((T, spec.n_in), dtype=torch.bfloat16, device="cuda"))
        dGs.append([torch.empty(s, dtype=torch.float32, device="cuda") for s in mod.core_shapes])
    for i, m in enumerate(mods):
        ttc.prepare_batch([m], Ts[i], [cores[i]], [Ds[i]], [saved[i]])
    ttc.forward_batch(mods, xs, cores, Ds, ys, saved, prepared=True)
    ttc.backward_data_batch(mods, xs, dys, cores, Ds, saved, scratch, dxs)
    for i, m in enumerate(mods):
        ttc.backward_cores_batch([m], Ts[i], [cores[i]], [Ds[i]], [saved[i]], [scratch[i]], [dGs[i]])
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy()
    for i, r in enumerate(refs):
        assert np.array_equal(f(ys[i]), r[0]) and np.array_equal(f(dxs[i]), r[1]), i
        for g, rr in zip(dGs[i], r[2]):
            assert np.array_equal(f(g), rr), i
