"""GPU parity of the TT-linear forward and backward against the fp64 oracle.

Every case draws seeded inputs (synth), runs the HIP path through the C ABI
and compares each output tensor with the oracle by relative L2 error
||gpu - ref|| / ||ref||: at most 1e-5 for fp32 activations, 2e-2 for bf16
storage with fp32 accumulation.  Gradient slices whose link diagonal entry is
zero must be exactly 0.0.  Unless a test says otherwise the layers are forced
onto the merged contraction order (the sequential order has its own tests in
test_gpu_sequential.py).
"""

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 0.15}


def _ttc():
    import tensor_train_compressed_tt_amd as ttc
    return ttc


def _rel(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    nr = np.linalg.norm(ref)
    if nr == 0.0:
        return 0.0 if np.all(got == 0) else np.inf
    return float(np.linalg.norm(got - ref) / nr)


def _to_dev(layer, dtype):
    dev = torch.device("cuda:0")
    cores = [torch.from_numpy(np.ascontiguousarray(c)).to(dev) for c in layer["cores"]]
    D = [torch.from_numpy(np.ascontiguousarray(v)).to(dev) for v in layer["D"]]
    if dtype == "bf16":
        x = torch.from_numpy(layer["x_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
        dy = torch.from_numpy(layer["dy_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
    elif dtype == "fp8":
        x = torch.from_numpy(layer["x_bits"]).to(dev).view(torch.float8_e4m3fn)
        dy = torch.from_numpy(layer["dy_bits"]).to(dev).view(torch.float8_e4m3fn)
    else:
        x = torch.from_numpy(layer["x"]).to(dev)
        dy = torch.from_numpy(layer["dy"]).to(dev)
    return cores, D, x, dy


MERGED, SEQUENTIAL = 1, 2  # TTC_PATH_MERGED, TTC_PATH_SEQUENTIAL


def _run(spec, layer, dtype, want_dx=True, path=MERGED):
    ttc = _ttc()
    tdt = {"bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn, "f32": torch.float32}[dtype]
    mod = ttc.TTLinear(spec.out_modes, spec.in_modes, spec.ranks, tdt, spec.in_first, path, spec.chain_perm)
    cores, D, x, dy = _to_dev(layer, dtype)
    y, saved = mod.forward(x, cores, D)
    dx, dG = mod.backward(x, dy, cores, D, saved, want_dx=want_dx)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy()
    return f(y), (f(dx) if dx is not None else None), [f(g) for g in dG]


def _check(spec, layer, dtype, want_dx=True, path=MERGED):
    y, dx, dG = _run(spec, layer, dtype, want_dx, path)
    x = layer["x"].astype(np.float64)
    dy = layer["dy"].astype(np.float64)
    Yr = oracle.tt_linear_forward(x, spec.out_modes, spec.in_modes, layer["cores"], layer["D"], spec.in_first,
                                  spec.chain_perm)
    dXr, dGr = oracle.tt_linear_backward(x, dy, spec.out_modes, spec.in_modes, layer["cores"], layer["D"],
                                         spec.in_first, spec.chain_perm)
    tol = TOL[dtype]
    errs = {"Y": _rel(y, Yr)}
    if want_dx:
        errs["dX"] = _rel(dx, dXr)
    for k in range(len(dG)):
        errs[f"dG{k}"] = _rel(dG[k], dGr[k])
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"rel-L2 above {tol}: {bad} (all: {errs})"
    # dead slices are exactly zero
    for k, v in enumerate(layer["D"]):
        dead = np.flatnonzero(v == 0)
        if dead.size:
            assert np.all(dG[k][:, :, dead] == 0.0), f"dG{k} dead slice not exactly 0"
            assert np.all(dG[k + 1][dead, :, :] == 0.0), f"dG{k + 1} dead slice not exactly 0"
    return errs


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_config0_single_layer(dtype):
    spec = synth.config_layers(0)[0]
    layer = synth.make_tt_layer(0, 0, spec, 64, 0.25, dtype)
    print(_check(spec, layer, dtype))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("in_first", [False, True])
@pytest.mark.parametrize("T", [1, 70, 200])
def test_tiny_odd_shapes(dtype, in_first, T):
    spec = synth.LayerSpec("tiny", (2, 3), (3, 2), 3, in_first)
    layer = synth.make_tt_layer(100, T, spec, T, 0.34, dtype)
    _check(spec, layer, dtype)


@pytest.mark.parametrize("modes", [((5,), (7,)), ((2, 2, 2, 2), (3,)), ((4,), (2, 3, 2, 2, 1))])
def test_chain_lengths(modes):
    spec = synth.LayerSpec("chain", modes[0], modes[1], 5)
    layer = synth.make_tt_layer(101, len(modes[0]) * 10 + len(modes[1]), spec, 130, 0.2, "f32")
    _check(spec, layer, "f32")


@pytest.mark.parametrize("rank", [1, 8, 16, 30, 33, 64, 100, 128])
def test_rank_range(rank):
    spec = synth.LayerSpec("r", (4, 6), (6, 4), rank)
    layer = synth.make_tt_layer(102, rank, spec, 150, 0.3, "f32")
    _check(spec, layer, "f32")


@pytest.mark.parametrize("dtype,li,T,rank", [
    ("bf16", 3, 2000, 30),  # 63 tiles of 32 tokens, 3 output steps: 3 column groups of one step
    ("f32", 3, 1000, 30),   # 32 tiles, 3 column groups
    ("bf16", 3, 1000, 64),  # rank 64: 6 output steps, 6 column groups
    ("bf16", 4, 100, 30),   # 4 tiles, 768 -> 3072: 12 column groups of one step
    ("bf16", 4, 1500, 30),  # 47 tiles: 5 column groups over 12 steps (3, 3, 2, 2, 2)
])
def test_forward_column_groups(dtype, li, T, rank):
    """With fewer token tiles than CUs the forward splits each tile's output
    steps over column groups (uneven ones included); Y, dX and every dG
    (through the saved Z, stored by the first group only) match the oracle."""
    spec = synth.config_layers(2, rank)[li]
    layer = synth.make_tt_layer(2, 500 + li, spec, T, 0.40, dtype)
    _check(spec, layer, dtype)


@pytest.mark.parametrize("li", range(6))
def test_config1_layers_fp32(li):
    spec = synth.config_layers(1)[li]
    layer = synth.make_tt_layer(1, li, spec, 333, 0.25, "f32")
    _check(spec, layer, "f32")


@pytest.mark.parametrize("rank", [8, 16, 30, 64])
@pytest.mark.parametrize("li", [0, 4, 5])
def test_config2_layers_bf16(rank, li):
    spec = synth.config_layers(2, rank)[li]
    layer = synth.make_tt_layer(2, 10 * rank + li, spec, 257, 0.40, "bf16")
    _check(spec, layer, "bf16")


def test_config1_full_tokens_one_layer():
    spec = synth.config_layers(1)[0]
    layer = synth.make_tt_layer(1, 0, spec, 4096, 0.25, "f32")
    print(_check(spec, layer, "f32"))


def test_config2_full_tokens_ffn1_r30():
    spec = synth.config_layers(2, 30)[4]
    layer = synth.make_tt_layer(2, 4, spec, 16384, 0.40, "bf16")
    print(_check(spec, layer, "bf16"))


@pytest.mark.parametrize("T", [16384, 16392])
def test_wide_input_row_pieces(T):
    """A 2304 -> 768 layer at the full token count and with a ragged last
    tile: its 4.5 KB rows take the forward's row-piece x loads (staged through
    LDS, the last batch of each row half past its end); bf16, rank 30."""
    spec = synth.LayerSpec("w2304", (12, 8, 8), (12, 12, 16), 30)
    layer = synth.make_tt_layer(2, 700, spec, T, 0.40, "bf16")
    print(_check(spec, layer, "bf16"))


def test_skip_dx():
    spec = synth.config_layers(0)[0]
    layer = synth.make_tt_layer(0, 1, spec, 100, 0.25, "f32")
    _check(spec, layer, "f32", want_dx=False)


def test_all_zero_link_removes_layer():
    spec = synth.LayerSpec("dead", (4, 6), (6, 4), 8)
    layer = synth.make_tt_layer(103, 0, spec, 90, 0.0, "f32")
    layer["D"][1][:] = 0.0
    y, dx, dG = _run(spec, layer, "f32")
    assert np.all(y == 0.0) and np.all(dx == 0.0)
    # both cores next to the dead link get exactly-zero gradients
    assert np.all(dG[1] == 0.0) and np.all(dG[2] == 0.0)


def test_split_link_all_dead():
    spec = synth.LayerSpec("deadsplit", (4, 6), (6, 4), 8)
    layer = synth.make_tt_layer(104, 0, spec, 90, 0.0, "bf16")
    layer["D"][1][:] = 0.0  # link 2 is the split between output and input modes
    y, dx, dG = _run(spec, layer, "bf16")
    assert np.all(y == 0.0) and np.all(dx == 0.0)
    for g in dG:
        assert np.all(g == 0.0)


def test_zero_tokens():
    ttc = _ttc()
    spec = synth.config_layers(0)[0]
    layer = synth.make_tt_layer(0, 2, spec, 0, 0.25, "f32")
    mod = ttc.TTLinear(spec.out_modes, spec.in_modes, spec.ranks, torch.float32)
    cores, D, x, dy = _to_dev(layer, "f32")
    y, saved = mod.forward(x, cores, D)
    dG = [torch.full(s, 7.0, device="cuda") for s in mod.core_shapes]
    mod.backward(x, dy, cores, D, saved, dG=dG)
    torch.cuda.synchronize()
    assert y.shape == (0, 768)
    for g in dG:
        assert torch.all(g == 0.0)


def test_bitwise_deterministic():
    spec = synth.config_layers(2, 30)[5]
    layer = synth.make_tt_layer(2, 5, spec, 1000, 0.40, "bf16")
    a = _run(spec, layer, "bf16")
    b = _run(spec, layer, "bf16")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    for g1, g2 in zip(a[2], b[2]):
        assert np.array_equal(g1, g2)


def test_prepared_and_split_stream_match_single_stream():
    """tt_linear_prepare + TTC_FLAG_PREPARED forward and the backward with a
    separate grad stream give bitwise the same results as the plain calls."""
    ttc = _ttc()
    spec = synth.config_layers(2, 30)[4]
    layer = synth.make_tt_layer(2, 77, spec, 700, 0.40, "bf16")
    ref = _run(spec, layer, "bf16")
    mod = ttc.TTLinear(spec.out_modes, spec.in_modes, spec.ranks, torch.bfloat16)
    cores, D, x, dy = _to_dev(layer, "bf16")
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    side.wait_stream(main)
    with torch.cuda.stream(side):
        saved = mod.prepare(700, cores, D)
        ev = torch.cuda.Event()
        ev.record(side)
    main.wait_event(ev)
    y, _ = mod.forward(x, cores, D, saved=saved, prepared=True)
    dx, dG = mod.backward(x, dy, cores, D, saved, grad_stream=side)
    main.wait_stream(side)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy()
    assert np.array_equal(f(y), ref[0]) and np.array_equal(f(dx), ref[1])
    for g, r in zip(dG, ref[2]):
        assert np.array_equal(f(g), r)


def test_backward_in_two_calls_matches_single_call():
    """tt_linear_bwd_data followed (on another stream, after an event) by
    tt_linear_bwd_cores gives bitwise the results of tt_linear_bwd, for an
    output-side and an input-side FFN layer; T = 0 zeroes dG."""
    ttc = _ttc()
    for li in (4, 5):
        spec = synth.config_layers(2, 30)[li]
        layer = synth.make_tt_layer(2, 90 + li, spec, 333, 0.40, "bf16")
        ref = _run(spec, layer, "bf16")
        mod = ttc.TTLinear(spec.out_modes, spec.in_modes, spec.ranks, torch.bfloat16, spec.in_first)
        cores, D, x, dy = _to_dev(layer, "bf16")
        y, saved = mod.forward(x, cores, D)
        _, cb = mod.workspace(333)
        scratch = torch.empty(cb, dtype=torch.uint8, device="cuda")
        dx = mod.backward_data(x, dy, cores, D, saved, scratch)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            dG = mod.backward_cores(333, cores, D, saved, scratch)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        f = lambda t: t.float().cpu().numpy()
        assert np.array_equal(f(y), ref[0]) and np.array_equal(f(dx), ref[1])
        for g, r in zip(dG, ref[2]):
            assert np.array_equal(f(g), r)
    dG = [torch.full(s, 5.0, device="cuda") for s in mod.core_shapes]
    mod.backward_cores(0, cores, D, saved, scratch, dG=dG)
    torch.cuda.synchronize()
    for g in dG:
        assert torch.all(g == 0.0)

def test_batched_prepare_and_core_gradients_match_single_layer_calls():
    """tt_linear_prepare_batch and tt_linear_bwd_cores_batch over layers of
    different shapes, chain orders and dtypes (and one with T = 0) give
    bitwise the results of the single-layer calls."""
    ttc = _ttc()
    cases = [(synth.config_layers(2, 30)[0], "bf16", 257), (synth.config_layers(2, 30)[4], "bf16", 257),
             (synth.config_layers(2, 16)[5], "bf16", 257), (synth.config_layers(1, 30)[4], "f32", 130),
             (synth.config_layers(0)[0], "f32", 0)]
    mods, data, refs = [], [], []
    for i, (spec, dt, T) in enumerate(cases):
        layer = synth.make_tt_layer(2, 300 + i, spec, T, 0.40, dt)
        in_first = spec.in_first
        tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        mod = ttc.TTLinear(spec.out_modes, spec.in_modes, spec.ranks, tdt, in_first)
        cores, D, x, dy = _to_dev(layer, dt)
        y, saved = mod.forward(x, cores, D)
        dx, dG = mod.backward(x, dy, cores, D, saved)
        torch.cuda.synchronize()
        refs.append((y.clone(), dx.clone(), [g.clone() for g in dG]))
        sb, cb = mod.workspace(T)
        mods.append(mod)
        data.append(dict(cores=cores, D=D, x=x, dy=dy, T=T,
                         saved=torch.empty(max(sb, 256), dtype=torch.uint8, device="cuda"),
                         scratch=torch.empty(max(cb, 256), dtype=torch.uint8, device="cuda"),
                         dG=[torch.full(sh, 9.0, device="cuda") for sh in mod.core_shapes]))
    # per-layer T differs, so call the ctypes level directly
    ttc.tt_linear_prepare_batch([m.desc for m in mods], [b["T"] for b in data],
                                [[c.data_ptr() for c in b["cores"]] for b in data],
                                [[v.data_ptr() for v in b["D"]] for b in data],
                                [b["saved"].data_ptr() for b in data], [b["saved"].numel() for b in data],
                                torch.cuda.current_stream().cuda_stream)
    ys, dxs = [], []
    for m, b in zip(mods, data):
        y, _ = m.forward(b["x"], b["cores"], b["D"], saved=b["saved"], prepared=True)
        dx = m.backward_data(b["x"], b["dy"], b["cores"], b["D"], b["saved"], b["scratch"])
        ys.append(y)
        dxs.append(dx)
    ttc.tt_linear_bwd_cores_batch([m.desc for m in mods], [b["T"] for b in data],
                                  [[c.data_ptr() for c in b["cores"]] for b in data],
                                  [[v.data_ptr() for v in b["D"]] for b in data],
                                  [b["saved"].data_ptr() for b in data], [b["saved"].numel() for b in data],
                                  [[g.data_ptr() for g in b["dG"]] for b in data],
                                  [b["scratch"].data_ptr() for b in data], [b["scratch"].numel() for b in data],
                                  torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for (ry, rdx, rdG), y, dx, b in zip(refs, ys, dxs, data):
        assert torch.equal(y, ry) and torch.equal(dx, rdx)
        for g, r in zip(b["dG"], rdG):
            assert torch.equal(g, r)
        if b["T"] == 0:
            for g in b["dG"]:
                assert torch.all(g == 0.0)

def test_batched_streaming_passes_match_single_layer_calls():
    """tt_linear_fwd_batch and tt_linear_bwd_data_batch (then the batched core
    gradients) over five same-form bf16 layers (two launches: four layers and
    one), an FFN layer, an fp32 layer and a zero-token layer in one call give
    bitwise the outputs of the single-layer calls."""
    ttc = _ttc()
    c2 = synth.config_layers(2, 30)
    cases = [(c2[i % 4], "bf16", 257) for i in range(5)] + [(c2[5], "bf16", 257),
                                                           (synth.config_layers(1, 30)[4], "f32", 130),
                                                           (c2[0], "bf16", 0)]
    mods, data, refs = [], [], []
    for i, (spec, dt, T) in enumerate(cases):
        layer = synth.make_tt_layer(2, 400 + i, spec, T, 0.40, dt)
        tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        mod = ttc.TTLinear(spec.out_modes, spec.in_modes, spec.ranks, tdt, spec.in_first)
        cores, D, x, dy = _to_dev(layer, dt)
        y, saved = mod.forward(x, cores, D)
        dx, dG = mod.backward(x, dy, cores, D, saved)
        torch.cuda.synchronize()
        refs.append((y.clone(), dx.clone(), [g.clone() for g in dG]))
        sb, cb = mod.workspace(T)
        mods.append(mod)
        data.append(dict(cores=cores, D=D, x=x, dy=dy, T=T,
                         y=torch.full((T, spec.n_out), 3.0, dtype=tdt, device="cuda"),
                         dx=torch.full((T, spec.n_in), 3.0, dtype=tdt, device="cuda"),
                         saved=torch.empty(max(sb, 256), dtype=torch.uint8, device="cuda"),
                         scratch=torch.empty(max(cb, 256), dtype=torch.uint8, device="cuda"),
                         dG=[torch.full(sh, 9.0, device="cuda") for sh in mod.core_shapes]))
    cur = torch.cuda.current_stream().cuda_stream
    Ts = [b["T"] for b in data]
    Gp = [[c.data_ptr() for c in b["cores"]] for b in data]
    Dp = [[v.data_ptr() for v in b["D"]] for b in data]
    ttc.tt_linear_fwd_batch([m.desc for m in mods], Ts, [b["x"].data_ptr() for b in data], Gp, Dp,
                            [b["y"].data_ptr() for b in data], [b["saved"].data_ptr() for b in data],
                            [b["saved"].numel() for b in data], cur)
    ttc.tt_linear_bwd_data_batch([m.desc for m in mods], Ts, [b["x"].data_ptr() for b in data],
                                 [b["dy"].data_ptr() for b in data], Gp, Dp, [b["saved"].data_ptr() for b in data],
                                 [b["saved"].numel() for b in data], [b["dx"].data_ptr() for b in data],
                                 [b["scratch"].data_ptr() for b in data], [b["scratch"].numel() for b in data], cur)
    ttc.tt_linear_bwd_cores_batch([m.desc for m in mods], Ts, Gp, Dp, [b["saved"].data_ptr() for b in data],
                                  [b["saved"].numel() for b in data], [[g.data_ptr() for g in b["dG"]] for b in data],
                                  [b["scratch"].data_ptr() for b in data], [b["scratch"].numel() for b in data], cur)
    torch.cuda.synchronize()
    for i, ((ry, rdx, rdG), b) in enumerate(zip(refs, data)):
        assert torch.equal(b["y"], ry), i
        assert torch.equal(b["dx"], rdx), i
        for g, r in zip(b["dG"], rdG):
            assert torch.equal(g, r), i

@pytest.mark.parametrize("deferred", [False, True])
def test_graph_replay_two_streams_matches_eager(deferred):
    """A captured two-layer step (merges and core-gradient tails on a side
    stream; the tails either per layer behind its data pass, or all together
    after the last data pass) replayed several times, with eager work and
    synchronisation in between, reproduces the eager results every time."""
    ttc = _ttc()
    specs = synth.config_layers(2, 16)[3:5]
    T = 300
    mods, data = [], []
    for i, spec in enumerate(specs):
        layer = synth.make_tt_layer(2, 200 + i, spec, T, 0.40, "bf16")
        mod = ttc.TTLinear(spec.out_modes, spec.in_modes, spec.ranks, torch.bfloat16)
        cores, D, x, dy = _to_dev(layer, "bf16")
        sb, cb = mod.workspace(T)
        bufs = dict(saved=torch.empty(sb, dtype=torch.uint8, device="cuda"),
                    scratch=torch.empty(cb, dtype=torch.uint8, device="cuda"),
                    y=torch.empty((T, spec.n_out), dtype=torch.bfloat16, device="cuda"),
                    dx=torch.empty((T, spec.n_in), dtype=torch.bfloat16, device="cuda"),
                    dG=[torch.empty(s, device="cuda") for s in mod.core_shapes])
        mods.append(mod)
        data.append((cores, D, x, dy, bufs))
    side = torch.cuda.Stream()

    def step():
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        evs = []
        with torch.cuda.stream(side):
            if deferred:
                ttc.prepare_batch(mods, T, [d[0] for d in data], [d[1] for d in data],
                                  [d[4]["saved"] for d in data])
                e = torch.cuda.Event()
                e.record(side)
                evs = [e] * len(mods)
            else:
                for mod, (cores, D, x, dy, b) in zip(mods, data):
                    mod.prepare(T, cores, D, saved=b["saved"])
                    e = torch.cuda.Event()
                    e.record(side)
                    evs.append(e)
        if deferred:
            main.wait_event(evs[0])
            ttc.forward_batch(mods, [d[2] for d in data], [d[0] for d in data], [d[1] for d in data],
                              [d[4]["y"] for d in data], [d[4]["saved"] for d in data], prepared=True)
        else:
            for mod, e, (cores, D, x, dy, b) in zip(mods, evs, data):
                main.wait_event(e)
                mod.forward(x, cores, D, out=b["y"], saved=b["saved"], prepared=True)
        if deferred:
            ttc.backward_data_batch(mods[::-1], [d[2] for d in data][::-1], [d[3] for d in data][::-1],
                                    [d[0] for d in data][::-1], [d[1] for d in data][::-1],
                                    [d[4]["saved"] for d in data][::-1], [d[4]["scratch"] for d in data][::-1],
                                    [d[4]["dx"] for d in data][::-1])
            side.wait_stream(main)
            with torch.cuda.stream(side):
                ttc.backward_cores_batch(mods, T, [d[0] for d in data], [d[1] for d in data],
                                         [d[4]["saved"] for d in data], [d[4]["scratch"] for d in data],
                                         [d[4]["dG"] for d in data])
        else:
            for mod, (cores, D, x, dy, b) in reversed(list(zip(mods, data))):
                mod.backward(x, dy, cores, D, b["saved"], dx=b["dx"], dG=b["dG"], scratch=b["scratch"],
                             grad_stream=side)
        main.wait_stream(side)

    def snapshot():
        out = []
        for _, (_, _, _, _, b) in zip(mods, data):
            out += [b["y"].float().cpu(), b["dx"].float().cpu()] + [g.cpu().clone() for g in b["dG"]]
        return out

    step()
    torch.cuda.synchronize()
    want = snapshot()
    g = torch.cuda.CUDAGraph()
    s0 = torch.cuda.Stream()
    s0.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s0):
        step()  # warm-up on the capture stream
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for _, (_, _, _, _, b) in zip(mods, data):  # eager work between replays
            b["y"].zero_()
            b["dx"].zero_()
            for t in b["dG"]:
                t.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for a, b2 in zip(got, want):
            assert torch.equal(a, b2), f"replay {rep} differs"


# ---- config 4: CodeBERT-large-shaped layers (d = 1024, FFN 4096, rank 64, half of D zeroed)

@pytest.mark.parametrize("li", [0, 4, 5])
def test_config4_layer_shapes(li):
    """Each of the three config-4 layer shapes, several token tiles and a ragged tail."""
    spec = synth.config_layers(4)[li]
    layer = synth.make_tt_layer(4, li, spec, 257, synth.CONFIG_ZERO_FRAC[4], "bf16")
    print(_check(spec, layer, "bf16"))


def test_config4_full_tokens_sampled_rows():
    """Full config-4 size (T = 16384) for the 1024 -> 4096 layer: Y and dX on
    seeded token samples (rows are independent, so this is exact), the core
    gradients in full."""
    spec = synth.config_layers(4)[4]
    T = synth.CONFIG_TOKENS[4]
    layer = synth.make_tt_layer(4, 4, spec, T, synth.CONFIG_ZERO_FRAC[4], "bf16")
    y, dx, dG = _run(spec, layer, "bf16")
    rows = np.sort(np.random.default_rng(4).choice(T, 512, replace=False))
    x = layer["x"].astype(np.float64)
    dy = layer["dy"].astype(np.float64)
    W = oracle.dense_weight(spec.out_modes, spec.in_modes, layer["cores"], layer["D"], spec.in_first)
    assert _rel(y[rows], x[rows] @ W.T) <= TOL["bf16"]
    assert _rel(dx[rows], dy[rows] @ W) <= TOL["bf16"]
    dGr = oracle.tt_linear_core_grads(x, dy, layer["cores"], layer["D"], spec.in_first)
    for k in range(len(dG)):
        assert _rel(dG[k], dGr[k]) <= TOL["bf16"], k
    for k, v in enumerate(layer["D"]):
        dead = np.flatnonzero(v == 0)
        assert np.all(dG[k][:, :, dead] == 0.0) and np.all(dG[k + 1][dead, :, :] == 0.0)


# ---- early-stage gradients: link diagonals and penalties -------------------------

def _rank_grads_case(spec, layer, dtype, gamma, beta):
    ttc = _ttc()
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    mod = ttc.TTLinear(spec.out_modes, spec.in_modes, spec.ranks, tdt, spec.in_first)
    cores, D, x, dy = _to_dev(layer, dtype)
    y, saved = mod.forward(x, cores, D)
    _, dG = mod.backward(x, dy, cores, D, saved)
    dD = mod.rank_grads(cores, D, dG, gamma, beta)
    torch.cuda.synchronize()
    xr = layer["x"].astype(np.float64)
    dyr = layer["dy"].astype(np.float64)
    dGr, dDr = oracle.early_stage_grads(xr, dyr, layer["cores"], layer["D"], gamma, beta, spec.in_first)
    tol = TOL[dtype]
    errs = {f"dG{k}": _rel(g.cpu().numpy(), r) for k, (g, r) in enumerate(zip(dG, dGr))}
    errs.update({f"dD{k}": _rel(v.cpu().numpy(), r) for k, (v, r) in enumerate(zip(dD, dDr))})
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"rel-L2 above {tol}: {bad} (all: {errs})"
    for v, d in zip(dD, layer["D"]):
        assert np.all(v.cpu().numpy()[d == 0] == 0.0), "pruned entry of dD not exactly 0"
    return errs


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("gamma,beta", [(0.0, 0.0), (0.02, 1e-3)])
def test_rank_grads_config0(dtype, gamma, beta):
    spec = synth.config_layers(0)[0]
    layer = synth.make_tt_layer(0, 5, spec, 64, 0.25, dtype)
    print(_rank_grads_case(spec, layer, dtype, gamma, beta))


@pytest.mark.parametrize("in_first", [False, True])
@pytest.mark.parametrize("modes", [((2, 3), (3, 2)), ((5,), (7,)), ((2, 2, 2, 2), (3,))])
def test_rank_grads_chain_orders_and_lengths(in_first, modes):
    spec = synth.LayerSpec("rg", modes[0], modes[1], 3, in_first)
    layer = synth.make_tt_layer(105, 3 * len(modes[0]) + int(in_first), spec, 90, 0.34, "f32")
    _rank_grads_case(spec, layer, "f32", 0.1, 0.01)


@pytest.mark.parametrize("li", [0, 4, 5])
def test_rank_grads_config2_layers(li):
    spec = synth.config_layers(2, 30)[li]
    layer = synth.make_tt_layer(2, 500 + li, spec, 512, 0.40, "bf16")
    _rank_grads_case(spec, layer, "bf16", 0.01, 1e-4)


def test_rank_grads_batch_matches_single_layer_calls():
    """tt_linear_rank_grads_batch over six layers (two launches of core lists
    would be needed above forty cores; here one) gives bitwise the results of
    per-layer calls, penalties included."""
    ttc = _ttc()
    specs = synth.config_layers(2, 16)
    mods, args, single = [], [], []
    for i, spec in enumerate(specs):
        layer = synth.make_tt_layer(2, 600 + i, spec, 200, 0.40, "bf16")
        mod = ttc.TTLinear(spec.out_modes, spec.in_modes, spec.ranks, torch.bfloat16, spec.in_first)
        cores, D, x, dy = _to_dev(layer, "bf16")
        y, saved = mod.forward(x, cores, D)
        _, dG = mod.backward(x, dy, cores, D, saved)
        dG2 = [g.clone() for g in dG]
        dD1 = mod.rank_grads(cores, D, dG, 0.05, 1e-3)
        mods.append(mod)
        args.append((cores, D, dG2, [torch.empty_like(v) for v in D]))
        single.append((dG, dD1))
    ttc.rank_grads_batch(mods, [a[0] for a in args], [a[1] for a in args], [a[2] for a in args],
                         [a[3] for a in args], 0.05, 1e-3)
    torch.cuda.synchronize()
    for (dG, dD1), (_, _, dG2, dD2) in zip(single, args):
        for a, b in zip(dG, dG2):
            assert torch.equal(a, b)
        for a, b in zip(dD1, dD2):
            assert torch.equal(a, b)
