"""GPU parity at the benchmarked sizes, in the launch configuration that
bench.py times, against the fp64 oracle.

bench.make_layers and bench.make_step build and run the step exactly as the
benchmark does: the merges of all layers in one batched call, the Q, K and V
forwards and backward data passes in one launch each, O, FFN1 and FFN2 one
after another, the core-gradient tails of all layers in one batched call on
the side stream, two input sets read by alternating steps.  Two eager steps
run (one per input set); the outputs of the second are compared with the
oracle:

* Y and dX on a seeded sample of token rows that always holds the first and
  the last 64-token tile (rows are independent, so the sample is exact for
  the rows it holds): one rel-L2 over the sample and a rel-L2 for every row;
* every core gradient in full, and its dead slices exactly 0.

Bounds: rel-L2 <= 2e-2 for bf16 storage with fp32 accumulation, <= 1e-5 for
fp32, per tensor and per row.
"""

import numpy as np
import pytest
import torch

import bench
import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}


def _rows(T, n=384, seed=0):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(T, min(n, T), replace=False).tolist())
    rows |= set(range(min(64, T))) | set(range(max(0, T - 64), T))
    return np.array(sorted(rows), dtype=np.int64)


def _rel(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    nr = np.linalg.norm(ref)
    if nr == 0.0:
        return 0.0 if np.all(got == 0) else np.inf
    return float(np.linalg.norm(got - ref) / nr)


def _row_rel(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return np.linalg.norm(got - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-300)


def _take(t, rows):
    return t[torch.from_numpy(rows).to(t.device)].float().cpu().numpy()


def _check_rows(name, got, ref, tol, rows):
    assert _rel(got, ref) <= tol, (name, _rel(got, ref))
    rr = _row_rel(got, ref)
    worst = int(np.argmax(rr))
    assert rr[worst] <= tol, f"{name}: row {rows[worst]} rel-L2 {rr[worst]:.3e} > {tol}"
    return float(rr.max())


def _check_step(layers, host, dtype, rows, full_dG=True):
    tol = TOL[dtype]
    report = []
    for L, h in zip(layers, host):
        spec = h["spec"]
        W = oracle.dense_weight(spec.out_modes, spec.in_modes, h["cores"], h["D"], spec.in_first)
        x = h["x"].astype(np.float64)
        dy = h["dy"].astype(np.float64)
        wy = _check_rows(f"{spec.name} Y", _take(L["y"], rows), x[rows] @ W.T, tol, rows)
        wx = _check_rows(f"{spec.name} dX", _take(L["dx"], rows), dy[rows] @ W, tol, rows)
        errs = []
        if full_dG:
            dGr = oracle.tt_linear_core_grads(x, dy, h["cores"], h["D"], spec.in_first)
            for k, r in enumerate(dGr):
                g = L["dG"][k].cpu().numpy()
                e = _rel(g, r)
                assert e <= tol, (spec.name, k, e)
                errs.append(e)
        for k, v in enumerate(h["D"]):
            dead = np.flatnonzero(v == 0)
            if dead.size:
                assert np.all(L["dG"][k].cpu().numpy()[:, :, dead] == 0.0), (spec.name, k)
                assert np.all(L["dG"][k + 1].cpu().numpy()[dead, :, :] == 0.0), (spec.name, k + 1)
        report.append((spec.name, round(wy, 5), round(wx, 5), round(max(errs), 5) if errs else None))
    print(report)


def _run_bench_step(cfg, rank, T, n_layers=None):
    dev = torch.device("cuda:0")
    layers, host = bench.make_layers(cfg, rank, T, dev, n_sets=2, keep_host=True, n_layers=n_layers)
    step, _, _ = bench.make_step(layers, T, None, bench.StepOptions())
    runner = bench.Runner(step)
    runner.eager_steps(2)
    torch.cuda.synchronize()
    return layers, host, step


@pytest.mark.parametrize("rank", [8, 16, 30, 64])
def test_config2_full_step_bench_launches(rank):
    """Config 2 at T = 16384: six bf16 layers, 40% of every diagonal zeroed."""
    T = synth.CONFIG_TOKENS[2]
    layers, host, _ = _run_bench_step(2, rank, T)
    _check_step(layers, host, "bf16", _rows(T, seed=rank))


@pytest.mark.parametrize("T", [16360, 16424])
def test_config2_ragged_tokens_bench_launches(T):
    """Config 2 at rank 30 with a ragged last tile of 40 tokens: 256 tiles
    (T = 16360; FFN2's dY pass in two column groups and its two-slab dX pass
    summing the dZ partials itself) and 257 tiles (T = 16424; three column
    groups), so the benchmark's launch forms (the eight-wave forward, the
    row-piece x loads of the 3072-wide input, the batched Q, K, V passes, the
    backward grids the planner picks for this T) all meet a ragged tail."""
    layers, host, _ = _run_bench_step(2, 30, T)
    _check_step(layers, host, "bf16", _rows(T, seed=T))


def test_config2_full_step_graph_replay_bitwise():
    """The step as the benchmark replays it (two steps per HIP graph) gives
    bitwise the eager results at T = 16384, rank 30."""
    T = synth.CONFIG_TOKENS[2]
    dev = torch.device("cuda:0")
    layers, _ = bench.make_layers(2, 30, T, dev, n_sets=2)
    step, _, _ = bench.make_step(layers, T, None, bench.StepOptions())
    runner = bench.Runner(step)
    runner.eager_steps(2)
    torch.cuda.synchronize()
    outs = lambda: [t for L in layers for t in [L["y"], L["dx"]] + L["dG"]]
    want = [t.clone() for t in outs()]
    runner.capture(pair=True)
    for rep in range(2):
        for t in outs():
            t.fill_(float("nan"))
        runner.replay_steps(2)
        torch.cuda.synchronize()
        for j, (a, b) in enumerate(zip(outs(), want)):
            assert torch.equal(a, b), (rep, j)


def test_config1_full_step_bench_launches():
    """Config 1 at T = 4096: six fp32 layers, rank 30, 25% of D zeroed."""
    T = synth.CONFIG_TOKENS[1]
    layers, host, _ = _run_bench_step(1, 30, T)
    _check_step(layers, host, "f32", _rows(T, seed=1))


def test_config4_full_encoder_bench_launches():
    """Config 4 at T = 16384: one CodeBERT-large-sized encoder (four
    1024->1024, 1024->4096 and 4096->1024), rank 64, half of D zeroed; core
    gradients in full for every layer."""
    T = synth.CONFIG_TOKENS[4]
    layers, host, _ = _run_bench_step(4, 64, T, n_layers=6)
    _check_step(layers, host, "bf16", _rows(T, seed=4))


def test_config2_full_step_with_embedding():
    """The benchmark's step with the TTM embedding (index built one step
    ahead) at T = 16384, rank 30: TT-linear outputs as above, embedding rows
    on the sample (bitwise equal for repeated ids), dF in full."""
    T = synth.CONFIG_TOKENS[2]
    dev = torch.device("cuda:0")
    layers, host = bench.make_layers(2, 30, T, dev, n_sets=2, keep_host=True)
    ttm, th = bench.make_ttm(T, dev, keep_host=True)
    step, _, _ = bench.make_step(layers, T, ttm, bench.StepOptions())
    runner = bench.Runner(step)
    runner.eager_steps(2)
    torch.cuda.synchronize()
    rows = _rows(T, seed=3)
    _check_step(layers, host, "bf16", rows)
    ids = th["ids"][1]
    E = oracle.ttm_table(th["cores"])
    out = _take(ttm["out"], rows)
    _check_rows("embedding rows", out, E[ids[rows]], 1e-5, rows)
    for k, r in enumerate(oracle.ttm_backward(ids, th["dout"][1], th["cores"])):
        assert _rel(ttm["dF"][k].cpu().numpy(), r) <= 1e-5, k
