"""GPU parity of a whole training step in the launch configurations that
bench.py times, against the fp64 oracle, at a size with several token tiles
and a ragged tail.

bench.make_layers / make_ttm / make_step build the step: the merges of six
TT-linear layers, their forwards (Q, K and V in one launch), the backward data
passes in reverse order and the batched core-gradient tails (or, pipelined,
each backward group's tail beside the next group's passes); with the
embedding, its lookup of an already indexed id batch and the index of the next
batch beside them (side stream) and its backward beside the tails.  Two steps
run, one per input set (the two id batches differ).  The eager steps are
checked against the oracle (relative L2: 2e-2 for the bf16 TT-linear outputs,
1e-5 for the fp32 embedding); every replay of the two-step HIP graph, with
eager work and synchronisation in between and the outputs overwritten with NaN
before it, must reproduce the eager results bitwise.
"""

import numpy as np
import pytest
import torch

import bench
import oracle

pytestmark = pytest.mark.gpu

T = 300  # several 64-token tiles and a ragged tail


def _rel(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    nr = np.linalg.norm(ref)
    if nr == 0.0:
        return 0.0 if np.all(got == 0) else np.inf
    return float(np.linalg.norm(got - ref) / nr)


def _check_layers(layers, host):
    for i, (L, h) in enumerate(zip(layers, host)):
        spec = h["spec"]
        x, dy = h["x"].astype(np.float64), h["dy"].astype(np.float64)
        W = oracle.dense_weight(spec.out_modes, spec.in_modes, h["cores"], h["D"], spec.in_first)
        assert _rel(L["y"].float().cpu().numpy(), x @ W.T) <= 2e-2, i
        assert _rel(L["dx"].float().cpu().numpy(), dy @ W) <= 2e-2, i
        for k, r in enumerate(oracle.tt_linear_core_grads(x, dy, h["cores"], h["D"], spec.in_first)):
            assert _rel(L["dG"][k].cpu().numpy(), r) <= 2e-2, (i, k)


def _check_ttm(ttm, th, s):
    E = oracle.ttm_table(th["cores"])
    ids = th["ids"][s]
    assert _rel(ttm["out"].cpu().numpy(), E[ids]) <= 1e-5, s
    for k, r in enumerate(oracle.ttm_backward(ids, th["dout"][s], th["cores"])):
        assert _rel(ttm["dF"][k].cpu().numpy(), r) <= 1e-5, (s, k)


OPTIONS = {
    "default": bench.StepOptions(),
    "single_stream": bench.StepOptions(single_stream=True),
    "index_in_step": bench.StepOptions(index_ahead=False),
    "merge_side": bench.StepOptions(merge_side=True),
    "qkv_unbatched": bench.StepOptions(qkv_batch=False),
    "pipeline": bench.StepOptions(pipeline=True),
}


@pytest.mark.parametrize("name", list(OPTIONS))
def test_bench_step_graph_matches_oracle_and_eager(name):
    dev = torch.device("cuda:0")
    layers, host = bench.make_layers(2, 30, T, dev, n_sets=2, keep_host=True)
    ttm, th = bench.make_ttm(T, dev, keep_host=True)
    step, _, _ = bench.make_step(layers, T, ttm, OPTIONS[name])
    runner = bench.Runner(step)

    runner.eager_steps(1)
    torch.cuda.synchronize()
    _check_layers(layers, host)
    _check_ttm(ttm, th, 0)
    runner.eager_steps(1)
    torch.cuda.synchronize()
    _check_layers(layers, host)  # set 1 holds the same activations at other addresses
    _check_ttm(ttm, th, 1)

    def outputs():
        return [t for L in layers for t in [L["y"], L["dx"]] + L["dG"]] + [ttm["out"]] + ttm["dF"]

    want = [t.cpu().clone() for t in outputs()]
    runner.capture(pair=True)
    for rep in range(3):
        for t in outputs():
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        runner.replay_steps(2)
        torch.cuda.synchronize()
        for j, (u, v) in enumerate(zip(outputs(), want)):
            assert torch.equal(u.cpu(), v), (rep, j)
        # eager work between replays
        layers[3]["mod"].forward(layers[3]["x"][0], layers[3]["cores"], layers[3]["D"])
        torch.cuda.synchronize()
