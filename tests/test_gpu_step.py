"""GPU parity of a whole training step in the launch configuration that
bench.py times, against the fp64 oracle.

One step: the embedding lookup of an already indexed id batch and the index of
the next batch (side stream), the merges of six TT-linear layers (main
stream), the forwards (Q, K and V in one launch), the backward data passes in
reverse order, the core-gradient tails of all layers (side stream) beside the
embedding backward.  Two steps, one per index buffer and each with its own id
batch, are captured into one HIP graph.  The eager steps are checked against
the oracle (relative L2: 2e-2 for the bf16 TT-linear outputs, 1e-5 for the
fp32 embedding); every replay of the graph, with eager work and
synchronisation in between and the outputs overwritten with NaN before it,
must reproduce the eager results bitwise.
"""

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

T = 300  # several 64-token tiles and a ragged tail
GROUPS = [[0, 1, 2], [3], [4], [5]]  # Q+K+V in one launch, then O, FFN1, FFN2


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


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def test_bench_step_graph_matches_oracle_and_eager():
    ttc = _ttc()
    dev = torch.device("cuda:0")
    specs = synth.config_layers(2, 30)
    host, layers = [], []
    for i, spec in enumerate(specs):
        L = synth.make_tt_layer(2, 300 + i, spec, T, 0.40, "bf16")
        mod = ttc.TTLinear(spec.out_modes, spec.in_modes, spec.ranks, torch.bfloat16, spec.in_first)
        sb, cb = mod.workspace(T)
        layers.append({
            "mod": mod, "cores": [_dev(c) for c in L["cores"]], "D": [_dev(v) for v in L["D"]],
            "x": torch.from_numpy(L["x_bits"].view(np.int16)).to(dev).view(torch.bfloat16),
            "dy": torch.from_numpy(L["dy_bits"].view(np.int16)).to(dev).view(torch.bfloat16),
            "y": torch.empty((T, spec.n_out), dtype=torch.bfloat16, device=dev),
            "dx": torch.empty((T, spec.n_in), dtype=torch.bfloat16, device=dev),
            "dG": [torch.empty(s, dtype=torch.float32, device=dev) for s in mod.core_shapes],
            "saved": torch.empty(sb, dtype=torch.uint8, device=dev),
            "scratch": torch.empty(cb, dtype=torch.uint8, device=dev),
        })
        host.append((spec, L))
    # two id batches over the same embedding cores, one per index buffer
    a = synth.make_ttm(3, T=T)
    b = synth.make_ttm(3, T=T, base=20241203)
    sp = a["spec"]
    emb = ttc.TTMEmbedding(sp.vocab_modes, sp.dim_modes, sp.ranks)
    F = [_dev(c) for c in a["cores"]]
    tsb, tcb = emb.workspace(T)
    ids = [_dev(a["ids"]), _dev(b["ids"])]
    dout = [_dev(a["dout"]), _dev(b["dout"])]
    saved2 = [torch.empty(tsb, dtype=torch.uint8, device=dev) for _ in range(2)]
    tscratch = torch.empty(tcb, dtype=torch.uint8, device=dev)
    out = [torch.empty((T, sp.dim), dtype=torch.float32, device=dev) for _ in range(2)]
    dF = [[torch.empty(c.shape, dtype=torch.float32, device=dev) for c in a["cores"]] for _ in range(2)]
    side = torch.cuda.Stream()
    mods = [L["mod"] for L in layers]
    col = lambda k: [L[k] for L in layers]

    def step(ph):
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        looked = torch.cuda.Event()
        with torch.cuda.stream(side):
            emb.lookup(T, F, None, saved2[ph], out=out[ph], scratch=tscratch)
            looked.record(side)
            emb.index(ids[1 - ph], saved=saved2[1 - ph])
        ttc.prepare_batch(mods, T, col("cores"), col("D"), col("saved"))
        main.wait_event(looked)
        for g in GROUPS:
            Ls = [layers[i] for i in g]
            if len(Ls) == 1:
                L = Ls[0]
                L["mod"].forward(L["x"], L["cores"], L["D"], out=L["y"], saved=L["saved"], prepared=True)
            else:
                ttc.forward_batch([L["mod"] for L in Ls], [L["x"] for L in Ls], [L["cores"] for L in Ls],
                                  [L["D"] for L in Ls], [L["y"] for L in Ls], [L["saved"] for L in Ls],
                                  prepared=True)
        for g in reversed(GROUPS):
            Ls = [layers[i] for i in g]
            if len(Ls) == 1:
                L = Ls[0]
                L["mod"].backward_data(L["x"], L["dy"], L["cores"], L["D"], L["saved"], L["scratch"], dx=L["dx"])
            else:
                ttc.backward_data_batch([L["mod"] for L in Ls], [L["x"] for L in Ls], [L["dy"] for L in Ls],
                                        [L["cores"] for L in Ls], [L["D"] for L in Ls],
                                        [L["saved"] for L in Ls], [L["scratch"] for L in Ls],
                                        [L["dx"] for L in Ls])
        side.wait_stream(main)
        emb.backward(ids[ph], dout[ph], F, None, saved2[ph], dF=dF[ph], scratch=tscratch)
        with torch.cuda.stream(side):
            ttc.backward_cores_batch(mods[::-1], T, col("cores")[::-1], col("D")[::-1], col("saved")[::-1],
                                     col("scratch")[::-1], col("dG")[::-1])
        main.wait_stream(side)

    def outputs():
        res = [t for L in layers for t in [L["y"], L["dx"]] + L["dG"]]
        return res + out + dF[0] + dF[1]

    def snapshot():
        return [t.cpu().clone() for t in outputs()]

    def poison():
        for t in outputs():
            t.fill_(float("nan"))

    emb.index(ids[0], saved=saved2[0])
    step(0)
    step(1)
    torch.cuda.synchronize()
    want = snapshot()

    # the eager steps against the oracle
    for i, (spec, L) in enumerate(host):
        x, dy = L["x"].astype(np.float64), L["dy"].astype(np.float64)
        W = oracle.dense_weight(spec.out_modes, spec.in_modes, L["cores"], L["D"], spec.in_first)
        assert _rel(layers[i]["y"].float().cpu().numpy(), x @ W.T) <= 2e-2, i
        assert _rel(layers[i]["dx"].float().cpu().numpy(), dy @ W) <= 2e-2, i
        if i in (0, 3):  # one layer of the batched Q/K/V launch, and O
            for k, r in enumerate(oracle.tt_linear_core_grads(x, dy, L["cores"], L["D"], spec.in_first)):
                assert _rel(layers[i]["dG"][k].cpu().numpy(), r) <= 2e-2, (i, k)
    E = oracle.ttm_table(a["cores"])
    for ph, m in enumerate((a, b)):
        assert _rel(out[ph].cpu().numpy(), E[m["ids"]]) <= 1e-5, ph
        for k, r in enumerate(oracle.ttm_backward(m["ids"], m["dout"], a["cores"])):
            assert _rel(dF[ph][k].cpu().numpy(), r) <= 1e-5, (ph, k)

    # both steps in one graph, as the bench replays them
    s0 = torch.cuda.Stream()
    s0.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s0):
        step(0)
        step(1)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(0)
        step(1)
    torch.cuda.synchronize()
    for rep in range(3):
        poison()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for j, (u, v) in enumerate(zip(got, want)):
            assert torch.equal(u, v), (rep, j)
        # eager work between replays
        layers[3]["mod"].forward(layers[3]["x"], layers[3]["cores"], layers[3]["D"])
        torch.cuda.synchronize()
