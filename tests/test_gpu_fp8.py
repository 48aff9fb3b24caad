"""GPU parity of the FP8 mixed-precision TT-linear (TTC_FP8) against the fp64
oracle.

FP8 mixed precision follows the CoMERA poster page (tables and figures on
FP8-mix tensor-vector products and FP8/FP32 training): activations x, dY, Y,
dX are stored as OCP e4m3, every MFMA operand is e4m3 (gfx950
v_mfma_f32_16x16x32_fp8_fp8), accumulation and the core gradients are fp32.
The oracle consumes the same e4m3-rounded x and dY (synth).

Tolerance, derived from the arithmetic rather than fitted: e4m3 keeps 3
mantissa bits, so one rounding has relative error at most u = 2^-4 and about
u / sqrt(3) = 3.6 % RMS over a binade.  Y passes through four roundings (the
packed A, the kept Z, the packed B, the stored Y), dX likewise (B, dZ, A,
dX), the core gradients through two or three (Z or dZ and an operand): about
7.2 % RMS for Y and dX and 5-6 % for dG.  The bound is twice that: rel-L2 <=
0.15 per tensor and per token row.  Dead slices must still be exactly 0 (the
operands' dead columns are exact zeros in any format).
"""

import numpy as np
import pytest
import torch

import bench
import oracle
import synth
from test_gpu_tt_linear import MERGED, SEQUENTIAL, _check

pytestmark = pytest.mark.gpu

TOL = 0.15


@pytest.mark.parametrize("rank", [8, 16, 30, 64])
@pytest.mark.parametrize("li", [0, 4, 5])
def test_config2_layers_fp8(li, rank):
    spec = synth.config_layers(2, rank)[li]
    layer = synth.make_tt_layer(2, 800 + 10 * rank + li, spec, 300, 0.40, "fp8")
    print(_check(spec, layer, "fp8"))


@pytest.mark.parametrize("T", [1, 8])
@pytest.mark.parametrize("li", [0, 4, 5])
def test_sequential_order_fp8(li, T):
    spec = synth.config_layers(2, 30)[li]
    layer = synth.make_tt_layer(2, 850 + li, spec, T, 0.40, "fp8")
    _check(spec, layer, "fp8", path=SEQUENTIAL)


def test_rank_above_64_takes_the_sequential_order():
    import tensor_train_compressed_tt_amd as ttc

    spec = synth.LayerSpec("r80", (2, 3), (3, 2), 80)
    d = ttc.make_linear_desc(spec.out_modes, spec.in_modes, spec.ranks, ttc.TTC_FP8)
    assert ttc.tt_linear_explain(d, 300).startswith("path=sequential")
    layer = synth.make_tt_layer(2, 860, spec, 40, 0.3, "fp8")
    _check(spec, layer, "fp8", path=0)  # AUTO


def _rows(T, n=256, seed=0):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(T, n, replace=False).tolist()) | set(range(64)) | set(range(T - 64, T))
    return np.array(sorted(rows), dtype=np.int64)


def _row_rel(got, ref):
    return np.linalg.norm(got - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-300)


@pytest.mark.parametrize("rank", [30, 64])
def test_config2_full_step_fp8_bench_launches(rank):
    """The benchmark's six-layer step with fp8 activations at T = 16384: Y and
    dX on sampled rows (per tensor and per row), every dG in full."""
    T = synth.CONFIG_TOKENS[2]
    dev = torch.device("cuda:0")
    layers, host = bench.make_layers(2, rank, T, dev, n_sets=2, keep_host=True, dtype="fp8")
    step, _, _ = bench.make_step(layers, T, None, bench.StepOptions())
    runner = bench.Runner(step)
    runner.eager_steps(2)
    torch.cuda.synchronize()
    rows = _rows(T, seed=rank)
    idx = torch.from_numpy(rows).to(dev)
    worst = []
    for L, h in zip(layers, host):
        s = h["spec"]
        W = oracle.dense_weight(s.out_modes, s.in_modes, h["cores"], h["D"])
        x, dy = h["x"].astype(np.float64), h["dy"].astype(np.float64)
        for name, got, ref in (("Y", L["y"], x[rows] @ W.T), ("dX", L["dx"], dy[rows] @ W)):
            g = got[idx].float().cpu().numpy()
            e = np.linalg.norm(g - ref) / np.linalg.norm(ref)
            rr = _row_rel(g, ref)
            assert e <= TOL and rr.max() <= TOL, (s.name, name, e, rr.max())
            worst.append((s.name, name, round(float(e), 4), round(float(rr.max()), 4)))
        for k, r in enumerate(oracle.tt_linear_core_grads(x, dy, h["cores"], h["D"])):
            g = L["dG"][k].cpu().numpy()
            e = np.linalg.norm(g - r) / np.linalg.norm(r)
            assert e <= TOL, (s.name, k, e)
            worst.append((s.name, f"dG{k}", round(float(e), 4)))
        for k, v in enumerate(h["D"]):
            dead = np.flatnonzero(v == 0)
            assert np.all(L["dG"][k].cpu().numpy()[:, :, dead] == 0.0)
            assert np.all(L["dG"][k + 1].cpu().numpy()[dead, :, :] == 0.0)
    print(worst)
