#!/usr/bin/env python3
"""TT-linear fwd+bwd throughput on one MI355X.

One step = the forward pass of six TT-linear layers shaped like one encoder
of the CoMERA pages' six-encoder transformer (Q, K, V, O 768->768 with modes
(12,8,8)x(12,8,8); FFN 768->3072 and 3072->768 with 3072 = (12,16,16)) and
their backward passes in reverse order (input gradients and core gradients),
over T = 128 x 128 = 16384 tokens; activations bf16 with fp32 accumulation,
TT rank 30 with 40% of every link diagonal zeroed.  That step is the headline
(`value`).  The same run also times the step with a TTM embedding lookup of
the step's T ids in front and its backward at the end (vocabulary 32^3 with
modes (32,32,32), rows of 768 = (12,8,8), ranks (1,16,16,1), Zipf(1.1) ids,
fp32), reported under `with_embedding` (--no-ttm skips it).

Inputs are seeded synthetic data resident in HBM.  Consecutive steps read two
different input sets (activations, output gradients, ids), so no step finds
the previous step's inputs in the 256 MB memory-side cache.

Prints one JSON line: the metric, the roofline of the dominant kernel and the
oracle's CPU baseline.  One GPU only: --gpus above 1 is refused.

The module-level helpers (make_layers, make_ttm, make_step) are the step the
benchmark times; the full-size parity tests drive the same code.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time
from dataclasses import dataclass

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "TT-linear fwd+bwd tokens/sec at d=768 r=30; achieved HBM GB/s % of peak"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, vendor figure
RG_GAMMA, RG_BETA = 1e-3, 1e-5  # early-stage penalty weights for --rank-grads (values do not change the cost)
N_SETS = 2  # input sets read by alternating steps


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 4])
    ap.add_argument("--rank", type=int, default=None)
    ap.add_argument("--layers", type=int, default=None, help="with --config 4: number of encoder layers (default 24)")
    ap.add_argument("--tokens", type=int, default=None,
                    help="tokens per step instead of the config's (batch x 128-token sequences, e.g. 128 for batch 1)")
    ap.add_argument("--eager", action="store_true", help="launch every call from Python instead of replaying a HIP graph")
    ap.add_argument("--single-stream", action="store_true",
                    help="run merges and core-gradient tails on the main stream too (no overlap)")
    ap.add_argument("--no-ttm", action="store_true", help="do not time the step with the embedding lookup")
    ap.add_argument("--ttm-mode", default="dedup", choices=["dedup", "unique", "plain"],
                    help="embedding lookup mode: distinct ids and shared prefixes (default), distinct ids only, "
                         "or every token on its own")
    ap.add_argument("--no-index-ahead", action="store_true",
                    help="build the embedding index inside the step's forward instead of one step ahead")
    ap.add_argument("--rank-grads", action="store_true",
                    help="also compute every layer's early-stage gradients (diagonals dD, penalties) after its dG")
    ap.add_argument("--graph-steps", type=int, default=2, choices=[1, 2],
                    help="steps per captured graph (2 needs an even --steps; otherwise 1)")
    ap.add_argument("--merge-side", action="store_true",
                    help="run the merges on the side stream and the embedding lookup on the main one")
    ap.add_argument("--pipeline", action="store_true",
                    help="merge only the first forward group's layers before it (the others beside it) and run "
                         "each backward group's core-gradient tail beside the next group's passes")
    ap.add_argument("--no-qkv-batch", action="store_true",
                    help="one launch per layer for the Q, K and V projections instead of one batched launch")
    ap.add_argument("--dtype", default=None, choices=["f32", "bf16", "fp8"],
                    help="activation storage instead of the config's (fp8: OCP e4m3 activations and MFMA operands)")
    ap.add_argument("--path", default="auto", choices=["auto", "merged", "sequential"],
                    help="contraction order of every layer (default: the planner's pick for the batch)")
    ap.add_argument("--one-input-set", action="store_true",
                    help="every step reads the same inputs (they may then hit in the memory-side cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=None,
                    help="tokens of the CPU-baseline sample (default: the whole step for configs 1 and 2, "
                         "2048 for config 4)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device to device three times (scale for the HBM byte counters)")
    return ap.parse_args(argv)


def copy_calibration(mib):
    import torch

    n = mib * 1024 * 1024 // 2
    x = torch.empty(n, dtype=torch.bfloat16, device="cuda").normal_()
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 2, "copies": 3}), flush=True)


# the sources that decide what the TT-linear kernels do and how they are launched
KERNEL_SOURCES = ("tt_linear.hip", "ttc_device.hpp", "tt_plan.cpp", "tt_plan.hpp")


def kernel_source_digest():
    """sha256 over the kernel sources, in KERNEL_SOURCES order."""
    import hashlib

    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "tensor_train_compressed_tt_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from its committed counter summary
    on the default workload (profiles/<kernel>_tt6_bf16_t16384_rank30_hbm_traffic.md),
    or None when that summary was taken on a different version of the kernel
    sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_tt6_bf16_t16384_rank30_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.strip().startswith("- "):
            k, v = line.strip()[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_sources_sha256") != kernel_source_digest() or "traffic_bytes_per_launch" not in fields:
        return None
    return float(fields["traffic_bytes_per_launch"])


def step_bytes(specs, Ds, T, es):
    """Algorithmic HBM bytes of one fwd+bwd per layer (kernel-level split).

    fwd:    read x, write Y, write Z (T x r_eff fp32)
    bwd_dy: read dY, read Z
    bwd_dx: read x, write dX
    """
    out = []
    for s, D in zip(specs, Ds):
        r_eff = int((D[s.split - 1] != 0).sum())
        out.append({
            "fwd": T * (s.n_in + s.n_out) * es + T * r_eff * 4,
            "bwd_dy": T * s.n_out * es + T * r_eff * 4,
            "bwd_dx": T * 2 * s.n_in * es,
            "r_eff": r_eff,
        })
    return out


def _blas_info():
    try:
        from threadpoolctl import threadpool_info

        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    except Exception:  # pragma: no cover
        blas = []
    if not blas:
        return "unknown", 1
    p = blas[0]
    return f"{p.get('internal_api', '?')} {p.get('version', '')}".strip(), int(p.get("num_threads", 1))


def cpu_baseline(host, T_cpu, min_s=10.0, max_reps=64):
    """The fp64 oracle, as it stands, on the first T_cpu tokens of every given
    layer, repeated until about min_s seconds of CPU work have run (the mean
    over the repetitions is reported); also the time of the same calls on 0
    tokens (the work that does not depend on the token count: weight
    reconstruction, core gradients)."""
    import numpy as np

    import oracle

    def run(Tn):
        t0 = time.perf_counter()
        for L in host:
            s = L["spec"]
            x = L["x"][:Tn].astype(np.float64)
            dy = L["dy"][:Tn].astype(np.float64)
            oracle.tt_linear_forward(x, s.out_modes, s.in_modes, L["cores"], L["D"], s.in_first)
            oracle.tt_linear_backward(x, dy, s.out_modes, s.in_modes, L["cores"], L["D"], s.in_first)
        return time.perf_counter() - t0

    t_fixed = run(0)
    times = [run(T_cpu)]
    while sum(times) < min_s and len(times) < max_reps:
        times.append(run(T_cpu))
    dt = sum(times) / len(times)
    blas, threads = _blas_info()
    return {"value": round(T_cpu / dt, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 oracle fwd+bwd of {len(host)} TT-linear layers on the first {T_cpu} tokens, "
                      f"{len(times)} repetitions ({sum(times):.1f} s wall, {dt:.2f} s each; the same calls on "
                      f"0 tokens take {t_fixed:.2f} s)",
            "blas": blas, "blas_threads": threads, "affinity_cores": len(os.sched_getaffinity(0)),
            "token_independent_s": round(t_fixed, 3), "wall_s": round(dt, 3), "repetitions": len(times)}


# ---- the step -------------------------------------------------------------------------

@dataclass
class StepOptions:
    single_stream: bool = False   # merges and core-gradient tails on the main stream
    qkv_batch: bool = True        # Q, K, V passes of an encoder in one launch each
    index_ahead: bool = True      # embedding index built one step ahead, beside the step
    merge_side: bool = False      # merges on the side stream, lookup on the main one
    rank_grads: bool = False      # early-stage gradients after the core gradients
    pipeline: bool = False        # later layers' merges and earlier layers' gradient tails beside the passes


PATHS = {"auto": 0, "merged": 1, "sequential": 2}


TORCH_DTYPES = {"f32": "float32", "bf16": "bfloat16", "fp8": "float8_e4m3fn"}


def make_layers(cfg, rank, T, dev, n_sets=N_SETS, keep_host=False, n_layers=None, clone_encoders=False,
                path="auto", dtype=None):
    """Device buffers of the step's TT-linear layers, in execution order.

    Every layer has its own seeded cores, diagonals, x and dY (synth), uploaded
    once and copied to n_sets device buffers (step s reads set s mod n_sets).
    With clone_encoders the activations of encoder e > 0 are device copies of
    encoder 0's (same shapes and values, separate memory; the cores are still
    drawn per layer).  keep_host keeps the fp32 host arrays for the oracle.
    """
    import numpy as np
    import torch

    import synth
    import tensor_train_compressed_tt_amd as ttc

    zf = synth.CONFIG_ZERO_FRAC[cfg]
    dt = dtype or synth.CONFIG_DTYPE[cfg]
    specs = synth.config_layers(cfg, rank)
    if n_layers is not None:
        specs = specs[:n_layers]
    tdt = getattr(torch, TORCH_DTYPES[dt])
    layers, host = [], []
    for li, spec in enumerate(specs):
        fresh = not (clone_encoders and li >= 6)
        L = synth.make_tt_layer(cfg, li, spec, T, zf, dt, acts=fresh)
        mod = ttc.TTLinear(spec.out_modes, spec.in_modes, spec.ranks, tdt, spec.in_first, PATHS[path],
                           spec.chain_perm)
        if fresh:
            if dt == "bf16":
                x = torch.from_numpy(L["x_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
                dy = torch.from_numpy(L["dy_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
            elif dt == "fp8":
                x = torch.from_numpy(L["x_bits"]).to(dev).view(torch.float8_e4m3fn)
                dy = torch.from_numpy(L["dy_bits"]).to(dev).view(torch.float8_e4m3fn)
            else:
                x = torch.from_numpy(L["x"]).to(dev)
                dy = torch.from_numpy(L["dy"]).to(dev)
        else:
            x, dy = layers[li % 6]["x"][0], layers[li % 6]["dy"][0]
        sb, cb = mod.workspace(T)
        layers.append({
            "spec": spec, "mod": mod,
            "cores": [torch.from_numpy(c).to(dev) for c in L["cores"]],
            "D": [torch.from_numpy(v).to(dev) for v in L["D"]],
            "x": [x if (s == 0 and fresh) else x.clone() for s in range(n_sets)],
            "dy": [dy if (s == 0 and fresh) else dy.clone() for s in range(n_sets)],
            "y": torch.empty((T, spec.n_out), dtype=tdt, device=dev),
            "dx": torch.empty((T, spec.n_in), dtype=tdt, device=dev),
            "dG": [torch.empty(s, dtype=torch.float32, device=dev) for s in mod.core_shapes],
            "dD": [torch.empty(v.shape, dtype=torch.float32, device=dev) for v in L["D"]],
            "saved": torch.empty(sb, dtype=torch.uint8, device=dev),
            "scratch": torch.empty(cb, dtype=torch.uint8, device=dev),
        })
        keep = {"spec": spec, "cores": L["cores"], "D": L["D"]}
        if keep_host and fresh:
            keep["x"], keep["dy"] = L["x"], L["dy"]
        host.append(keep)
        del L
    return layers, host


def make_ttm(T, dev, mode="dedup", n_sets=N_SETS, keep_host=False):
    """The embedding of the step: one set of cores, n_sets id batches and row
    gradients (set 0 from the base seed, set s from the base seed + s)."""
    import torch

    import synth
    import tensor_train_compressed_tt_amd as ttc

    sets = [synth.make_ttm(3, T=T, base=synth.BASE_SEED + s) for s in range(n_sets)]
    sp = sets[0]["spec"]
    emb = ttc.TTMEmbedding(sp.vocab_modes, sp.dim_modes, sp.ranks,
                           mode={"dedup": 0, "unique": 1, "plain": 2}[mode])
    tsb, tcb = emb.workspace(T)
    ttm = {"emb": emb, "F": [torch.from_numpy(c).to(dev) for c in sets[0]["cores"]],
           "ids": [torch.from_numpy(w["ids"]).to(dev) for w in sets],
           "dout": [torch.from_numpy(w["dout"]).to(dev) for w in sets],
           "out": torch.empty((T, sp.dim), dtype=torch.float32, device=dev),
           "dF": [torch.empty(c.shape, dtype=torch.float32, device=dev) for c in sets[0]["cores"]],
           "saved": torch.empty(tsb, dtype=torch.uint8, device=dev),
           # one index buffer per phase: the next step's index is built into the other
           "saved2": [torch.empty(tsb, dtype=torch.uint8, device=dev) for _ in range(2)],
           "scratch": torch.empty(tcb, dtype=torch.uint8, device=dev), "dim": sp.dim}
    host = None
    if keep_host:
        host = {"cores": sets[0]["cores"], "ids": [w["ids"] for w in sets], "dout": [w["dout"] for w in sets]}
    return ttm, host


def launch_groups(n_layers, qkv_batch=True):
    """Launch groups of the streaming passes.  Within one encoder the Q, K and
    V projections are independent (separate outputs), so each of their passes
    is one batched launch; O, FFN1 and FFN2 depend on what comes before them
    in the encoder and run one after another."""
    fwd = []
    for e in range(n_layers // 6):
        qkv = [6 * e, 6 * e + 1, 6 * e + 2]
        fwd += ([qkv] if qkv_batch else [[i] for i in qkv]) + [[6 * e + 3], [6 * e + 4], [6 * e + 5]]
    fwd += [[i] for i in range(6 * (n_layers // 6), n_layers)]
    return fwd, [g[::-1] for g in fwd[::-1]]


def make_step(layers, T, ttm=None, opts=StepOptions()):
    """step(ph): one fwd+bwd pass over every layer (and the embedding) reading
    input set ph mod n_sets.  Consecutive steps must alternate ph = 0, 1, ...
    when the embedding index is built ahead (call ttm_first_index first).
    Returns (step, fwd_groups, bwd_groups)."""
    import torch

    import tensor_train_compressed_tt_amd as ttc

    n_sets = len(layers[0]["x"])
    fwd_groups, bwd_groups = launch_groups(len(layers), opts.qkv_batch and not opts.single_stream)
    mods = [L["mod"] for L in layers]
    col = lambda k: [L[k] for L in layers]
    pick = lambda k, idx: [layers[i][k] for i in idx]
    every = [i for g in fwd_groups for i in g]
    # merged on the main stream before the first forward; the others beside it
    first = list(fwd_groups[0]) if opts.pipeline else every
    rest = [i for i in every if i not in first]
    ahead = ttm is not None and opts.index_ahead and not opts.single_stream
    side = torch.cuda.Stream()  # default priority

    def ttm_fwd(ph):
        if ttm is None:
            return
        s = ph % len(ttm["ids"])
        if ahead:
            ttm["emb"].lookup(T, ttm["F"], None, ttm["saved2"][ph % 2], out=ttm["out"], scratch=ttm["scratch"])
        else:
            ttm["emb"].forward(ttm["ids"][s], ttm["F"], None, out=ttm["out"], saved=ttm["saved"],
                               scratch=ttm["scratch"])

    def ttm_index_next(ph):
        nxt = ph + 1
        ttm["emb"].index(ttm["ids"][nxt % len(ttm["ids"])], saved=ttm["saved2"][nxt % 2])

    def ttm_bwd(ph):
        if ttm is not None:
            s = ph % len(ttm["ids"])
            ttm["emb"].backward(ttm["ids"][s], ttm["dout"][s], ttm["F"], None,
                                ttm["saved2"][ph % 2] if ahead else ttm["saved"], dF=ttm["dF"],
                                scratch=ttm["scratch"])

    def fwd_group(g, s):
        Ls = [layers[i] for i in g]
        if len(Ls) == 1:
            L = Ls[0]
            L["mod"].forward(L["x"][s], L["cores"], L["D"], out=L["y"], saved=L["saved"], prepared=True)
        else:
            ttc.forward_batch([L["mod"] for L in Ls], [L["x"][s] for L in Ls], [L["cores"] for L in Ls],
                              [L["D"] for L in Ls], [L["y"] for L in Ls], [L["saved"] for L in Ls], prepared=True)

    def bwd_group(g, s):
        Ls = [layers[i] for i in g]
        if len(Ls) == 1:
            L = Ls[0]
            L["mod"].backward_data(L["x"][s], L["dy"][s], L["cores"], L["D"], L["saved"], L["scratch"], dx=L["dx"])
        else:
            ttc.backward_data_batch([L["mod"] for L in Ls], [L["x"][s] for L in Ls], [L["dy"][s] for L in Ls],
                                    [L["cores"] for L in Ls], [L["D"] for L in Ls], [L["saved"] for L in Ls],
                                    [L["scratch"] for L in Ls], [L["dx"] for L in Ls])

    def cores_tail(idx):
        ttc.backward_cores_batch([mods[i] for i in idx], T, pick("cores", idx), pick("D", idx), pick("saved", idx),
                                 pick("scratch", idx), pick("dG", idx))

    def rank_grads():
        if opts.rank_grads:
            ttc.rank_grads_batch(mods, col("cores"), col("D"), col("dG"), col("dD"), RG_GAMMA, RG_BETA)

    def merge(idx):
        if idx:
            ttc.prepare_batch([mods[i] for i in idx], T, pick("cores", idx), pick("D", idx), pick("saved", idx))

    def step_single(ph):
        s = ph % n_sets
        ttm_fwd(ph)
        for L in layers:
            L["mod"].forward(L["x"][s], L["cores"], L["D"], out=L["y"], saved=L["saved"])
        for L in reversed(layers):
            L["mod"].backward(L["x"][s], L["dy"][s], L["cores"], L["D"], L["saved"], dx=L["dx"], dG=L["dG"],
                              scratch=L["scratch"])
        rank_grads()
        ttm_bwd(ph)

    def step_overlap(ph):
        # Merges depend only on the cores and D, the core-gradient tails
        # produce only dG.  The main stream carries the merges and then the
        # dependent chain of streaming passes (forward over the layers, dX
        # backward through them in reverse order, then the embedding's
        # backward).  The side stream carries the embedding lookup beside the
        # merges (the forwards wait for it), the next batch's index beside the
        # forwards, and the core-gradient tails after the last dX pass, beside
        # the embedding's backward.  With the index built in the step (no index
        # ahead) the lookup is the longer of the two and runs on the main
        # stream, the merges beside it.  Pipelined (an option, slower on
        # MI355X: the streaming passes place one work-group per CU and lose
        # whole CUs to the latency-bound tails beside them), only the first
        # forward group's layers are merged on the main stream, the others
        # beside that group's forward, and each backward group's tail runs as
        # soon as its data pass is done, beside the next group's passes.
        s = ph % n_sets
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        merged = torch.cuda.Event()
        if ttm is None:
            merge(first)
            with torch.cuda.stream(side):
                merge(rest)
                merged.record(side)
        elif ahead and not opts.merge_side:
            looked = torch.cuda.Event()
            with torch.cuda.stream(side):
                ttm_fwd(ph)
                looked.record(side)
                merge(rest)
                merged.record(side)
                ttm_index_next(ph)
            merge(first)
            main.wait_event(looked)
        else:
            with torch.cuda.stream(side):
                merge(every)
                merged.record(side)
                if ahead:
                    ttm_index_next(ph)
            ttm_fwd(ph)
            main.wait_event(merged)
        waited = False
        for g in fwd_groups:
            if not waited and any(i in rest for i in g):
                main.wait_event(merged)
                waited = True
            fwd_group(g, s)
        for g in bwd_groups:
            bwd_group(g, s)
            if opts.pipeline:
                side.wait_stream(main)
                with torch.cuda.stream(side):
                    cores_tail(g)
        side.wait_stream(main)
        ttm_bwd(ph)
        with torch.cuda.stream(side):
            if not opts.pipeline:
                cores_tail([i for g in bwd_groups for i in g])
            rank_grads()
        main.wait_stream(side)

    step = step_single if opts.single_stream else step_overlap
    if ahead:
        step.first_index = lambda: ttm["emb"].index(ttm["ids"][0], saved=ttm["saved2"][0])
    else:
        step.first_index = lambda: None
    return step, fwd_groups, bwd_groups


class Runner:
    """Runs a step eagerly or from captured HIP graphs, keeping the phase
    (input set and index buffer) alternating from one step to the next."""

    def __init__(self, step, eager=False, graph_steps=2):
        self.step, self.eager, self.graph_steps = step, eager, graph_steps
        self.ph = 0
        self.graphs = None
        step.first_index()

    def eager_steps(self, n):
        for _ in range(n):
            self.step(self.ph)
            self.ph ^= 1

    def capture(self, pair):
        import torch

        assert self.ph == 0
        self.pair = pair
        self.graphs = []
        for k in range(1 if pair else 2):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                if pair:
                    self.step(0)
                    self.step(1)
                else:
                    self.step(k)
            self.graphs.append(g)
        torch.cuda.synchronize()

    def replay_steps(self, n):
        """n steps from the graphs (n even with a two-step graph)."""
        if self.pair:
            assert n % 2 == 0 and self.ph == 0
            for _ in range(n // 2):
                self.graphs[0].replay()
        else:
            for _ in range(n):
                self.graphs[self.ph].replay()
                self.ph ^= 1


def time_step(step, steps, warmup, eager=False, graph_steps=2):
    """ms per step over exactly `steps` timed steps (HIP events around the whole
    run, after `warmup` untimed steps)."""
    import torch

    r = Runner(step, eager, graph_steps)
    w = max(2, warmup + (warmup & 1))  # even: the timed run starts at phase 0
    r.eager_steps(w)
    torch.cuda.synchronize()
    run = r.eager_steps
    pair = graph_steps == 2 and steps % 2 == 0
    if not eager:
        r.capture(pair)
        r.replay_steps(w)
        torch.cuda.synchronize()
        run = r.replay_steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    run(steps)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    info = {"launch": "eager" if eager else "hip_graph_replay",
            "steps_per_graph": None if eager else (2 if pair else 1)}
    return start.elapsed_time(end) / steps, wall, info, r


def trace_kernels(runner, steps):
    """Per-kernel HIP-event durations of `steps` eager steps (the library
    records a start and a stop event around every kernel on its stream)."""
    import torch

    import tensor_train_compressed_tt_amd as ttc

    if runner.ph:
        runner.eager_steps(1)
    torch.cuda.synchronize()
    ttc.trace_start()
    runner.eager_steps(steps)
    torch.cuda.synchronize()
    ttc.trace_stop()
    return ttc.trace_records()


def kernel_table(recs, steps, sizes, groups, ttm_sizes):
    """Per-kernel totals from trace records: ms, launches, algorithmic bytes."""
    fg, bg = groups
    layer_of = {"fwd": fg, "bwd_dy": bg, "bwd_dx": bg}
    per, counts = {}, {}
    for name, ms in recs:
        d = per.setdefault(name, {"ms": 0.0, "bytes": 0.0, "launches": 0})
        d["ms"] += ms
        k = counts.get(name, 0)
        counts[name] = k + 1
        d["launches"] += 1
        if name in layer_of:
            grp = layer_of[name][k % len(layer_of[name])]
            d["bytes"] += sum(sizes[i].get(name, 0) for i in grp)
        elif name in ttm_sizes:
            d["bytes"] += ttm_sizes[name]
    for name in layer_of:  # layers on the sequential order launch none of these
        assert counts.get(name, 0) in (0, len(layer_of[name]) * steps), (name, counts.get(name))
    for d in per.values():
        d["avg_us"] = 1e3 * d["ms"] / d["launches"]
        d["gbps"] = d["bytes"] / (d["ms"] / 1e3) / 1e9 if d["bytes"] else None
        d["ms_per_step"] = d["ms"] / steps
    return per


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    import synth

    cfg = args.config
    rank = args.rank if args.rank is not None else (64 if cfg == 4 else 30)
    T = args.tokens if args.tokens is not None else synth.CONFIG_TOKENS[cfg]
    if not 1 <= T <= 16384:
        sys.exit("--tokens must be in [1, 16384] (the embedding sorts at most 16384 ids per call)")
    dt = args.dtype or synth.CONFIG_DTYPE[cfg]
    es = {"f32": 4, "bf16": 2, "fp8": 1}[dt]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    n_layers = 6 * (args.layers if args.layers is not None else 24) if cfg == 4 else None
    cpu_T = None if args.no_cpu_baseline else min(T, args.cpu_tokens or (2048 if cfg == 4 else T))
    n_sets = 1 if args.one_input_set else N_SETS

    # ---- inputs, resident in HBM ----------------------------------------------------
    t_setup = time.perf_counter()
    layers, host = make_layers(cfg, rank, T, dev, n_sets=n_sets, keep_host=cpu_T is not None, n_layers=n_layers,
                               clone_encoders=(cfg == 4), path=args.path, dtype=dt)
    print(f"# {len(layers)} layers ready in {time.perf_counter() - t_setup:.1f} s", file=sys.stderr, flush=True)
    specs = [L["spec"] for L in layers]
    sizes = step_bytes(specs, [h["D"] for h in host], T, es)
    opts = StepOptions(single_stream=args.single_stream, qkv_batch=not args.no_qkv_batch,
                       index_ahead=not args.no_index_ahead, merge_side=args.merge_side, rank_grads=args.rank_grads,
                       pipeline=args.pipeline)
    tt_bytes = sum(s["fwd"] + s["bwd_dy"] + s["bwd_dx"] for s in sizes)

    # ---- headline: the TT-linear layers alone -----------------------------------------
    step, fg, bg = make_step(layers, T, None, opts)
    ms_per_step, wall, launch, runner = time_step(step, args.steps, args.warmup, args.eager, args.graph_steps)
    tokens_per_s = T / (ms_per_step / 1e3)
    step_gbps = tt_bytes / (ms_per_step / 1e3) / 1e9
    per = kernel_table(trace_kernels(runner, args.steps), args.steps, sizes, (fg, bg), {})
    stream_kernels = [k for k in ("fwd", "bwd_dy", "bwd_dx") if k in per]
    roof = None  # every layer on the sequential order: latency-bound, no streaming kernel
    if stream_kernels:
        dom = max(stream_kernels, key=lambda k: per[k]["ms"])
        roof = {
            "bound": "hbm",
            "kernel": dom,
            "achieved": round(per[dom]["gbps"], 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(per[dom]["gbps"] / HBM_PEAK_GBPS, 4),
            # the counter summaries were taken on the default workload only
            "traffic": measured_traffic(dom)
            if (cfg, rank, T, args.rank_grads, n_sets, dt) == (2, 30, 16384, False, 2, "bf16") else None,
            "avg_launch_us": round(per[dom]["avg_us"], 2),
            "algorithmic_bytes_per_launch": round(per[dom]["bytes"] / per[dom]["launches"]),
        }

    # ---- the same step with the embedding lookup and its backward ----------------------
    with_emb = None
    if not args.no_ttm:
        ttm, _ = make_ttm(T, dev, args.ttm_mode, n_sets=n_sets)
        stepe, fge, bge = make_step(layers, T, ttm, opts)
        ms_e, _, _, runner_e = time_step(stepe, args.steps, args.warmup, args.eager, args.graph_steps)
        ttm_sizes = {"ttm_sort": T * 8, "ttm_gather": T * ttm["dim"] * 4, "ttm_seg": T * ttm["dim"] * 4}
        pere = kernel_table(trace_kernels(runner_e, args.steps), args.steps, sizes, (fge, bge), ttm_sizes)
        tk = [k for k in pere if k.startswith("ttm_")]
        t_ms = sum(pere[k]["ms_per_step"] for k in tk)
        tb = sum(ttm_sizes.values())
        eb = tt_bytes + tb
        with_emb = {
            "ms_per_step": round(ms_e, 5), "tokens_per_s": round(T / (ms_e / 1e3), 1),
            "algorithmic_bytes_per_step": eb, "hbm_gbps_step": round(eb / (ms_e / 1e3) / 1e9, 1),
            "hbm_frac_step": round(eb / (ms_e / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
            "embedding_kernel_us_per_step": round(1e3 * t_ms, 2), "embedding_algorithmic_bytes": tb,
            "embedding_gbps": round(tb / (t_ms / 1e3) / 1e9, 1),
            "embedding_index": "built one step ahead on the side stream"
            if (opts.index_ahead and not opts.single_stream) else "built in the step's forward",
            "embedding": "TTM 32^3 x 768, modes (32,32,32)x(12,8,8), ranks (1,16,16,1), fp32, Zipf(1.1) ids, "
                         f"lookup mode {args.ttm_mode}",
            "kernels_us_per_step": {k: round(1e3 * v["ms_per_step"], 2) for k, v in pere.items()},
        }

    cpu = None
    if cpu_T is not None:
        cpu = cpu_baseline(host[:6], cpu_T)

    wl = {1: "one encoder's TT-linear set", 2: "one encoder's TT-linear set",
          4: "CodeBERT-large-sized encoder stack"}[cfg] + f", {dt}"
    shapes = "4x 768->768, 768->3072, 3072->768" if cfg != 4 else \
        f"{len(layers) // 6}x (4x 1024->1024, 1024->4096, 4096->1024)"
    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic",
        "config": {
            "workload": f"{wl}: {len(specs)} TT-linear layers (fwd then bwd in reverse), {shapes}, "
                        f"{dt} activations, fp32 accumulate, T={T} tokens, TT rank {rank}, "
                        f"{int(synth.CONFIG_ZERO_FRAC[cfg] * 100)}% of each link diagonal zeroed",
            "tokens": T,
            "rank": rank,
            "layers": len(specs),
            "input_sets": n_sets,
            "path": args.path,
            "planned": sorted({__import__("tensor_train_compressed_tt_amd").tt_linear_explain(L["mod"].desc, T).split()[0][5:]
                               for L in layers}),
            "qkv_batched": not (args.no_qkv_batch or args.single_stream),
            "rank_grads": bool(args.rank_grads),
            "streams": 1 if args.single_stream else 2,
            "pipelined_merges_and_tails": bool(args.pipeline and not args.single_stream),
            **launch,
        },
        "hbm_gbps_step": round(step_gbps, 1),
        "hbm_frac_step": round(step_gbps / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_step": tt_bytes,
        "kernels": {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in per.items()},
        "with_embedding": with_emb,
        "roofline": roof,
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
