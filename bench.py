#!/usr/bin/env python3
"""TT-linear fwd+bwd throughput on one MI355X.

One step = a TTM embedding lookup of the step's T ids (vocabulary 32^3 with
modes (32,32,32), rows of 768 = (12,8,8), ranks (1,16,16,1), Zipf(1.1) ids),
the forward pass of six TT-linear layers shaped like one encoder of the
CoMERA pages' six-encoder transformer (Q, K, V, O 768->768 with modes
(12,8,8)x(12,8,8); FFN 768->3072 and 3072->768 with 3072 = (12,16,16)),
their backward passes in reverse order (input gradients and core gradients)
and the embedding's backward into its core gradients, over T = 128 x 128 =
16384 tokens; TT-linear activations bf16 with fp32 accumulation, TT rank 30
with 40% of every link diagonal zeroed; the embedding is fp32.  Inputs are
seeded synthetic data already resident in HBM.  --no-ttm drops the
embedding from the step.

Prints one JSON line: the metric, the roofline of the dominant kernel and the
oracle's CPU baseline.  One GPU only: --gpus above 1 is refused.
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "TT-linear fwd+bwd tokens/sec at d=768 r=30; achieved HBM GB/s % of peak"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, vendor figure
RG_GAMMA, RG_BETA = 1e-3, 1e-5  # early-stage penalty weights for --rank-grads (values do not change the cost)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 4])
    ap.add_argument("--rank", type=int, default=None)
    ap.add_argument("--layers", type=int, default=None, help="with --config 4: number of encoder layers")
    ap.add_argument("--tokens", type=int, default=None,
                    help="tokens per step instead of the config's (batch x 128-token sequences, e.g. 128 for batch 1)")
    ap.add_argument("--eager", action="store_true", help="launch every call from Python instead of replaying a HIP graph")
    ap.add_argument("--single-stream", action="store_true",
                    help="run merges and core-gradient tails on the main stream too (no overlap)")
    ap.add_argument("--no-ttm", action="store_true", help="time the TT-linear layers only")
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
    ap.add_argument("--no-qkv-batch", action="store_true",
                    help="one launch per layer for the Q, K and V projections instead of one batched launch")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=1024)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device to device three times (scale for the HBM byte counters)")
    return ap.parse_args()


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


def step_bytes(layers, T, es):
    """Algorithmic HBM bytes of one fwd+bwd per layer (kernel-level split).

    fwd:    read x, write Y, write Z (T x r_eff fp32)
    bwd_dy: read dY, read Z
    bwd_dx: read x, write dX
    """
    out = []
    for L in layers:
        s = L["spec"]
        r_eff = int((L["D"][len(s.out_modes) - 1 if not s.in_first else len(s.in_modes) - 1] != 0).sum())
        out.append({
            "fwd": T * (s.n_in + s.n_out) * es + T * r_eff * 4,
            "bwd_dy": T * s.n_out * es + T * r_eff * 4,
            "bwd_dx": T * 2 * s.n_in * es,
            "r_eff": r_eff,
        })
    return out


def cpu_baseline(layers_host, T_cpu, ttm_host=None):
    """The fp64 oracle, as it stands, on the first T_cpu tokens of every layer
    (and of the embedding lookup when the step has one)."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    t0 = time.perf_counter()
    for L in layers_host:
        s = L["spec"]
        x = L["x"][:T_cpu].astype(np.float64)
        dy = L["dy"][:T_cpu].astype(np.float64)
        oracle.tt_linear_forward(x, s.out_modes, s.in_modes, L["cores"], L["D"], s.in_first)
        oracle.tt_linear_backward(x, dy, s.out_modes, s.in_modes, L["cores"], L["D"], s.in_first)
    what = f"all {len(layers_host)} TT-linear layers"
    if ttm_host is not None:
        oracle.ttm_forward(ttm_host["ids"][:T_cpu], ttm_host["cores"])
        oracle.ttm_backward(ttm_host["ids"][:T_cpu], ttm_host["dout"][:T_cpu], ttm_host["cores"])
        what = "the TTM embedding lookup and " + what
    dt = time.perf_counter() - t0
    return {"value": T_cpu / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 oracle fwd+bwd of {what} on the first {T_cpu} tokens "
                      f"({dt:.1f} s wall)"}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import synth
    import tensor_train_compressed_tt_amd as ttc

    cfg = args.config
    rank = args.rank if args.rank is not None else (64 if cfg == 4 else 30)
    T = args.tokens if args.tokens is not None else synth.CONFIG_TOKENS[cfg]
    if not 1 <= T <= 16384:
        sys.exit("--tokens must be in [1, 16384] (the embedding sorts at most 16384 ids per call)")
    zf = synth.CONFIG_ZERO_FRAC[cfg]
    dt = synth.CONFIG_DTYPE[cfg]
    specs = synth.config_layers(cfg, rank)
    if cfg == 4 and args.layers is not None:
        specs = specs[: 6 * args.layers]
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    es = 2 if dt == "bf16" else 4
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- inputs, resident in HBM ------------------------------------------------
    layers, host = [], []
    max_scratch = 0
    for li, spec in enumerate(specs):
        L = synth.make_tt_layer(cfg, li, spec, T, zf, dt)
        mod = ttc.TTLinear(spec.out_modes, spec.in_modes, spec.ranks, tdt, spec.in_first)
        cores = [torch.from_numpy(c).to(dev) for c in L["cores"]]
        D = [torch.from_numpy(v).to(dev) for v in L["D"]]
        if dt == "bf16":
            x = torch.from_numpy(L["x_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
            dy = torch.from_numpy(L["dy_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            x = torch.from_numpy(L["x"]).to(dev)
            dy = torch.from_numpy(L["dy"]).to(dev)
        sb, cb = mod.workspace(T)
        max_scratch = max(max_scratch, cb)
        layers.append({
            "scratch": torch.empty(cb, dtype=torch.uint8, device=dev) if not args.single_stream else None,
            "spec": spec, "mod": mod, "cores": cores, "D": D, "x": x, "dy": dy,
            "y": torch.empty((T, spec.n_out), dtype=tdt, device=dev),
            "dx": torch.empty((T, spec.n_in), dtype=tdt, device=dev),
            "dG": [torch.empty(s, dtype=torch.float32, device=dev) for s in mod.core_shapes],
            "dD": [torch.empty(v.shape, dtype=torch.float32, device=dev) for v in D],
            "saved": torch.empty(sb, dtype=torch.uint8, device=dev),
        })
        keep = {"spec": spec, "cores": L["cores"], "D": L["D"]}
        if not args.no_cpu_baseline and len(host) < 6:
            keep["x"] = L["x"][: args.cpu_tokens].copy()
            keep["dy"] = L["dy"][: args.cpu_tokens].copy()
        host.append(keep)
        del L
    scratch = torch.empty(max_scratch, dtype=torch.uint8, device=dev) if args.single_stream else None
    sizes = step_bytes(host, T, es)

    # ---- the embedding lookup of the step's T ids ------------------------------
    ttm = None
    ttm_host = None
    if not args.no_ttm:
        w = synth.make_ttm(3, T=T)
        sp = w["spec"]
        emb = ttc.TTMEmbedding(sp.vocab_modes, sp.dim_modes, sp.ranks,
                               mode={"dedup": 0, "unique": 1, "plain": 2}[args.ttm_mode])
        tsb, tcb = emb.workspace(T)
        ttm = {"emb": emb, "F": [torch.from_numpy(c).to(dev) for c in w["cores"]],
               "ids": torch.from_numpy(w["ids"]).to(dev), "dout": torch.from_numpy(w["dout"]).to(dev),
               "out": torch.empty((T, sp.dim), dtype=torch.float32, device=dev),
               "dF": [torch.empty(c.shape, dtype=torch.float32, device=dev) for c in w["cores"]],
               "saved": torch.empty(tsb, dtype=torch.uint8, device=dev),
               # the index of the next step's ids is built into the other buffer
               "saved2": [torch.empty(tsb, dtype=torch.uint8, device=dev) for _ in range(2)],
               "scratch": torch.empty(tcb, dtype=torch.uint8, device=dev), "d": len(sp.vocab_modes),
               "dim": sp.dim}
        if not args.no_cpu_baseline:
            ttm_host = {"ids": w["ids"][: args.cpu_tokens].copy(), "dout": w["dout"][: args.cpu_tokens].copy(),
                        "cores": w["cores"]}
        del w

    ahead = ttm is not None and not args.no_index_ahead and not args.single_stream
    phase = [0]  # which of the two index buffers the current step looks up

    def ttm_saved():
        return ttm["saved2"][phase[0]] if ahead else ttm["saved"]

    def ttm_fwd():
        if ttm is None:
            return
        if ahead:
            ttm["emb"].lookup(T, ttm["F"], None, ttm_saved(), out=ttm["out"], scratch=ttm["scratch"])
        else:
            ttm["emb"].forward(ttm["ids"], ttm["F"], None, out=ttm["out"], saved=ttm["saved"],
                               scratch=ttm["scratch"])

    def ttm_index_next():
        # the next step's ids are known before it starts (this synthetic
        # workload repeats the same batch)
        ttm["emb"].index(ttm["ids"], saved=ttm["saved2"][1 - phase[0]])

    def ttm_bwd():
        if ttm is not None:
            ttm["emb"].backward(ttm["ids"], ttm["dout"], ttm["F"], None, ttm_saved(), dF=ttm["dF"],
                                scratch=ttm["scratch"])
    side = torch.cuda.Stream()  # default priority

    def step_single():
        ttm_fwd()
        for L in layers:
            L["mod"].forward(L["x"], L["cores"], L["D"], out=L["y"], saved=L["saved"])
        for L in reversed(layers):
            L["mod"].backward(L["x"], L["dy"], L["cores"], L["D"], L["saved"], dx=L["dx"], dG=L["dG"],
                              scratch=scratch)
        ttm_bwd()

    mods = [L["mod"] for L in layers]
    all_cores = [L["cores"] for L in layers]
    all_D = [L["D"] for L in layers]
    # Launch groups of the streaming passes.  Within one encoder the Q, K and V
    # projections are independent (same input, separate outputs), so each of
    # their passes is one batched launch; O, FFN1 and FFN2 depend on what comes
    # before them in the encoder and run one after another.
    fwd_groups = []
    for e in range(len(layers) // 6):
        qkv = [6 * e, 6 * e + 1, 6 * e + 2]
        fwd_groups += ([[i] for i in qkv] if args.no_qkv_batch else [qkv]) + [[6 * e + 3], [6 * e + 4], [6 * e + 5]]
    bwd_groups = [g[::-1] for g in fwd_groups[::-1]]

    def fwd_group(g):
        if len(g) == 1:
            L = layers[g[0]]
            L["mod"].forward(L["x"], L["cores"], L["D"], out=L["y"], saved=L["saved"], prepared=True)
        else:
            Ls = [layers[i] for i in g]
            ttc.forward_batch([L["mod"] for L in Ls], [L["x"] for L in Ls], [L["cores"] for L in Ls],
                              [L["D"] for L in Ls], [L["y"] for L in Ls], [L["saved"] for L in Ls], prepared=True)

    def bwd_group(g):
        if len(g) == 1:
            L = layers[g[0]]
            L["mod"].backward_data(L["x"], L["dy"], L["cores"], L["D"], L["saved"], L["scratch"], dx=L["dx"])
        else:
            Ls = [layers[i] for i in g]
            ttc.backward_data_batch([L["mod"] for L in Ls], [L["x"] for L in Ls], [L["dy"] for L in Ls],
                                    [L["cores"] for L in Ls], [L["D"] for L in Ls], [L["saved"] for L in Ls],
                                    [L["scratch"] for L in Ls], [L["dx"] for L in Ls])

    def step_overlap():
        # The merges depend only on the cores and D, the core-gradient tails
        # produce only dG; each is one batched call for all layers.  The main
        # stream carries the merges and then the dependent chain of streaming
        # passes (forward over the layers, dX backward through them in reverse
        # order, then the embedding's backward).  The side stream carries the
        # embedding lookup beside the merges (the forwards wait for it), the
        # next batch's index beside the forwards, and the tails after the last
        # dX pass, beside the embedding's backward, so no side-stream work sits
        # between two streaming passes.  With the index built in the step
        # (no index ahead) the lookup is the longer of the two and runs on the
        # main stream, the merges beside it.
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        if ahead and not args.merge_side:
            # the lookup of the already indexed batch (shorter than the merges)
            # on the side stream, then the index of the next batch (sort,
            # distinct ids, prefix tree) beside this step's streaming passes;
            # the forwards follow the merges on the main stream
            looked = torch.cuda.Event()
            with torch.cuda.stream(side):
                ttm_fwd()
                looked.record(side)
                ttm_index_next()
            ttc.prepare_batch(mods, T, all_cores, all_D, [L["saved"] for L in layers])
            main.wait_event(looked)
        else:
            merged = torch.cuda.Event()
            with torch.cuda.stream(side):
                ttc.prepare_batch(mods, T, all_cores, all_D, [L["saved"] for L in layers])
                merged.record(side)
                if ahead:
                    ttm_index_next()
            ttm_fwd()
            main.wait_event(merged)
        for g in fwd_groups:
            fwd_group(g)
        for g in bwd_groups:
            bwd_group(g)
        side.wait_stream(main)
        ttm_bwd()
        with torch.cuda.stream(side):
            ttc.backward_cores_batch(mods[::-1], T, all_cores[::-1], all_D[::-1],
                                     [L["saved"] for L in layers][::-1], [L["scratch"] for L in layers][::-1],
                                     [L["dG"] for L in layers][::-1])
            if args.rank_grads:
                ttc.rank_grads_batch(mods, all_cores, all_D, [L["dG"] for L in layers], [L["dD"] for L in layers],
                                     RG_GAMMA, RG_BETA)
        main.wait_stream(side)
        phase[0] = 1 - phase[0]

    step = step_single if args.single_stream else step_overlap

    # ---- warm-up, optional graph capture --------------------------------------------
    if ahead:
        ttm["emb"].index(ttm["ids"], saved=ttm["saved2"][0])  # the first step's index
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    graph = None
    if not args.eager:
        # with the index built one step ahead, the step alternates between two
        # index buffers: one graph per phase, replayed in turn, or one graph of
        # both steps (no drain between the two)
        pair = args.graph_steps == 2 and args.steps % 2 == 0
        graphs = []
        for _ in range(1 if pair else 2 if ahead else 1):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step()
                if pair:
                    step()
            graphs.append(g)
        torch.cuda.synchronize()
        turn = [0]

        def replay():
            graphs[turn[0]].replay()
            turn[0] = (turn[0] + 1) % len(graphs)

        graph = graphs[0]
        for _ in range(max(1, args.warmup) * len(graphs)):
            replay()
        torch.cuda.synchronize()
    run = replay if graph is not None else step
    launches = args.steps // 2 if graph is not None and pair else args.steps

    # ---- timed region -----------------------------------------------------------------
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(launches):
        run()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = start.elapsed_time(end) / args.steps
    tokens_per_s = T / (ms_per_step / 1e3)
    bytes_per_step = sum(s["fwd"] + s["bwd_dy"] + s["bwd_dx"] for s in sizes)
    # embedding: read the ids, write the rows; read the row gradients
    ttm_sizes = {} if ttm is None else {"ttm_sort": T * 8, "ttm_gather": T * ttm["dim"] * 4,
                                        "ttm_seg": T * ttm["dim"] * 4}
    bytes_per_step += sum(ttm_sizes.values())
    step_gbps = bytes_per_step / (ms_per_step / 1e3) / 1e9

    # ---- per-kernel durations: the same steps, launched eagerly with HIP events
    # recorded by the library around every kernel on its launch stream -----------------
    ttc.trace_start()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ttc.trace_stop()
    recs = ttc.trace_records()
    per = {}
    # layers of the k-th launch of a streaming kernel within one step: the
    # forward runs over the launch groups in order, the backward passes in
    # reverse (one launch per layer in the single-stream step)
    nl = len(layers)
    if args.single_stream:
        fg = [[i] for i in range(nl)]
        bg = fg[::-1]
    else:
        fg, bg = fwd_groups, bwd_groups
    layer_of = {"fwd": fg, "bwd_dy": bg, "bwd_dx": bg}
    ttm_names = {"ttm_sort", "ttm_lists", "ttm_level", "ttm_gather", "ttm_seg", "ttm_bwd_level", "ttm_reduce"}
    counts = {}
    for name, ms in recs:
        d = per.setdefault(name, {"ms": 0.0, "bytes": 0.0, "launches": 0})
        d["ms"] += ms
        k = counts.get(name, 0)
        counts[name] = k + 1
        d["launches"] += 1
        if name in layer_of:
            grp = layer_of[name][k % len(layer_of[name])]
            d["bytes"] += sum(sizes[i].get(name, 0) for i in grp)
        elif name in ttm_names:
            d["bytes"] += ttm_sizes.get(name, 0)
    for name in layer_of:
        assert counts.get(name, 0) == len(layer_of[name]) * args.steps, (name, counts.get(name))
    for d in per.values():
        d["avg_us"] = 1e3 * d["ms"] / d["launches"]
        d["gbps"] = d["bytes"] / (d["ms"] / 1e3) / 1e9 if d["bytes"] else None
        d["ms_per_step"] = d["ms"] / args.steps
    stream_kernels = ["fwd", "bwd_dy", "bwd_dx"]
    dom = max(stream_kernels, key=lambda k: per[k]["ms"])
    roof = {
        "bound": "hbm",
        "kernel": dom,
        "achieved": round(per[dom]["gbps"], 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(per[dom]["gbps"] / HBM_PEAK_GBPS, 4),
        # the counter summaries were taken on the default workload only
        "traffic": measured_traffic(dom) if (cfg, rank, T, args.rank_grads) == (2, 30, 16384, False) else None,
        "avg_launch_us": round(per[dom]["avg_us"], 2),
        "algorithmic_bytes_per_launch": round(per[dom]["bytes"] / per[dom]["launches"]),
    }

    ttm_summary = None
    if ttm is not None:
        tk = [k for k in per if k.startswith("ttm_")]
        t_ms = sum(per[k]["ms_per_step"] for k in tk)
        tb = sum(ttm_sizes.values())
        ttm_summary = {"kernel_us_per_step": round(1e3 * t_ms, 2), "algorithmic_bytes": tb,
                       "gbps": round(tb / (t_ms / 1e3) / 1e9, 1)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(host[:6], min(args.cpu_tokens, T), ttm_host)

    wl = {1: "one encoder's TT-linear set, fp32", 2: "one encoder's TT-linear set, bf16",
          4: "CodeBERT-large-sized encoder stack"}[cfg]
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
            "workload": f"{wl}{'' if ttm is None else ' + TTM embedding lookup of the same tokens'}: {len(specs)} TT-linear layers (fwd then bwd in reverse), "
                        f"{'4x 768->768, 768->3072, 3072->768' if cfg != 4 else '24x (4x 1024->1024, 1024->4096, 4096->1024)'}, "
                        f"{dt} activations, fp32 accumulate, T={T} tokens, TT rank {rank}, "
                        f"{int(zf * 100)}% of each link diagonal zeroed",
            "tokens": T,
            "rank": rank,
            "layers": len(specs),
            "launch": "eager" if graph is None else "hip_graph_replay",
            "steps_per_graph": None if graph is None else (2 if pair else 1),
            "qkv_batched": not (args.no_qkv_batch or args.single_stream),
            "embedding_index": None if ttm is None else ("built one step ahead on the side stream" if ahead
                                                         else "built in the step's forward"),
            "merges": "side stream, beside the embedding lookup" if (args.merge_side or not ahead)
                      else "main stream, the embedding lookup beside them on the side stream",
            "rank_grads": bool(args.rank_grads and not args.single_stream),
            "streams": 1 if args.single_stream else 2,
            "embedding": None if ttm is None else "TTM 32^3 x 768, modes (32,32,32)x(12,8,8), ranks (1,16,16,1), "
                                                  f"fp32, Zipf(1.1) ids, lookup mode {args.ttm_mode}",
        },
        "hbm_gbps_step": round(step_gbps, 1),
        "hbm_frac_step": round(step_gbps / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_step": bytes_per_step,
        "kernels": {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in per.items()},
        "embedding": ttm_summary,
        "roofline": roof,
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
