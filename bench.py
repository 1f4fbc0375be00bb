"""Benchmark of the N:M sparse x dense product on one MI355X.

Default workload: ViT-B/16 FC1 at batch 64 -- W 3072x768 int8 at 2:4,
X 768x12608 int8, fused bias + requant to int8 (the headline metric).  A
step is one nm_spmm call (load, decode, sparse MFMA, epilogue, store) over
one batch; the weights are packed once beforehand (nm_pack is offline, timed
separately and reported as `pack_ms`).  Inputs rotate over >= 1 GiB of
independent buffer sets so no timed call is served from the 256 MB
Infinity Cache.

Prints ONE JSON line on stdout.  `roofline.achieved` is the algorithmic
bytes of one launch divided by the average launch duration measured with HIP
events around the timed launches (on the stream the kernel runs on);
`cpu_baseline` times the CPU oracle on a bounded row sample of the same
workload.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0                              # MI355X HBM3E
MFMA_PEAK_TOPS = {"i8": 5000.0, "f16": 2500.0, "bf16": 2500.0}   # dense, per dtype
METRIC = "N:M SpMM dense-equivalent TOPS + % of MI355X roofline (int8 2:4, ViT-B FC1)"


def _layers():
    import nm_inputs
    out = {nm_inputs.headline().name: nm_inputs.headline()}
    for layers in nm_inputs.all_configs().values():
        for L in layers:
            out.setdefault(L.name, L)
    return out


def _traffic(kernel_name: str, launches_per_step: int = 1):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(kernel_name)
    except ValueError:
        return None
    if not rec or rec.get("source_sha") != _source_sha(kernel_name):
        return None
    return rec.get("bytes_per_launch")


# the source files a kernel variant is built from (its counters go stale
# when one of them changes); variants not listed hash every source
KERNEL_SOURCES = {
    "smfmac_i8_2of4_persistent": ["semi_structured_sparse_nm_amd/csrc/nm_spmm_smfmac_i8p.hip",
                                  "semi_structured_sparse_nm_amd/csrc/nm_common.hpp", "include/nm_sparse.h"],
    "smfmac_i8_2of4_stationary": ["semi_structured_sparse_nm_amd/csrc/nm_spmm_smfmac_i8ws.hip",
                                  "semi_structured_sparse_nm_amd/csrc/nm_common.hpp", "include/nm_sparse.h"],
}


def _source_sha(kernel_name: str = "") -> str:
    h = hashlib.sha256()
    files = KERNEL_SOURCES.get(kernel_name)
    if files is None:
        csrc = os.path.join("semi_structured_sparse_nm_amd", "csrc")
        files = [os.path.join(csrc, f) for f in sorted(os.listdir(os.path.join(ROOT, csrc)))]
    for f in files:
        h.update(os.path.basename(f).encode())
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def cpu_baseline(L, inp, target_s: float = 12.0):
    """Time the CPU oracle (direct compressed loop + epilogue) on a row sample."""
    import numpy as np
    import oracle
    vals, idx = oracle.compress(inp["W"], L.N, L.M, L.dt)
    threads = oracle.max_threads()

    def run(rows):
        t = time.perf_counter()
        acc = oracle.spmm_direct(vals, idx, inp["X"], L.R, L.K, L.N, L.M, L.dt, rows=rows)
        if L.out == "i8":
            oracle.requant_i8(acc, inp["bias"][rows], inp["scale"][rows])
        return time.perf_counter() - t

    n = max(threads, 8)
    rows = np.arange(n) % L.R
    dt = run(rows)
    n2 = int(min(L.R, max(n, n * target_s / max(dt, 1e-3) * 0.8)))
    n2 = max(threads, (n2 // threads) * threads)
    rows = (np.arange(n2) * (L.R // max(1, n2))) % L.R
    # repeat the sample until about target_s of CPU time has been measured
    reps, total = 0, 0.0
    while total < target_s and reps < 100:
        total += run(rows)
        reps += 1
    dense_ops = 2.0 * L.K * L.T * n2 * reps
    return {"value": dense_ops / total / 1e12, "unit": "TOPS (dense-equivalent)", "cores": threads,
            "kind": "oracle",
            "sample": f"{n2} of {L.R} rows x all {L.T} tokens of {L.name}, {reps} pass(es) "
                      f"(direct compressed-index loop + epilogue, {total:.1f} s)"}


def run_stack(args):
    """The 48-layer mixed-N:M ViT-B int8 stack (12 blocks x qkv / proj / fc1 /
    fc2, per-layer N:M drawn with seed 0), run back to back on one stream.

    Reports every layer's time (a HIP graph of `reps` launches of that layer
    alone), their sum, and the time of one pass of the whole stack (a HIP
    graph of the 48 launches in order, replayed).  Inputs are seeded int8
    tensors drawn on the GPU (timing only; parity of every shape is covered
    by the tests)."""
    import torch

    import nm_inputs
    import semi_structured_sparse_nm_amd as nm

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev)
    layers = nm_inputs.config4()
    built = []
    for i, L in enumerate(layers):
        gen.manual_seed(1000 + i)
        W = torch.randint(-127, 128, (L.R, L.K), dtype=torch.int8, device=dev, generator=gen)
        X = torch.randint(-127, 128, (L.K, L.T), dtype=torch.int8, device=dev, generator=gen)
        b = torch.randint(-2000, 2000, (L.R,), dtype=torch.int32, device=dev, generator=gen)
        sc = torch.full((L.R,), 1.0 / 4096, dtype=torch.float32, device=dev)
        p = nm.pack(W, L.N, L.M)
        Y = torch.empty((L.R, L.T), dtype=torch.int8, device=dev)
        built.append((L, p, X, b, sc, Y))
    torch.cuda.synchronize()

    def launch(item):
        L, p, X, b, sc, Y = item
        nm.spmm(p, X, bias=b, scale=sc, out_dtype=torch.int8, out=Y)

    def graph_time(items, reps):
        for it in items:
            launch(it)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            with torch.cuda.graph(g, stream=st):
                for _ in range(reps):
                    for it in items:
                        launch(it)
        torch.cuda.current_stream().wait_stream(st)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps      # microseconds per repetition

    per = []
    for it in built:
        L = it[0]
        us = graph_time([it], 20)
        ops, nbytes, dense = nm_inputs.ops_and_bytes(L)
        t_roof = max(nbytes / 8e12, ops / 5e15) * 1e6
        per.append({"layer": L.name, "R": L.R, "K": L.K, "N": L.N, "M": L.M,
                    "kernel": nm.variant(it[1], L.T, torch.int8), "us": round(us, 2),
                    "t_roof_us": round(t_roof, 3), "roofline_fraction": round(t_roof / us, 4)})
    pass_us = graph_time(built, 5)
    dense_total = sum(nm_inputs.ops_and_bytes(L)[2] for L in layers)
    roof_total = sum(r["t_roof_us"] for r in per)
    out = {"stack": "vitb_int8_mixed_nm_48_layers", "tokens": nm_inputs.VIT_B_TOKENS,
           "pass_us": round(pass_us, 1), "sum_of_layers_us": round(sum(r["us"] for r in per), 1),
           "sum_of_rooflines_us": round(roof_total, 1), "roofline_fraction": round(roof_total / pass_us, 4),
           "dense_equivalent_TOPS": round(dense_total / (pass_us * 1e-6) / 1e12, 1),
           "layers": per}
    text = json.dumps(out)
    if args.details:
        json.dump(out, open(args.details, "w"), indent=1)
    print(text, flush=True)


def run_sweep(args):
    """Every layer of the single-layer workloads (ViT-Tiny slice, ViT-B int8 at
    four N:M, Swin-T fp16 stages, LLaMA-7B fp16 / bf16 decode and prefill),
    each timed on its own: inputs drawn on the GPU (timing only; parity of
    every shape is covered by the tests), buffer sets rotated over
    `--rotate-gib` so no timed launch is served from the Infinity Cache, a HIP
    graph of `reps` launches replayed.  One JSON line per layer, then a
    summary line."""
    import torch

    import nm_inputs
    import semi_structured_sparse_nm_amd as nm

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev)
    tdt = {"i8": torch.int8, "f16": torch.float16, "bf16": torch.bfloat16, "i32": torch.int32,
           "f32": torch.float32}
    cfgs = nm_inputs.all_configs()
    want = [c for c in args.sweep.split(",") if c]
    rows = []
    for cfg in want:
        for i, L in enumerate(cfgs[cfg]):
            gen.manual_seed(2000 + 100 * int(cfg) + i)
            if L.dt == "i8":
                W = torch.randint(-127, 128, (L.R, L.K), dtype=torch.int8, device=dev, generator=gen)
            else:
                W = (torch.randn((L.R, L.K), device=dev, generator=gen) * 0.02).to(tdt[L.dt])
            p = nm.pack(W, L.N, L.M)
            del W
            bias = scale = None
            if L.out == "i8":
                bias = torch.randint(-2000, 2000, (L.R,), dtype=torch.int32, device=dev, generator=gen)
                scale = torch.full((L.R,), 1.0 / 4096, dtype=torch.float32, device=dev)
            ebx = torch.empty(0, dtype=tdt[L.dt]).element_size()
            eby = torch.empty(0, dtype=tdt[L.out]).element_size()
            footprint = p.values.numel() + (0 if p.meta is None else p.meta.numel()) + \
                L.K * L.T * ebx + L.R * L.T * eby
            nsets = max(2, math.ceil(args.rotate_gib * 2**30 / footprint))
            sets = []
            for _ in range(nsets):
                if L.dt == "i8":
                    X = torch.randint(-127, 128, (L.K, L.T), dtype=torch.int8, device=dev, generator=gen)
                else:
                    X = torch.randn((L.K, L.T), device=dev, generator=gen).to(tdt[L.dt])
                pm = None if p.meta is None else p.meta.clone()
                ps = nm.Packed(p.rows, p.K, p.N, p.M, p.dtype, p.values.clone(), pm, p.format_version)
                sets.append((ps, X, torch.empty((L.R, L.T), dtype=tdt[L.out], device=dev)))
            need = nm.workspace_size(p, L.T, tdt[L.out])
            ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
            reps = max(nsets, 20)

            def launch(j):
                ps, X, Y = sets[j % nsets]
                nm.spmm(ps, X, bias=bias, scale=scale, out_dtype=tdt[L.out], out=Y, workspace=ws)

            for j in range(nsets):
                launch(j)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            st = torch.cuda.Stream()
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                with torch.cuda.graph(g, stream=st):
                    for j in range(reps):
                        launch(j)
            torch.cuda.current_stream().wait_stream(st)
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            ops, nbytes, dense = nm_inputs.ops_and_bytes(L)
            t_hbm = nbytes / (HBM_PEAK_GBS * 1e9) * 1e6
            t_mfma = ops / (MFMA_PEAK_TOPS[L.dt] * 1e12) * 1e6
            row = {"config": cfg, "layer": L.name, "R": L.R, "K": L.K, "T": L.T, "N": L.N, "M": L.M,
                   "in": L.dt, "out": L.out, "kernel": nm.variant(p, L.T, tdt[L.out]), "us": round(us, 2),
                   "bound": "hbm" if t_hbm >= t_mfma else "mfma", "t_roof_us": round(max(t_hbm, t_mfma), 3),
                   "roofline_fraction": round(max(t_hbm, t_mfma) / us, 4),
                   "dense_equivalent_TOPS": round(dense / (us * 1e-6) / 1e12, 1),
                   "effective_GBps": round(nbytes / (us * 1e-6) / 1e9, 1), "rotation_sets": nsets}
            rows.append(row)
            print(json.dumps(row), flush=True)
            del sets, g, ws, p
            torch.cuda.empty_cache()
    summary = {"sweep": want, "layers": len(rows),
               "sum_us": round(sum(r["us"] for r in rows), 1),
               "sum_roof_us": round(sum(r["t_roof_us"] for r in rows), 1)}
    summary["roofline_fraction_of_sums"] = round(summary["sum_roof_us"] / max(summary["sum_us"], 1e-9), 4)
    print(json.dumps(summary), flush=True)
    if args.details:
        json.dump({"summary": summary, "layers": rows}, open(args.details, "w"), indent=1)


def run_lut(args):
    """Latency look-up table for the mixed-N:M ViT-B stack: measure every
    (layer shape, N:M) of the stack's choice set, time stacks of four
    different seeded N:M draws, calibrate the per-launch gap on the first
    and report how well the table predicts the other three."""
    import torch

    import nm_inputs
    from semi_structured_sparse_nm_amd.lut import LayerShape, measure_layers, time_stack

    torch.cuda.set_device(0)
    T = nm_inputs.VIT_B_TOKENS
    choices = [(1, 4), (2, 4), (4, 8), (8, 8)]
    shapes = [LayerShape(R, K, T, n, m) for (R, K) in nm_inputs.VIT_B_LAYERS.values() for n, m in choices]
    lut = measure_layers(shapes, reps=20)
    print(json.dumps({"lut_entries": len(lut)}), file=sys.stderr, flush=True)

    def stack(seed):
        out = []
        for i, (n, m) in enumerate(nm_inputs.stack_nm(seed)):
            R, K = list(nm_inputs.VIT_B_LAYERS.values())[i % 4]
            out.append(LayerShape(R, K, T, n, m))
        return out

    measured = {}
    for seed in range(4):
        measured[seed] = time_stack(stack(seed), reps=3, seed=seed)
        print(json.dumps({"stack_seed": seed, "measured_us": round(measured[seed], 1)}), file=sys.stderr, flush=True)
    raw = {seed: lut.predict(stack(seed)) for seed in range(4)}
    gap = lut.calibrate(stack(0), measured[0])
    val = []
    for seed in range(1, 4):
        pred = lut.predict(stack(seed))
        val.append({"seed": seed, "measured_us": round(measured[seed], 1), "predicted_us": round(pred, 1),
                    "uncalibrated_us": round(raw[seed], 1),
                    "error": round((pred - measured[seed]) / measured[seed], 4)})
    out = {"lut": "vitb_int8_mixed_nm_stack", "entries": len(lut), "tokens": T,
           "calibration": {"seed": 0, "measured_us": round(measured[0], 1), "gap_us_per_launch": round(gap, 2)},
           "validation": val,
           "max_abs_error": round(max(abs(v["error"]) for v in val), 4)}
    print(json.dumps(out), flush=True)
    if args.details:
        json.dump({"result": out, "lut": json.loads(lut.to_json())}, open(args.details, "w"), indent=1)


def run_chain(args):
    """The ViT-B MLP in int8 on the device: FC1 (3072 x 768, 2:4) with GELU
    fused and requantised to int8, whose [3072][T] output is FC2's (768 x
    3072, 2:4) activation as it stands, T = 12608.  Timed as HIP-graph
    replays over rotated operand sets (>= 1 GiB, every set with its own
    packed weights): the two-layer chain, FC1 with GELU alone, FC1 with the
    plain requantisation alone (the activation's cost is the difference) and
    FC2 alone.  Inputs follow nm_inputs.mlp_chain; parity of this
    configuration is covered by the tests (sampled token columns at full
    size)."""
    import torch

    import nm_inputs
    import semi_structured_sparse_nm_amd as nm

    import numpy as np

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    T = nm_inputs.VIT_B_TOKENS
    c = nm_inputs.mlp_chain(3072, 768, T, 2, 4, 0, "vitb_mlp")
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    p1, p2 = nm.pack(d(c.W1), 2, 4), nm.pack(d(c.W2), 2, 4)
    X0, b1, s1, b2, s2 = d(c.X), d(c.b1), d(c.s_deq1), d(c.b2), d(c.scale2)
    foot = 3072 * 768 // 2 * 5 // 4 + 768 * 3072 // 2 * 5 // 4 + 768 * T + 3072 * T + 768 * T
    nsets = max(2, math.ceil(args.rotate_gib * 2**30 / foot))
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)

    def clone(p):
        return nm.Packed(p.rows, p.K, p.N, p.M, p.dtype, p.values.clone(),
                         None if p.meta is None else p.meta.clone(), p.format_version)

    sets = []
    for i in range(nsets):
        X = X0 if i == 0 else X0[:, torch.randperm(T, device=dev, generator=gen)].contiguous()
        sets.append((clone(p1), clone(p2), X, torch.empty((3072, T), dtype=torch.int8, device=dev),
                     torch.empty((768, T), dtype=torch.int8, device=dev)))
    torch.cuda.synchronize()

    def fc1(j, act="gelu"):
        q1, q2, X, H, Y = sets[j % nsets]
        nm.spmm(q1, X, bias=b1, scale=s1, out_dtype=torch.int8, out=H, act=act, out_scale=c.os1)

    def fc2(j):
        q1, q2, X, H, Y = sets[j % nsets]
        nm.spmm(q2, H, bias=b2, scale=s2, out_dtype=torch.int8, out=Y)

    def graph_us(fn, reps):
        for j in range(nsets):
            fn(j)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            with torch.cuda.graph(g, stream=st):
                for j in range(reps):
                    fn(j)
        torch.cuda.current_stream().wait_stream(st)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    reps = max(nsets, 20)
    chain = graph_us(lambda j: (fc1(j), fc2(j)), reps)
    fc1_gelu = graph_us(fc1, reps)
    fc1_plain = graph_us(lambda j: fc1(j, "none"), reps)
    fc2_us = graph_us(fc2, reps)
    L1 = nm_inputs.Layer("vitb_fc1_2of4_gelu", 3072, 768, T, 2, 4, "i8", "i8")
    L2 = nm_inputs.Layer("vitb_fc2_2of4", 768, 3072, T, 2, 4, "i8", "i8")
    roof, dense = 0.0, 0.0
    for L in (L1, L2):
        ops, nbytes, dn = nm_inputs.ops_and_bytes(L)
        roof += max(nbytes / (HBM_PEAK_GBS * 1e9), ops / (MFMA_PEAK_TOPS["i8"] * 1e12)) * 1e6
        dense += dn
    out = {"chain": "vitb_mlp_fc1_gelu_fc2_int8_2of4", "tokens": T, "rotated_sets": nsets,
           "chain_us": round(chain, 2), "fc1_gelu_us": round(fc1_gelu, 2), "fc1_plain_us": round(fc1_plain, 2),
           "gelu_cost_us": round(fc1_gelu - fc1_plain, 2), "fc2_us": round(fc2_us, 2),
           "kernels": {"fc1_gelu": nm.variant(p1, T, torch.int8, act="gelu"),
                       "fc1_plain": nm.variant(p1, T, torch.int8), "fc2": nm.variant(p2, T, torch.int8)},
           "sum_roof_us": round(roof, 2), "roofline_fraction": round(roof / chain, 4),
           "dense_equivalent_TOPS": round(dense / (chain * 1e-6) / 1e12, 1)}
    if args.details:
        json.dump(out, open(args.details, "w"), indent=1)
    print(json.dumps(out), flush=True)


def run_search(args):
    """Latency-constrained layer-wise N:M search over the 48 ViT-B layers
    (choices 1:4, 2:4, 4:8, 8:8): latencies from a freshly measured look-up
    table (calibrated on one measured stack), quality proxy = retained
    weight energy of seeded synthetic weights; for three budgets, the exact,
    greedy and evolutionary solvers, and the evolutionary assignment's stack
    timed on the GPU against its budget."""
    import numpy as np
    import torch

    import nm_inputs
    from semi_structured_sparse_nm_amd.lut import LayerShape, measure_layers, time_stack
    from semi_structured_sparse_nm_amd.search import (Problem, retained_energy, solve_evolutionary, solve_exact,
                                                      solve_greedy)

    torch.cuda.set_device(0)
    T = nm_inputs.VIT_B_TOKENS
    choices = [(1, 4), (2, 4), (4, 8), (8, 8)]
    dims = list(nm_inputs.VIT_B_LAYERS.values())
    shapes = [LayerShape(R, K, T, n, m) for (R, K) in dims for n, m in choices]
    lut = measure_layers(shapes, reps=20)
    layer_dims = [dims[i % 4] for i in range(48)]

    def stack(assign):
        return [LayerShape(R, K, T, *choices[c]) for (R, K), c in zip(layer_dims, assign)]

    calib = [c for c in np.random.default_rng(0).integers(0, 4, 48)]
    lut.calibrate(stack(calib), time_stack(stack(calib), reps=3))
    rng = np.random.default_rng(2024)
    energy, score = [], np.zeros((48, 4))
    for l, (R, K) in enumerate(layer_dims):
        W = rng.standard_normal((R, K)) * 0.02
        energy.append(float((W * W).sum()))
        for c, (n, m) in enumerate(choices):
            score[l, c] = retained_energy(W, n, m)
    score *= (np.array(energy) / sum(energy))[:, None]     # model-level retained energy fraction
    # a layer's latency in the stack: its table entry plus the calibrated gap
    lat = np.array([[lut.lookup(LayerShape(R, K, T, *nm)) + lut.gap_us for nm in choices]
                    for (R, K) in layer_dims])
    fastest, dense = lat.min(axis=1).sum(), lat[:, 3].sum()
    results = []
    for frac in (0.25, 0.5, 0.75):
        budget = fastest + frac * (dense - fastest)
        p = Problem(score, lat, budget)
        ex, gr = solve_exact(p, res=0.01), solve_greedy(p)
        t0 = time.perf_counter()
        ev = solve_evolutionary(p, pop=64, generations=200, seed=0)
        ev_s = time.perf_counter() - t0
        measured = time_stack(stack(ev.choice), reps=3, seed=11)
        results.append({"budget_us": round(budget, 1), "exact_value": round(ex.value, 5),
                        "greedy_value": round(gr.value, 5), "evolutionary_value": round(ev.value, 5),
                        "evolutionary_predicted_us": round(ev.latency, 1), "evolutionary_measured_us": round(measured, 1),
                        "measured_over_budget": round(measured / budget - 1, 4), "evolutionary_s": round(ev_s, 2),
                        "choice_counts": {f"{n}:{m}": int(sum(1 for c in ev.choice if choices[c] == (n, m)))
                                          for n, m in choices}})
        print(json.dumps(results[-1]), file=sys.stderr, flush=True)
    out = {"search": "vitb_int8_48_layers", "choices": ["1:4", "2:4", "4:8", "8:8"],
           "objective": "retained weight energy (proxy)", "all_fastest_us": round(fastest, 1),
           "all_dense_us": round(dense, 1), "gap_us_per_launch": round(lut.gap_us, 2), "budgets": results}
    print(json.dumps(out), flush=True)
    if args.details:
        json.dump(out, open(args.details, "w"), indent=1)


def run_hybrid(args):
    """Three-layer format product (nm_hybrid_spmm) on the ~50% unstructured
    LLaMA-7B projections and the 4:8 ViT-B FC1, one JSON line per workload,
    each timed as a HIP graph of back-to-back calls over rotating buffer sets,
    with comparison paths timed the same way: the same weight dense through
    torch.matmul (hipBLASLt), and for the 4:8 weight the library's own 4:8
    path (nm_spmm)."""
    import numpy as np
    import torch

    import nm_inputs
    import semi_structured_sparse_nm_amd as nm

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_mib:
        src = torch.ones(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    names = [L.name for L in nm_inputs.hybrid_workloads()]
    want = names if args.hybrid == "all" else args.hybrid.split(",")
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}

    def to_dev(a, dt):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if dt == "bf16":
            t = t.view(torch.bfloat16)
        return t.to(dev)

    def graph_us(fn, nsets, reps):
        for i in range(3):
            fn(i % nsets)
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                for i in range(reps):
                    fn(i % nsets)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    for L in nm_inputs.hybrid_workloads():
        if L.name not in want:
            continue
        inp = nm_inputs.hybrid_inputs(L)
        W, X = inp["W"], inp["X"]
        Wd = to_dev(W, L.dt)
        t0 = time.perf_counter()
        h = nm.pack_hybrid(Wd, device=dev)
        pack_s = time.perf_counter() - t0
        nnz = int(((W.view(np.uint16) & 0x7FFF) != 0).sum())
        Xd = to_dev(X, L.dt)
        odt = tdt[L.out]
        yb = torch.empty(0, dtype=odt).element_size()
        fmt_bytes = h.nbytes()
        nbytes = fmt_bytes + L.K * L.T * 2 + L.R * L.T * yb
        nsets = max(2, math.ceil(args.rotate_gib * 2**30 / nbytes))
        sets = []
        for _ in range(nsets):
            hs = nm.Hybrid(h.rows, h.K, h.dtype, *(None if getattr(h, n) is None else getattr(h, n).clone()
                                                   for n in nm.HYBRID_BUFFERS), h.n_fill, h.n_res,
                           h.format_version)
            sets.append((hs, Xd.clone(), torch.empty((L.R, L.T), dtype=odt, device=dev)))

        def hy(i):
            hs, Xi, Yi = sets[i]
            nm.spmm_hybrid(hs, Xi, out_dtype=odt, out=Yi)
        us = graph_us(hy, nsets, args.steps)
        # dense reference path: the same weight, all K columns, through torch.matmul
        dsets = [(Wd.clone(), Xd.clone(), torch.empty((L.R, L.T), dtype=tdt[L.dt], device=dev))
                 for _ in range(max(2, math.ceil(args.rotate_gib * 2**30 / (L.R * L.K * 2))))]

        def dense(i):
            Wi, Xi, Yi = dsets[i]
            torch.matmul(Wi, Xi, out=Yi)
        dense_us = graph_us(dense, len(dsets), args.steps)
        del dsets
        nm48_us = None
        if L.pattern == "4of8":
            p = nm.pack(Wd, 4, 8)
            psets = [(nm.Packed(p.rows, p.K, 4, 8, p.dtype, p.values.clone(), p.meta.clone(), p.format_version),
                      Xd.clone(), torch.empty((L.R, L.T), dtype=odt, device=dev)) for _ in range(nsets)]
            ws = torch.empty(max(1, nm.workspace_size(p, L.T, odt)), dtype=torch.uint8, device=dev)

            def nm48(i):
                ps, Xi, Yi = psets[i]
                nm.spmm(ps, Xi, out_dtype=odt, out=Yi, workspace=ws)
            nm48_us = round(graph_us(nm48, nsets, args.steps), 3)
            del psets
        t_s = us * 1e-6
        t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
        line = {
            "metric": "three-layer format SpMM: effective GB/s of the format's bytes + % of MI355X HBM roofline",
            "value": round(nbytes / t_s / 1e9, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": 3, "ms_per_step": round(us * 1e-3, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": L.dt, "data": "synthetic",
            "config": {"workload": L.name, "R": L.R, "K": L.K, "T": L.T, "pattern": L.pattern, "out": L.out,
                       "nonzeros": nnz, "slot_filled": h.n_fill, "residual": h.n_res},
            "roofline": {"bound": "hbm", "achieved": round(nbytes / t_s / 1e9, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(t_hbm / t_s, 4), "traffic": None,
                         "t_roof_us": round(t_hbm * 1e6, 3)},
            "format_bytes": fmt_bytes, "dense_weight_bytes": L.R * L.K * 2,
            "dense_equiv_TOPS": round(2 * L.R * L.K * L.T / t_s / 1e12, 3),
            "us_hybrid": round(us, 3), "us_dense_torch_matmul": round(dense_us, 3),
            "speedup_vs_dense": round(dense_us / us, 3), "us_library_4of8": nm48_us,
            "rotation_sets": nsets, "launch": "hip-graph", "pack_host_s": round(pack_s, 3),
        }
        print(json.dumps(line), flush=True)
        del sets


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="vitb_fc1_2of4_i8")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--rotate-gib", type=float, default=1.0)
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of a HIP graph")
    ap.add_argument("--details", default="", help="write a JSON file of extra figures here")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB three times (a known-size "
                         "reference for HBM byte counters)")
    ap.add_argument("--stack", action="store_true",
                    help="time the 48-layer mixed-N:M ViT-B int8 stack instead of one layer")
    ap.add_argument("--lut", action="store_true",
                    help="build the latency look-up table of the mixed ViT-B stack and validate it on "
                         "stacks of other N:M draws")
    ap.add_argument("--search", action="store_true",
                    help="latency-constrained layer-wise N:M search over the ViT-B stack, solutions timed")
    ap.add_argument("--layout", choices=["kt", "tk"], default="kt",
                    help="operand layout of the default benchmark: X [K][T] (kt) or the PyTorch-linear "
                         "X [T][K], Y [T][R] (tk)")
    ap.add_argument("--chain", action="store_true",
                    help="time the int8 ViT-B MLP: FC1 with GELU fused, chained into FC2 on the device")
    ap.add_argument("--floor", action="store_true",
                    help="also time a one-element kernel the same way (the per-call launch floor)")
    ap.add_argument("--hybrid", default="",
                    help="time the three-layer format product: 'all' or comma-separated workload names")
    ap.add_argument("--sweep", default="",
                    help="comma-separated workload sets to time layer by layer (1, 2, 3, 5)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the product shards by output rows or tokens with no exchange, but no "
              "multi-GPU launcher is provided", file=sys.stderr)
        sys.exit(2)
    if args.stack:
        run_stack(args)
        return
    if args.sweep:
        run_sweep(args)
        return
    if args.hybrid:
        run_hybrid(args)
        return
    if args.lut:
        run_lut(args)
        return
    if args.search:
        run_search(args)
        return
    if args.chain:
        run_chain(args)
        return

    import numpy as np
    import torch

    import nm_inputs
    import semi_structured_sparse_nm_amd as nm

    L = _layers()[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_mib:
        src = torch.ones(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    inp = nm_inputs.make_inputs(L, seed=0)
    tdt = {"i8": torch.int8, "f16": torch.float16, "bf16": torch.bfloat16}[L.dt]
    odt = {"i8": torch.int8, "i32": torch.int32, "f16": torch.float16, "bf16": torch.bfloat16,
           "f32": torch.float32}[L.out]

    def to_dev(a, dt):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if dt == "bf16":
            t = t.view(torch.bfloat16)
        return t.to(dev)

    W = to_dev(inp["W"], L.dt)
    X0 = to_dev(inp["X"], L.dt)
    bias = None if inp["bias"] is None else torch.from_numpy(inp["bias"]).to(dev)
    scale = None if inp["scale"] is None else torch.from_numpy(inp["scale"]).to(dev)

    # pack once (offline step), timed on its own
    p = nm.pack(W, L.N, L.M)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        p = nm.pack(W, L.N, L.M)
    e1.record()
    torch.cuda.synchronize()
    pack_ms = e0.elapsed_time(e1) / 5

    ops, nbytes, dense_ops = nm_inputs.ops_and_bytes(L)
    footprint = p.values.numel() + (0 if p.meta is None else p.meta.numel()) + \
        X0.numel() * X0.element_size() + L.R * L.T * torch.empty(0, dtype=odt).element_size()
    nsets = max(2, math.ceil(args.rotate_gib * 2**30 / footprint))
    sets = []
    for i in range(nsets):
        pv = p.values.clone()
        pm = None if p.meta is None else p.meta.clone()
        ps = nm.Packed(p.rows, p.K, p.N, p.M, p.dtype, pv, pm, p.format_version)
        tk = args.layout == "tk"
        Xi = X0.t().contiguous() if tk else X0.clone()
        Yi = torch.empty((L.T, L.R) if tk else (L.R, L.T), dtype=odt, device=dev)
        sets.append((ps, Xi, Yi))
    need = nm.workspace_size_tk(p, L.T, odt) if args.layout == "tk" else nm.workspace_size(p, L.T, odt)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    variant = nm.variant_tk(p, L.T, odt) if args.layout == "tk" else nm.variant(p, L.T, odt)

    def step(i):
        ps, Xi, Yi = sets[i % nsets]
        if args.layout == "tk":
            nm.linear(ps, Xi, bias=bias, scale=scale, out_dtype=odt, out=Yi, workspace=ws)
        else:
            nm.spmm(ps, Xi, bias=bias, scale=scale, out_dtype=odt, out=Yi, workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # The timed launches are captured once into a HIP graph and replayed, so
    # the GPU runs them back to back without host launch gaps; the events
    # bracket the replay on the stream the kernels run on, and the per-launch
    # average is what rocprofv3's kernel trace reports for the same command.
    def timed(seq):
        graph = None
        if not args.no_graph:
            try:
                s = torch.cuda.Stream()
                s.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(s):
                    graph = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(graph, stream=s):
                        for i in seq:
                            step(i)
                torch.cuda.current_stream().wait_stream(s)
                torch.cuda.synchronize()
                graph.replay()          # warm the graph once
                torch.cuda.synchronize()
            except Exception as ex:     # noqa: BLE001 - fall back to eager launches
                print(f"bench.py: graph capture unavailable ({ex}); timing eager launches", file=sys.stderr)
                graph = None
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        if graph is not None:
            graph.replay()
        else:
            for i in seq:
                step(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / len(seq), graph is not None

    ms, graphed = timed(list(range(args.steps)))
    # warm (no rotation) figure, labelled as such
    warm_ms, _ = timed([0] * args.steps)
    # launch floor: a one-element kernel (torch's elementwise add) captured and
    # replayed the same way, per call
    floor_us = None
    if args.floor:
        z = torch.zeros(1, device=dev)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                for _ in range(args.steps):
                    z.add_(1.0)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f0.record()
        g.replay()
        f1.record()
        torch.cuda.synchronize()
        floor_us = f0.elapsed_time(f1) * 1e3 / args.steps

    # quick parity spot check of the timed configuration on sampled rows
    parity = None
    try:
        import oracle
        rows = np.array([0, L.R // 2, L.R - 1])
        ps, Xi, Yi = sets[0]
        step(0)
        torch.cuda.synchronize()
        got = (Yi.t() if args.layout == "tk" else Yi)[torch.from_numpy(rows).to(dev)].cpu()
        if L.out == "bf16":
            got = got.view(torch.int16).numpy().view(np.uint16)
            got = oracle.to_f64(got, "bf16")
        else:
            got = got.numpy()
        if L.dt == "i8":
            ref = oracle.reference(inp["W"], inp["X"], L.N, L.M, L.dt, L.out, bias=inp["bias"],
                                   scale=inp["scale"], rows=rows)
            parity = "bit-exact" if np.array_equal(got, ref) else "MISMATCH"
        else:
            ref = oracle.reference(inp["W"], inp["X"], L.N, L.M, L.dt, "f64", rows=rows)
            err = float(np.abs(got.astype(np.float64) - ref).max() / np.abs(ref).max())
            parity = f"max-abs-normalised error {err:.2e}"
    except Exception as ex:  # noqa: BLE001 - reported, not fatal
        parity = f"not checked: {ex}"

    t_s = ms * 1e-3
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = ops / (MFMA_PEAK_TOPS[L.dt] * 1e12)
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    if bound == "hbm":
        achieved, peak, unit = nbytes / t_s / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        achieved, peak, unit = ops / t_s / 1e12, MFMA_PEAK_TOPS[L.dt], "TFLOP/s" if L.dt != "i8" else "TOPS"
    traffic = _traffic(variant)
    roof = {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic,
            "t_roof_us": round(max(t_hbm, t_mfma) * 1e6, 3),
            "roofline_fraction": round(max(t_hbm, t_mfma) / t_s, 4)}

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(L, inp)

    line = {
        "metric": METRIC, "value": round(dense_ops / t_s / 1e12, 2),
        "unit": "TOPS (dense-equivalent)", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": L.dt, "data": "synthetic",
        "config": {"workload": L.name, "R": L.R, "K": L.K, "T": L.T, "N": L.N, "M": L.M,
                   "in": L.dt, "out": L.out,
                   "epilogue": "bias+requant" if L.out == "i8" else "none",
                   "parallelism": "single-gpu", "layout": "T x K" if args.layout == "tk" else "K x T"},
        "roofline": roof, "cpu_baseline": cpu,
        "kernel": variant, "rotation_sets": nsets, "launch": "hip-graph" if graphed else "eager", "warm_ms_per_step": round(warm_ms, 5),
        "effective_GBps": round(nbytes / t_s / 1e9, 1), "pack_ms": round(pack_ms, 4),
        "parity": parity,
    }
    if floor_us is not None:
        line["launch_floor_us_per_call"] = round(floor_us, 3)
        line["us_per_call"] = round(ms * 1e3, 3)
    print(json.dumps(line), flush=True)
    if args.details:
        json.dump(line, open(args.details, "w"), indent=1)


if __name__ == "__main__":
    main()
