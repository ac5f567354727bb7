#!/usr/bin/env python3
"""Benchmark of the union-expert MoE verify step on one MI355X.

A step is one speculative verify step of the whole hot path over one batch
of synthetic input: cost-aware draft selection (select_drafts) for the
step's draft tree(s), then the MoE-layer verify call (router GEMV, routing,
expert union and grouping, SwiGLU FFN over the unique experts) for the
T = gamma + 1 verified tokens at every MoE layer of the model (94 for the
Qwen3-235B shape).  The layers cycle over several distinct device-resident
layers (each far larger than the caches), so expert weights are cold at
every call.

The headline value is the achieved HBM rate on unique-expert bytes (GB/s):
the bytes of the union experts' weights (+ shared expert, + fp8 scales) over
the step time.  Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verify µs/MoE layer + achieved HBM GB/s (% of peak) on unique-expert bytes"
HBM_PEAK_GBS = 8000.0
MODEL_LAYERS = {"qwen3_bf16": 94, "gptoss_bf16": 36, "deepseek_fp8": 58, "qwen3_batch4_bf16": 94, "tiny_f32": 4}


def err(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--model-layers", type=int, default=0,
                    help="MoE layers verified per step (default: the model's MoE layer count)")
    ap.add_argument("--workload", default="qwen3_bf16")
    ap.add_argument("--layers", type=int, default=8, help="distinct layers cycled by the steps")
    ap.add_argument("--trees", type=int, default=1, help="draft trees selected per step")
    ap.add_argument("--bias", action="store_true", help="turn the reuse-aware soft bias on")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU budget of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile-pass", action="store_true")
    return ap.parse_args()


def main() -> int:
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        return 2
    import numpy as np
    import torch

    import moe_speculative_decoding_router_amd as m
    import synth

    dev = torch.device("cuda:0")
    wl = synth.WORKLOADS[args.workload]
    T, L = wl.T, max(1, args.layers)

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # ---------------- inputs (seeded, synthetic, resident in HBM) ----------------
    err(f"[bench] building {L} {wl.name} layers on the device")
    layers = []
    for l in range(L):
        x, _, Wr = synth.layer_inputs(wl, l)
        if wl.wdtype == "f32":
            raise SystemExit("bench.py measures the bf16/fp8 workloads")
        W = m.pack_layer_tensors(synth.fill_layer_device(wl, l, dev), wl.wdtype)
        torch.cuda.synchronize()
        lw = m.LayerWeights(H=wl.H, I=wl.I, E=wl.E, k=wl.k, wdtype=wl.wdtype, Wr=to_dev(Wr), **W)
        layers.append((lw, to_dev(x)))
    bias = None
    if args.bias:
        rng = synth.rng_for(0, wl.cid, 999)
        bias = m.Bias(cap=2 * wl.k, alpha=0.5, w_conf=to_dev(rng.random(T).astype(np.float32)))
    trees = synth.draft_trees(seed=0, nt=args.trees, n_layers=MODEL_LAYERS[wl.name], E=wl.E, k=wl.k)
    P_d, F_d = to_dev(trees.P), to_dev(trees.F.view(np.int32))
    S_d = torch.empty((args.trees, 4), dtype=torch.int32, device=dev)
    wsp = m.alloc_workspace(layers[0][0], T, bias, device=dev)
    y = torch.empty((T, wl.H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    ML = args.model_layers or MODEL_LAYERS[wl.name]

    def step(i, events=None):
        m.select_drafts(trees.parent, P_d, F_d, 4, out=S_d)
        for j in range(ML):
            lw, x = layers[(i * ML + j) % L]
            m.verify_layer(x, lw, bias, out=y, workspace=wsp, events=events[j] if events else None)

    # union size per layer -> unique-expert bytes
    be = m.expert_bytes(wl.H, wl.I, wl.wdtype)
    esz = {"bf16": 2, "fp8": 1}[wl.wdtype]
    gu_bytes_e = 2 * wl.I * wl.H * esz + ((2 * wl.I // 128) * (wl.H // 128) * 4 if wl.wdtype == "fp8" else 0)
    d_bytes_e = wl.H * wl.I * esz + ((wl.H // 128) * (wl.I // 128) * 4 if wl.wdtype == "fp8" else 0)
    U = []
    for i in range(L):
        m.verify_layer(layers[i][1], layers[i][0], bias, out=y, workspace=wsp)
        torch.cuda.synchronize()
        U.append(int(wsp.aux.union_size.item()))
    n_sh = 1 if wl.shared else 0
    bytes_layer = [(u + n_sh) * be for u in U]
    err(f"[bench] unions per layer: {U}")

    # ---------------- timed region ----------------
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms_step = total_ms / args.steps
    total_bytes = sum(bytes_layer[(i * ML + j) % L] for i in range(args.steps) for j in range(ML))
    value = total_bytes / (total_ms * 1e-3) / 1e9
    err(f"[bench] {args.steps} steps x {ML} layers in {total_ms:.3f} ms -> {ms_step * 1e3:.1f} us/step, "
        f"{ms_step * 1e3 / ML:.1f} us/layer, {value:.0f} GB/s")

    # ---------------- per-kernel profile region (events between stages) ----------------
    # The same steps again with HIP events recorded on the stream between the
    # stages of every verify call (the events add a little time of their own).
    stage_ms = None
    if not args.no_profile_pass:
        PS = min(args.steps, 4)
        evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(m.NUM_STAGES + 1)] for _ in range(ML)]
               for _ in range(PS)]
        sel0 = [torch.cuda.Event(enable_timing=True) for _ in range(PS)]
        for e in [e for st in evs for row in st for e in row] + sel0:   # torch creates the HIP event at first record
            e.record(stream)
        torch.cuda.synchronize()
        for i in range(PS):
            sel0[i].record(stream)
            step(i, events=evs[i])
        torch.cuda.synchronize()
        stage_ms = np.array([[evs[i][j][q].elapsed_time(evs[i][j][q + 1]) for q in range(m.NUM_STAGES)]
                             for i in range(PS) for j in range(ML)])
        sel_ms = np.array([sel0[i].elapsed_time(evs[i][0][0]) for i in range(PS)])
        layer_ms = stage_ms.sum(axis=1)
        lidx = [(i * ML + j) % L for i in range(PS) for j in range(ML)]
        step_bytes = np.array([bytes_layer[q] for q in lidx], dtype=np.float64)
        gu_bytes = np.array([(U[q] + n_sh) * gu_bytes_e for q in lidx], dtype=np.float64)
        d_bytes = np.array([(U[q] + n_sh) * d_bytes_e for q in lidx], dtype=np.float64)

    # ---------------- CPU oracle baseline (bounded sample) ----------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_seconds, U[0], be, n_sh)

    us_layer = float(layer_ms.mean() * 1e3) if stage_ms is not None else None
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.wdtype,
        "data": "synthetic (seeded structured router logits, planted router, counter-generated weights)",
        "config": {"workload": wl.name, "H": wl.H, "I": wl.I, "E": wl.E, "k": wl.k, "T": T,
                   "shared_expert": wl.shared, "moe_layers_per_step": ML, "distinct_layers_cycled": L,
                   "trees_per_step": args.trees, "bias": bool(args.bias)},
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "unique_experts_per_layer": round(float(np.mean(U)), 2),
        "unique_expert_MB_per_layer": round(float(np.mean(bytes_layer)) / 1e6, 1),
        "us_per_step": round(ms_step * 1e3, 2),
        "verify_us_per_layer_incl_select": round(ms_step * 1e3 / ML, 2),
    }
    if stage_ms is not None:
        gu_ms = stage_ms[:, 2]
        d_ms = stage_ms[:, 3]
        ffn_ms = gu_ms + d_ms
        out["verify_us_per_layer_profiled"] = round(us_layer, 2)
        out["verify_GBs"] = round(float(step_bytes.sum() / (layer_ms.sum() * 1e-3) / 1e9), 1)
        out["ffn_GBs"] = round(float(step_bytes.sum() / (ffn_ms.sum() * 1e-3) / 1e9), 1)
        out["stages_us"] = {name: round(float(stage_ms[:, j].mean() * 1e3), 2)
                            for j, name in enumerate(m.STAGE_NAMES)}
        out["stages_us"]["select_drafts"] = round(float(sel_ms.mean() * 1e3), 2)
        ach = float(gu_bytes.mean() / (gu_ms.mean() * 1e-3) / 1e9)
        out["roofline"] = {"kernel": "ffn gate_up (ffn_mfma_kernel, gate-up instance)", "bound": "hbm",
                           "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
                           "bytes_per_launch": round(float(gu_bytes.mean())), "avg_us": round(float(gu_ms.mean() * 1e3), 2)}
        out["roofline_down"] = {"achieved": round(float(d_bytes.mean() / (d_ms.mean() * 1e-3) / 1e9), 1),
                                "avg_us": round(float(d_ms.mean() * 1e3), 2)}
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)
    return 0


def cpu_baseline(wl, budget_s, U0, be, n_sh):
    """The CPU oracle (plain NumPy, float64) on layer 0 of the same workload:
    router logits, routing, and the per-token dense loop over each token's
    top-k experts.  Weight regeneration/decoding is outside the timing."""
    import numpy as np
    import synth
    from oracle import fp as ofp
    from oracle import moe as omoe
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    x, _, Wr = synth.layer_inputs(wl, 0)
    logits = omoe.router_logits(x, Wr).astype(np.float32)
    r = omoe.route(logits, wl.k)
    t_regen = time.perf_counter()
    cache = {}
    for e in list(omoe.expert_union(r.topk_idx)) + ([wl.E] if wl.shared else []):
        raw = synth.host_expert_raw(wl, 0, int(e))
        if wl.wdtype == "bf16":
            gu, d = ofp.bf16_to_f64(raw["gu"]), ofp.bf16_to_f64(raw["d"])
        else:
            gu, d = ofp.dequant_block128(raw["gu"], raw["s_gu"]), ofp.dequant_block128(raw["d"], raw["s_d"])
        cache[int(e)] = (gu[:wl.I], gu[wl.I:], d)
    t_regen = time.perf_counter() - t_regen
    shared = cache[wl.E] if wl.shared else None
    reps, t_total = 0, 0.0
    while t_total < budget_s or reps == 0:
        t = time.perf_counter()
        lg = omoe.router_logits(x, Wr).astype(np.float32)
        rr = omoe.route(lg, wl.k)
        omoe.moe_layer(x, rr.topk_idx, rr.topk_w, lambda e: cache[e], shared=shared)
        t_total += time.perf_counter() - t
        reps += 1
    per_layer = t_total / reps
    U = len(omoe.expert_union(r.topk_idx))
    gbs = (U + n_sh) * be / per_layer / 1e9
    err(f"[bench] cpu oracle: {per_layer * 1e3:.1f} ms/layer ({reps} reps), {gbs:.2f} GB/s, {threads} threads")
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"layer 0 of {wl.name} (union {U} experts), {reps} repetitions of router logits + "
                      f"routing + per-token dense float64 loop; {per_layer * 1e3:.1f} ms/layer; expert "
                      f"regeneration and decoding ({t_regen:.1f} s) untimed"}


if __name__ == "__main__":
    sys.exit(main())
