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
    ap.add_argument("--workload", default="qwen3_batch4_bf16",
                    help="headline workload (default: the largest one-GPU configuration, 4 sequences x 5 tokens)")
    ap.add_argument("--also", default="qwen3_bf16,deepseek_fp8,gptoss_bf16",
                    help="comma-separated workloads measured after the headline and reported under 'workloads' "
                         "('' for none)")
    ap.add_argument("--no-calib", action="store_true", help="skip the wide-range cost-model calibration")
    ap.add_argument("--layers", type=int, default=8, help="distinct layers cycled by the steps")
    ap.add_argument("--trees", type=int, default=1, help="draft trees selected per step")
    ap.add_argument("--bias", action="store_true", help="turn the reuse-aware soft bias on")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU budget of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before the workload, copy this many MiB device to device once (a plain copy of "
                         "known size, the calibration of the HBM byte counters)")
    ap.add_argument("--no-ab", action="store_true",
                    help="skip the batched workload's width/depth and bias A/B runs (profiling runs)")
    ap.add_argument("--ablation", action="store_true",
                    help="also run the EcoSpec gamma sweep and static-cost ablation (field 'ablation')")
    return ap.parse_args()


def main() -> int:
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the path has no multi-GPU code); got --gpus {args.gpus}",
              file=sys.stderr)
        return 2
    import numpy as np
    import torch

    import moe_speculative_decoding_router_amd as m
    import synth

    dev = torch.device("cuda:0")
    if args.copy_probe_mib > 0:
        nb = args.copy_probe_mib << 20
        src = torch.ones(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        err(f"[bench] copy probe: {nb} bytes device to device")
        del src, dst

    head = measure_workload(m, synth, args, args.workload, dev, headline=True)
    subs = {}
    for name in [w for w in args.also.split(",") if w and w != args.workload]:
        subs[name] = measure_workload(m, synth, args, name, dev, headline=False)
    out = head.pop("_line")
    out["read_stream"] = read_stream(m, torch, dev)
    if subs:
        out["workloads"] = subs
    if not args.no_cpu_baseline:
        wl = synth.WORKLOADS[args.workload]
        be = m.expert_bytes(wl.H, wl.I, wl.wdtype)
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, be, 1 if wl.shared else 0)
    print(json.dumps(out), flush=True)
    return 0


def measure_workload(m, synth, args, name, dev, headline):
    """Times `args.steps` verify steps of workload `name` (after
    `args.warmup` untimed ones) and returns its record.  The headline record
    carries the bench line's fields under '_line'; every record carries the
    per-kernel figures, its roofline fraction and the cost-model fit."""
    import numpy as np
    import torch

    wl = synth.WORKLOADS[name]
    if wl.wdtype == "f32":
        raise SystemExit("bench.py measures the bf16/fp8 workloads")
    T, L = wl.T, max(1, args.layers)

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # ---------------- inputs (seeded, synthetic, resident in HBM) ----------------
    err(f"[bench] building {L} {wl.name} layers on the device")
    layers = []
    for l in range(L):
        x, _, Wr = synth.layer_inputs(wl, l)
        W = m.pack_layer_tensors(synth.fill_layer_device(wl, l, dev), wl.wdtype)
        torch.cuda.synchronize()
        lw = m.LayerWeights(H=wl.H, I=wl.I, E=wl.E, k=wl.k, wdtype=wl.wdtype, Wr=to_dev(Wr), **W)
        layers.append((lw, to_dev(x)))
    bias = None
    if args.bias and headline:
        rng = synth.rng_for(0, wl.cid, 999)
        bias = m.Bias(cap=2 * wl.k, alpha=0.5, w_conf=to_dev(rng.random(T).astype(np.float32)))
    ML = args.model_layers or MODEL_LAYERS[wl.name]
    trees = synth.draft_trees(seed=0, nt=args.trees, n_layers=ML, E=wl.E, k=wl.k)
    P_d, F_d = to_dev(trees.P), to_dev(trees.F.view(np.int32))
    S_d = torch.empty((args.trees, 4), dtype=torch.int32, device=dev)
    wsp = m.alloc_workspace(layers[0][0], T, bias, device=dev)
    y = torch.empty((T, wl.H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i, evs=None):
        m.select_drafts(trees.parent, P_d, F_d, 4, out=S_d)
        for j in range(ML):
            lw, x = layers[(i * ML + j) % L]
            m.verify_layer(x, lw, bias, out=y, workspace=wsp, events=None if evs is None else evs.get((i, j)))

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
    err(f"[bench] {wl.name}: unions per layer: {U}")

    # ---------------- timed region ----------------
    # Every EV_STRIDE-th verify call of the region (the stride is coprime with
    # the cycled layer count, so every layer is sampled) carries a start/end
    # event pair per stage, recorded by the kernel launches themselves on the
    # stream the kernels run on; the per-kernel durations come from the same
    # region as the headline value.  (Event pairs on every call would add
    # about 30 us of packet gaps per call.)
    calls = [(i, j) for i in range(args.steps) for j in range(ML)]
    EV_STRIDE = 31 if len(calls) >= 4 * 31 else 1   # short runs: every call
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    NS = m.NUM_STAGES
    sampled = [c for n, c in enumerate(calls) if n % EV_STRIDE == EV_STRIDE // 2]
    evs = {c: [torch.cuda.Event(enable_timing=True) for _ in range(2 * NS)] for c in sampled}
    for e in (e for row in evs.values() for e in row):   # torch creates the HIP event at its first record
        e.record(stream)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        step(i, evs)
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms_step = total_ms / args.steps
    total_bytes = sum(bytes_layer[(i * ML + j) % L] for i in range(args.steps) for j in range(ML))
    value = total_bytes / (total_ms * 1e-3) / 1e9
    err(f"[bench] {wl.name}: {args.steps} steps x {ML} layers in {total_ms:.3f} ms -> {ms_step * 1e3:.1f} us/step, "
        f"{ms_step * 1e3 / ML:.1f} us/layer, {value:.0f} GB/s")
    # kernel durations [sampled calls, stages] in ms
    stage_ms = np.array([[evs[c][2 * q].elapsed_time(evs[c][2 * q + 1]) for q in range(NS)] for c in sampled])
    lidx = [(i * ML + j) % L for (i, j) in sampled]
    kbytes = {  # algorithmic bytes per launch of each kernel
        "router": np.array([wl.E * wl.H * 4 + T * wl.H * 4 + T * wl.E * 4 for _ in lidx], dtype=np.float64),
        "gate_up": np.array([(U[q] + n_sh) * gu_bytes_e for q in lidx], dtype=np.float64),
        "down": np.array([(U[q] + n_sh) * d_bytes_e for q in lidx], dtype=np.float64),
    }
    ffn_ms = stage_ms[:, 2] + stage_ms[:, 3]
    ffn_bytes = kbytes["gate_up"] + kbytes["down"]
    # router + gate-up + down of one verify call (the stages that run kernels
    # for matrix-core weights; a stage without a kernel records its events
    # back to back, which reads a few microseconds)
    call_us = (stage_ms[:, 0] + stage_ms[:, 2] + stage_ms[:, 3]) * 1e3
    kernels = {}
    for q, kname in enumerate(m.STAGE_NAMES):
        if kname not in kbytes:
            continue
        gbs = float(kbytes[kname].sum() / (stage_ms[:, q].sum() * 1e-3) / 1e9)
        kernels[kname] = {"avg_us": round(float(stage_ms[:, q].mean() * 1e3), 2), "launches": len(lidx),
                          "bytes_per_launch": round(float(kbytes[kname].mean())), "GBs": round(gbs, 1),
                          "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    gu = kernels["gate_up"]
    ffn_gbs = float(ffn_bytes.sum() / (ffn_ms.sum() * 1e-3) / 1e9)
    rec = {
        "workload": wl.name, "T": T, "dtype": wl.wdtype,
        "unique_experts_per_layer": round(float(np.mean(U)), 2),
        "unique_expert_MB_per_layer": round(float(np.mean(bytes_layer)) / 1e6, 1),
        "verify_us_per_layer_incl_select": round(ms_step * 1e3 / ML, 2),
        "GBs": round(value, 1), "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "ms_per_step": round(ms_step, 5), "moe_layers_per_step": ML,
        "verify_kernel_us_per_layer_p10_p50_p90": [round(float(v), 2) for v in np.percentile(call_us, [10, 50, 90])],
        "kernels": kernels,
        "ffn_us_per_layer": round(float(ffn_ms.mean() * 1e3), 2),
        "ffn_GBs": round(ffn_gbs, 1), "ffn_frac_of_hbm_peak": round(ffn_gbs / HBM_PEAK_GBS, 4),
        "roofline": {"kernel": "gateup_kernel", "bound": "hbm", "achieved": gu["GBs"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gu["GBs"] / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(wl.name, "gate_up")},
        "kernel_events": f"start/end events on 1 in {EV_STRIDE} verify calls of the timed region "
                         f"({len(sampled)} calls)",
    }
    if not args.no_calib:
        rec["cost_model"] = calibrate_cost_model(m, synth, wl, layers, dev)
    if headline:
        rec["select_4096_trees"] = select_timing(m, synth, wl, dev, stream, nt=4096)
        rec["expand_4096_trees"] = expand_timing(m, synth, wl, dev, stream, rec.get("cost_model"), nt=4096)
        if wl.n_seq > 1 and not args.no_ab:
            rec["config_ab"] = config_ab(m, synth, wl, layers, dev)
        if args.ablation:
            rec["ablation"] = ablation(m, synth, wl, layers, ML, dev, stream)
        line = {
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
                       "sequences": wl.n_seq, "shared_expert": wl.shared, "moe_layers_per_step": ML,
                       "distinct_layers_cycled": L, "trees_per_step": args.trees, "bias": bias is not None},
            "roofline": dict(rec["roofline"], kernel="gateup_kernel (router top-k + union + gate/up SwiGLU over "
                                                     "the union experts)",
                             bytes_per_launch=gu["bytes_per_launch"], avg_us=gu["avg_us"]),
        }
        line.update({k: v for k, v in rec.items() if k not in ("roofline", "ms_per_step", "dtype", "T")})
        rec["_line"] = line
    del layers, wsp, y
    import gc
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def calibrate_cost_model(m, synth, wl, layers, dev, Ts=(1, 2, 3, 4, 5, 6, 8, 10, 12, 16, 20), reps=5):
    """Cost model of the expansion step ([S2-MoE] component 1, Fig. 6):
    verify latency = a + T_exp * (unique experts).  The verify kernels
    (router + gate-up + down, start/end events, median of `reps` calls) run
    on the resident layers for T = 1 .. 20 tokens of one sequence, each layer
    with the router planted for those tokens, so the union spans a wide
    range; least-squares fit of the kernel time against the number of
    experts streamed (union + shared expert)."""
    import dataclasses
    import numpy as np
    import torch

    NS = m.NUM_STAGES
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * NS)]
    for e in ev:  # torch creates the HIP event at its first record
        e.record()
    torch.cuda.synchronize()
    n_sh = 1 if wl.shared else 0
    us_all, u_all, t_all = [], [], []
    for T in Ts:
        for l, (lw, _) in enumerate(layers):
            x, _, Wr = synth.layer_inputs(wl, l, T=T, n_seq=1)
            lw2 = dataclasses.replace(lw, Wr=torch.from_numpy(Wr).to(dev))
            xd = torch.from_numpy(x).to(dev)
            ws = m.alloc_workspace(lw2, T, None, device=dev)
            y = torch.empty((T, wl.H), dtype=torch.float32, device=dev)
            times = []
            for _ in range(reps + 1):
                m.verify_layer(xd, lw2, out=y, workspace=ws, events=ev)
                torch.cuda.synchronize()
                times.append(sum(ev[2 * q].elapsed_time(ev[2 * q + 1]) for q in (0, 2, 3)) * 1e3)
            us_all.append(float(np.median(times[1:])))
            u_all.append(int(ws.aux.union_size.item()) + n_sh)
            t_all.append(T)
    us, u = np.array(us_all), np.array(u_all, dtype=np.float64)
    b, a = np.polyfit(u, us, 1)
    pred = a + b * u
    r2 = 1.0 - float(((us - pred) ** 2).sum() / ((us - us.mean()) ** 2).sum())
    mape = float(np.mean(np.abs(us - pred) / us))
    err(f"[bench] {wl.name}: cost model T_exp {b:.3f} us/expert, intercept {a:.2f} us, R2 {r2:.4f}, "
        f"MAPE {mape:.4f}, experts {int(u.min())}..{int(u.max())}")
    t_arr = np.array(t_all)
    per_T = [[int(T), round(float(u[t_arr == T].mean()), 2), round(float(us[t_arr == T].mean()), 1)] for T in Ts]
    return {"t_exp_us_per_unique_expert": round(float(b), 3), "intercept_us": round(float(a), 2),
            "r2": round(r2, 4), "mape": round(mape, 4), "points": len(us_all),
            "tokens": list(Ts), "experts_streamed_range": [int(u.min()), int(u.max())],
            "per_T_experts_us": per_T,
            "note": "verify kernel time (router + gate-up + down) against experts streamed, T = 1..20 "
                    "tokens of one sequence on each cycled layer, median of 5 calls"}


ABLATION_SCATTER, ABLATION_RHO = 2.0, 0.8


def ablation(m, synth, wl, layers, ML, dev, stream, n_trees=8, n_layers=8):
    """EcoSpec variants on synthetic trees ([EcoSpec] section 4.3): for
    gamma = 3..6 the drafts chosen by the marginal cost (select_drafts), by
    the static whole-footprint cost (select_drafts_static) and by confidence
    alone (the static selection with empty footprints: top-gamma by P) are
    verified together with the root token, each token routed to its own
    predicted experts (a perfect predictor), on n_layers of the model's
    layers; reports the unique experts per layer (from the library), the
    verify kernel time per layer (router + gate-up + down events) and the
    expected accepted drafts (the sum of P over the chosen nodes, which is
    the expectation for a prefix-closed choice).  The trees scatter their
    branches over the experts ([EcoSpec] section 1: candidates close in
    probability, far apart in expert space): synth.draft_trees with a path
    context that follows each branch."""
    import numpy as np
    import torch
    trees = synth.draft_trees(seed=11, nt=n_trees, n_layers=ML, E=wl.E, k=wl.k, rate=wl.rate, with_own=True,
                              branch_scatter=ABLATION_SCATTER, branch_rho=ABLATION_RHO)
    P_d = torch.from_numpy(trees.P).to(dev)
    F_d = torch.from_numpy(trees.F.view(np.int32)).to(dev)
    Z_d = torch.zeros_like(F_d)
    rng = synth.rng_for(0, wl.cid, 777)
    NS = m.NUM_STAGES
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * NS)]
    for e in evs:
        e.record(stream)
    torch.cuda.synchronize()
    res = {"gamma": [3, 4, 5, 6], "trees": n_trees, "layers": n_layers,
           "branch_scatter": ABLATION_SCATTER, "branch_rho": ABLATION_RHO,
           "note": "tokens routed to their predicted experts; unique experts and kernel us per layer; "
                   "expected accepted drafts = sum of P over the chosen nodes"}
    for mode in ("marginal", "static", "confidence"):
        U_m, us_m, acc_m = [], [], []
        for gamma in res["gamma"]:
            if mode == "marginal":
                S = m.select_drafts(trees.parent, P_d, F_d, gamma)
            else:
                S = m.select_drafts(trees.parent, P_d, F_d if mode == "static" else Z_d, gamma, static=True)
            S = S.cpu().numpy()
            acc_m.append(round(float(np.mean([trees.P[t][S[t]].sum() for t in range(n_trees)])), 3))
            us, uu = [], []
            for t in range(n_trees):
                sets = np.concatenate([trees.root_own[t][None], trees.own[t][S[t]]], axis=0)
                T = sets.shape[0]
                for j in range(n_layers):
                    lm = j * ML // n_layers                     # model layer of the footprints
                    lw, _ = layers[j % len(layers)]             # resident weights
                    lg = synth.logits_for_sets(rng, sets, lm, wl.E)
                    x = rng.standard_normal((T, wl.H)).astype(np.float32)
                    Wr = torch.from_numpy(synth.planted_router(x, lg)).to(dev)
                    lw2 = m.LayerWeights(H=lw.H, I=lw.I, E=lw.E, k=lw.k, wdtype=lw.wdtype, Wr=Wr, W_gu=lw.W_gu,
                                         W_d=lw.W_d, s_gu=lw.s_gu, s_d=lw.s_d, Wsh_gu=lw.Wsh_gu, Wsh_d=lw.Wsh_d,
                                         ssh_gu=lw.ssh_gu, ssh_d=lw.ssh_d)
                    wsp = m.alloc_workspace(lw2, T, None, device=dev)
                    m.verify_layer(torch.from_numpy(x).to(dev), lw2, workspace=wsp, events=evs)
                    torch.cuda.synchronize()
                    us.append(sum(evs[2 * q].elapsed_time(evs[2 * q + 1]) for q in (0, 2, 3)) * 1e3)
                    uu.append(int(wsp.aux.union_size.item()))
            U_m.append(round(float(np.mean(uu)), 2))
            us_m.append(round(float(np.mean(us)), 1))
        res[mode] = {"unique_experts_per_layer": U_m, "verify_kernel_us_per_layer": us_m,
                     "expected_accepted_drafts": acc_m}
        err(f"[bench] ablation {mode}: U {U_m} us {us_m} accepted {acc_m}")
    return res


KERNEL_SOURCES = ("ffn.hip", "route_block.h", "common.h", "internal.h")


def kernel_source_digest():
    """sha256 over the sources the FFN kernels are compiled from."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "moe_speculative_decoding_router_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary of
    this workload (FETCH_SIZE and WRITE_SIZE scaled by what they count for a
    plain device-to-device copy of known size in the same runs), or None when the
    summary is missing or the kernel source changed since the counters were
    taken."""
    path = os.path.join(ROOT, "profiles", f"pmc_{workload}.md")
    try:
        lines = open(path).read().splitlines()
        digest = kernel_source_digest()
    except OSError:
        return None
    kv = {}
    for ln in lines:
        if ln.startswith("- ") and ": " in ln:
            key, val = ln[2:].split(": ", 1)
            kv[key.strip("` ")] = val.strip("` ")
    if kv.get("kernel source sha256") != digest:
        return None
    v = kv.get(f"{kernel} HBM bytes per launch")
    return int(float(v)) if v else None


def read_stream(m, torch, dev, gib=4, reps=10):
    """Context for the roofline: the streaming ceiling measured with the
    library's read probe (moe_stream_read: the FFN kernels' load pattern, one
    workgroup of 8 waves per compute unit, every byte folded into a
    checksum) over `gib` GiB, best of `reps` launches."""
    t = torch.ones((gib << 30) // 4, dtype=torch.int32, device=dev)
    chk = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(2):
        m.stream_read(t, chk)
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        m.stream_read(t, chk)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        best = ms if best is None or ms < best else best
    del t
    gbs = (gib << 30) / (best * 1e-3) / 1e9
    err(f"[bench] read stream (moe_stream_read, {gib} GiB): {gbs:.0f} GB/s")
    return {"GBs": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "kernel": f"read_probe_kernel (moe_stream_read) over {gib} GiB, best of {reps}"}


def config_ab(m, synth, wl, layers, dev, reps=15):
    """The batched workload's A/B runs on the same expert weights, each layer
    with the router planted for the arm's tokens: width against depth at
    T = 2 ([W-vs-D] section 1: two consecutive tokens of one sequence, whose
    routes are correlated, against one token from each of two sequences) and
    the reuse bias off, on pooled over the call and on per sequence at the
    workload's T ([S2-MoE] component 2, cap 2k, alpha 0.5).  Reports unique experts and the verify kernel time
    (router + gate-up + down events, median of reps calls) per layer."""
    import dataclasses
    import numpy as np
    import torch

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def arm(T, n_seq, with_bias, per_sequence=False):
        U, us = [], []
        for l, (lw, _) in enumerate(layers):
            x, _, Wr = synth.layer_inputs(wl, l, T=T, n_seq=n_seq)
            lw2 = dataclasses.replace(lw, Wr=to_dev(Wr))
            xd = to_dev(x)
            bias = None
            if with_bias:
                rng = synth.rng_for(0, wl.cid, 999)
                offsets = list(range(0, T + 1, T // n_seq)) if per_sequence else None
                bias = m.Bias(cap=2 * wl.k, alpha=0.5, w_conf=to_dev(rng.random(T).astype(np.float32)),
                              offsets=offsets)
            ws = m.alloc_workspace(lw2, T, bias, device=dev)
            y = torch.empty((T, wl.H), dtype=torch.float32, device=dev)
            m.verify_layer(xd, lw2, bias, out=y, workspace=ws)
            torch.cuda.synchronize()
            U.append(int(ws.aux.union_size.item()))
            times = []
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * m.NUM_STAGES)]
            for e in ev:  # torch creates the HIP event at its first record
                e.record()
            torch.cuda.synchronize()
            for _ in range(reps):
                m.verify_layer(xd, lw2, bias, out=y, workspace=ws, events=ev)
                torch.cuda.synchronize()
                times.append(sum(ev[2 * q].elapsed_time(ev[2 * q + 1]) for q in (0, 2, 3)) * 1e3)
            us.append(float(np.median(times)))
        return {"unique_experts_per_layer": round(float(np.mean(U)), 2),
                "verify_kernel_us_per_layer": round(float(np.mean(us)), 1), "unions": U}

    res = {"width_vs_depth_T2": {"depth_one_sequence": arm(2, 1, False), "width_two_sequences": arm(2, 2, False)},
           "reuse_bias": {"off": arm(wl.T, wl.n_seq, False), "on": arm(wl.T, wl.n_seq, True),
                          "on_per_sequence": arm(wl.T, wl.n_seq, True, per_sequence=True)}}
    wd, rb = res["width_vs_depth_T2"], res["reuse_bias"]
    err(f"[bench] T=2 depth: U {wd['depth_one_sequence']['unique_experts_per_layer']}, "
        f"{wd['depth_one_sequence']['verify_kernel_us_per_layer']} us; width: U "
        f"{wd['width_two_sequences']['unique_experts_per_layer']}, {wd['width_two_sequences']['verify_kernel_us_per_layer']} us")
    err(f"[bench] bias off: U {rb['off']['unique_experts_per_layer']}, {rb['off']['verify_kernel_us_per_layer']} us; "
        f"on (pooled): U {rb['on']['unique_experts_per_layer']}, {rb['on']['verify_kernel_us_per_layer']} us; "
        f"on (per sequence): U {rb['on_per_sequence']['unique_experts_per_layer']}, "
        f"{rb['on_per_sequence']['verify_kernel_us_per_layer']} us")
    return res


def expand_timing(m, synth, wl, dev, stream, cost_model, nt=4096, reps=20):
    """expand_drafts (S2-MoE utility expansion) on a batch of nt draft trees of
    this workload's shape, one launch for the batch.  The cost model's terms
    come from the calibration when it ran (T_exp per streamed expert; T_AR =
    the verify time of one token per layer times the model's layers), else
    6 us per expert and 60 us per layer; the draft cost is zero."""
    import numpy as np
    import torch
    ML = MODEL_LAYERS[wl.name]
    t_exp, t_layer = 6.0, 60.0
    if cost_model:
        t_exp = float(cost_model["t_exp_us_per_unique_expert"])
        t_layer = float(cost_model["per_T_experts_us"][0][2])
    t_ar = ML * t_layer
    base = min(nt, 256)
    trees = synth.draft_trees(seed=5, nt=base, n_layers=ML, E=wl.E, k=wl.k)
    reps_t = (nt + base - 1) // base
    P_d = torch.from_numpy(np.ascontiguousarray(np.tile(trees.P, (reps_t, 1))[:nt])).to(dev)
    F = np.ascontiguousarray(np.tile(trees.F, (reps_t, 1, 1))[:nt])
    F_d = torch.from_numpy(F.view(np.int32)).to(dev)
    for _ in range(3):
        S, cnt = m.expand_drafts(trees.parent, P_d, F_d, t_ar, t_exp)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pad = torch.empty(1 << 28, dtype=torch.uint8, device=dev)  # queue ahead, as in select_timing
    for _ in range(40):
        pad.fill_(1)
    a.record(stream)
    for _ in range(reps):
        S, cnt = m.expand_drafts(trees.parent, P_d, F_d, t_ar, t_exp)
    b.record(stream)
    torch.cuda.synchronize()
    del pad
    us = a.elapsed_time(b) / reps * 1e3
    nbytes = F.nbytes + nt * F.shape[1] * 4
    joined = float(cnt.float().mean())
    err(f"[bench] expand_drafts, {nt} trees: {us:.1f} us per launch, {nbytes / (us * 1e-6) / 1e9:.0f} GB/s, "
        f"{joined:.2f} nodes joined per tree")
    return {"trees": nt, "distinct_trees": base, "nodes_per_tree": int(F.shape[1]), "words_per_footprint": int(F.shape[2]),
            "t_ar_us": round(t_ar, 1), "t_exp_us": round(t_exp, 3), "nodes_joined_per_tree": round(joined, 3),
            "us_per_launch": round(us, 2), "bytes_read": int(nbytes), "GBs": round(nbytes / (us * 1e-6) / 1e9, 1)}


def select_timing(m, synth, wl, dev, stream, nt=4096, reps=20):
    """select_drafts on a batch of nt draft trees of this workload's shape
    (depth 3, top-2: 14 nodes; footprints over the model's MoE layers), gamma
    4; one launch for the batch.  Reported with the bytes of P and the
    footprints, which the kernel reads once."""
    import numpy as np
    import torch
    # 256 distinct trees tiled to nt (the kernel's work does not depend on
    # the trees being distinct; generating 4096 takes about a minute)
    base = min(nt, 256)
    trees = synth.draft_trees(seed=5, nt=base, n_layers=MODEL_LAYERS[wl.name], E=wl.E, k=wl.k)
    reps_t = (nt + base - 1) // base
    P = np.ascontiguousarray(np.tile(trees.P, (reps_t, 1))[:nt])
    F = np.ascontiguousarray(np.tile(trees.F, (reps_t, 1, 1))[:nt])
    P_d = torch.from_numpy(P).to(dev)
    F_d = torch.from_numpy(F.view(np.int32)).to(dev)
    S_d = torch.empty((nt, 4), dtype=torch.int32, device=dev)
    for _ in range(3):
        m.select_drafts(trees.parent, P_d, F_d, 4, out=S_d)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # a few ms of fills ahead of the timed launches, so that they are all
    # queued before the first one starts and the events see device time only
    # (a launch takes less than the binding's host work per call)
    pad = torch.empty(1 << 28, dtype=torch.uint8, device=dev)
    for _ in range(40):
        pad.fill_(1)
    a.record(stream)
    for _ in range(reps):
        m.select_drafts(trees.parent, P_d, F_d, 4, out=S_d)
    b.record(stream)
    torch.cuda.synchronize()
    del pad
    us = a.elapsed_time(b) / reps * 1e3
    nbytes = F.nbytes + P.nbytes
    err(f"[bench] select_drafts, {nt} trees: {us:.1f} us per launch, {nbytes / (us * 1e-6) / 1e9:.0f} GB/s")
    return {"trees": nt, "distinct_trees": base, "nodes_per_tree": int(P.shape[1]), "words_per_footprint": int(F.shape[2]),
            "us_per_launch": round(us, 2), "bytes_read": int(nbytes),
            "GBs": round(nbytes / (us * 1e-6) / 1e9, 1)}


def cpu_threads():
    """Threads the CPU oracle may use: the process's CPU share
    (OMP_NUM_THREADS when the environment sets it, else the CPUs this
    process may run on)."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    n = int(env) if env.isdigit() and int(env) > 0 else len(os.sched_getaffinity(0))
    return max(1, n)


def cpu_baseline(wl, budget_s, be, n_sh):
    """The CPU oracle (plain NumPy, float64) on layer 0 of the same workload:
    router logits, routing, and the per-token dense loop over each token's
    top-k experts, with the BLAS thread pool set to the process's CPU share
    and then to one thread.  Weight regeneration and decoding are outside the
    timing."""
    import numpy as np
    import synth
    from oracle import fp as ofp
    from oracle import moe as omoe
    from threadpoolctl import threadpool_info, threadpool_limits
    threads = cpu_threads()
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
    U = len(omoe.expert_union(r.topk_idx))

    def one_layer():
        lg = omoe.router_logits(x, Wr).astype(np.float32)
        rr = omoe.route(lg, wl.k)
        omoe.moe_layer(x, rr.topk_idx, rr.topk_w, lambda e: cache[e], shared=shared)

    with threadpool_limits(limits=threads):
        used = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        reps, t_total = 0, 0.0
        while t_total < budget_s or reps == 0:
            t = time.perf_counter()
            one_layer()
            t_total += time.perf_counter() - t
            reps += 1
    per_layer = t_total / reps
    gbs = (U + n_sh) * be / per_layer / 1e9
    err(f"[bench] cpu oracle: {per_layer * 1e3:.1f} ms/layer ({reps} reps), {gbs:.2f} GB/s, {used} threads")
    # the same on one thread
    with threadpool_limits(limits=1):
        reps1, t1 = 0, 0.0
        while t1 < budget_s / 4 or reps1 == 0:
            t = time.perf_counter()
            one_layer()
            t1 += time.perf_counter() - t
            reps1 += 1
    t1 /= reps1
    single = {"value": round((U + n_sh) * be / t1 / 1e9, 3), "ms_per_layer": round(t1 * 1e3, 1), "reps": reps1}
    err(f"[bench] cpu oracle, 1 thread: {t1 * 1e3:.1f} ms/layer")
    # the selection oracle ([EcoSpec] section 3.3) per batch of 16 trees
    from oracle import select as osel
    trees = synth.draft_trees(seed=5, nt=16, n_layers=MODEL_LAYERS[wl.name], E=wl.E, k=wl.k)
    t = time.perf_counter()
    osel.select_drafts_batch(trees.P, trees.F, 4)
    sel_ms = (time.perf_counter() - t) * 1e3
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": int(used), "kind": "oracle",
            "sample": f"layer 0 of {wl.name} (union {U} experts{' + shared' if n_sh else ''}), {reps} repetitions "
                      f"of router logits + routing + per-token dense float64 loop; {per_layer * 1e3:.1f} ms/layer; "
                      f"expert regeneration and decoding ({t_regen:.1f} s) untimed",
            "ms_per_layer": round(per_layer * 1e3, 1), "os_cpu_count": os.cpu_count(),
            "threads_note": "BLAS threads = the process's CPU share (OMP_NUM_THREADS, else its CPU affinity)",
            "single_thread": single, "select_ms_per_16_trees": round(sel_ms, 2)}


if __name__ == "__main__":
    sys.exit(main())
