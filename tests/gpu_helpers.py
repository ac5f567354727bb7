"""Shared helpers of the GPU parity tests: build device layers from the seeded
generators, run the verify layer through the C ABI, and compare with the
oracle (routing bit for bit given the device logits; outputs to tolerance)."""
from __future__ import annotations

import sys
from dataclasses import replace

import numpy as np

import moe_speculative_decoding_router_amd as m
import synth
from oracle import fp as ofp
from oracle import moe as omoe

# Output tolerances, max |y - y_oracle| <= TOL * RMS(y_oracle), by weight format.
TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 5e-2}
# Tighter bound when activations enter the products as a bf16 high/low pair
# (2T <= 16, i.e. T <= 8): weights are exact, activations carry ~2^-16 relative error, and
# accumulation is float32, so errors stay orders of magnitude below 1e-3.
TOL_SPLIT = 1e-3


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dev():
    import torch
    return torch.device("cuda:0")


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch_dev())


def expert_fn_raw(wl: synth.Workload, layer: int):
    """Oracle expert accessor: regenerate the expert's codes on the host and
    decode them with the oracle's own format decoders (cached)."""
    cache = {}
    I = wl.I

    def get(e):
        if e not in cache:
            raw = synth.host_expert_raw(wl, layer, e)
            if wl.wdtype == "bf16":
                gu = ofp.bf16_to_f64(raw["gu"])
                d = ofp.bf16_to_f64(raw["d"])
            else:
                gu = ofp.dequant_block128(raw["gu"], raw["s_gu"])
                d = ofp.dequant_block128(raw["d"], raw["s_d"])
            cache[e] = (gu[:I], gu[I:], d)
        return cache[e]
    return get


def device_layer(wl: synth.Workload, layer: int, Wr: np.ndarray):
    W = m.pack_layer_tensors(synth.fill_layer_device(wl, layer, torch_dev()), wl.wdtype)
    return m.LayerWeights(H=wl.H, I=wl.I, E=wl.E, k=wl.k, wdtype=wl.wdtype, Wr=to_dev(Wr), **W)


def bias_parts(bias_np):
    """(cap, alpha, w_conf[, offsets]) -> cap, alpha, w_conf, offsets or None."""
    cap, alpha, w_conf = bias_np[:3]
    return cap, alpha, w_conf, (bias_np[3] if len(bias_np) > 3 else None)


def run_layer(layer_w, x: np.ndarray, bias_np=None):
    import torch
    bias = None
    if bias_np is not None:
        cap, alpha, w_conf, offsets = bias_parts(bias_np)
        bias = m.Bias(cap=cap, alpha=alpha, w_conf=to_dev(w_conf.astype(np.float32)), offsets=offsets)
    y, aux = m.verify_layer(to_dev(x), layer_w, bias)
    torch.cuda.synchronize()
    out = {f: getattr(aux, f).cpu().numpy() for f in m.Aux.__dataclass_fields__}
    out["y"] = y.cpu().numpy()
    return out


def check_routing(out, k, E, bias_np=None, x=None, Wr=None):
    """Routing, union and CSR bit for bit against the oracle given the
    device's float32 logits; gate weights to 1e-6; router GEMV to 1e-5."""
    logits = out["logits"]
    if x is not None:
        ref = omoe.router_logits(x, Wr)
        assert np.abs(logits - ref).max() <= 1e-5 * np.abs(ref).max(), "router logits"
    if bias_np is None:
        r = omoe.route(logits, k)
        assert int(out["pstar_size"][0]) == 0, "P* size without the bias"
    else:
        cap, alpha, w_conf, offsets = bias_parts(bias_np)
        r_own = omoe.route(logits, k, w_conf=w_conf, cap=cap, alpha=alpha, offsets=offsets)
        # one preferred set per sequence (one for the pooled call)
        own_sets = r_own.bias.pstar if offsets is not None else [r_own.bias.pstar]
        own_g = r_own.bias.g if offsets is not None else r_own.bias.g[None]
        dev_sets = []
        for sq, (ps_own, g) in enumerate(zip(own_sets, own_g)):
            npst = int(out["pstar_size"][sq])
            gpu_pstar = out["pstar"][sq * cap:sq * cap + npst]
            assert np.array_equal(gpu_pstar, np.sort(gpu_pstar)), "P* ascending"
            # P* depends on exp(): compare it where the importance gap at the
            # cap boundary is clear; the remaining steps are checked given the
            # device P*
            order = omoe.order_desc(g)
            pos = [e for e in order if g[e] > 0]
            if len(pos) > cap:
                gap = g[pos[cap - 1]] - g[pos[cap]]
                if gap > 1e-5 * g.max():
                    assert np.array_equal(gpu_pstar, np.sort(ps_own)), f"P* of sequence {sq}"
            else:
                assert np.array_equal(gpu_pstar, np.sort(ps_own)), f"P* of sequence {sq}"
            dev_sets.append(gpu_pstar)
        r = omoe.route(logits, k, w_conf=w_conf, cap=cap, alpha=alpha,
                       pstar=dev_sets if offsets is not None else dev_sets[0], offsets=offsets)
    assert np.array_equal(out["topk_idx"], r.topk_idx), "top-k"
    assert np.abs(out["topk_w"] - r.topk_w).max() <= 1e-6, "gate weights"
    U = omoe.expert_union(r.topk_idx)
    nU = int(out["union_size"][0])
    assert nU == len(U), f"union size {nU} vs {len(U)}"
    assert np.array_equal(out["union_experts"][:nU], U), "union"
    c = omoe.csr(r.topk_idx, r.topk_w)
    assert np.array_equal(out["csr_ptr"][:nU + 1], c.ptr), "csr_ptr"
    assert np.array_equal(out["csr_tok"], c.tok), "csr_tok"
    assert np.abs(out["csr_w"] - c.w).max() <= 1e-6, "csr_w"
    return r


def check_output(out, y_ref, wdtype, split):
    y = out["y"]
    rms = float(np.sqrt((y_ref ** 2).mean()))
    err = float(np.abs(y - y_ref).max())
    log(f"    max|y - y_oracle| = {err:.3e}, RMS(y_oracle) = {rms:.3e}, ratio {err / rms:.2e}")
    assert err <= TOL[wdtype] * rms, f"output error {err} > {TOL[wdtype]} * RMS {rms}"
    if split and wdtype != "f32":  # 2T <= 16: activations as a bf16 high/low pair
        assert err <= TOL_SPLIT * rms, f"output error {err} > {TOL_SPLIT} * RMS {rms}"
    return err / rms


def verify_workload(wl: synth.Workload, layer: int = 0, bias_np=None, T=None, n_seq=None, check_y=True):
    """Build one layer of a bf16/fp8 workload on the device, run it and check
    it against the oracle.  Returns (out, oracle routing)."""
    T = wl.T if T is None else T
    x, _, Wr = synth.layer_inputs(wl, layer, T=T, n_seq=n_seq)
    lw = device_layer(wl, layer, Wr)
    out = run_layer(lw, x, bias_np)
    r = check_routing(out, wl.k, wl.E, bias_np, x, Wr)
    if check_y:
        get = expert_fn_raw(wl, layer)
        shared = get(wl.E) if wl.shared else None
        y_ref = omoe.moe_layer(x, r.topk_idx, r.topk_w, get, shared=shared)
        check_output(out, y_ref, wl.wdtype, split=2 * T <= 16)
    del lw
    return out, r


def small(wl_name: str, **kw) -> synth.Workload:
    return replace(synth.WORKLOADS[wl_name], **kw)
