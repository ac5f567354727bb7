"""GPU parity of moe_verify_layer through the C ABI against the CPU oracle:
routing, union and CSR bit for bit (given the device logits), outputs within
the format's tolerance, at small sizes spanning several tiles and ragged
tails, and at the full configuration sizes."""
import ctypes

import numpy as np
import pytest

import synth
from oracle import moe as omoe

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import moe_speculative_decoding_router_amd as m  # noqa: E402
from gpu_helpers import (check_output, check_routing, log, run_layer, small, to_dev,  # noqa: E402
                         verify_workload)


def f32_layer(Wr, Wgu, Wd, k, shared=None):
    E, H = Wr.shape
    I = Wd.shape[2]
    kw = {}
    if shared is not None:
        kw = dict(Wsh_gu=to_dev(shared[0]), Wsh_d=to_dev(shared[1]))
    return m.LayerWeights(H=H, I=I, E=E, k=k, wdtype="f32", Wr=to_dev(Wr), W_gu=to_dev(Wgu),
                          W_d=to_dev(Wd), **kw)


def f32_expert_fn(Wgu, Wd, I):
    return lambda e: (Wgu[e, :I].astype(np.float64), Wgu[e, I:].astype(np.float64), Wd[e].astype(np.float64))


def test_tiny_f32_config():
    log("case tiny_f32 (T=5, H=256, E=8, k=2, I=512)")
    wl = synth.WORKLOADS["tiny_f32"]
    x, Wr, Wgu, Wd = synth.tiny_f32_arrays(wl)
    out = run_layer(f32_layer(Wr, Wgu, Wd, wl.k), x)
    r = check_routing(out, wl.k, wl.E, None, x, Wr)
    y_ref = omoe.moe_layer(x, r.topk_idx, r.topk_w, f32_expert_fn(Wgu, Wd, wl.I))
    check_output(out, y_ref, "f32", split=True)


def one_hot_case(L, H, I, seed, shared=False):
    """x = one-hot rows, so the device logits equal the chosen values exactly."""
    T, E = L.shape
    rng = np.random.default_rng(seed)
    x = np.zeros((T, H), np.float32)
    x[np.arange(T), np.arange(T)] = 1.0
    Wr = (0.02 * rng.standard_normal((E, H))).astype(np.float32)
    Wr[:, :T] = L.T
    Wgu = (0.05 * rng.standard_normal((E, 2 * I, H))).astype(np.float32)
    Wd = (0.05 * rng.standard_normal((E, H, I))).astype(np.float32)
    sh = None
    if shared:
        sh = ((0.05 * rng.standard_normal((2 * I, H))).astype(np.float32),
              (0.05 * rng.standard_normal((H, I))).astype(np.float32))
    return x, Wr, Wgu, Wd, sh


def test_fig5_worked_example_on_device():
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "fig5_reuse_gating.json")))
    L = np.array(g["logits"], np.float32)
    facts = g["page_facts"]
    log("case fig5 worked example (E=8, T=4, k=2), without and with the reuse bias")
    x, Wr, Wgu, Wd, _ = one_hot_case(L, 64, 32, 1)
    lw = f32_layer(Wr, Wgu, Wd, facts["k"])
    out = run_layer(lw, x)
    assert np.array_equal(out["logits"], L)
    check_routing(out, 2, 8)
    assert int(out["union_size"][0]) == facts["unique_experts_without_bias"]
    bias = (g["cap"], g["alpha"], np.array(g["w_conf"], np.float32))
    out = run_layer(lw, x, bias)
    r = check_routing(out, 2, 8, bias)
    assert int(out["union_size"][0]) == facts["unique_experts_with_bias"]
    assert sorted(out["pstar"][:int(out["pstar_size"][0])].tolist()) == facts["preferred_set_zero_based"]
    y_ref = omoe.moe_layer(x, r.topk_idx, r.topk_w, f32_expert_fn(Wgu, Wd, 32))
    check_output(out, y_ref, "f32", split=True)


def test_exact_ties_and_k_equals_E():
    log("case exact ties")
    L = np.array([[1, 3, 3, 2, 3, 0, 3, 3], [0, 0, 0, 0, 0, 0, 0, 0], [2, 2, 5, 5, 1, 1, 5, 0]], np.float32)
    x, Wr, Wgu, Wd, sh = one_hot_case(L, 32, 32, 2, shared=True)
    for k in (1, 3, 8):
        out = run_layer(f32_layer(Wr, Wgu, Wd, k, shared=sh), x)
        r = check_routing(out, k, 8)
        shared = (sh[0][:32].astype(np.float64), sh[0][32:].astype(np.float64), sh[1].astype(np.float64))
        y_ref = omoe.moe_layer(x, r.topk_idx, r.topk_w, f32_expert_fn(Wgu, Wd, 32), shared=shared)
        check_output(out, y_ref, "f32", split=True)
    assert out["union_size"][0] == 8


@pytest.mark.parametrize("bias_on", [False, True])
def test_f32_route_kernel_max_experts(bias_on):
    """Float32 weights route in the standalone route kernel: E = 512 experts
    (8 entries per lane), k = 32 (radix selection; k + 1 with the bias),
    T = 9."""
    log(f"case f32 E=512 k=32 T=9 bias={bias_on}")
    rng = np.random.default_rng(77)
    T, H, I, E, k = 9, 64, 32, 512, 32
    x = rng.standard_normal((T, H)).astype(np.float32)
    Wr = (0.5 * rng.standard_normal((E, H))).astype(np.float32)
    Wgu = (0.05 * rng.standard_normal((E, 2 * I, H))).astype(np.float32)
    Wd = (0.05 * rng.standard_normal((E, H, I))).astype(np.float32)
    bias = (64, 0.5, rng.random(T).astype(np.float32)) if bias_on else None
    out = run_layer(f32_layer(Wr, Wgu, Wd, k), x, bias)
    r = check_routing(out, k, E, bias, x, Wr)
    y_ref = omoe.moe_layer(x, r.topk_idx, r.topk_w, f32_expert_fn(Wgu, Wd, I))
    check_output(out, y_ref, "f32", split=True)


SMALL_BF16 = dict(H=512, I=384, E=32, k=4, rate=0.05, cid=10)


@pytest.mark.parametrize("T", [1, 5, 8, 9, 16, 17, 20, 33, 64])
def test_bf16_small_shapes(T):
    log(f"case bf16 small T={T}")
    wl = small("qwen3_bf16", T=T, **SMALL_BF16)
    verify_workload(wl)


@pytest.mark.parametrize("T", [5, 20])
def test_bf16_small_with_bias(T):
    log(f"case bf16 small with bias T={T}")
    wl = small("qwen3_bf16", T=T, **SMALL_BF16)
    rng = np.random.default_rng(T)
    verify_workload(wl, bias_np=(8, 0.5, rng.random(T).astype(np.float32)))


@pytest.mark.parametrize("T", [1, 5])
def test_bf16_top1_routing(T):
    """k = 1: one expert per token, gate weight exactly 1."""
    log(f"case bf16 top-1 T={T}")
    wl = small("qwen3_bf16", T=T, **{**SMALL_BF16, "k": 1})
    out, _ = verify_workload(wl)
    assert np.all(out["topk_w"] == 1.0)


def test_identical_tokens_one_expert_set():
    """Every token the same: the union is one token's k experts, and every
    output row is the same bits (token columns never mix)."""
    log("case bf16 identical tokens")
    wl = small("qwen3_bf16", T=6, **SMALL_BF16)
    x, _, Wr = synth.layer_inputs(wl, 0)
    x = np.repeat(x[:1], wl.T, axis=0)
    from gpu_helpers import device_layer, expert_fn_raw
    lw = device_layer(wl, 0, Wr)
    out = run_layer(lw, x)
    r = check_routing(out, wl.k, wl.E, None, x, Wr)
    assert int(out["union_size"][0]) == wl.k
    y_ref = omoe.moe_layer(x, r.topk_idx, r.topk_w, expert_fn_raw(wl, 0))
    check_output(out, y_ref, "bf16", split=2 * wl.T <= 16)
    for t in range(1, wl.T):
        assert np.array_equal(out["y"][t], out["y"][0]), t


@pytest.mark.parametrize("E,k,bias", [(64, 20, False), (64, 16, True), (512, 8, False), (512, 32, True)])
def test_bf16_wide_routing(E, k, bias):
    """Selections past 16 ranks (radix search) and 8 entries per lane (E = 512)."""
    log(f"case bf16 routing E={E} k={k} bias={bias}")
    wl = small("qwen3_bf16", H=256, I=128, E=E, k=k, T=5, rate=0.05, cid=13)
    bias_np = (2 * k, 0.5, np.random.default_rng(E + k).random(5).astype(np.float32)) if bias else None
    verify_workload(wl, bias_np=bias_np)


@pytest.mark.parametrize("T,shared", [(1, True), (5, True), (5, False), (12, True), (40, True), (64, True)])
def test_fp8_small(T, shared):
    log(f"case fp8 small T={T} shared={shared}")
    wl = small("deepseek_fp8", H=512, I=256, E=32, k=8, T=T, shared=shared, cid=11)
    verify_workload(wl)


def _random_shape(seed):
    """Seeded shape within the documented limits: bf16 H % 64, I % 32; fp8
    H, I % 128; 1 <= k <= min(E, 32), E <= 512, 1 <= T <= 64; the shared
    expert and the reuse bias on or off."""
    rng = np.random.default_rng(1000 + seed)
    fp8 = seed % 3 == 2
    H = int(rng.integers(1, 9)) * (128 if fp8 else 64)
    I = int(rng.integers(1, 9)) * (128 if fp8 else 32)
    E = int(rng.choice([8, 16, 40, 96, 200, 512]))
    k = int(rng.integers(1, min(E, 32) + 1))
    T = int(rng.integers(1, 65))
    shared = bool(rng.integers(0, 2))
    bias = None
    if rng.integers(0, 2):  # reuse bias: k <= cap <= E, 0 <= alpha < 1
        bias = (int(rng.integers(k, E + 1)), float(rng.random()), rng.random(T).astype(np.float32))
    return fp8, H, I, E, k, T, shared, bias


@pytest.mark.parametrize("seed", range(24))
def test_random_shapes(seed):
    fp8, H, I, E, k, T, shared, bias = _random_shape(seed)
    log(f"case random seed={seed}: {'fp8' if fp8 else 'bf16'} H={H} I={I} E={E} k={k} T={T} shared={shared} "
        f"bias={None if bias is None else bias[:2]}")
    if fp8:
        wl = small("deepseek_fp8", H=H, I=I, E=E, k=k, T=T, shared=shared, cid=40 + seed)
    else:
        wl = small("qwen3_bf16", H=H, I=I, E=E, k=k, T=T, shared=shared, rate=0.05, cid=40 + seed)
    verify_workload(wl, bias_np=bias)


def test_fp8_small_with_bias():
    log("case fp8 small with bias T=5")
    wl = small("deepseek_fp8", H=512, I=256, E=32, k=8, T=5, shared=True, cid=11)
    verify_workload(wl, bias_np=(16, 0.5, np.random.default_rng(5).random(5).astype(np.float32)))


def test_bf16_all_limits():
    """E = 512, k = 32, T = 64 with the bias (cap 64): the largest routing
    tables, the radix selection and up to 512 union slots in one call."""
    log("case bf16 E=512 k=32 T=64 bias")
    wl = small("qwen3_bf16", H=256, I=128, E=512, k=32, T=64, rate=0.05, cid=18)
    verify_workload(wl, bias_np=(64, 0.5, np.random.default_rng(64).random(64).astype(np.float32)))


@pytest.mark.parametrize("T", [20, 32, 64])
def test_bf16_wide_operand(T):
    """H = 4096 with 20, 32 and 64 token columns: the activation operand does
    not fit in LDS whole.  At T = 20 each workgroup still runs whole items,
    with the operand of one unit in four read from L2; at T = 32 the
    contraction of each item is split over 4 workgroups and finished by the
    SwiGLU combine; at T = 64 no slice fits and the operand is read from L2
    with the tail items handed out by tickets (I = 1024 gives the 16 experts
    enough items)."""
    I = 1024 if T == 64 else 256
    log(f"case bf16 H=4096 I={I} T={T}")
    wl = small("qwen3_bf16", H=4096, I=I, E=16, k=4, T=T, rate=0.05, cid=14)
    verify_workload(wl)


@pytest.mark.parametrize("H,T", [(4096, 24), (2880, 24), (2880, 32), (2048, 40)])
def test_bf16_operand_partly_from_l2(H, T):
    """Whole items per workgroup with part of the activation operand read from
    L2: H = 4096, T = 24 reads two units in four from L2; H = 2880 (90
    units, not a multiple of the 4-unit batch) reads one in four at T = 24
    and two in four at T = 32, so the last batch of every item is partial;
    H = 2048, T = 40 (three column tiles, 2-unit batches) reads one in two."""
    log(f"case bf16 H={H} T={T} operand partly from L2")
    wl = small("qwen3_bf16", H=H, I=256, E=16, k=4, T=T, rate=0.05, cid=17)
    verify_workload(wl)


@pytest.mark.parametrize("H,T", [(7168, 6), (7168, 8), (7168, 12), (7168, 16), (7040, 8), (7168, 20), (7040, 24)])
def test_fp8_operand_partly_from_l2(H, T):
    """fp8 with the DeepSeek hidden size past the 5 tokens whose operand fits
    in LDS: whole items per workgroup, the operand of one unit in two
    (2-unit batches of 128-wide blocks) read from L2, with one column tile
    (T <= 16) and with two (T = 20, 24); H = 7040 has 55 blocks, so the last
    batch of every item is partial."""
    log(f"case fp8 H={H} T={T} operand partly from L2")
    wl = small("deepseek_fp8", H=H, I=256, E=16, k=4, T=T, shared=True, cid=18)
    verify_workload(wl)


def test_fp8_split_contraction():
    """fp8 with 40 token columns at H = 2048: contraction split over 2
    workgroups (per-block scales applied per part)."""
    log("case fp8 H=2048 T=40")
    wl = small("deepseek_fp8", H=2048, I=256, E=16, k=4, T=40, shared=True, cid=15)
    verify_workload(wl)


def test_bf16_gptoss_contraction_tail():
    log("case bf16 H=I=2880 (90 k-steps, uneven split), E=16")
    wl = small("gptoss_bf16", E=16, cid=12)
    verify_workload(wl)


@pytest.mark.parametrize("kind", ["bf16", "fp8", "f32"])
def test_output_over_the_input(kind):
    """y may share memory with x: x is consumed by the router kernel (the
    float32 path: by its gate-up) before y is cleared or written, so the
    call with out = x gives the same bits as with a separate output."""
    import torch
    log(f"case {kind} output over the input")
    if kind == "f32":
        wl = synth.WORKLOADS["tiny_f32"]
        x, Wr, Wgu, Wd = synth.tiny_f32_arrays(wl)
        lw = f32_layer(Wr, Wgu, Wd, wl.k)
    else:
        wl = small("deepseek_fp8" if kind == "fp8" else "qwen3_bf16", H=2816 if kind == "fp8" else 2112, I=256,
                   E=16, k=4, T=5, shared=kind == "fp8", rate=0.05, cid=20)
        x, _, Wr = synth.layer_inputs(wl, 0)
        from gpu_helpers import device_layer
        lw = device_layer(wl, 0, Wr)
    ref, _ = m.verify_layer(to_dev(x), lw)
    xy = to_dev(x)
    y, _ = m.verify_layer(xy, lw, out=xy)
    torch.cuda.synchronize()
    assert y.data_ptr() == xy.data_ptr()
    assert np.array_equal(y.cpu().numpy(), ref.cpu().numpy())


def test_down_two_and_three_piece_row_groups():
    """bf16 at H = 2112 (132 row groups): no grid of 224-256 workgroups keeps
    every row group to two pieces, so 256 workgroups leave 12 groups with two
    pieces (added into y by the atomics) and 120 with three (the counted
    fix-up) in the same call; the output matches the oracle and two runs
    give identical bits."""
    log("case bf16 H=2112 T=5 (two- and three-piece down row groups)")
    wl = small("qwen3_bf16", H=2112, I=256, E=16, k=4, T=5, rate=0.05, cid=19)
    verify_workload(wl)
    x, _, Wr = synth.layer_inputs(wl, 0)
    from gpu_helpers import device_layer
    lw = device_layer(wl, 0, Wr)
    a = run_layer(lw, x)
    b = run_layer(lw, x)
    assert np.array_equal(a["y"], b["y"])


@pytest.mark.parametrize("case", ["fp8_straddle", "bf16_multi_group"])
def test_down_shared_row_groups(case):
    """Down kernel with row groups shared between workgroups.  fp8 at
    H = 2816 (88 row groups of 2 row tiles over one workgroup per CU): most
    workgroups' ranges straddle two row groups and are streamed as one
    window.  bf16 at H = 7168 (448 row groups): each workgroup owns one or
    two whole row groups between two pieces, so a range spans two windows."""
    if case == "fp8_straddle":
        log("case fp8 H=2816 T=5 (down ranges straddle row groups)")
        wl = small("deepseek_fp8", H=2816, I=256, E=16, k=4, T=5, shared=True, cid=16)
    else:
        log("case bf16 H=7168 T=5 (several row groups per down workgroup)")
        wl = small("qwen3_bf16", H=7168, I=256, E=16, k=4, T=5, rate=0.05, cid=17)
    verify_workload(wl)


def test_deterministic_two_runs():
    log("case determinism")
    wl = small("qwen3_bf16", T=5, **SMALL_BF16)
    x, _, Wr = synth.layer_inputs(wl, 0)
    from gpu_helpers import device_layer
    lw = device_layer(wl, 0, Wr)
    a = run_layer(lw, x)
    b = run_layer(lw, x)
    for key in ("y", "logits", "topk_idx", "topk_w", "csr_tok", "csr_w"):
        assert np.array_equal(a[key], b[key]), key


def test_side_stream_matches_current_stream():
    """verify_layer launched on another stream (a torch.cuda.Stream, then its
    raw handle), with the workspace and output allocated by the call: the
    same bits as on the current stream."""
    log("case side stream")
    wl = small("qwen3_bf16", T=5, **SMALL_BF16)
    x, _, Wr = synth.layer_inputs(wl, 0)
    from gpu_helpers import device_layer
    lw = device_layer(wl, 0, Wr)
    xd = to_dev(x)
    y0, a0 = m.verify_layer(xd, lw)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    y1, a1 = m.verify_layer(xd, lw, stream=side)
    y2, a2 = m.verify_layer(xd, lw, stream=side.cuda_stream)
    side.synchronize()
    assert torch.equal(y0, y1) and torch.equal(y0, y2)
    assert torch.equal(a0.topk_idx, a1.topk_idx) and torch.equal(a0.csr_tok, a2.csr_tok)
    ti = a0.topk_idx.unsqueeze(0).contiguous()
    c0, r0 = m.union_stats(ti, wl.E)
    torch.cuda.synchronize()
    c1, r1 = m.union_stats(ti, wl.E, stream=side)
    side.synchronize()
    assert torch.equal(c0, c1) and torch.equal(r0, r1) and int(c1[0]) == int(a0.union_size[0])


@pytest.mark.parametrize("wdtype", ["bf16", "f32"])
def test_stage_events_bracket_the_kernels(wdtype):
    """Per-stage start/end events: the kernels that run have positive
    durations, a stage without a kernel spans only its two back-to-back event
    records (a few microseconds), and timing does not change the result."""
    log(f"case stage events ({wdtype})")
    if wdtype == "bf16":
        wl = small("qwen3_bf16", T=5, **SMALL_BF16)
        x, _, Wr = synth.layer_inputs(wl, 0)
        from gpu_helpers import device_layer
        lw = device_layer(wl, 0, Wr)
    else:
        wl = synth.WORKLOADS["tiny_f32"]
        x, Wr, Wgu, Wd = synth.tiny_f32_arrays(wl)
        lw = f32_layer(Wr, Wgu, Wd, wl.k)
    ref = run_layer(lw, x)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * m.NUM_STAGES)]
    stream = torch.cuda.current_stream()
    for e in evs:
        e.record(stream)
    torch.cuda.synchronize()
    wsp = m.alloc_workspace(lw, x.shape[0])
    y, _ = m.verify_layer(to_dev(x), lw, workspace=wsp, events=evs)
    torch.cuda.synchronize()
    ms = {name: evs[2 * i].elapsed_time(evs[2 * i + 1]) for i, name in enumerate(m.STAGE_NAMES)}
    log(f"    stage ms {ms}")
    assert ms["router"] > 0 and ms["gate_up"] > 0 and ms["down"] > 0
    if wdtype == "bf16":
        assert ms["combine"] < 0.02
    else:
        assert ms["combine"] > 0 and ms["route"] > 0
    assert np.array_equal(y.cpu().numpy(), ref["y"])
    with pytest.raises(ValueError):
        m.verify_layer(to_dev(x), lw, workspace=wsp, events=evs[:-1])


def test_workspace_error_through_real_library():
    wl = small("qwen3_bf16", T=5, **SMALL_BF16)
    x, _, Wr = synth.layer_inputs(wl, 0)
    from gpu_helpers import device_layer
    lw = device_layer(wl, 0, Wr)
    wsp = m.alloc_workspace(lw, 5)
    xd = to_dev(x)
    y = torch.empty_like(xd)
    # the binding refuses a workspace below what the call needs ...
    short = m.Workspace(ws=wsp.ws, nbytes=wsp.nbytes - 1024, aux=wsp.aux)
    with pytest.raises(ValueError, match="workspace"):
        m.verify_layer(xd, lw, workspace=short)
    # ... and so does the C ABI itself, before anything is enqueued
    L = lw._c()
    stream = torch.cuda.current_stream().cuda_stream
    rc = m.lib().moe_verify_layer(ctypes.byref(L), xd.data_ptr(), 5, None, y.data_ptr(), None,
                                  wsp.ws.data_ptr(), wsp.nbytes - 1024, stream)
    assert rc == -3 and b"workspace" in m.lib().moe_last_error()
    rc = m.lib().moe_verify_layer(ctypes.byref(L), xd.data_ptr(), 5, None, y.data_ptr(), None,
                                  wsp.ws.data_ptr(), wsp.nbytes, stream)
    torch.cuda.synchronize()
    assert rc == 0


# ---------------------------------------------------------------------------
# Full configuration sizes
# ---------------------------------------------------------------------------
def test_full_qwen3_bf16_layer():
    log("case full qwen3_bf16 layer 0")
    out, r = verify_workload(synth.WORKLOADS["qwen3_bf16"])
    log(f"    union {int(out['union_size'][0])} experts")


def test_full_gptoss_bf16_layer():
    log("case full gptoss_bf16 layer 0")
    verify_workload(synth.WORKLOADS["gptoss_bf16"])


def test_full_deepseek_fp8_layer():
    log("case full deepseek_fp8 layer 0 (256 experts + shared)")
    verify_workload(synth.WORKLOADS["deepseek_fp8"])


@pytest.mark.parametrize("bias_on", [False, True])
def test_full_qwen3_batch4_layer(bias_on):
    log(f"case full qwen3_batch4 layer 0 (T=20), bias={bias_on}")
    wl = synth.WORKLOADS["qwen3_batch4_bf16"]
    bias = None
    if bias_on:
        rng = synth.rng_for(0, wl.cid, 999)
        bias = (16, 0.5, rng.random(wl.T).astype(np.float32))
    out, r = verify_workload(wl, bias_np=bias)
    log(f"    union {int(out['union_size'][0])} experts")


def test_full_qwen3_batch4_layer_bias_per_sequence():
    """The batched layer with the reuse bias computed per sequence (the 4
    sequences of 5 tokens each have their own importance and preferred set)
    on layers 0 and 5, against the oracle; no sequence's expert set grows."""
    wl = synth.WORKLOADS["qwen3_batch4_bf16"]
    rng = synth.rng_for(0, wl.cid, 999)
    w_conf = rng.random(wl.T).astype(np.float32)
    offsets = [0, 5, 10, 15, 20]
    for layer in (0, 5):
        log(f"case full qwen3_batch4 layer {layer} (T=20), bias per sequence")
        out, r = verify_workload(wl, layer=layer, bias_np=(16, 0.5, w_conf, offsets))
        idx0 = omoe.topk(out["logits"], wl.k)
        for s in range(4):
            a, b = offsets[s], offsets[s + 1]
            assert set(r.topk_idx[a:b].ravel()) <= set(idx0[a:b].ravel())
        pooled = omoe.route(out["logits"], wl.k, w_conf=w_conf, cap=16, alpha=0.5)
        log(f"    union {int(out['union_size'][0])} experts per sequence, "
            f"{len(omoe.expert_union(pooled.topk_idx))} pooled, {len(omoe.expert_union(idx0))} unbiased")


@pytest.mark.parametrize("seed", range(6))
def test_bias_random_sequences(seed):
    """Random segmentations (empty sequences included) with the per-sequence
    bias, on bf16 layers (routing fused into the gate-up kernel) and on
    float32 layers (the standalone route kernel)."""
    rng = np.random.default_rng(900 + seed)
    T = int(rng.integers(2, 40))
    S = int(rng.integers(1, min(T, 9) + 1))
    cuts = np.sort(rng.integers(0, T + 1, size=S - 1))
    offsets = [0] + [int(c) for c in cuts] + [T]
    w_conf = rng.random(T).astype(np.float32)
    if seed % 2 == 0:
        wl = small("qwen3_bf16", T=T, H=512, I=256, E=int(rng.choice([16, 64, 160])), k=int(rng.integers(1, 9)),
                   n_seq=1, cid=30 + seed)
        cap = int(rng.integers(wl.k, min(wl.E, 3 * wl.k) + 1))
        log(f"case bf16 T={T} E={wl.E} k={wl.k} cap={cap} offsets={offsets}")
        verify_workload(wl, bias_np=(cap, 0.5, w_conf, offsets))
    else:
        H, I, E, k = 64, 32, int(rng.choice([8, 100, 512])), int(rng.integers(1, 9))
        cap = int(rng.integers(k, min(E, 3 * k) + 1))
        log(f"case f32 T={T} E={E} k={k} cap={cap} offsets={offsets}")
        x = rng.standard_normal((T, H)).astype(np.float32)
        Wr = (0.5 * rng.standard_normal((E, H))).astype(np.float32)
        Wgu = (0.05 * rng.standard_normal((E, 2 * I, H))).astype(np.float32)
        Wd = (0.05 * rng.standard_normal((E, H, I))).astype(np.float32)
        bias = (cap, 0.7, w_conf, offsets)
        out = run_layer(f32_layer(Wr, Wgu, Wd, k), x, bias)
        r = check_routing(out, k, E, bias, x, Wr)
        y_ref = omoe.moe_layer(x, r.topk_idx, r.topk_w, f32_expert_fn(Wgu, Wd, I))
        check_output(out, y_ref, "f32", split=True)


@pytest.mark.parametrize("part", [0, 1])
def test_deepseek_fp8_stack(part):
    """The 16-layer DeepSeek-shaped fp8 stack (256 experts + shared):
    routing, union and CSR bit for bit against the oracle on every layer,
    outputs on the first, middle and last layers."""
    wl = synth.WORKLOADS["deepseek_fp8"]
    L = wl.n_layers
    for layer in range(part * L // 2, (part + 1) * L // 2):
        out_check = layer in (0, L // 2, L - 1)
        log(f"case deepseek_fp8 stack layer {layer}{' with outputs' if out_check else ''}")
        verify_workload(wl, layer=layer, check_y=out_check)


@pytest.mark.parametrize("bias_on,part", [(False, 0), (False, 1), (True, 0), (True, 1)])
def test_qwen3_batch4_stack(bias_on, part):
    """The 40-layer batched Qwen3 stack (4 sequences x 5 tokens), without
    and with the reuse bias (cap 16, alpha 0.5): routing, union and CSR bit
    for bit on every layer, outputs on the first, middle and last layers."""
    wl = synth.WORKLOADS["qwen3_batch4_bf16"]
    L = wl.n_layers
    bias = None
    if bias_on:
        rng = synth.rng_for(0, wl.cid, 999)
        bias = (16, 0.5, rng.random(wl.T).astype(np.float32))
    for layer in range(part * L // 2, (part + 1) * L // 2):
        out_check = layer in (0, L // 2, L - 1)
        log(f"case qwen3_batch4 stack layer {layer} bias={bias_on}{' with outputs' if out_check else ''}")
        verify_workload(wl, layer=layer, bias_np=bias, check_y=out_check)
