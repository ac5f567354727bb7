"""Ragged, confidence-gated verify end to end on the GPU ([W-vs-D] section
2, ragged speculation): per-sequence depths from gate_depths, one
moe_verify_layer call over the sum of (d_s + 1) tokens grouped by sequence
with the reuse bias computed per sequence, and union_stats_segments on the
call's own selections; each step checked against the oracle."""
import numpy as np
import pytest

import synth
from oracle import moe as omoe
from oracle import ragged as orag

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import moe_speculative_decoding_router_amd as m  # noqa: E402
from gpu_helpers import (check_output, check_routing, device_layer, expert_fn_raw, log, run_layer,  # noqa: E402
                         small, to_dev)


@pytest.mark.parametrize("seed", range(3))
def test_ragged_chain(seed):
    S, Dmax, t_base, t_exp = 6, 5, 10.0, 1.0
    wl = small("qwen3_bf16", H=512, I=256, E=64, k=4, T=S * (Dmax + 1), n_seq=S, rate=0.05, cid=40)
    rng = synth.rng_for(0, 40, seed)
    # every sequence's root and Dmax drafts: correlated tokens per sequence
    L = synth.structured_logits(rng, S, Dmax + 1, wl.E, wl.rate)
    x_all = rng.standard_normal((S * (Dmax + 1), wl.H)).astype(np.float32)
    Wr = synth.planted_router(x_all, L)
    # predicted experts of each token (one layer) and cumulative confidences
    pred = omoe.topk(L.astype(np.float32), wl.k)
    bits = np.zeros((S * (Dmax + 1), wl.E), dtype=bool)
    for r in range(S * (Dmax + 1)):
        bits[r, pred[r]] = True
    Ep = synth.pack_bits(bits, wl.E // 32).reshape(S, Dmax + 1, wl.E // 32)
    edge = rng.uniform(0.3, 1.0, size=(S, Dmax + 1)).astype(np.float32)
    c = np.cumprod(edge, axis=1).astype(np.float32)
    c[:, 0] = 0.0

    # 1. depths
    d_dev = m.gate_depths(to_dev(c), to_dev(np.ascontiguousarray(Ep).view(np.int32)), t_base, t_exp)
    torch.cuda.synchronize()
    d = d_dev.cpu().numpy().tolist()
    assert d == orag.gate_depths(c, Ep, t_base, t_exp)
    assert len(set(d)) > 1, "the case should be ragged"
    log(f"case ragged chain seed {seed}: depths {d}")

    # 2. one verify call over the chosen tokens, grouped by sequence
    rows = [s * (Dmax + 1) + j for s in range(S) for j in range(d[s] + 1)]
    offsets = np.concatenate([[0], np.cumsum([ds + 1 for ds in d])]).astype(np.int32).tolist()
    x = x_all[rows]
    T = len(rows)
    w_conf = np.concatenate([np.concatenate([[1.0], c[s, 1:d[s] + 1]]) for s in range(S)]).astype(np.float32)
    bias = (8, 0.5, w_conf, offsets)
    lw = device_layer(wl, 0, Wr)
    out = run_layer(lw, x, bias)
    r = check_routing(out, wl.k, wl.E, bias, x, Wr)
    y_ref = omoe.moe_layer(x, r.topk_idx, r.topk_w, expert_fn_raw(wl, 0))
    check_output(out, y_ref, "bf16", split=2 * T <= 16)

    # 3. per-sequence unique experts of the call's own selections
    per, total = m.union_stats_segments(to_dev(out["topk_idx"][None]), wl.E, offsets)
    torch.cuda.synchronize()
    rp, rt = orag.segment_union_stats(r.topk_idx[None], np.array(offsets), wl.E)
    assert np.array_equal(per.cpu().numpy(), rp) and np.array_equal(total.cpu().numpy(), rt)
    assert int(total[0].item()) == int(out["union_size"][0])
    log(f"    T={T}, unique experts per sequence {rp[0].tolist()}, call {int(rt[0])}")
