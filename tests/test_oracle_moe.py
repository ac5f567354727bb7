"""Pins of the MoE verify-layer oracle against the pages, closed forms,
invariants, library routines and brute force (CPU only)."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special

from oracle import fp, moe

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rand_experts(rng, E, H, I, scale=0.05):
    return [(rng.standard_normal((I, H)) * scale, rng.standard_normal((I, H)) * scale,
             rng.standard_normal((H, I)) * scale) for _ in range(E)]


# ---------------------------------------------------------------------------
# The pages' worked example (S2-MoE component 2, Fig. 5)
# ---------------------------------------------------------------------------
def test_fig5_union_six_then_four():
    g = load("fig5_reuse_gating.json")
    facts = g["page_facts"]
    L = np.array(g["logits"], dtype=np.float32)
    k = facts["k"]
    r0 = moe.route(L, k)
    assert len(moe.expert_union(r0.topk_idx)) == facts["unique_experts_without_bias"]
    r1 = moe.route(L, k, w_conf=np.array(g["w_conf"]), cap=g["cap"], alpha=g["alpha"])
    assert len(moe.expert_union(r1.topk_idx)) == facts["unique_experts_with_bias"]
    assert sorted(r1.bias.pstar.tolist()) == facts["preferred_set_zero_based"]
    for t in facts["tokens_keeping_their_choice_zero_based"]:
        assert set(r1.topk_idx[t]) == set(r0.topk_idx[t])
    moved = facts["token_moved_onto_preferred_set_zero_based"]
    assert set(r1.topk_idx[moved]) != set(r0.topk_idx[moved])
    assert set(r1.topk_idx[moved]) - set(r0.topk_idx[moved]) <= set(r1.bias.pstar.tolist())


# ---------------------------------------------------------------------------
# Top-k (R2) and gate weights (R3)
# ---------------------------------------------------------------------------
def test_topk_exact_ties_lowest_index():
    L = np.array([[1.0, 3.0, 3.0, 2.0, 3.0]], dtype=np.float32)
    assert moe.topk(L, 1).tolist() == [[1]]
    assert moe.topk(L, 2).tolist() == [[1, 2]]
    assert moe.topk(L, 3).tolist() == [[1, 2, 4]]
    assert moe.topk(L, 4).tolist() == [[1, 2, 4, 3]]
    assert moe.topk(np.zeros((1, 6), np.float32), 3).tolist() == [[0, 1, 2]]


def test_topk_matches_bruteforce_with_many_ties():
    rng = np.random.default_rng(1)
    for _ in range(200):
        E = int(rng.integers(2, 9))
        k = int(rng.integers(1, E + 1))
        row = rng.integers(-2, 3, size=E).astype(np.float32)
        # brute force: the k-subset, in rank order, whose elements beat every
        # element outside it under (value desc, index asc)
        best = None
        for perm in itertools.permutations(range(E), k):
            ok = all((row[perm[i]] > row[perm[i + 1]]) or
                     (row[perm[i]] == row[perm[i + 1]] and perm[i] < perm[i + 1])
                     for i in range(k - 1))
            rest = [e for e in range(E) if e not in perm]
            ok = ok and all((row[perm[-1]] > row[e]) or (row[perm[-1]] == row[e] and perm[-1] < e)
                            for e in rest)
            if ok:
                assert best is None
                best = list(perm)
        assert moe.topk(row[None], k)[0].tolist() == best


def test_gate_weights_sum_to_one_and_equal_selected_softmax():
    rng = np.random.default_rng(2)
    L = rng.standard_normal((7, 16)).astype(np.float32) * 3
    idx = moe.topk(L, 4)
    w = moe.gate_weights(L, idx)
    assert np.all(np.abs(w.sum(axis=1) - 1.0) <= 1e-12)
    # closed form via a library softmax over the selected logits only
    sel = np.take_along_axis(L.astype(np.float64), idx.astype(np.int64), axis=1)
    assert np.allclose(w, scipy.special.softmax(sel, axis=1), rtol=0, atol=1e-14)
    # weights are non-increasing along the rank order
    assert np.all(np.diff(w, axis=1) <= 1e-15)


def test_router_logits_textbook():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 64)).astype(np.float32)
    Wr = rng.standard_normal((8, 64)).astype(np.float32)
    ref = np.array([[math.fsum(float(a) * float(b) for a, b in zip(x[t], Wr[e])) for e in range(8)]
                    for t in range(5)])
    assert np.allclose(moe.router_logits(x, Wr), ref, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# Union, reuse ratio, CSR
# ---------------------------------------------------------------------------
def test_identical_tokens_union_is_k_and_reuse_is_one_over_T():
    figs = load("page_figures.json")["reuse_ratio_ideal"]
    rng = np.random.default_rng(4)
    row = rng.standard_normal(64).astype(np.float32)
    L = np.repeat(row[None], figs["s"], axis=0)
    idx = moe.topk(L, figs["k"])
    assert len(moe.expert_union(idx)) == figs["k"]
    assert moe.reuse_ratio(idx) == pytest.approx(figs["ratio"], abs=0)


def test_ar_decode_touches_k_experts():
    figs = load("page_figures.json")["ar_decode_experts"]
    rng = np.random.default_rng(5)
    L = rng.standard_normal((1, 128)).astype(np.float32)
    assert len(moe.expert_union(moe.topk(L, figs["k"]))) == figs["experts_per_layer"]


def test_union_bounds_random():
    rng = np.random.default_rng(6)
    for _ in range(300):
        T = int(rng.integers(1, 12))
        E = int(rng.integers(1, 40))
        k = int(rng.integers(1, E + 1))
        L = rng.integers(-3, 4, size=(T, E)).astype(np.float32)
        idx = moe.topk(L, k)
        U = moe.expert_union(idx)
        assert k <= len(U) <= min(E, T * k)
        assert list(U) == sorted(set(idx.ravel().tolist()))


def test_csr_layout_is_the_unique_grouping():
    rng = np.random.default_rng(7)
    for _ in range(100):
        T, E, k = int(rng.integers(1, 10)), int(rng.integers(2, 20)), 0
        k = int(rng.integers(1, E + 1))
        L = rng.standard_normal((T, E)).astype(np.float32)
        idx = moe.topk(L, k)
        w = moe.gate_weights(L, idx)
        c = moe.csr(idx, w)
        assert c.ptr[0] == 0 and c.ptr[-1] == T * k and np.all(np.diff(c.ptr) > 0)
        # every token appears exactly k times, once per selected expert
        assert np.bincount(c.tok, minlength=T).tolist() == [k] * T
        for u, e in enumerate(c.union):
            toks = c.tok[c.ptr[u]:c.ptr[u + 1]].tolist()
            assert toks == sorted(t for t in range(T) if e in idx[t])
            for p, t in zip(range(c.ptr[u], c.ptr[u + 1]), toks):
                j = list(idx[t]).index(e)
                assert c.w[p] == w[t, j]


def test_union_stats_counts_and_exact_ratio():
    rng = np.random.default_rng(8)
    a = np.stack([moe.topk(rng.standard_normal((5, 32)).astype(np.float32), 4) for _ in range(6)])
    counts, reuse = moe.union_stats(a)
    for l in range(6):
        assert counts[l] == len(set(a[l].ravel().tolist()))
        # float32 division of small integers is correctly rounded: compare to
        # the exact rational rounded once
        assert reuse[l] == np.float32(counts[l] / 20)


def test_union_stats_ignores_entries_outside_the_experts():
    # one rule for both statistics calls: an entry outside [0, E) names no
    # expert, so it adds nothing to the union; T k stays the denominator
    E = 16
    a = np.array([[[3, -1], [3, 16], [5, 99]],          # {3, 5}
                  [[-7, -7], [16, 17], [40, 16]],       # nothing in range
                  [[0, 15], [15, 0], [1, 2]]], dtype=np.int32)  # {0, 1, 2, 15}
    counts, reuse = moe.union_stats(a, E)
    assert counts.tolist() == [2, 0, 4]
    assert reuse.tolist() == [np.float32(2 / 6), 0.0, np.float32(4 / 6)]
    # brute force on random rows with a third of the entries out of range
    rng = np.random.default_rng(31)
    b = rng.integers(-20, 2 * E, size=(40, 7, 3)).astype(np.int32)
    c2, _ = moe.union_stats(b, E)
    for l in range(40):
        assert c2[l] == len({int(e) for e in b[l].ravel() if 0 <= e < E})
    # without E every entry counts (the verify layer's own selections are in range)
    c3, _ = moe.union_stats(a)
    assert c3.tolist() == [5, 4, 4]


# ---------------------------------------------------------------------------
# Expert FFN and layer output
# ---------------------------------------------------------------------------
def test_silu_closed_form_values():
    # SiLU(ln 3) = ln3 * 3/4, SiLU(-ln 3) = -ln3 / 4, SiLU(0) = 0
    z = np.array([math.log(3.0), -math.log(3.0), 0.0])
    assert np.allclose(moe.silu(z), [0.75 * math.log(3.0), -0.25 * math.log(3.0), 0.0], atol=1e-15)


def test_swiglu_diagonal_closed_form_and_torch():
    torch = pytest.importorskip("torch")
    H = 4
    x = np.array([math.log(3.0), -math.log(3.0), 0.0, 1.0])
    Wg, Wu, Wd = np.eye(H), 2.0 * np.eye(H), np.diag([1.0, 1.0, 1.0, -1.0])
    y = moe.swiglu(Wg, Wu, Wd, x)
    silu1 = 1.0 / (1.0 + math.exp(-1.0))
    expect = [0.75 * math.log(3) * 2 * math.log(3), -0.25 * math.log(3) * -2 * math.log(3), 0.0, -silu1 * 2.0]
    assert np.allclose(y, expect, atol=1e-14)
    rng = np.random.default_rng(9)
    Wg, Wu, Wd = rand_experts(rng, 1, 32, 48, 0.3)[0]
    xr = rng.standard_normal(32)
    tx = torch.tensor(xr, dtype=torch.float64)
    ref = torch.tensor(Wd) @ (torch.nn.functional.silu(torch.tensor(Wg) @ tx) * (torch.tensor(Wu) @ tx))
    assert np.allclose(moe.swiglu(Wg, Wu, Wd, xr), ref.numpy(), rtol=1e-12, atol=1e-14)


def test_k_equals_E_is_dense_softmax_mixture():
    rng = np.random.default_rng(10)
    T, H, I, E = 3, 16, 24, 5
    ex = rand_experts(rng, E, H, I, 0.2)
    x = rng.standard_normal((T, H))
    L = rng.standard_normal((T, E)).astype(np.float32)
    idx = moe.topk(L, E)
    y = moe.moe_layer(x, idx, moe.gate_weights(L, idx), lambda e: ex[e])
    p = scipy.special.softmax(L.astype(np.float64), axis=1)
    for t in range(T):
        ref = sum(p[t, e] * (ex[e][2] @ (scipy.special.expit(ex[e][0] @ x[t]) * (ex[e][0] @ x[t]) *
                                         (ex[e][1] @ x[t]))) for e in range(E))
        assert np.allclose(y[t], ref, rtol=1e-12, atol=1e-14)


def test_T1_is_standard_moe_and_union_path_equals_per_token_loop():
    rng = np.random.default_rng(11)
    T, H, I, E, k = 6, 16, 12, 10, 3
    ex = rand_experts(rng, E, H, I, 0.3)
    x = rng.standard_normal((T, H))
    L = rng.standard_normal((T, E)).astype(np.float32)
    idx = moe.topk(L, k)
    w = moe.gate_weights(L, idx)
    y = moe.moe_layer(x, idx, w, lambda e: ex[e])
    # union path: each unique expert applied once to all of its tokens
    c = moe.csr(idx, w)
    y2 = np.zeros_like(y)
    for u, e in enumerate(c.union):
        toks = c.tok[c.ptr[u]:c.ptr[u + 1]]
        Xe = x[toks]                                         # [n_u, H]
        He = scipy.special.expit(Xe @ ex[e][0].T) * (Xe @ ex[e][0].T) * (Xe @ ex[e][1].T)
        np.add.at(y2, toks, c.w[c.ptr[u]:c.ptr[u + 1], None] * (He @ ex[e][2].T))
    assert np.allclose(y, y2, rtol=1e-12, atol=1e-14)
    # T = 1: the union is the token's own top-k
    y1 = moe.moe_layer(x[:1], idx[:1], w[:1], lambda e: ex[e])
    assert np.allclose(y1[0], y[0], rtol=0, atol=0)
    assert len(moe.expert_union(idx[:1])) == k


def test_layer_is_linear_in_gate_weights_and_shared_expert_adds():
    rng = np.random.default_rng(12)
    T, H, I, E, k = 4, 8, 8, 6, 2
    ex = rand_experts(rng, E, H, I, 0.3)
    sh = rand_experts(rng, 1, H, I, 0.3)[0]
    x = rng.standard_normal((T, H))
    idx = moe.topk(rng.standard_normal((T, E)).astype(np.float32), k)
    w1, w2 = rng.random((T, k)), rng.random((T, k))
    f = lambda w, s=None: moe.moe_layer(x, idx, w, lambda e: ex[e], shared=s)
    assert np.allclose(f(w1 + w2), f(w1) + f(w2), rtol=1e-12, atol=1e-14)
    assert np.allclose(f(2.5 * w1), 2.5 * f(w1), rtol=1e-12, atol=1e-14)
    assert np.allclose(f(np.zeros((T, k))), 0.0)
    ys = f(w1, sh) - f(w1)
    for t in range(T):
        assert np.allclose(ys[t], moe.swiglu(*sh, x[t]), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# Reuse-aware bias (R4-R7)
# ---------------------------------------------------------------------------
def _random_bias_case(rng):
    T = int(rng.integers(1, 21))
    E = int(rng.integers(3, 64))
    k = int(rng.integers(1, min(E, 9)))
    cap = int(rng.integers(k, E + 1))
    alpha = float(rng.choice([0.0, 0.25, 0.5, 0.9, 0.999]))
    L = (rng.standard_normal((T, E)) * rng.choice([0.3, 1.0, 3.0])).astype(np.float32)
    if rng.random() < 0.3:
        L = np.round(L).astype(np.float32)          # many exact ties
    w = rng.random(T)
    return L, w, k, cap, alpha


def test_bias_alpha_zero_is_unbiased():
    rng = np.random.default_rng(13)
    for _ in range(100):
        L, w, k, cap, _ = _random_bias_case(rng)
        b = moe.reuse_bias(L, w, k, cap, 0.0)
        assert np.array_equal(b.topk_idx, moe.topk(L, k))
        assert np.array_equal(b.topk_w, moe.gate_weights(L, moe.topk(L, k)))


def test_bias_never_grows_union_and_keeps_top1():
    rng = np.random.default_rng(14)
    for _ in range(400):
        L, w, k, cap, alpha = _random_bias_case(rng)
        b = moe.reuse_bias(L, w, k, cap, alpha)
        U0 = set(moe.expert_union(moe.topk(L, k)).tolist())
        U1 = set(moe.expert_union(b.topk_idx).tolist())
        assert U1 <= U0                                  # S2-MoE comp. 2: cost never above the estimate
        top1 = moe.topk(L, 1)[:, 0]
        for t in range(L.shape[0]):
            assert top1[t] in b.topk_idx[t]              # alpha < 1 keeps the top-1 expert
        assert set(b.pstar.tolist()) <= U0
        assert len(b.pstar) <= cap


def test_bias_unchanged_sets_keep_their_weights():
    rng = np.random.default_rng(15)
    for _ in range(100):
        L, w, k, cap, alpha = _random_bias_case(rng)
        b = moe.reuse_bias(L, w, k, cap, alpha)
        idx0 = moe.topk(L, k)
        w0 = moe.gate_weights(L, idx0)
        for t in range(L.shape[0]):
            if set(b.topk_idx[t]) == set(idx0[t]):
                assert np.allclose(np.sort(b.topk_w[t]), np.sort(w0[t]), rtol=1e-14, atol=0)  # same set, other sum order


def test_bias_k_equals_E_and_zero_confidence():
    L = np.array([[1.0, 2.0, 3.0]], dtype=np.float32)
    b = moe.reuse_bias(L, np.array([1.0]), 3, 3, 0.5)
    assert b.lam.tolist() == [0.0]
    b = moe.reuse_bias(np.ones((2, 5), np.float32), np.zeros(2), 2, 3, 0.5)
    assert len(b.pstar) == 0 and np.array_equal(b.topk_idx, moe.topk(np.ones((2, 5), np.float32), 2))


def test_bias_float32_steps_by_hand():
    # l = [3, 1, 2, 0.5], k = 1: d = l(1) - l(2) = 1, lambda = 0.5, P* = {0}
    L = np.array([[3.0, 1.0, 2.0, 0.5], [0.0, 1.0, 0.25, 0.75]], dtype=np.float32)
    b = moe.reuse_bias(L, np.array([1.0, 0.0]), 1, 1, 0.5)
    assert b.pstar.tolist() == [0]
    assert b.lam.tolist() == [0.5, 0.125]               # 0.5*(3-2), 0.5*(1-0.75)
    assert b.biased[0].tolist() == [3.5, 1.0, 2.0, 0.5]
    assert b.biased[1].tolist() == [0.125, 1.0, 0.25, 0.75]
    # importance: token 0 (w=1) selects expert 0 with softmax prob p0
    p0 = math.exp(3) / (math.exp(3) + math.exp(1) + math.exp(2) + math.exp(0.5))
    assert b.g[0] == pytest.approx(p0, rel=1e-15) and b.g[1:].tolist() == [0.0, 0.0, 0.0]


# ---------------------------------------------------------------------------
# Reuse bias with the tokens grouped by sequence (R16)
# ---------------------------------------------------------------------------
def _random_offsets(rng, T):
    S = int(rng.integers(1, 6))
    cuts = np.sort(rng.integers(0, T + 1, size=S - 1))
    return np.concatenate([[0], cuts, [T]]).astype(np.int32)     # may hold empty sequences


def test_segments_one_sequence_is_the_pooled_bias():
    rng = np.random.default_rng(40)
    for _ in range(100):
        L, w, k, cap, alpha = _random_bias_case(rng)
        T = L.shape[0]
        b = moe.reuse_bias(L, w, k, cap, alpha)
        sb = moe.reuse_bias_segments(L, w, k, cap, alpha, [0, T])
        assert np.array_equal(sb.topk_idx, b.topk_idx) and np.array_equal(sb.topk_w, b.topk_w)
        assert np.array_equal(sb.pstar[0], b.pstar) and np.array_equal(sb.biased, b.biased)


def test_segments_each_sequence_union_never_grows():
    # the bias only moves a token onto experts that its own sequence's
    # tokens already chose, so no sequence's expert set grows, and neither
    # does the call's
    rng = np.random.default_rng(41)
    for _ in range(300):
        L, w, k, cap, alpha = _random_bias_case(rng)
        T = L.shape[0]
        off = _random_offsets(rng, T)
        sb = moe.reuse_bias_segments(L, w, k, cap, alpha, off)
        idx0 = moe.topk(L, k)
        for s in range(len(off) - 1):
            a, b = off[s], off[s + 1]
            U0 = {int(e) for e in idx0[a:b].ravel()}
            assert {int(e) for e in sb.topk_idx[a:b].ravel()} <= U0
            assert set(sb.pstar[s].tolist()) <= U0 and len(sb.pstar[s]) <= cap
            if a == b:
                assert len(sb.pstar[s]) == 0
        assert set(moe.expert_union(sb.topk_idx).tolist()) <= set(moe.expert_union(idx0).tolist())
        top1 = idx0[:, 0]
        assert all(top1[t] in sb.topk_idx[t] for t in range(T))


def test_segments_fig5_inside_one_sequence_and_independence():
    g = load("fig5_reuse_gating.json")
    facts = g["page_facts"]
    fig = np.array(g["logits"], dtype=np.float32)
    rng = np.random.default_rng(42)
    before = rng.standard_normal((3, 8)).astype(np.float32)
    after = rng.standard_normal((2, 8)).astype(np.float32)
    L = np.concatenate([before, fig, after])
    w = np.concatenate([rng.random(3), np.array(g["w_conf"]), rng.random(2)])
    off = [0, 3, 7, 9]
    sb = moe.reuse_bias_segments(L, w, facts["k"], g["cap"], g["alpha"], off)
    mid = sb.topk_idx[3:7]
    assert len(moe.expert_union(moe.topk(fig, facts["k"]))) == facts["unique_experts_without_bias"]
    assert len(moe.expert_union(mid)) == facts["unique_experts_with_bias"]
    assert sorted(sb.pstar[1].tolist()) == facts["preferred_set_zero_based"]
    # the other sequences' tokens and confidences do not reach this one
    L2 = L.copy()
    L2[:3] = rng.standard_normal((3, 8)).astype(np.float32) * 3
    L2[7:] = -L2[7:]
    w2 = w.copy()
    w2[[0, 8]] = [5.0, 0.0]
    sb2 = moe.reuse_bias_segments(L2, w2, facts["k"], g["cap"], g["alpha"], off)
    assert np.array_equal(sb2.topk_idx[3:7], mid) and np.array_equal(sb2.topk_w[3:7], sb.topk_w[3:7])


def test_pooled_bias_crosses_sequences_and_per_sequence_does_not():
    # sequence A: one token on {0, 1}; sequence B: two confident tokens on
    # {2, 3}.  Pooled, P* = {2, 3} pulls A's token onto expert 2, which only
    # B uses; per sequence, A's preferred set is its own {0, 1}.
    L = np.zeros((3, 8), dtype=np.float32)
    L[0, :3] = [3.0, 2.0, 1.9]
    L[1, 2:4] = [5.0, 4.9]
    L[2, 2:4] = [5.0, 4.8]
    w = np.array([0.1, 1.0, 1.0])
    pooled = moe.reuse_bias(L, w, 2, 2, 0.9)
    per = moe.reuse_bias_segments(L, w, 2, 2, 0.9, [0, 1, 3])
    assert sorted(pooled.pstar.tolist()) == [2, 3]
    assert sorted(pooled.topk_idx[0].tolist()) == [0, 2]
    assert sorted(per.pstar[0].tolist()) == [0, 1] and sorted(per.pstar[1].tolist()) == [2, 3]
    assert sorted(per.topk_idx[0].tolist()) == [0, 1]
    assert len(moe.expert_union(pooled.topk_idx)) == 3 and len(moe.expert_union(per.topk_idx)) == 4


def test_segment_offsets_validated():
    L = np.zeros((4, 6), dtype=np.float32)
    for bad in ([0, 5], [1, 4], [0, 3, 2, 4], [0]):
        with pytest.raises(ValueError):
            moe.reuse_bias_segments(L, np.ones(4), 2, 3, 0.5, bad)


# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------
def test_e4m3fn_spec_values():
    g = load("e4m3fn_values.json")
    for code, val in g["values"].items():
        got = fp.e4m3fn_value(int(code, 16))
        assert got == val and math.copysign(1, got) == math.copysign(1, val)
    for code in g["nan_codes"]:
        assert math.isnan(fp.e4m3fn_value(int(code, 16)))
    finite = fp.E4M3FN_TABLE[~np.isnan(fp.E4M3FN_TABLE)]
    assert finite.max() == 448.0 and finite.min() == -448.0
    assert len(set(finite.tolist())) == 253           # 254 finite codes, +0 and -0 equal


def test_dequant_block_scales_layout():
    rows, cols = 256, 384
    codes = np.full((rows, cols), 0x38, dtype=np.uint8)   # every weight 1.0
    s = np.arange(1, 2 * 3 + 1, dtype=np.float32).reshape(2, 3)
    W = fp.dequant_block128(codes, s)
    assert W[0, 0] == 1 and W[127, 127] == 1 and W[128, 0] == 4 and W[0, 128] == 2 and W[255, 383] == 6


def test_bf16_decode():
    assert fp.bf16_to_f64(np.array([0x3F80, 0xC000, 0x0000, 0x3F81], np.uint16)).tolist() == \
        [1.0, -2.0, 0.0, 1.0 + 2 ** -7]
