"""The seeded input generators: counter generator against its published
definition, the C host fill against the NumPy definition, structure of the
synthetic logits, planted router and draft trees (CPU only)."""
import json
import os

import numpy as np
import pytest

import synth
from oracle import fp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_reference_outputs():
    with open(os.path.join(GOLDEN, "splitmix64_seed1234567.json")) as f:
        g = json.load(f)
    got = synth.splitmix64_sequence(g["seed"], len(g["outputs"]))
    assert [int(v) for v in got] == [int(v) for v in g["outputs"]]


def test_bf16_round_to_nearest_even():
    one = np.float32(1.0)
    cases = {1.0: 0x3F80, 1.0 + 2 ** -8: 0x3F80, 1.0 + 3 * 2 ** -8: 0x3F82,
             1.0 + 2 ** -8 + 2 ** -20: 0x3F81, -2.0: 0xC000, 0.0: 0x0000}
    for v, bits in cases.items():
        assert int(synth.f32_to_bf16_rne(np.array([v], np.float32))[0]) == bits, v
    assert one == 1


def test_e4m3fn_encode_roundtrip_and_ties():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = fp.e4m3fn_to_f64(codes).astype(np.float32)
    back = synth.f32_to_e4m3fn_rne(vals)
    assert np.array_equal(back, codes)
    # midpoints between neighbours round to the even code
    pos = np.array(sorted(set(fp.E4M3FN_TABLE[:0x7F].tolist())))
    for a, b in zip(pos[:-1], pos[1:]):
        mid = np.float32((a + b) / 2)
        c = int(synth.f32_to_e4m3fn_rne(np.array([mid]))[0])
        ca = int(synth.f32_to_e4m3fn_rne(np.array([a], np.float32))[0])
        cb = int(synth.f32_to_e4m3fn_rne(np.array([b], np.float32))[0])
        assert c == (ca if ca % 2 == 0 else cb)
    assert int(synth.f32_to_e4m3fn_rne(np.array([1000.0], np.float32))[0]) == 0x7E


@pytest.mark.parametrize("kind", ["bf16", "fp8", "scale"])
def test_host_fill_matches_numpy_definition(kind):
    n = 50_000 if kind != "scale" else 500
    out = synth.host_fill(kind, 3, n, seed=0, layer=7, expert0=11, matrix=1)
    for j in range(3):
        sid = synth.stream_id(0, 7, 11 + j, 1)
        ref = {"bf16": synth.counter_bf16, "fp8": synth.counter_fp8,
               "scale": synth.counter_scales}[kind](sid, 0, n)
        assert np.array_equal(out[j], ref)


def test_weight_statistics():
    w = synth.host_fill("bf16", 1, 1_000_000, 0, 0, 0, 0)[0]
    v = fp.bf16_to_f64(w)
    assert abs(v.std() - 0.02) < 2e-4 and abs(v.mean()) < 1e-4
    q = fp.e4m3fn_to_f64(synth.host_fill("fp8", 1, 1_000_000, 0, 0, 0, 0)[0])
    assert abs(q.std() - 64) < 1.0 and np.abs(q).max() <= 224


def test_planted_router_reproduces_logits():
    rng = synth.rng_for(0, 1, 0)
    x = rng.standard_normal((5, 512)).astype(np.float32)
    L = synth.structured_logits(rng, 1, 5, 64, 0.05)
    Wr = synth.planted_router(x, L)
    assert np.allclose(x.astype(np.float64) @ Wr.astype(np.float64).T, L, atol=1e-4)


def test_draft_trees_structure():
    tr = synth.draft_trees(seed=0, nt=16, n_layers=36, E=128, k=4)
    assert tr.parent.tolist() == [-1, -1, 0, 0, 1, 1, 2, 2, 3, 3, 4, 4, 5, 5]
    assert tr.F.shape == (16, 14, 144)
    for i, p in enumerate(tr.parent):
        if p >= 0:
            assert np.all(tr.P[:, i] <= tr.P[:, p])
            assert np.all((tr.F[:, p] & ~tr.F[:, i]) == 0)     # parent footprint within child's
    depth = np.array([1, 1, 2, 2, 2, 2, 3, 3, 3, 3, 3, 3, 3, 3])
    pc = np.unpackbits(tr.F.view(np.uint8), axis=-1).sum(-1)
    assert np.all(pc <= depth[None] * 36 * 4) and np.all(pc >= 36 * 4)


def test_tree_own_sets_and_logits_for_sets():
    a = synth.draft_trees(seed=0, nt=5, n_layers=4, E=16, k=2)
    b = synth.draft_trees(seed=0, nt=5, n_layers=4, E=16, k=2, with_own=True)
    assert np.array_equal(a.F, b.F) and np.array_equal(a.P, b.P)      # the trees do not change

    def per_layer(bits):
        return np.unpackbits(bits.view(np.uint8), bitorder="little")[:64].reshape(4, 16)
    rng = np.random.default_rng(0)
    for t in range(5):
        assert (per_layer(b.root_own[t]).sum(1) == 2).all()
        for i, pi in enumerate(b.parent):
            assert (per_layer(b.own[t, i]).sum(1) == 2).all()
            assert np.array_equal(b.F[t, i], b.own[t, i] | (b.F[t, pi] if pi >= 0 else 0))
        sets = np.concatenate([b.root_own[t][None], b.own[t]], axis=0)
        for layer in range(4):
            lg = synth.logits_for_sets(rng, sets, layer, 16)
            top = np.argsort(-lg, axis=1)[:, :2]
            for r in range(sets.shape[0]):
                assert set(top[r].tolist()) == set(np.nonzero(per_layer(sets[r])[layer])[0].tolist())


def test_draft_trees_branch_scatter():
    """With a path context per branch, a child routes close to its parent and
    siblings route apart; without it the trees are the same as before."""
    a = synth.draft_trees(seed=3, nt=8, n_layers=6, E=64, k=4, with_own=True)
    b = synth.draft_trees(seed=3, nt=8, n_layers=6, E=64, k=4, with_own=True, branch_scatter=0.0)
    assert np.array_equal(a.F, b.F) and np.array_equal(a.P, b.P) and np.array_equal(a.own, b.own)
    def parent_vs_sibling(tr):
        own = np.unpackbits(tr.own.view(np.uint8), axis=-1, bitorder="little").astype(bool)

        def overlap(i, j):
            return float((own[:, i] & own[:, j]).sum(axis=-1).mean())
        par = tr.parent
        pc = np.mean([overlap(i, par[i]) for i in range(len(par)) if par[i] >= 0])
        sib = np.mean([overlap(i, i + 1) for i in range(0, len(par), 2)])
        return pc / sib

    plain = synth.draft_trees(seed=3, nt=64, n_layers=6, E=64, k=4, with_own=True)
    scat = synth.draft_trees(seed=3, nt=64, n_layers=6, E=64, k=4, with_own=True, branch_scatter=2.0, branch_rho=0.8)
    assert np.array_equal(scat.P, plain.P)           # the probabilities are drawn as before
    assert 0.9 < parent_vs_sibling(plain) < 1.1      # one context per tree: no branch structure
    assert parent_vs_sibling(scat) > 1.2
