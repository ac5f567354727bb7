"""Pins of the EcoSpec greedy-selection oracle (CPU only)."""
import itertools

import numpy as np
import pytest

import synth
from oracle import select


def sets_to_bits(sets, nbits):
    W = (nbits + 31) // 32
    b = np.zeros((len(sets), nbits), dtype=bool)
    for i, s in enumerate(sets):
        for p in s:
            b[i, p] = True
    return synth.pack_bits(b, W)


def pseudocode_with_sets(P, sets, gamma, eps):
    """The selection written with Python sets of (layer, expert) pairs, the
    representation the page's pseudocode uses (no bitsets, no popcount)."""
    S, B = [], set()
    while len(S) < gamma:
        cand = [t for t in range(len(P)) if t not in S]
        scores = [np.float32(np.float32(P[t]) / (np.float32(len(sets[t] - B)) + np.float32(eps)))
                  for t in cand]
        top = max(scores)
        best = min(t for t, s in zip(cand, scores) if s == top)
        S.append(best)
        B |= sets[best]
    return S


def random_tree_case(rng, N, nbits):
    parent = [-1] + [int(rng.integers(-1, i)) for i in range(1, N)]
    own = [set(rng.choice(nbits, size=min(nbits, int(rng.integers(0, 5))), replace=False).tolist())
           for _ in range(N)]
    P = np.zeros(N, np.float32)
    sets = []
    for i in range(N):
        e = np.float32(rng.uniform(0.3, 1.0))
        if parent[i] < 0:
            P[i] = e
            sets.append(set(own[i]))
        else:
            P[i] = np.float32(P[parent[i]] * e)
            sets.append(own[i] | sets[parent[i]])
    return parent, P, sets


def test_matches_set_pseudocode_random():
    rng = np.random.default_rng(20)
    for _ in range(300):
        N, nbits = int(rng.integers(1, 12)), int(rng.integers(1, 100))
        _, P, sets = random_tree_case(rng, N, nbits)
        gamma = int(rng.integers(0, N + 1))
        F = sets_to_bits(sets, nbits)
        assert select.select_drafts(P, F, gamma) == pseudocode_with_sets(P, sets, gamma, 1e-6)


def test_bruteforce_unique_greedy_sequence_tiny_trees():
    rng = np.random.default_rng(21)
    for _ in range(60):
        N = int(rng.integers(1, 8))
        gamma = int(rng.integers(1, min(N, 4) + 1))
        nbits = 24
        _, P, sets = random_tree_case(rng, N, nbits)
        if rng.random() < 0.3:                       # force exact score ties
            P[:] = np.float32(0.5)
        F = sets_to_bits(sets, nbits)
        valid = [seq for seq in itertools.permutations(range(N), gamma)
                 if select.is_greedy_sequence(seq, P, F)]
        assert len(valid) == 1
        assert list(valid[0]) == select.select_drafts(P, F, gamma)


def test_prefix_closed_on_generated_trees():
    trees = synth.draft_trees(seed=0, nt=200, n_layers=8, E=32, k=4)
    for tr in range(200):
        for gamma in (1, 2, 4, 6, 14):
            S = select.select_drafts(trees.P[tr], trees.F[tr], gamma)
            seen = set()
            for t in S:
                p = int(trees.parent[t])
                assert p < 0 or p in seen, (tr, gamma, S)
                seen.add(t)


def test_prefix_closed_for_every_subset_size_bruteforce():
    # every gamma-subset the greedy returns is closed under taking parents
    rng = np.random.default_rng(22)
    for _ in range(100):
        N = int(rng.integers(2, 9))
        parent, P, sets = random_tree_case(rng, N, 40)
        F = sets_to_bits(sets, 40)
        for gamma in range(1, N + 1):
            S = set(select.select_drafts(P, F, gamma))
            assert all(parent[t] < 0 or parent[t] in S for t in S)


def test_special_cases():
    rng = np.random.default_rng(23)
    N, nbits = 9, 64
    same = [set(range(10))] * N
    P = rng.uniform(0.1, 1, N).astype(np.float32)
    P[3] = P[5]                                          # a tie in P
    F = sets_to_bits(same, nbits)
    expect = sorted(range(N), key=lambda t: (-P[t], t))[:5]
    assert select.select_drafts(P, F, 5) == expect       # equal footprints: top-gamma by P
    # equal P: greedy fewest-new-pairs
    sizes = [5, 3, 8, 1, 3, 2]
    sets = [set(range(100 * i, 100 * i + s)) for i, s in enumerate(sizes)]
    Pe = np.full(len(sets), 0.5, np.float32)
    assert select.select_drafts(Pe, sets_to_bits(sets, 600), 6) == [3, 5, 1, 4, 0, 2]
    # an empty footprint costs nothing and wins even with a tiny P
    sets = [set(range(5)), set(), set(range(3))]
    Pz = np.array([0.9, 1e-3, 0.8], np.float32)
    assert select.select_drafts(Pz, sets_to_bits(sets, 8), 1) == [1]
    # then node 2 (0.8 / 3 > 0.9 / 5); node 0 then pays only for its 2 pairs
    # that node 2 did not bring in (score 0.45)
    assert select.select_drafts(Pz, sets_to_bits(sets, 8), 3) == [1, 2, 0]
    assert select.select_drafts(Pz, sets_to_bits(sets, 8), 0) == []
    with pytest.raises(ValueError):
        select.select_drafts(Pz, sets_to_bits(sets, 8), 4)


def test_score_is_float32():
    from fractions import Fraction
    for P, c in ((0.5, 3), (0.7, 0), (0.123, 1000), (1.0, 4608)):
        got = select.score(np.float32(P), c, 1e-6)
        assert got.dtype == np.float32
        # two float32 operations, each correctly rounded: check each rounding
        # against the exact rational value and the float32 neighbours
        d = np.float32(c) + np.float32(1e-6)
        d_exact = Fraction(c) + Fraction(float(np.float32(1e-6)))
        for val, exact in ((d, d_exact), (got, Fraction(float(np.float32(P))) / Fraction(float(d)))):
            up = np.nextafter(val, np.float32(np.inf))
            dn = np.nextafter(val, np.float32(-np.inf))
            err = abs(Fraction(float(val)) - exact)
            assert err <= abs(Fraction(float(up)) - exact) and err <= abs(Fraction(float(dn)) - exact)


def test_static_cost_is_a_sort_and_agrees_on_disjoint_footprints():
    rng = np.random.default_rng(31)
    for _ in range(200):
        N, nbits = int(rng.integers(1, 12)), int(rng.integers(1, 100))
        _, P, sets = random_tree_case(rng, N, nbits)
        gamma = int(rng.integers(0, N + 1))
        F = sets_to_bits(sets, nbits)
        got = select.select_drafts(P, F, gamma, static=True)
        # closed form: top-gamma of P / (|F| + eps), float32, ties to the lower index
        s = [np.float32(np.float32(P[t]) / (np.float32(len(sets[t])) + np.float32(1e-6))) for t in range(N)]
        assert got == sorted(range(N), key=lambda t: (-s[t], t))[:gamma]
    # pairwise disjoint footprints: the marginal cost equals the static one
    for _ in range(100):
        N = int(rng.integers(1, 10))
        sizes = rng.integers(0, 6, N)
        starts = np.concatenate([[0], np.cumsum(sizes)[:-1]])
        sets = [set(range(int(a), int(a + b))) for a, b in zip(starts, sizes)]
        nbits = max(1, int(sizes.sum()))
        P = rng.uniform(0.05, 1.0, N).astype(np.float32)
        F = sets_to_bits(sets, nbits)
        g = int(rng.integers(0, N + 1))
        assert select.select_drafts(P, F, g, static=True) == select.select_drafts(P, F, g)
