"""Pins of the S^2-MoE utility-expansion oracle (CPU only)."""
import numpy as np

import synth
from oracle import expand


def sets_to_bits(sets, nbits):
    W = (nbits + 31) // 32
    b = np.zeros((len(sets), nbits), dtype=bool)
    for i, s in enumerate(sets):
        for p in s:
            b[i, p] = True
    return synth.pack_bits(b, W)


def random_tree(rng, N, nbits):
    parent = [-1] + [int(rng.integers(-1, i)) for i in range(1, N)]
    own = [set(rng.choice(nbits, size=min(nbits, int(rng.integers(0, 6))), replace=False).tolist())
           for _ in range(N)]
    P = np.zeros(N, np.float32)
    sets = []
    for i in range(N):
        e = np.float32(rng.uniform(0.3, 1.0))
        P[i] = e if parent[i] < 0 else np.float32(P[parent[i]] * e)
        sets.append(set(own[i]) if parent[i] < 0 else own[i] | sets[parent[i]])
    return parent, P, sets


def jacobi_closure(parent, P, sets, t_ar, t_exp, cd):
    """Least fixed point by simultaneous rounds over Python sets: every node
    that is eligible and passes the test against the current union joins at
    once.  A different schedule from the oracle's in-order passes; both
    compute the least fixed point of the same monotone test."""
    S = set()
    while True:
        B = set().union(*[sets[j] for j in S]) if S else set()
        new = {i for i in range(len(P)) if i not in S and (parent[i] < 0 or parent[i] in S)
               and expand.accepts(P[i], len(sets[i] - B), t_ar, t_exp, cd[i])}
        if not new:
            return S
        S |= new


def test_free_experts_take_every_node_in_order():
    rng = np.random.default_rng(1)
    parent, P, sets = random_tree(rng, 14, 90)
    F = sets_to_bits(sets, 90)
    assert expand.expand(parent, P, F, 1.0, 0.0, np.zeros(14, np.float32)) == list(range(14))


def test_no_benefit_takes_nothing():
    rng = np.random.default_rng(2)
    parent, P, sets = random_tree(rng, 14, 90)
    F = sets_to_bits(sets, 90)
    assert expand.expand(parent, P, F, 0.0, 1.0, np.full(14, 0.25, np.float32)) == []


def test_hand_chain():
    # chain 0 -> 1 -> 2 with own experts {0,1}, {2}, {3,4,5}; path footprints
    # are unions.  T_AR = 10, T_exp = 2, no draft cost.
    parent = [-1, 0, 1]
    sets = [{0, 1}, {0, 1, 2}, {0, 1, 2, 3, 4, 5}]
    F = sets_to_bits(sets, 8)
    P = np.array([0.9, 0.5, 0.4], np.float32)
    cd = np.zeros(3, np.float32)
    # node 0: 9 >= 2*2 = 4 joins; node 1: 5 >= 1*2 joins; node 2: 4 >= 3*2 = 6 fails
    assert expand.expand(parent, P, F, 10.0, 2.0, cd) == [0, 1]
    # a larger saving per step lets node 2 in: 0.4 * 15 = 6 >= 6 (the boundary counts)
    assert expand.expand(parent, P, F, 15.0, 2.0, cd) == [0, 1, 2]
    # draft cost alone can stop a node that brings no new expert
    sets2 = [{0, 1}, {0, 1}, {0, 1}]
    F2 = sets_to_bits(sets2, 8)
    assert expand.expand(parent, P, F2, 10.0, 2.0, np.array([0.0, 6.0, 0.0], np.float32)) == [0]


def test_reuse_beats_equal_confidence():
    # children 1 and 2 of the root have equal probability; 1 reuses the
    # experts of node 0, 2 brings three new ones.  T_AR = 10:
    #   T_exp = 2: node 0 9 >= 3*2 joins, node 1 5 >= 0 joins, node 2 5 < 3*2 stays out
    #   T_exp = 1: node 2 5 >= 3*1 joins as well
    parent = [-1, -1, -1]
    sets = [{0, 1, 2}, {0, 1, 2}, {3, 4, 5}]
    F = sets_to_bits(sets, 8)
    P = np.array([0.9, 0.5, 0.5], np.float32)
    cd = np.zeros(3, np.float32)
    assert expand.expand(parent, P, F, 10.0, 2.0, cd) == [0, 1]
    assert expand.expand(parent, P, F, 10.0, 1.0, cd) == [0, 1, 2]


def test_matches_jacobi_closure_and_is_a_fixed_point():
    rng = np.random.default_rng(3)
    for _ in range(300):
        N, nbits = int(rng.integers(1, 15)), int(rng.integers(1, 80))
        parent, P, sets = random_tree(rng, N, nbits)
        F = sets_to_bits(sets, nbits)
        t_ar = float(rng.uniform(0.5, 20.0))
        t_exp = float(rng.uniform(0.0, 3.0))
        cd = rng.uniform(0.0, 2.0, N).astype(np.float32)
        got = expand.expand(parent, P, F, t_ar, t_exp, cd)
        assert len(got) == len(set(got))
        assert set(got) == jacobi_closure(parent, P, sets, t_ar, t_exp, cd)
        # prefix-closed, in join order
        seen = set()
        for i in got:
            assert parent[i] < 0 or parent[i] in seen
            seen.add(i)
        # nothing outside passes at the end
        B = set().union(*[sets[j] for j in got]) if got else set()
        for i in range(N):
            if i not in seen and (parent[i] < 0 or parent[i] in seen):
                assert not expand.accepts(P[i], len(sets[i] - B), t_ar, t_exp, cd[i])


def test_monotone_in_benefit_and_cost():
    rng = np.random.default_rng(4)
    for _ in range(100):
        N, nbits = int(rng.integers(2, 15)), int(rng.integers(8, 80))
        parent, P, sets = random_tree(rng, N, nbits)
        F = sets_to_bits(sets, nbits)
        cd = rng.uniform(0.0, 1.0, N).astype(np.float32)
        a = set(expand.expand(parent, P, F, 5.0, 1.0, cd))
        assert a <= set(expand.expand(parent, P, F, 8.0, 1.0, cd))      # more saving per step
        assert set(expand.expand(parent, P, F, 5.0, 1.5, cd)) <= a      # dearer experts


def test_batch_shape_and_padding():
    trees = synth.draft_trees(seed=5, nt=6, n_layers=4, E=16, k=2)
    cd = np.full(trees.P.shape, 0.05, np.float32)
    out = expand.expand_batch(trees.parent, trees.P, trees.F, 4.0, 0.2, cd)
    assert out.shape == trees.P.shape
    for t in range(6):
        o = expand.expand(trees.parent, trees.P[t], trees.F[t], 4.0, 0.2, cd[t])
        assert out[t, :len(o)].tolist() == o and (out[t, len(o):] == -1).all()
