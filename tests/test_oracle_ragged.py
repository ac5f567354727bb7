"""Pins of the ragged / confidence-gated verify oracle (CPU only)."""
import numpy as np

import synth
from oracle import moe as omoe
from oracle import ragged


def bits(sets, nbits):
    W = (nbits + 31) // 32
    b = np.zeros((len(sets), nbits), dtype=bool)
    for i, s in enumerate(sets):
        for p in s:
            b[i, p] = True
    return synth.pack_bits(b, W)


def case(rng, S, Dmax, nbits):
    E = np.stack([bits([set(rng.choice(nbits, size=min(nbits, int(rng.integers(1, 6))), replace=False).tolist())
                        for _ in range(Dmax + 1)], nbits) for _ in range(S)])
    q = rng.uniform(0.2, 1.0, (S, Dmax + 1)).astype(np.float32)
    c = np.cumprod(q, axis=1).astype(np.float32)
    c[:, 0] = 1.0
    return c, E


def test_hand_example_gives_ragged_depths():
    # sequence 0 reuses its root's experts with high confidence, sequence 1
    # brings new experts with low confidence (t_base 10, t_exp 1):
    # common depth 2 (3.81 / 18 beats 3.0 / 16 and 2 / 14); truncating
    # sequence 0 loses tokens without saving experts; truncating sequence 1
    # twice raises 0.2117 -> 0.2375 -> 0.2643.
    E = np.stack([bits([{0, 1}, {0, 1}, {0, 1}], 8), bits([{2, 3}, {4, 5}, {6, 7}], 8)])
    c = np.array([[1.0, 0.9, 0.8], [1.0, 0.1, 0.01]], np.float32)
    assert ragged.gate_depths(c, E, 10.0, 1.0) == [2, 0]


def test_free_experts_take_full_depth_and_useless_drafts_none():
    rng = np.random.default_rng(1)
    for _ in range(50):
        S, Dmax = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        c, E = case(rng, S, Dmax, 64)
        assert ragged.gate_depths(c, E, 5.0, 0.0) == [Dmax] * S           # time fixed: depth only adds
        c0 = c.copy()
        c0[:, 1:] = 0.0
        assert ragged.gate_depths(c0, E, 5.0, 1.0) == [0] * S              # drafts never pay off


def test_invariants_random():
    rng = np.random.default_rng(2)
    for _ in range(200):
        S, Dmax, nbits = int(rng.integers(1, 6)), int(rng.integers(0, 6)), int(rng.integers(4, 100))
        c, E = case(rng, S, Dmax, nbits)
        t_base, t_exp = float(rng.uniform(1, 50)), float(rng.uniform(0, 2))
        d = ragged.gate_depths(c, E, t_base, t_exp)
        ths = [ragged.throughput(c, E, [D] * S, t_base, t_exp) for D in range(Dmax + 1)]
        Dstar = int(np.argmax(ths))                                         # first maximum
        assert all(0 <= v <= Dstar for v in d)
        assert ragged.throughput(c, E, d, t_base, t_exp) >= ths[Dstar]


def test_throughput_counts_distinct_pairs():
    E = np.stack([bits([{0, 1, 2}, {2, 3}], 40), bits([{1, 30}, {39}], 40)])
    c = np.array([[1.0, 0.5], [1.0, 0.25]], np.float32)
    # all tokens: pairs {0,1,2,3,30,39} = 6; tokens (1 + 0.5) + (1 + 0.25) = 2.75
    assert ragged.throughput(c, E, [1, 1], 4.0, 0.5) == np.float32(2.75) / np.float32(7.0)
    # roots only: pairs {0,1,2,30} = 4
    assert ragged.throughput(c, E, [0, 0], 4.0, 0.5) == np.float32(2.0) / np.float32(6.0)


def test_segment_union_stats():
    rng = np.random.default_rng(3)
    E, k = 64, 4
    off = np.array([0, 3, 4, 9, 9 + 2])                                    # ragged segments
    T = int(off[-1])
    idx = np.stack([np.stack([rng.choice(E, k, replace=False) for _ in range(T)]) for _ in range(5)])
    per, tot = ragged.segment_union_stats(idx, off, E)
    counts, _ = omoe.union_stats(idx)
    assert np.array_equal(tot, counts)
    for s in range(len(off) - 1):
        c1, _ = omoe.union_stats(idx[:, off[s]:off[s + 1]])
        assert np.array_equal(per[:, s], c1)
    assert (per.max(axis=1) <= tot).all() and (tot <= per.sum(axis=1)).all()


def test_segment_union_stats_ignores_out_of_range_and_empty_segments():
    E = 10
    idx = np.array([[[1, 2], [2, -1], [10, 3], [9, 0]]], dtype=np.int32)   # one layer, T = 4, k = 2
    off = np.array([0, 2, 2, 4])                                              # segment 1 is empty
    per, tot = ragged.segment_union_stats(idx, off, E)
    assert per.tolist() == [[2, 0, 3]]        # {1, 2}; {}; {3, 9, 0}
    assert tot.tolist() == [5]                # {0, 1, 2, 3, 9}
    counts, _ = omoe.union_stats(idx, E)
    assert tot.tolist() == counts.tolist()
