"""Oracle for EcoSpec cost-aware greedy draft selection (test infrastructure only).

[EcoSpec] = the review of "Less Experts, Faster Decoding: Cost-Aware
Speculative Decoding for Mixture-of-Experts".

§3.2 (global expert buffer): the buffer B holds the (layer, expert) pairs
already covered by the drafts chosen so far in this speculative step; it
starts empty and is rebuilt every step, so a node pays only for experts no
earlier choice has brought in.

§3.3 (score equation and greedy selection): node t scores
    S(t) = P(t) / (DeltaCost(t | B) + eps)
where P(t) is the product of draft probabilities along the path from the
root to t and DeltaCost(t | B) is the number of (layer, expert) pairs of t's
whole-path predicted footprint not yet in B.  The greedy step takes the best
remaining node gamma times, adding its footprint to B after each pick.

Readings:
  R8   eps is unspecified beyond preventing division by zero: parameter,
       default 1e-6.
  R9   nodes are numbered in BFS order (parent index < child index); equal
       scores go to the lowest node index.
  R10  B starts empty; the root's own experts are not pre-loaded.
  R11  a node's footprint is the union of the predicted per-layer top-k of
       the node and of its draft ancestors (root excluded), given as bitsets.
  R17  DeltaCost is a count (the garbled formula lost its cardinality bars;
       the text defines it as a number of new experts).
  Arithmetic: c = popcount(F_t & ~B) is exact; the score is
  float32(P_t) / (float32(c) + float32(eps)), two IEEE float32 operations,
  each rounded to nearest.
"""
from __future__ import annotations

from typing import List, Sequence

import numpy as np


def new_pairs(F_t: np.ndarray, B: np.ndarray) -> int:
    """|footprint \\ B| for bitsets given as uint32 word arrays."""
    return int(sum(int(f & ~b & 0xFFFFFFFF).bit_count() for f, b in zip(F_t.tolist(), B.tolist())))


def score(P_t, c: int, eps: float) -> np.float32:
    return np.float32(np.float32(P_t) / (np.float32(c) + np.float32(eps)))


def popcounts(words: np.ndarray) -> np.ndarray:
    """Number of set bits of each row of a [..., W] uint32 bitset array."""
    w = np.ascontiguousarray(np.asarray(words, dtype=np.uint32))
    return np.unpackbits(w.view(np.uint8), axis=-1).sum(axis=-1).astype(np.int64)


def select_drafts(P: np.ndarray, F: np.ndarray, gamma: int, eps: float = 1e-6, static: bool = False) -> List[int]:
    """Cost-aware selection for one tree; returns node ids in pick order.

    P: [N] float32 path probabilities; F: [N, W] uint32 path footprints.
    Each round scores every node at once, S = P / (|F \\ B| + eps) in
    float32 (§3.3), with the nodes already taken scored -inf, and takes the
    first node in (score desc, index asc) order; its footprint then joins
    the buffer B, which starts empty (§3.2).  static: the ablation of
    [EcoSpec] section 4.3, where the cost is the size of the whole path
    footprint (B stays empty)."""
    P = np.asarray(P, dtype=np.float32)
    F = np.asarray(F, dtype=np.uint32)
    N = P.shape[0]
    if not 0 <= gamma <= N:
        raise ValueError("need 0 <= gamma <= N")
    B = np.zeros(F.shape[1], dtype=np.uint32)
    taken = np.zeros(N, dtype=bool)
    picks: List[int] = []
    node = np.arange(N)
    for _ in range(gamma):
        cost = popcounts(F & ~B[None, :]).astype(np.float32)          # new (layer, expert) pairs
        score = P / (cost + np.float32(eps))                             # two float32 operations
        score = np.where(taken, np.float32(-np.inf), score)
        pick = int(np.lexsort((node, -score))[0])                        # score desc, then index asc
        picks.append(pick)
        taken[pick] = True
        if not static:
            B = B | F[pick]
    return picks


def select_drafts_batch(P: np.ndarray, F: np.ndarray, gamma: int, eps: float = 1e-6,
                        static: bool = False) -> np.ndarray:
    """select_drafts for each of nt trees: P [nt, N], F [nt, N, W] -> [nt, gamma]."""
    return np.array([select_drafts(P[i], F[i], gamma, eps, static) for i in range(P.shape[0])],
                    dtype=np.int32).reshape(P.shape[0], gamma)


def is_greedy_sequence(seq: Sequence[int], P: np.ndarray, F: np.ndarray, eps: float = 1e-6) -> bool:
    """True iff every element of ``seq`` is the best remaining node (ties to
    the lowest index) given the footprints of the elements before it."""
    P = np.asarray(P, dtype=np.float32)
    F = np.asarray(F, dtype=np.uint32)
    B = np.zeros(F.shape[1], dtype=np.uint32)
    used = set()
    for pick in seq:
        if pick in used:
            return False
        scores = {t: score(P[t], new_pairs(F[t], B), eps) for t in range(len(P)) if t not in used}
        top = max(scores.values())
        if pick != min(t for t, s in scores.items() if s == top):
            return False
        used.add(pick)
        B |= F[pick]
    return True
