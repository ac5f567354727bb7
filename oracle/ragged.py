"""Oracle for ragged, confidence-gated verify (test infrastructure only).

[W-vs-D] = the summary of the width-vs-depth article (batch versus
speculation for MoE on one GPU), section 2 (where to spend depth): sequences
differ widely in how many drafted tokens get accepted; the draft model's
cumulative confidence is a calibrated signal; confidence gating gives every
sequence its own depth in one verify step, by choosing one batch-wide depth
from the live sequences' confidences and then truncating each sequence
greedily while that raises the expected throughput.  Verifying sequences of
different depths in one call is ragged speculation.

Readings (the page gives no formulas):
  R24  sequence s verifies its root (bonus) token plus its first d_s drafts;
       c[s, j] (j = 1..Dmax) is the draft model's cumulative confidence of
       the first j drafts, so the expected tokens produced are
       A_s(d) = 1 + c[s, 1] + ... + c[s, d].
  R25  the expected step time is t_base + t_exp * U, with U the number of
       distinct (layer, expert) pairs over all verified tokens (the cost
       model of the expansion step: one calibrated latency per expert
       brought in); throughput = sum_s A_s / step time.
  R26  float32 throughout: A_s summed over j ascending, the total over s
       ascending, time = fl(t_base + fl(t_exp * U)), throughput =
       fl(total / time); a change is taken only if it raises the throughput
       strictly.  The batch-wide depth is the smallest D in 0..Dmax with the
       largest throughput; then, in sequence order, each d_s is lowered one
       step at a time while that strictly raises the throughput.
  Experts of a token are given as bitsets of (layer, expert) pairs
  E[s, j] (j = 0 is the root token, always verified).

Segmented statistics: for a call whose tokens are grouped by sequence
(segment offsets, R27: tokens of sequence s are rows off[s] .. off[s+1]-1),
the unique experts per (layer, sequence) and per layer overall.
"""
from __future__ import annotations

from typing import List

import numpy as np


def _popcount_words(words: np.ndarray) -> int:
    return int(sum(int(w).bit_count() for w in np.asarray(words, dtype=np.uint64).tolist()))


def throughput(c: np.ndarray, E: np.ndarray, d: List[int], t_base: float, t_exp: float) -> np.float32:
    """Expected tokens per unit time for depths d (R24-R26)."""
    S = len(d)
    total = np.float32(0.0)
    union = np.zeros(E.shape[-1], dtype=np.uint32)
    for s in range(S):
        a = np.float32(1.0)
        for j in range(1, d[s] + 1):
            a = np.float32(a + np.float32(c[s, j]))
        total = np.float32(total + a)
        for j in range(0, d[s] + 1):
            union |= E[s, j]
    U = _popcount_words(union)
    time = np.float32(np.float32(t_base) + np.float32(np.float32(t_exp) * np.float32(U)))
    return np.float32(total / time)


def gate_depths(c: np.ndarray, E: np.ndarray, t_base: float, t_exp: float) -> List[int]:
    """Confidence-gated depths for S sequences.

    c: [S, Dmax + 1] float32 cumulative confidences (column 0 unused);
    E: [S, Dmax + 1, W] uint32 expert bitsets of each sequence's root (j = 0)
    and drafts (j = 1..Dmax)."""
    c = np.asarray(c, dtype=np.float32)
    E = np.asarray(E, dtype=np.uint32)
    S, D1 = c.shape
    Dmax = D1 - 1
    best_D, best = 0, None
    for D in range(Dmax + 1):                         # batch-wide depth
        th = throughput(c, E, [D] * S, t_base, t_exp)
        if best is None or th > best:
            best_D, best = D, th
    d = [best_D] * S
    for s in range(S):                                # greedy per-sequence truncation
        while d[s] > 0:
            trial = list(d)
            trial[s] -= 1
            th = throughput(c, E, trial, t_base, t_exp)
            if th > best:
                d, best = trial, th
            else:
                break
    return d


def segment_union_stats(topk_idx: np.ndarray, offsets: np.ndarray, E: int):
    """topk_idx [nL, T, k] of a call whose tokens are grouped by sequence
    (offsets [S + 1], R27) -> (per_seq [nL, S] int32 unique experts of each
    sequence's tokens, total [nL] int32 unique experts of the call)."""
    topk_idx = np.asarray(topk_idx)
    nL = topk_idx.shape[0]
    S = len(offsets) - 1
    per = np.zeros((nL, S), dtype=np.int32)
    tot = np.zeros(nL, dtype=np.int32)
    for l in range(nL):
        tot[l] = len(set(int(e) for e in topk_idx[l].ravel().tolist() if 0 <= e < E))
        for s in range(S):
            rows = topk_idx[l, offsets[s]:offsets[s + 1]]
            per[l, s] = len(set(int(e) for e in rows.ravel().tolist() if 0 <= e < E))
    return per, tot
