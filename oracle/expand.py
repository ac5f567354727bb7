"""Oracle for S^2-MoE routing-aware adaptive expansion (test infrastructure only).

[S2-MoE] = the walkthrough of S^2-MoE (self-speculative decoding for MoE on
edge devices), component 1 (routing-aware adaptive speculative expansion).

The page prices adding draft token i to the expansion set S by the experts
it would bring in that no token of S has activated yet, each new expert
costing one calibrated latency unit T_exp, plus the draft-side cost of the
token's descendants:
    DeltaC(i | S) = |E_i \\ union_{j in S} E_j| * T_exp
    C_i           = DeltaC(i | S) + C_i^draft
and weighs it against the expected saving p_i * T_AR (acceptance
probability times one autoregressive step):
    U_i = p_i * T_AR / C_i.
Candidates are examined in draft-generation order and taken while U_i >= 1.

Readings:
  R21  "until no candidate satisfies the condition": passes over the
       candidates in generation order repeat until a whole pass adds none.
       Adding a token only removes experts from the others' new sets, so
       the test is monotone in S and the final set is the unique least
       fixed point, whatever the order.
  R22  a node can be taken only once its parent is in S (a node whose
       parent is not verified can never be accepted; the set stays
       prefix-closed, as the draft tree of [EcoSpec] section 3.3).
  R23  U_i >= 1 is decided as the float32 comparison
       fl(p_i * T_AR) >= fl(fl(c_i * T_exp) + C_i^draft), each operation
       rounded to nearest (no fused multiply-add); c_i is the exact count.
  E_i is given as a bitset of (layer, expert) pairs.  With a prefix-closed S
  a node's own pairs and its whole-path pairs give the same count, so the
  path footprints of the selection input serve unchanged.
"""
from __future__ import annotations

from typing import List, Sequence

import numpy as np

from .select import new_pairs


def accepts(p, c: int, t_ar, t_exp, c_draft) -> bool:
    """U >= 1 in the float32 form of R23."""
    num = np.float32(np.float32(p) * np.float32(t_ar))
    den = np.float32(np.float32(np.float32(c) * np.float32(t_exp)) + np.float32(c_draft))
    return bool(num >= den)


def expand(parent: Sequence[int], P: np.ndarray, F: np.ndarray, t_ar: float, t_exp: float,
           c_draft: np.ndarray) -> List[int]:
    """Utility-driven expansion of one draft tree; returns node ids in the
    order they join S.

    parent: [N] BFS order, -1 = child of the root; P: [N] float32 acceptance
    (path) probabilities; F: [N, W] uint32 footprints; c_draft: [N] float32."""
    P = np.asarray(P, dtype=np.float32)
    F = np.asarray(F, dtype=np.uint32)
    cd = np.asarray(c_draft, dtype=np.float32)
    N = len(parent)
    B = np.zeros(F.shape[1], dtype=np.uint32)
    inS = [False] * N
    order: List[int] = []
    while True:
        added = False
        for i in range(N):                      # one pass in generation order
            if inS[i] or (parent[i] >= 0 and not inS[parent[i]]):
                continue
            if accepts(P[i], new_pairs(F[i], B), t_ar, t_exp, cd[i]):
                inS[i] = True
                order.append(i)
                B |= F[i]
                added = True
        if not added:
            return order


def expand_batch(parent, P, F, t_ar, t_exp, c_draft) -> np.ndarray:
    """expand for nt trees: P [nt, N], F [nt, N, W], c_draft [nt, N] ->
    [nt, N] int32, the join order padded with -1."""
    nt, N = np.asarray(P).shape
    out = np.full((nt, N), -1, dtype=np.int32)
    for t in range(nt):
        o = expand(parent, P[t], F[t], t_ar, t_exp, c_draft[t])
        out[t, :len(o)] = o
    return out
