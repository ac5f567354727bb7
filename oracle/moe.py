"""Oracle for the MoE-layer verify step (test infrastructure only).

Pages cited:
  [EcoSpec]  the review of "Less Experts, Faster Decoding: Cost-Aware
             Speculative Decoding for Mixture-of-Experts" (EcoSpec);
  [S2-MoE]   the walkthrough of S^2-MoE (self-speculative decoding for MoE
             on edge devices): motivation (challenge 2, reuse ratio) and
             component 2 (reuse-aware expert gating, Fig. 5);
  [W-vs-D]   the summary of the width-vs-depth article (MoE co-activation).

What the method computes, in the pages' terms: verifying the speculated
tokens at one MoE layer costs the union of the experts those tokens route to
([EcoSpec] §2, verify-union equation; [S2-MoE] motivation, challenge 2), so
the layer's output is the ordinary MoE output of every token; only the cost
depends on the union.  The oracle is therefore the plain definition: route
each token, then a per-token dense loop over that token's own top-k experts.

Readings taken where the pages are silent (each is a parameter or a
documented choice; tests pin them):
  R1  softmax routing: router logits -> softmax -> top-k ([EcoSpec] §3.1
      describes this pipeline; no other router function appears).
  R2  top-k order is (logit descending, expert index ascending); selection
      compares logits, never probabilities.
  R3  gate weights are the softmax over all experts renormalised over the
      selected k (equivalently a softmax over the selected logits).
  R4  expert importance g_e = sum_b w_b * softmax(l_b)_e * [e in TopK_b]
      ([S2-MoE] component 2, step 1; the displayed formula is missing).
  R5  preferred set P* = first `cap` experts by (g descending, index
      ascending) among experts with g_e > 0 (step 2; formula missing).
  R6  bias lambda_b = alpha * (l_b,(1) - l_b,(k+1)) added to the logits of
      the experts in P* (step 3; proportional to the top-1 / (k+1)-th margin),
      computed in float32 as three separately rounded operations; lambda = 0
      when k == E.
  R7  the biased logits decide the selection only; gate weights are R3 on
      the original logits over the new selection.
  R13 the always-on shared expert has weight 1, is outside the union and
      outside the union statistics.
  R16 bias aggregation runs over all tokens of the call, unless the call's
      tokens are grouped by sequence (segment offsets, as in a ragged or
      batched verify call): then the importance and the preferred set are
      those of each sequence's own tokens, and a token is biased toward its
      own sequence's preferred set (each sequence verifies its own drafts;
      [W-vs-D] section 2, ragged speculation; [S2-MoE] component 2, steps
      1-2, whose candidate set is one sequence's drafts).
  R20 expert FFN = SwiGLU: W_d (SiLU(W_g x) * (W_u x)), SiLU(z) = z / (1 + e^-z).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Optional, Tuple

import numpy as np

ExpertFn = Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray]]


# ----------------------------------------------------------------------------
# Routing
# ----------------------------------------------------------------------------
def router_logits(x: np.ndarray, Wr: np.ndarray) -> np.ndarray:
    """l[t, e] = sum_h x[t, h] * Wr[e, h], accumulated in float64.

    [EcoSpec] §3.1 (per-layer routing logits over E experts);
    [S2-MoE] component 2, step 1 (the target gate's logits l_b)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(Wr, dtype=np.float64).T


def softmax(logits: np.ndarray) -> np.ndarray:
    """Softmax over the last axis in float64."""
    l = np.asarray(logits, dtype=np.float64)
    z = np.exp(l - l.max(axis=-1, keepdims=True))
    return z / z.sum(axis=-1, keepdims=True)


def order_desc(row: np.ndarray) -> np.ndarray:
    """Expert indices sorted by (value descending, index ascending) (R2).

    A stable sort of the negated values keeps equal values in index order."""
    return np.argsort(-np.asarray(row), kind="stable")


def topk(logits: np.ndarray, k: int) -> np.ndarray:
    """Per-token top-k expert indices, [T, k] int32, in rank order (R2).

    [EcoSpec] §3.1 (top-K per layer, K equal to the model's routing k);
    [EcoSpec] §2 (S_l(x_t), the experts token t routes to at layer l)."""
    l = np.asarray(logits)
    E = l.shape[-1]
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    return np.stack([order_desc(row)[:k] for row in l]).astype(np.int32)


def gate_weights(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Gate weights [T, k]: softmax over all experts, renormalised over each
    token's selected experts (R3).  float64."""
    p = softmax(logits)
    sel = np.take_along_axis(p, np.asarray(idx, dtype=np.int64), axis=-1)
    return sel / sel.sum(axis=-1, keepdims=True)


@dataclass
class BiasResult:
    g: np.ndarray            # [E] float64 expert importance (R4)
    pstar: np.ndarray        # [<= cap] int32 preferred experts, in (g desc, idx asc) order (R5)
    lam: np.ndarray          # [T] float32 per-token bias size (R6)
    biased: np.ndarray       # [T, E] float32 biased logits (R6)
    topk_idx: np.ndarray     # [T, k] int32 selection on the biased logits
    topk_w: np.ndarray       # [T, k] float64 gate weights on the original logits (R7)


def expert_importance(logits: np.ndarray, idx: np.ndarray, w_conf: np.ndarray) -> np.ndarray:
    """g_e = sum_b w_b * softmax(l_b)_e * [e in TopK_b] (R4), float64.

    [S2-MoE] component 2, step 1: confidence-weighted aggregation of each
    draft token's gate preference; high-confidence tokens count more."""
    T, E = np.asarray(logits).shape
    p = softmax(logits)
    g = np.zeros(E, dtype=np.float64)
    for b in range(T):
        for e in idx[b]:
            g[e] += float(w_conf[b]) * p[b, e]
    return g


def preferred_set(g: np.ndarray, cap: int) -> np.ndarray:
    """P* = first `cap` experts by (g desc, index asc) with g > 0 (R5).

    [S2-MoE] component 2, step 2: a bounded global set, cap >= k."""
    order = order_desc(g)
    return np.array([e for e in order if g[e] > 0][:cap], dtype=np.int32)


def bias_from_pstar(logits32: np.ndarray, pstar: np.ndarray, k: int, alpha: float):
    """Per-token bias and biased logits given P* (R6), in float32.

    [S2-MoE] component 2, step 3: an additive bias on the logits of the
    preferred experts, sized per token by the gap between its top-1 score and
    its (k+1)-th score.  float32: d = l_(1) - l_(k+1); lambda = alpha * d;
    l'_e = l_e + lambda for e in P*.  No fused multiply-add."""
    l = np.asarray(logits32, dtype=np.float32)
    T, E = l.shape
    a = np.float32(alpha)
    lam = np.zeros(T, dtype=np.float32)
    out = l.copy()
    inP = np.zeros(E, dtype=bool)
    inP[np.asarray(pstar, dtype=np.int64)] = True
    for b in range(T):
        if k < E:
            order = order_desc(l[b])
            d = np.float32(l[b, order[0]] - l[b, order[k]])
            lam[b] = np.float32(a * d)
        for e in range(E):
            if inP[e]:
                out[b, e] = np.float32(l[b, e] + lam[b])
    return lam, out


def reuse_bias(logits32: np.ndarray, w_conf: np.ndarray, k: int, cap: int, alpha: float,
               pstar: Optional[np.ndarray] = None) -> BiasResult:
    """Reuse-aware soft routing bias ([S2-MoE] component 2, steps 1-3, Fig. 5).

    logits32 are the router's float32 logits.  If ``pstar`` is given it is
    used instead of the one computed here (P* depends on exp(), so a parity
    check can take P* from the device and check the remaining steps bit for
    bit)."""
    l = np.asarray(logits32, dtype=np.float32)
    T, E = l.shape
    if not (k <= cap <= E):
        raise ValueError("need k <= cap <= E")
    if not (0.0 <= alpha < 1.0):
        raise ValueError("need 0 <= alpha < 1")
    idx0 = topk(l, k)
    g = expert_importance(l, idx0, w_conf)
    ps = preferred_set(g, cap) if pstar is None else np.asarray(pstar, dtype=np.int32)
    lam, biased = bias_from_pstar(l, ps, k, alpha)
    idx1 = topk(biased, k)
    w1 = gate_weights(l, idx1)
    return BiasResult(g=g, pstar=ps, lam=lam, biased=biased, topk_idx=idx1, topk_w=w1)


@dataclass
class SegmentBiasResult:
    offsets: np.ndarray      # [S + 1] token offsets of the sequences
    g: np.ndarray            # [S, E] float64 importance of each sequence's tokens (R4, R16)
    pstar: list              # S arrays, each sequence's preferred set (R5)
    lam: np.ndarray          # [T] float32 per-token bias size (R6)
    biased: np.ndarray       # [T, E] float32 biased logits (R6)
    topk_idx: np.ndarray     # [T, k] int32
    topk_w: np.ndarray       # [T, k] float64 (R7)


def check_offsets(offsets, T: int) -> np.ndarray:
    off = np.asarray(offsets, dtype=np.int64)
    if off.ndim != 1 or len(off) < 2 or off[0] != 0 or off[-1] != T or np.any(np.diff(off) < 0):
        raise ValueError("offsets must be non-decreasing from 0 to T")
    return off


def reuse_bias_segments(logits32: np.ndarray, w_conf: np.ndarray, k: int, cap: int, alpha: float,
                        offsets, pstar=None) -> SegmentBiasResult:
    """Reuse-aware soft bias with the tokens grouped by sequence (R16): the
    pooled bias of ``reuse_bias`` applied to each sequence's rows
    offsets[s] .. offsets[s+1]-1 on their own.  ``pstar`` (optional) gives
    each sequence's preferred set instead of the computed one."""
    l = np.asarray(logits32, dtype=np.float32)
    T, E = l.shape
    off = check_offsets(offsets, T)
    S = len(off) - 1
    if not (k <= cap <= E):
        raise ValueError("need k <= cap <= E")
    if not (0.0 <= alpha < 1.0):
        raise ValueError("need 0 <= alpha < 1")
    g = np.zeros((S, E), dtype=np.float64)
    ps = []
    lam = np.zeros(T, dtype=np.float32)
    biased = l.copy()
    idx = np.zeros((T, k), dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float64)
    for s in range(S):
        a, b = int(off[s]), int(off[s + 1])
        if a == b:
            ps.append(np.zeros(0, dtype=np.int32))
            continue
        r = reuse_bias(l[a:b], np.asarray(w_conf)[a:b], k, cap, alpha,
                       pstar=None if pstar is None else pstar[s])
        g[s], lam[a:b], biased[a:b], idx[a:b], w[a:b] = r.g, r.lam, r.biased, r.topk_idx, r.topk_w
        ps.append(r.pstar)
    return SegmentBiasResult(offsets=off.astype(np.int32), g=g, pstar=ps, lam=lam, biased=biased,
                             topk_idx=idx, topk_w=w)


# ----------------------------------------------------------------------------
# Union and grouping
# ----------------------------------------------------------------------------
def expert_union(topk_idx: np.ndarray) -> np.ndarray:
    """Ascending union of the experts the verified tokens route to.

    [EcoSpec] §2: E_verify = union over t in S of S_l(x_t)."""
    return np.array(sorted({int(e) for e in np.asarray(topk_idx).ravel()}), dtype=np.int32)


def reuse_ratio(topk_idx: np.ndarray) -> float:
    """|union| / (s * k) ([S2-MoE] motivation, challenge 2), float64."""
    s, k = np.asarray(topk_idx).shape
    return len(expert_union(topk_idx)) / (s * k)


@dataclass
class CSR:
    union: np.ndarray   # [U] ascending expert ids
    ptr: np.ndarray     # [U + 1]
    tok: np.ndarray     # [T * k] token ids, ascending within each expert
    w: np.ndarray       # [T * k] gate weight of (token, expert)


def csr(topk_idx: np.ndarray, topk_w: np.ndarray) -> CSR:
    """Token-by-expert grouping: for each union expert in ascending order, the
    tokens (ascending) that route to it and their gate weights.  This is the
    grouping that lets each unique expert be applied once to all of its
    tokens ([EcoSpec] §1-§2: the weights to load are the union)."""
    idx = np.asarray(topk_idx)
    T, k = idx.shape
    U = expert_union(idx)
    ptr = [0]
    tok, w = [], []
    for e in U:
        for t in range(T):
            for j in range(k):
                if idx[t, j] == e:
                    tok.append(t)
                    w.append(topk_w[t, j])
        ptr.append(len(tok))
    return CSR(union=U, ptr=np.array(ptr, dtype=np.int32), tok=np.array(tok, dtype=np.int32),
               w=np.array(w, dtype=np.float64))


def union_stats(topk_idx_layers: np.ndarray, E: Optional[int] = None):
    """Per layer: number of unique experts and reuse ratio |U| / (T k).

    Counts are integers; the ratio is the correctly rounded float32 quotient
    of two small integers ([S2-MoE] motivation, challenge 2).  With ``E``
    given, entries outside [0, E) name no expert and are left out of the
    union (the denominator stays T k: it counts the routing slots)."""
    a = np.asarray(topk_idx_layers)
    nL, T, k = a.shape

    counts = np.zeros(nL, dtype=np.int32)
    for l in range(nL):
        named = [int(e) for e in a[l].ravel() if E is None or 0 <= e < E]
        counts[l] = len(set(named))
    reuse = np.array([np.float32(c) / np.float32(T * k) for c in counts], dtype=np.float32)
    return counts, reuse


# ----------------------------------------------------------------------------
# Expert FFN and the layer output
# ----------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def swiglu(Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray, x: np.ndarray) -> np.ndarray:
    """One expert on one token (R20): Wd @ (SiLU(Wg @ x) * (Wu @ x))."""
    x = np.asarray(x, dtype=np.float64)
    return Wd @ (silu(Wg @ x) * (Wu @ x))


def moe_layer(x: np.ndarray, topk_idx: np.ndarray, topk_w: np.ndarray, expert: ExpertFn,
              shared: Optional[Tuple[np.ndarray, np.ndarray, np.ndarray]] = None,
              tokens: Optional[np.ndarray] = None) -> np.ndarray:
    """Layer output as a per-token dense loop over each token's own top-k.

    y_t = sum_j w_tj * FFN_{e_tj}(x_t)  (+ FFN_shared(x_t), weight 1, R13).
    ``expert(e)`` returns float64 (Wg [I,H], Wu [I,H], Wd [H,I]).  ``tokens``
    restricts the loop to a subset of tokens (rows of the result for other
    tokens are left zero)."""
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    y = np.zeros((T, H), dtype=np.float64)
    rows = range(T) if tokens is None else [int(t) for t in tokens]
    for t in rows:
        for j in range(topk_idx.shape[1]):
            Wg, Wu, Wd = expert(int(topk_idx[t, j]))
            y[t] += float(topk_w[t, j]) * swiglu(Wg, Wu, Wd, x[t])
        if shared is not None:
            y[t] += swiglu(shared[0], shared[1], shared[2], x[t])
    return y


@dataclass
class Routing:
    logits: np.ndarray
    topk_idx: np.ndarray
    topk_w: np.ndarray
    bias: Optional[BiasResult]


def route(logits32: np.ndarray, k: int, w_conf: Optional[np.ndarray] = None, cap: int = 0,
          alpha: float = 0.0, pstar=None, offsets=None) -> Routing:
    """Routing of one call: top-k and gate weights, with the optional reuse
    bias when ``w_conf`` is given, pooled over the call or, with sequence
    ``offsets``, per sequence (then ``pstar`` is a list, one set per
    sequence)."""
    l = np.asarray(logits32, dtype=np.float32)
    if w_conf is None:
        idx = topk(l, k)
        return Routing(l, idx, gate_weights(l, idx), None)
    if offsets is not None:
        b = reuse_bias_segments(l, w_conf, k, cap, alpha, offsets, pstar=pstar)
    else:
        b = reuse_bias(l, w_conf, k, cap, alpha, pstar=pstar)
    return Routing(l, b.topk_idx, b.topk_w, b)
