"""Seeded synthetic inputs for the MoE verify layer and for draft selection.

This module is the only code that both the CPU oracle and the HIP library's
tests/bench use.  It holds input generation only and none of the method's
arithmetic (no routing, no top-k of router logits, no union, no FFN, no
selection).  Every random value comes from one of two sources:

* ``numpy.random.Generator(PCG64)`` streams spawned from
  ``SeedSequence(seed)`` for activations, logit structure and draft trees;
* a counter-based generator for expert weights, defined below, implemented
  three times from the same definition: NumPy (``counter_*`` functions, the
  executable definition), plain C with OpenMP (``hostfill.c``) and HIP
  (``devfill.hip``).  The C and HIP fills are checked bit for bit against
  the NumPy definition.

Counter-based weight generator (SplitMix64, Steele, Lea & Flood, OOPSLA 2014)
------------------------------------------------------------------------------
``mix64`` is SplitMix64's output function.  The n-th output (n = 0, 1, ...)
of a SplitMix64 generator seeded with state ``s`` is
``mix64(s + (n + 1) * GAMMA)`` (mod 2**64).

* stream id ``sid = seed<<48 | layer<<32 | expert<<16 | matrix`` (16 bits each);
* stream state ``s = mix64(sid)``;
* element n of the stream draws ``v = mix64(s + (n + 1) * GAMMA)``;
* Irwin-Hall integer ``z = sum of the four 16-bit lanes of v - 131070``
  (|z| <= 131070, mean 0, std 65536/sqrt(3) up to 1e-5);
* bf16 weights: ``bf16_rne(float32(z) * c)`` with
  ``c = float32(std * sqrt(3) / 65536)``;
* fp8 weights: ``e4m3fn_rne(float32(z) * c8)`` with
  ``c8 = float32(64 * sqrt(3) / 65536)`` (|value| <= 222 < 448, no saturation);
  block scales ``(std / 64) * {0.5, 1, 2}[(v >> 32) % 3]`` from the scale
  matrix's own stream, one per 128 x 128 block, row-major over blocks.

Matrix ids: 0 = gate/up rows [2I, H], 1 = down [H, I], 2 = gate/up scales,
3 = down scales.  The always-on shared expert uses ``expert = E``.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
MASK64 = (1 << 64) - 1
IH_CENTER = 131070          # 4 * 65535 / 2
MAT_GU, MAT_D, MAT_GU_SCALE, MAT_D_SCALE = 0, 1, 2, 3

_HERE = os.path.dirname(os.path.abspath(__file__))


# ----------------------------------------------------------------------------
# Counter-based generator: executable definition in NumPy
# ----------------------------------------------------------------------------
def mix64(z):
    """SplitMix64 output function on uint64 arrays (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        return z ^ (z >> np.uint64(31))


def splitmix64_sequence(seed: int, n: int) -> np.ndarray:
    """First n outputs of a SplitMix64 generator seeded with ``seed``."""
    idx = np.arange(1, n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(np.uint64(seed & MASK64) + idx * np.uint64(GAMMA))


def stream_id(seed: int, layer: int, expert: int, matrix: int) -> int:
    for v in (seed, layer, expert, matrix):
        if not 0 <= v < 1 << 16:
            raise ValueError("stream id fields must fit in 16 bits")
    return (seed << 48) | (layer << 32) | (expert << 16) | matrix


def stream_state(sid: int) -> int:
    return int(mix64(np.array([sid], dtype=np.uint64))[0])


def counter_u64(sid: int, start: int, n: int) -> np.ndarray:
    """Raw 64-bit draws for elements start .. start+n-1 of stream ``sid``."""
    s = np.uint64(stream_state(sid))
    idx = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(s + idx * np.uint64(GAMMA))


def irwin_hall(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, dtype=np.uint64)
    m = np.uint64(0xFFFF)
    s = (v & m) + ((v >> np.uint64(16)) & m) + ((v >> np.uint64(32)) & m) + (v >> np.uint64(48))
    return s.astype(np.int64) - IH_CENTER


def bf16_scale(std: float) -> np.float32:
    return np.float32(std * math.sqrt(3.0) / 65536.0)


def fp8_scale() -> np.float32:
    return np.float32(64.0 * math.sqrt(3.0) / 65536.0)


def f32_to_bf16_rne(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest even (finite input)."""
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return (u >> np.uint64(16)).astype(np.uint16)


def f32_to_e4m3fn_rne(a: np.ndarray) -> np.ndarray:
    """float32 -> OCP FP8 E4M3FN code (uint8), round to nearest even, saturating
    to +-448.  E4M3FN: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits,
    no infinities, S.1111.111 is NaN."""
    a = np.asarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.int64)
    sign = ((u >> 31) & 1).astype(np.uint8)
    mag = np.abs(a).astype(np.float32)
    mu = mag.view(np.uint32).astype(np.int64)
    e = (mu >> 23) - 127
    mant = mu & 0x7FFFFF
    # normal range: keep 3 mantissa bits
    r = mant >> 20
    rem = mant & 0xFFFFF
    up = (rem > 0x80000) | ((rem == 0x80000) & ((r & 1) == 1))
    r = r + up
    e_n = np.where(r == 8, e + 1, e)
    r = np.where(r == 8, 0, r)
    code_n = ((e_n + 7) << 3) | r
    code_n = np.minimum(code_n, 0x7E)
    # subnormal range (|a| < 2^-6): multiples of 2^-9, ties to even
    q = np.rint(mag.astype(np.float64) * 512.0).astype(np.int64)
    code = np.where(e >= -6, code_n, q)
    return (code.astype(np.uint8) | (sign << 7)).astype(np.uint8)


def counter_bf16(sid: int, start: int, n: int, std: float = 0.02) -> np.ndarray:
    z = irwin_hall(counter_u64(sid, start, n)).astype(np.float32)
    return f32_to_bf16_rne(z * bf16_scale(std))


def counter_fp8(sid: int, start: int, n: int) -> np.ndarray:
    z = irwin_hall(counter_u64(sid, start, n)).astype(np.float32)
    return f32_to_e4m3fn_rne(z * fp8_scale())


def counter_scales(sid: int, start: int, n: int, std: float = 0.02) -> np.ndarray:
    v = counter_u64(sid, start, n)
    sel = ((v >> np.uint64(32)) % np.uint64(3)).astype(np.int64)
    base = np.float32(std / 64.0)
    mult = np.array([0.5, 1.0, 2.0], dtype=np.float32)
    return (base * mult[sel]).astype(np.float32)


# ----------------------------------------------------------------------------
# Native fills (C on the host, HIP on the device)
# ----------------------------------------------------------------------------
_host_lib = None
_dev_lib = None


def _load(name):
    path = os.path.join(_HERE, name)
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run __graft_entry__.build()")
    return ctypes.CDLL(path)


def host_lib():
    global _host_lib
    if _host_lib is None:
        lib = _load("libsynthhost.so")
        u64, i64, f32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
        lib.synth_host_fill_bf16.argtypes = [vp, u64, i64, i64, i64, f32]
        lib.synth_host_fill_fp8.argtypes = [vp, u64, i64, i64, i64, f32]
        lib.synth_host_fill_scales.argtypes = [vp, u64, i64, i64, i64, f32]
        _host_lib = lib
    return _host_lib


def dev_lib():
    global _dev_lib
    if _dev_lib is None:
        lib = _load("libsynthdev.so")
        u64, i64, f32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
        for fn in ("synth_dev_fill_bf16", "synth_dev_fill_fp8", "synth_dev_fill_scales"):
            getattr(lib, fn).argtypes = [vp, u64, i64, i64, i64, f32, vp]
            getattr(lib, fn).restype = ctypes.c_int
        _dev_lib = lib
    return _dev_lib


def sid_base(seed: int, layer: int, expert0: int, matrix: int) -> int:
    """Stream id of expert ``expert0``; expert e0+j uses base + (j << 16)."""
    return stream_id(seed, layer, expert0, matrix)


def host_fill(kind: str, n_exp: int, per_exp: int, seed: int, layer: int,
              expert0: int, matrix: int, std: float = 0.02) -> np.ndarray:
    """Fill [n_exp, per_exp] on the host with the counter generator."""
    lib = host_lib()
    base = sid_base(seed, layer, expert0, matrix)
    if kind == "bf16":
        out = np.empty((n_exp, per_exp), dtype=np.uint16)
        lib.synth_host_fill_bf16(out.ctypes.data, base, n_exp, per_exp, 0, float(bf16_scale(std)))
    elif kind == "fp8":
        out = np.empty((n_exp, per_exp), dtype=np.uint8)
        lib.synth_host_fill_fp8(out.ctypes.data, base, n_exp, per_exp, 0, float(fp8_scale()))
    elif kind == "scale":
        out = np.empty((n_exp, per_exp), dtype=np.float32)
        lib.synth_host_fill_scales(out.ctypes.data, base, n_exp, per_exp, 0, float(np.float32(std / 64.0)))
    else:
        raise ValueError(kind)
    return out


def dev_fill(kind: str, ptr: int, n_exp: int, per_exp: int, seed: int, layer: int,
             expert0: int, matrix: int, stream: int = 0, std: float = 0.02) -> None:
    """Fill a device buffer [n_exp, per_exp] with the counter generator."""
    lib = dev_lib()
    base = sid_base(seed, layer, expert0, matrix)
    if kind == "bf16":
        rc = lib.synth_dev_fill_bf16(ptr, base, n_exp, per_exp, 0, float(bf16_scale(std)), stream)
    elif kind == "fp8":
        rc = lib.synth_dev_fill_fp8(ptr, base, n_exp, per_exp, 0, float(fp8_scale()), stream)
    elif kind == "scale":
        rc = lib.synth_dev_fill_scales(ptr, base, n_exp, per_exp, 0, float(np.float32(std / 64.0)), stream)
    else:
        raise ValueError(kind)
    if rc != 0:
        raise RuntimeError(f"synth device fill failed ({rc})")


# ----------------------------------------------------------------------------
# Structured router logits, activations and planted router weights
# ----------------------------------------------------------------------------
def rng_for(seed: int, *path: int) -> np.random.Generator:
    """Independent PCG64 stream for a (config, layer, sequence, ...) path."""
    ss = np.random.SeedSequence(seed)
    for p in path:
        ss = ss.spawn(p + 1)[p]
    return np.random.Generator(np.random.PCG64(ss))


def structured_logits(rng: np.random.Generator, n_seq: int, t_per_seq: int, E: int,
                      rate: float, a_pop: float = 1.5, a_seq: float = 1.0,
                      a_tok: float = 0.7) -> np.ndarray:
    """Router logits with skewed expert popularity and correlated tokens.

    logit[t, e] = a_pop * exp(-rate * rank(e)) + a_seq * s_seq[e] + a_tok * n[t, e]
    where rank is a random permutation (popularity rank of each expert), s_seq
    is one N(0,1) vector per sequence and n is N(0,1) noise per token.  Rows are
    ordered sequence-major (tokens of sequence 0 first)."""
    rank = rng.permutation(E).astype(np.float64)
    pop = a_pop * np.exp(-rate * rank)
    out = np.empty((n_seq * t_per_seq, E), dtype=np.float64)
    for s in range(n_seq):
        shared = rng.standard_normal(E)
        noise = rng.standard_normal((t_per_seq, E))
        out[s * t_per_seq:(s + 1) * t_per_seq] = pop + a_seq * shared + a_tok * noise
    return out


def planted_router(x: np.ndarray, target_logits: np.ndarray) -> np.ndarray:
    """Router matrix Wr [E, H] (float32) with x @ Wr.T == target_logits in
    exact arithmetic: Wr = L^T (x x^T)^-1 x, computed in float64."""
    x64 = np.asarray(x, dtype=np.float64)
    L = np.asarray(target_logits, dtype=np.float64)
    G = x64 @ x64.T
    return (L.T @ np.linalg.solve(G, x64)).astype(np.float32)


# ----------------------------------------------------------------------------
# Draft trees for cost-aware selection
# ----------------------------------------------------------------------------
@dataclass
class DraftTrees:
    parent: np.ndarray      # [N] int32, BFS order, -1 = child of the root
    P: np.ndarray           # [nt, N] float32 path probabilities
    F: np.ndarray           # [nt, N, W] uint32 path footprints (bit = layer*E + expert)
    n_layers: int
    E: int
    k: int
    own: Optional[np.ndarray] = None        # [nt, N, W] each node's own per-layer experts
    root_own: Optional[np.ndarray] = None   # [nt, W] the root token's per-layer experts


def tree_parents(depth: int, branch: int) -> np.ndarray:
    """Parent array of a full tree without its root, in BFS order."""
    parents = []
    level_start, level_size = 0, 0
    for d in range(depth):
        if d == 0:
            new = [-1] * branch
        else:
            new = [level_start + i // branch for i in range(level_size * branch)]
        level_start = len(parents)
        parents.extend(new)
        level_size = len(new)
    return np.array(parents, dtype=np.int32)


def draft_trees(seed: int, nt: int, depth: int = 3, branch: int = 2, n_layers: int = 36,
                E: int = 128, k: int = 4, rate: float = 0.05, p_lo: float = 0.3,
                stream: int = 0, chunk: int = 256, with_own: bool = False,
                branch_scatter: float = 0.0, branch_rho: float = 0.5) -> DraftTrees:
    """Batch of nt draft trees.

    Each node draws its own per-layer set of k distinct experts, sampled
    without replacement with weights exp(popularity + per-tree context +
    per-node noise) (Gumbel-top-k sampling), so nodes of one tree are
    correlated through the shared per-tree context.  A node's footprint is
    the union of its own sets and those of its ancestors, the root excluded.
    Edge probabilities are U(p_lo, 1); P is their running product in
    float32 (so P(child) <= P(parent)).  with_own also returns each node's
    own sets and a root token's sets (same model and tree context, drawn from
    a separate stream, so the trees themselves do not change).

    branch_scatter > 0 adds branch_scatter * b_i to every node's weights,
    where b_i is a path context that follows the tree: b_i = z_i for a child
    of the root and b_i = rho b_parent + sqrt(1 - rho^2) z_i below it, with
    z_i ~ N(0, 1) per (node, layer, expert).  Siblings then route apart
    while a child stays close to its parent: draft candidates that are close
    in probability but spread over the experts.  Its draws come from a
    stream of their own, so the trees without it do not change."""
    parent = tree_parents(depth, branch)
    N = len(parent)
    W = (n_layers * E + 31) // 32
    P = np.empty((nt, N), dtype=np.float32)
    F = np.zeros((nt, N, W), dtype=np.uint32)
    OWN = np.zeros((nt, N, W), dtype=np.uint32) if with_own else None
    ROOT = np.zeros((nt, W), dtype=np.uint32) if with_own else None
    rng_root = rng_for(seed, 3, stream, 1) if with_own else None
    rng_branch = rng_for(seed, 3, stream, 2) if branch_scatter > 0 else None
    rng = rng_for(seed, 3, stream)
    rank = rng.permutation(E).astype(np.float64)
    pop = 1.5 * np.exp(-rate * rank)
    for c0 in range(0, nt, chunk):
        c = min(chunk, nt - c0)
        ctx = rng.standard_normal((c, 1, n_layers, E))
        noise = 0.7 * rng.standard_normal((c, N, n_layers, E))
        gumbel = -np.log(-np.log(rng.uniform(1e-300, 1.0, size=(c, N, n_layers, E))))
        keys = pop + ctx + noise + gumbel
        if branch_scatter > 0:
            z = rng_branch.standard_normal((c, N, n_layers, E))
            b = np.zeros_like(z)
            for i in range(N):
                pi = parent[i]
                b[:, i] = z[:, i] if pi < 0 else branch_rho * b[:, pi] + math.sqrt(1.0 - branch_rho ** 2) * z[:, i]
            keys = keys + branch_scatter * b
        sel = np.argpartition(-keys, k - 1, axis=-1)[..., :k]
        own = np.zeros((c, N, n_layers, E), dtype=bool)
        np.put_along_axis(own, sel, True, axis=-1)
        own = own.reshape(c, N, n_layers * E)
        edge = rng.uniform(p_lo, 1.0, size=(c, N)).astype(np.float32)
        bits = np.zeros_like(own)
        for i in range(N):
            pi = parent[i]
            if pi < 0:
                bits[:, i] = own[:, i]
                P[c0:c0 + c, i] = edge[:, i]
            else:
                bits[:, i] = own[:, i] | bits[:, pi]
                P[c0:c0 + c, i] = (P[c0:c0 + c, pi] * edge[:, i]).astype(np.float32)
        F[c0:c0 + c] = pack_bits(bits, W)
        if with_own:
            OWN[c0:c0 + c] = pack_bits(own, W)
            rk = pop + ctx[:, 0] + 0.7 * rng_root.standard_normal((c, n_layers, E)) \
                - np.log(-np.log(rng_root.uniform(1e-300, 1.0, size=(c, n_layers, E))))
            rsel = np.argpartition(-rk, k - 1, axis=-1)[..., :k]
            rbits = np.zeros((c, n_layers, E), dtype=bool)
            np.put_along_axis(rbits, rsel, True, axis=-1)
            ROOT[c0:c0 + c] = pack_bits(rbits.reshape(c, n_layers * E), W)
    return DraftTrees(parent=parent, P=P, F=F, n_layers=n_layers, E=E, k=k, own=OWN, root_own=ROOT)


def logits_for_sets(rng: np.random.Generator, sets: np.ndarray, layer: int, E: int) -> np.ndarray:
    """Router logits [T, E] whose per-token top sets are given: row t has
    values 10 + U(0, 1) on the experts of bit row sets[t] at `layer` (bits
    layer * E .. layer * E + E - 1 of the packed words) and 0.1 * N(0, 1)
    elsewhere, so the top-|set| of each row is exactly its set."""
    T = sets.shape[0]
    bits = np.unpackbits(sets.view(np.uint8), axis=-1, bitorder="little")[:, layer * E:(layer + 1) * E].astype(bool)
    out = 0.1 * rng.standard_normal((T, E))
    out[bits] = 10.0 + rng.uniform(0.0, 1.0, int(bits.sum()))
    return out


def pack_bits(bits: np.ndarray, W: int) -> np.ndarray:
    """[..., nbits] bool -> [..., W] uint32, bit b in word b//32, LSB first."""
    nb = bits.shape[-1]
    pad = W * 32 - nb
    b = np.concatenate([bits, np.zeros(bits.shape[:-1] + (pad,), dtype=bool)], axis=-1)
    b = b.reshape(bits.shape[:-1] + (W, 32)).astype(np.uint64)
    weights = (np.uint64(1) << np.arange(32, dtype=np.uint64))
    return (b * weights).sum(axis=-1).astype(np.uint32)


# ----------------------------------------------------------------------------
# Workloads: the verify-layer configurations, their inputs and weights
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    """One verify-layer configuration (shapes, weight format, routing skew)."""
    name: str
    H: int
    I: int
    E: int
    k: int
    T: int
    wdtype: str              # 'f32' | 'bf16' | 'fp8'
    rate: float = 0.05       # popularity decay rate of the logit generator
    n_seq: int = 1           # sequences sharing the T tokens (T // n_seq each)
    shared: bool = False     # one always-on shared expert
    n_layers: int = 1
    seed: int = 0
    cid: int = 0             # configuration id used in the seed path


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", H=256, I=512, E=8, k=2, T=5, wdtype="f32", cid=0),
    "qwen3_bf16": Workload("qwen3_bf16", H=4096, I=1536, E=128, k=8, T=5, wdtype="bf16", rate=0.05, cid=1),
    "gptoss_bf16": Workload("gptoss_bf16", H=2880, I=2880, E=128, k=4, T=5, wdtype="bf16", rate=0.05, cid=2),
    "deepseek_fp8": Workload("deepseek_fp8", H=7168, I=2048, E=256, k=8, T=5, wdtype="fp8", rate=0.01,
                             shared=True, n_layers=16, cid=3),
    "qwen3_batch4_bf16": Workload("qwen3_batch4_bf16", H=4096, I=1536, E=128, k=8, T=20, wdtype="bf16",
                                  rate=0.05, n_seq=4, n_layers=40, cid=4),
}


def tiny_f32_arrays(wl: Workload):
    """Tiny float32 layer drawn with NumPy (seed wl.seed) in the order x, Wr,
    gate, up, down; weights ~N(0, 0.02), x ~N(0, 1).  W_gu = [gate; up]."""
    rng = np.random.default_rng(wl.seed)
    x = rng.standard_normal((wl.T, wl.H)).astype(np.float32)
    Wr = (0.02 * rng.standard_normal((wl.E, wl.H))).astype(np.float32)
    gate = (0.02 * rng.standard_normal((wl.E, wl.I, wl.H))).astype(np.float32)
    up = (0.02 * rng.standard_normal((wl.E, wl.I, wl.H))).astype(np.float32)
    down = (0.02 * rng.standard_normal((wl.E, wl.H, wl.I))).astype(np.float32)
    return x, Wr, np.concatenate([gate, up], axis=1), down


def layer_inputs(wl: Workload, layer: int, T: Optional[int] = None, n_seq: Optional[int] = None):
    """x [T, H] float32, target logits [T, E] float64 and planted router
    Wr [E, H] float32 for one layer (structured logits, planted router)."""
    T = wl.T if T is None else T
    n_seq = wl.n_seq if n_seq is None else n_seq
    rng = rng_for(wl.seed, wl.cid, layer, T, n_seq)
    x = rng.standard_normal((T, wl.H)).astype(np.float32)
    L = structured_logits(rng, n_seq, T // n_seq, wl.E, wl.rate)
    return x, L, planted_router(x, L)


def fill_layer_device(wl: Workload, layer: int, device, stream: int = 0) -> dict:
    """Expert weights of one layer written on the device by the counter fill.
    Returns torch tensors W_gu, W_d (+ s_gu, s_d, shared expert)."""
    import torch
    E, H, I = wl.E, wl.H, wl.I
    out = {}
    if wl.wdtype == "bf16":
        nE = E + (1 if wl.shared else 0)
        gu = torch.empty((nE, 2 * I, H), dtype=torch.int16, device=device)
        d = torch.empty((nE, H, I), dtype=torch.int16, device=device)
        dev_fill("bf16", gu.data_ptr(), nE, 2 * I * H, wl.seed, layer, 0, MAT_GU, stream)
        dev_fill("bf16", d.data_ptr(), nE, H * I, wl.seed, layer, 0, MAT_D, stream)
        out.update(W_gu=gu[:E], W_d=d[:E])
        if wl.shared:
            out.update(Wsh_gu=gu[E], Wsh_d=d[E])
    elif wl.wdtype == "fp8":
        nE = E + (1 if wl.shared else 0)
        gu = torch.empty((nE, 2 * I, H), dtype=torch.uint8, device=device)
        d = torch.empty((nE, H, I), dtype=torch.uint8, device=device)
        sgu = torch.empty((nE, 2 * I // 128, H // 128), dtype=torch.float32, device=device)
        sd = torch.empty((nE, H // 128, I // 128), dtype=torch.float32, device=device)
        dev_fill("fp8", gu.data_ptr(), nE, 2 * I * H, wl.seed, layer, 0, MAT_GU, stream)
        dev_fill("fp8", d.data_ptr(), nE, H * I, wl.seed, layer, 0, MAT_D, stream)
        dev_fill("scale", sgu.data_ptr(), nE, sgu[0].numel(), wl.seed, layer, 0, MAT_GU_SCALE, stream)
        dev_fill("scale", sd.data_ptr(), nE, sd[0].numel(), wl.seed, layer, 0, MAT_D_SCALE, stream)
        out.update(W_gu=gu[:E], W_d=d[:E], s_gu=sgu[:E], s_d=sd[:E])
        if wl.shared:
            out.update(Wsh_gu=gu[E], Wsh_d=d[E], ssh_gu=sgu[E], ssh_d=sd[E])
    else:
        raise ValueError("device fill covers bf16 and fp8 layers")
    return out


def host_expert_raw(wl: Workload, layer: int, expert: int) -> dict:
    """Raw weight codes of one expert regenerated on the host (expert == E is
    the shared expert): 'gu' [2I, H], 'd' [H, I] (bf16 bits or fp8 codes) and
    for fp8 the block scales 's_gu', 's_d'."""
    H, I = wl.H, wl.I
    kind = "bf16" if wl.wdtype == "bf16" else "fp8"
    out = {"gu": host_fill(kind, 1, 2 * I * H, wl.seed, layer, expert, MAT_GU)[0].reshape(2 * I, H),
           "d": host_fill(kind, 1, H * I, wl.seed, layer, expert, MAT_D)[0].reshape(H, I)}
    if wl.wdtype == "fp8":
        out["s_gu"] = host_fill("scale", 1, (2 * I // 128) * (H // 128), wl.seed, layer, expert,
                                MAT_GU_SCALE)[0].reshape(2 * I // 128, H // 128)
        out["s_d"] = host_fill("scale", 1, (H // 128) * (I // 128), wl.seed, layer, expert,
                               MAT_D_SCALE)[0].reshape(H // 128, I // 128)
    return out
