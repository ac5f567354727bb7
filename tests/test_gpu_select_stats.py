"""GPU parity of select_drafts and union_stats (bit for bit against the
oracle) and of the device weight fill against the host generator."""
import numpy as np
import pytest

import synth
from oracle import expand as oexp
from oracle import moe as omoe
from oracle import ragged as orag
from oracle import select as osel

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import moe_speculative_decoding_router_amd as m  # noqa: E402
from gpu_helpers import log, to_dev  # noqa: E402


def run_select(trees, gamma, eps=1e-6, static=False):
    S = m.select_drafts(trees.parent, to_dev(trees.P), to_dev(trees.F.view(np.int32)), gamma, eps, static=static)
    torch.cuda.synchronize()
    return S.cpu().numpy()


def check_select_tiled(trees, gamma, ref, static=False):
    """The batch as given (one workgroup per tree below 512 trees) and tiled
    8 times (one wave per tree from 512 trees on, for N <= 16 and W <= 512):
    every tree's selection equals the oracle's."""
    for reps in (1, 8):
        P = np.ascontiguousarray(np.tile(trees.P, (reps, 1)))
        F = np.ascontiguousarray(np.tile(trees.F, (reps, 1, 1)))
        S = m.select_drafts(trees.parent, to_dev(P), to_dev(F.view(np.int32)), gamma, 1e-6, static=static)
        torch.cuda.synchronize()
        assert np.array_equal(S.cpu().numpy(), np.tile(ref, (reps, 1))), f"batch of {P.shape[0]} trees"


@pytest.mark.parametrize("gamma", [0, 1, 4, 14])
def test_select_gptoss_trees(gamma):
    log(f"case select_drafts gptoss trees nt=128 (and 1024) gamma={gamma}")
    trees = synth.draft_trees(seed=0, nt=128, n_layers=36, E=128, k=4)
    check_select_tiled(trees, gamma, osel.select_drafts_batch(trees.P, trees.F, gamma))


@pytest.mark.parametrize("gamma", [1, 4, 6])
def test_select_static_cost(gamma):
    log(f"case select_drafts_static gptoss trees nt=128 (and 1024) gamma={gamma}")
    trees = synth.draft_trees(seed=0, nt=128, n_layers=36, E=128, k=4)
    check_select_tiled(trees, gamma, osel.select_drafts_batch(trees.P, trees.F, gamma, static=True), static=True)


def test_select_ties_and_odd_widths():
    log("case select_drafts ties / odd W, nt=64 (and 512)")
    trees = synth.draft_trees(seed=1, nt=64, n_layers=5, E=37, k=3)   # W = 6 words
    trees.P[:] = np.float32(0.5)
    check_select_tiled(trees, 5, osel.select_drafts_batch(trees.P, trees.F, 5))
    trees.F[:] = trees.F[:, :1]                                          # all footprints equal
    trees.P[:] = np.random.default_rng(3).uniform(0.1, 1, trees.P.shape).astype(np.float32)
    check_select_tiled(trees, 7, osel.select_drafts_batch(trees.P, trees.F, 7))


def test_select_register_resident_ragged_batch():
    """One wave per tree, four trees per workgroup: 515 trees leave the last
    workgroup with three idle waves; N = 1 and N = 2 trees included."""
    log("case select_drafts register-resident nt=515, N in {1, 2, 5}")
    rng = np.random.default_rng(77)
    for N, W, gamma in ((1, 3, 1), (2, 40, 2), (5, 100, 3)):
        F = np.packbits(rng.random((515, N, W * 32)) < 0.2, axis=2, bitorder="little").view(np.uint32)
        F = np.ascontiguousarray(F.reshape(515, N, W))
        P = np.ascontiguousarray(rng.uniform(0.05, 1.0, (515, N)).astype(np.float32))
        parent = np.array([-1] + [(i - 1) // 2 for i in range(1, N)], dtype=np.int32)
        for static in (False, True):
            S = m.select_drafts(parent, to_dev(P), to_dev(F.view(np.int32)), gamma, 1e-6, static=static)
            torch.cuda.synchronize()
            assert np.array_equal(S.cpu().numpy(), osel.select_drafts_batch(P, F, gamma, static=static))


@pytest.mark.parametrize("N,W", [(16, 1), (16, 64), (9, 65), (16, 130), (12, 200), (16, 256), (15, 300), (16, 512),
                                 (3, 7)])
def test_select_register_resident_shapes(N, W):
    """Every register width of the one-wave-per-tree kernel (64, 128, 192,
    256, 384 and 512 words, partial last blocks, N up to 16) on 64 random
    trees tiled to 512, marginal and static cost, gamma 4 and N; ties in P."""
    log(f"case select_drafts register-resident N={N} W={W}")
    rng = np.random.default_rng(1000 + 7 * N + W)
    nt = 64
    F = (rng.random((nt, N, W * 32)) < 0.3)
    F = np.packbits(F, axis=2, bitorder="little").view(np.uint32).reshape(nt, N, W)
    P = rng.choice(np.array([0.25, 0.5, 0.75, 1.0], dtype=np.float32), size=(nt, N))
    parent = np.array([-1] + [(i - 1) // 2 for i in range(1, N)], dtype=np.int32)
    trees = type("Trees", (), {})()
    trees.parent, trees.P, trees.F = parent, np.ascontiguousarray(P), np.ascontiguousarray(F)
    for gamma in sorted({min(4, N), N}):
        for static in (False, True):
            check_select_tiled(trees, gamma, osel.select_drafts_batch(trees.P, trees.F, gamma, static=static),
                               static=static)


def test_select_large_batch_sampled():
    log("case select_drafts nt=4096 (sampled check)")
    trees = synth.draft_trees(seed=2, nt=4096, n_layers=36, E=128, k=4)
    S = run_select(trees, 4)
    idx = np.random.default_rng(0).choice(4096, 256, replace=False)
    ref = osel.select_drafts_batch(trees.P[idx], trees.F[idx], 4)
    assert np.array_equal(S[idx], ref)
    # every selection is prefix-closed on the tree
    for row in S:
        seen = set()
        for t in row:
            p = trees.parent[t]
            assert p < 0 or p in seen
            seen.add(int(t))


@pytest.mark.parametrize("t_ar,t_exp,with_cd", [(300.0, 1.0, True), (600.0, 1.0, False), (40.0, 0.05, True),
                                                (1.0, 0.0, False), (0.0, 1.0, True)])
def test_expand_gptoss_trees(t_ar, t_exp, with_cd):
    log(f"case expand_drafts gptoss trees nt=256 t_ar={t_ar} t_exp={t_exp} c_draft={with_cd}")
    trees = synth.draft_trees(seed=4, nt=256, n_layers=36, E=128, k=4)
    cd = (np.random.default_rng(9).uniform(0, 20, trees.P.shape).astype(np.float32) if with_cd
          else np.zeros(trees.P.shape, np.float32))
    ref = oexp.expand_batch(trees.parent, trees.P, trees.F, t_ar, t_exp, cd)
    # as given (one workgroup per tree) and tiled to 512 trees (one wave per tree)
    for reps in (1, 2):
        P = np.ascontiguousarray(np.tile(trees.P, (reps, 1)))
        F = np.ascontiguousarray(np.tile(trees.F, (reps, 1, 1)))
        C = np.ascontiguousarray(np.tile(cd, (reps, 1)))
        S, cnt = m.expand_drafts(trees.parent, to_dev(P), to_dev(F.view(np.int32)), t_ar, t_exp,
                                 to_dev(C) if with_cd else None)
        torch.cuda.synchronize()
        assert np.array_equal(S.cpu().numpy(), np.tile(ref, (reps, 1))), f"batch of {P.shape[0]} trees"
        assert np.array_equal(cnt.cpu().numpy(), np.tile((ref >= 0).sum(axis=1), reps))
    log(f"    nodes per tree: mean {float((ref >= 0).sum(axis=1).mean()):.2f}")


@pytest.mark.parametrize("N,W", [(16, 1), (16, 64), (9, 65), (12, 200), (16, 256), (15, 300), (16, 512), (1, 5)])
def test_expand_register_resident_shapes(N, W):
    """Every register width of the one-wave-per-tree expansion on random
    BFS trees (515 trees: the last workgroup is partly idle), draft costs,
    and costs that let some but not all nodes join, over several passes."""
    log(f"case expand_drafts register-resident N={N} W={W}")
    rng = np.random.default_rng(3000 + 11 * N + W)
    nt = 515
    F = np.packbits(rng.random((nt, N, W * 32)) < 0.05, axis=2, bitorder="little").view(np.uint32)
    F = np.ascontiguousarray(F.reshape(nt, N, W))
    P = np.ascontiguousarray(rng.uniform(0.05, 1.0, (nt, N)).astype(np.float32))
    cd = np.ascontiguousarray(rng.uniform(0, 2, (nt, N)).astype(np.float32))
    parent = np.array([-1] + [int(rng.integers(0, i)) for i in range(1, N)], dtype=np.int32)
    t_exp = 1.0
    t_ar = float(np.median(np.unpackbits(F.view(np.uint8), axis=2).sum(axis=2)) * 1.5 + 2)
    S, cnt = m.expand_drafts(parent, to_dev(P), to_dev(F.view(np.int32)), t_ar, t_exp, to_dev(cd))
    torch.cuda.synchronize()
    ref = oexp.expand_batch(parent, P, F, t_ar, t_exp, cd)
    assert np.array_equal(S.cpu().numpy(), ref)
    assert np.array_equal(cnt.cpu().numpy(), (ref >= 0).sum(axis=1))
    joined = (ref >= 0).sum(axis=1)
    log(f"    nodes per tree: mean {float(joined.mean()):.2f}, max {int(joined.max())}")


def test_expand_odd_shapes():
    log("case expand_drafts odd W, deep trees")
    trees = synth.draft_trees(seed=6, nt=32, depth=5, branch=2, n_layers=5, E=37, k=3)  # N = 62, W = 6
    cd = np.random.default_rng(1).uniform(0, 0.5, trees.P.shape).astype(np.float32)
    S, cnt = m.expand_drafts(trees.parent, to_dev(trees.P), to_dev(trees.F.view(np.int32)), 12.0, 0.4, to_dev(cd))
    torch.cuda.synchronize()
    assert np.array_equal(S.cpu().numpy(), oexp.expand_batch(trees.parent, trees.P, trees.F, 12.0, 0.4, cd))


def _random_trees(seed):
    """Seeded random trees within the documented limits: BFS parents
    (parent[i] in [-1, i)), footprints that contain the parent's (a node's
    own bits OR its parent's), probabilities with ties on odd seeds."""
    rng = np.random.default_rng(500 + seed)
    while True:
        N, W = int(rng.integers(1, 160)), int(rng.integers(1, 64))
        if N * W + W + 3 * N + N // 32 + 1 <= 16384:
            break
    nt = int(rng.integers(1, 48))
    parent = np.array([-1] + [int(rng.integers(-1, i)) for i in range(1, N)], np.int32)
    own = (rng.integers(0, 2**32, (nt, N, W), dtype=np.uint64) & rng.integers(0, 2**32, (nt, N, W), dtype=np.uint64)
           & rng.integers(0, 2**32, (nt, N, W), dtype=np.uint64)).astype(np.uint32)
    F = own.copy()
    for i in range(N):
        if parent[i] >= 0:
            F[:, i] |= F[:, parent[i]]
    P = rng.random((nt, N)).astype(np.float32)
    if seed % 2:
        P = (np.round(P * 4) / 4).astype(np.float32)
    return parent, P, F


@pytest.mark.parametrize("seed", range(10))
def test_random_trees(seed):
    """select_drafts (marginal and static cost) and expand_drafts on random
    tree shapes, bit for bit against the oracle."""
    parent, P, F = _random_trees(seed)
    nt, N, W = F.shape
    rng = np.random.default_rng(seed)
    gamma = int(rng.integers(0, N + 1))
    log(f"case random trees seed={seed}: nt={nt} N={N} W={W} gamma={gamma}")
    Pd, Fd = to_dev(P), to_dev(F.view(np.int32))
    for static in (False, True):
        S = m.select_drafts(parent, Pd, Fd, gamma, static=static)
        torch.cuda.synchronize()
        assert np.array_equal(S.cpu().numpy(), osel.select_drafts_batch(P, F, gamma, static=static)), static
    # the expert cost is scaled to the footprint density (about 4 W own bits
    # per node) so that some expansions grow and some stop
    cd = rng.uniform(0, 2, P.shape).astype(np.float32)
    t_ar = float(rng.uniform(1, 40))
    t_exp = float(t_ar * rng.uniform(0, 0.5) / (4 * W))
    S, cnt = m.expand_drafts(parent, Pd, Fd, t_ar, t_exp, to_dev(cd))
    torch.cuda.synchronize()
    ref = oexp.expand_batch(parent, P, F, t_ar, t_exp, cd)
    assert np.array_equal(S.cpu().numpy(), ref)
    assert np.array_equal(cnt.cpu().numpy(), (ref >= 0).sum(axis=1))


@pytest.mark.parametrize("depth,branch,static", [(5, 2, False), (5, 2, True), (3, 4, False)])
def test_select_trees_beyond_the_lds_stage(depth, branch, static):
    """Trees whose full-model footprints exceed the 64 KB LDS stage (62 or 84
    nodes x 376 words, Qwen3-shaped: 94 layers x 128 experts) are read from
    global memory every round: select_drafts, its static-cost ablation and
    expand_drafts bit for bit against the oracle, and the choice is
    prefix-closed."""
    trees = synth.draft_trees(seed=21, nt=24, depth=depth, branch=branch, n_layers=94, E=128, k=8)
    nt, N, W = trees.F.shape
    assert N * W + W + N + N // 32 > 16384
    log(f"case select beyond LDS: N={N} W={W} static={static}")
    Pd, Fd = to_dev(trees.P), to_dev(trees.F.view(np.int32))
    S = m.select_drafts(trees.parent, Pd, Fd, 6, static=static)
    torch.cuda.synchronize()
    S = S.cpu().numpy()
    assert np.array_equal(S, osel.select_drafts_batch(trees.P, trees.F, 6, static=static))
    if not static:
        for row in S:
            chosen = set(row.tolist())
            assert all(trees.parent[t] < 0 or trees.parent[t] in chosen for t in chosen)
        E_cnt, t_ar = 8 * 94, 30.0
        S2, cnt = m.expand_drafts(trees.parent, Pd, Fd, t_ar, t_ar / (2 * E_cnt))
        torch.cuda.synchronize()
        ref = oexp.expand_batch(trees.parent, trees.P, trees.F, t_ar, t_ar / (2 * E_cnt), np.zeros_like(trees.P))
        assert np.array_equal(S2.cpu().numpy(), ref)
        assert np.array_equal(cnt.cpu().numpy(), (ref >= 0).sum(axis=1))


def chains(seed, S, Dmax, n_layers, E, k):
    """S sequences of Dmax chained drafts: cumulative confidences and the
    expert bitsets of each sequence's root and drafts."""
    tr = synth.draft_trees(seed=seed, nt=S, depth=Dmax, branch=1, n_layers=n_layers, E=E, k=k, with_own=True)
    c = np.concatenate([np.ones((S, 1), np.float32), tr.P], axis=1)
    Ep = np.concatenate([tr.root_own[:, None], tr.own], axis=1)
    return c, Ep


@pytest.mark.parametrize("S,Dmax,t_base,t_exp", [(4, 8, 400.0, 1.0), (16, 6, 200.0, 0.5), (64, 4, 1000.0, 1.0),
                                                 (8, 12, 50.0, 0.05), (3, 0, 10.0, 1.0), (5, 5, 100.0, 0.0)])
def test_gate_depths(S, Dmax, t_base, t_exp):
    log(f"case gate_depths S={S} Dmax={Dmax} t_base={t_base} t_exp={t_exp}")
    c, Ep = chains(S + 31 * Dmax, S, Dmax, 36, 128, 4)
    d = m.gate_depths(to_dev(c), to_dev(Ep.view(np.int32)), t_base, t_exp)
    torch.cuda.synchronize()
    ref = orag.gate_depths(c, Ep, t_base, t_exp)
    assert d.cpu().numpy().tolist() == ref
    log(f"    depths {ref}")


def test_union_stats_segments():
    log("case union_stats_segments")
    rng = np.random.default_rng(12)
    E, k, nL = 128, 8, 12
    off = np.array([0, 5, 6, 6, 14, 20], dtype=np.int32)           # ragged, one empty segment
    T = int(off[-1])
    L = np.stack([synth.structured_logits(rng, 1, T, E, 0.05) for _ in range(nL)]).astype(np.float32)
    idx = np.stack([omoe.topk(L[l], k) for l in range(nL)]).astype(np.int32)
    per, tot = m.union_stats_segments(to_dev(idx), E, off)
    torch.cuda.synchronize()
    rp, rt = orag.segment_union_stats(idx, off, E)
    assert np.array_equal(per.cpu().numpy(), rp) and np.array_equal(tot.cpu().numpy(), rt)


@pytest.mark.parametrize("seed", range(8))
def test_random_ragged(seed):
    """union_stats_segments on random segmentations (empty segments, entries
    outside [0, E) that must be ignored) and gate_depths on random chains
    and costs, bit for bit against the oracle."""
    rng = np.random.default_rng(700 + seed)
    S = int(rng.integers(1, 65))
    sizes = rng.integers(0, 3, S)
    sizes[rng.integers(0, S)] += 1                     # at least one token
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    T = int(off[-1])
    E = int(rng.choice([8, 37, 128, 300, 512]))
    k = int(rng.integers(1, min(E, 32) + 1))
    nL = int(rng.integers(1, 20))
    idx = np.stack([np.stack([rng.choice(E, k, replace=False) for _ in range(T)]) for _ in range(nL)]).astype(np.int32)
    bad = rng.random(idx.shape) < 0.02
    idx[bad] = rng.choice([-1, E, E + 7], int(bad.sum()))
    log(f"case random ragged seed={seed}: S={S} T={T} E={E} k={k} nL={nL}")
    per, tot = m.union_stats_segments(to_dev(idx), E, off)
    torch.cuda.synchronize()
    rp, rt = orag.segment_union_stats(idx, off, E)
    assert np.array_equal(per.cpu().numpy(), rp) and np.array_equal(tot.cpu().numpy(), rt)
    # depth gating: S2 sequences, random depth bound, costs around the break-even
    S2, Dmax = int(rng.integers(1, 65)), int(rng.integers(0, 13))
    c, Ep = chains(800 + seed, S2, Dmax, 36, 128, 4) if Dmax > 0 else (np.ones((S2, 1), np.float32), None)
    if Ep is None:
        Ep = chains(800 + seed, S2, 1, 36, 128, 4)[1][:, :1]
    t_base, t_exp = float(rng.uniform(10, 1000)), float(rng.uniform(0, 2))
    d = m.gate_depths(to_dev(c), to_dev(np.ascontiguousarray(Ep).view(np.int32)), t_base, t_exp)
    torch.cuda.synchronize()
    assert d.cpu().numpy().tolist() == orag.gate_depths(c, Ep, t_base, t_exp)


@pytest.mark.parametrize("E,T,k", [(128, 5, 8), (128, 20, 8), (300, 7, 3), (8, 4, 2)])
def test_union_stats(E, T, k):
    log(f"case union_stats E={E} T={T} k={k}")
    rng = np.random.default_rng(E + T)
    nL = 40
    L = np.stack([synth.structured_logits(rng, 1, T, E, 0.05) for _ in range(nL)]).astype(np.float32)
    idx = np.stack([omoe.topk(L[l], k) for l in range(nL)])
    idx[0] = idx[0][:1]                          # identical tokens: union == k
    # entries outside [0, E) name no expert and are ignored (layers 1 and 2)
    idx[1, 0, 0] = -1
    idx[1, T - 1, k - 1] = E
    idx[2, :, :] = E + 7
    idx[2, 0, 0] = 0
    counts, reuse = m.union_stats(to_dev(idx), E)
    torch.cuda.synchronize()
    rc, rr = omoe.union_stats(idx, E)
    assert np.array_equal(counts.cpu().numpy(), rc)
    assert np.array_equal(reuse.cpu().numpy(), rr)
    assert counts[0].item() == k
    assert counts[2].item() == 1


@pytest.mark.parametrize("kind", ["bf16", "fp8", "scale"])
def test_device_fill_matches_host_generator(kind):
    n_exp, per = 3, 100_003 if kind != "scale" else 997
    dt = {"bf16": torch.int16, "fp8": torch.uint8, "scale": torch.float32}[kind]
    buf = torch.empty((n_exp, per), dtype=dt, device="cuda:0")
    synth.dev_fill(kind, buf.data_ptr(), n_exp, per, seed=0, layer=5, expert0=9, matrix=1)
    torch.cuda.synchronize()
    host = synth.host_fill(kind, n_exp, per, seed=0, layer=5, expert0=9, matrix=1)
    assert np.array_equal(buf.cpu().numpy().view(host.dtype), host)


def expected_pack(src, gate_up, esz):
    """The tile layout as the header describes it, written with NumPy."""
    E, R, K = src.shape
    KT = 32 if esz == 2 else 64
    out = np.empty(E * R * K * esz, dtype=np.uint8)
    b = src.view(np.uint8).reshape(E, R, K * esz)
    q = 0
    for e in range(E):
        if gate_up:   # row tile major, then K-tile
            order = [(rt, kt) for rt in range(R // 16) for kt in range(K // KT)]
        else:         # groups of 4 row tiles, then K-tile, then the tile in the group
            order = [(4 * grp + r, kt) for grp in range(R // 64) for kt in range(K // KT) for r in range(4)]
        for rt, kt in order:
            for l in range(64):
                m_, g = l % 16, l // 16
                if gate_up:
                    row = 8 * rt + m_ if m_ < 8 else R // 2 + 8 * rt + (m_ - 8)
                else:
                    row = 16 * rt + m_
                k = kt * KT + g * (KT // 4)
                out[q * 16:(q + 1) * 16] = b[e, row, k * esz:k * esz + 16]
                q += 1
    return out


@pytest.mark.parametrize("wdtype,gate_up", [("bf16", True), ("bf16", False), ("fp8", True), ("fp8", False)])
def test_pack_layout(wdtype, gate_up):
    rng = np.random.default_rng(7)
    E, R, K = 2, 128, 256
    if wdtype == "bf16":
        src = rng.integers(0, 1 << 16, size=(E, R, K), dtype=np.uint16)
        t = to_dev(src.view(np.int16))
    else:
        src = rng.integers(0, 256, size=(E, R, K), dtype=np.uint8)
        t = to_dev(src)
    out = m.pack_weights(t, wdtype, gate_up)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint8).ravel()
    assert np.array_equal(got, expected_pack(src, gate_up, 2 if wdtype == "bf16" else 1))


@pytest.mark.parametrize("nbytes", [16, 1008, 1040, 5 * 2**20 + 48, 256 * 2**20])
def test_stream_read_checksum(nbytes):
    """The read probe touches every byte once: its XOR checksum equals the
    host's, for sizes below one chunk, ragged tails and several passes."""
    log(f"case stream_read {nbytes} bytes")
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    src = to_dev(host.view(np.int32))
    chk = torch.zeros(1, dtype=torch.int32, device=src.device)
    m.stream_read(src, chk)
    torch.cuda.synchronize()
    want = int(np.bitwise_xor.reduce(host)) if host.size else 0
    assert (int(chk.item()) & 0xFFFFFFFF) == want
