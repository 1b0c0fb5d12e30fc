"""Pins of the oracle's routing and schedule against brute force, closed forms, library routines
and the pages' printed schedule example. CPU only."""
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
import synth


def brute_topk(row, K):
    """Pure-Python selection: repeatedly take the largest remaining logit (lowest index on ties,
    NaN last)."""
    left = list(range(len(row)))
    out = []
    for _ in range(K):
        best = None
        for e in left:
            v = row[e]
            if best is None:
                best = e
                continue
            b = row[best]
            if math.isnan(b) and not math.isnan(v):
                best = e
            elif not math.isnan(v) and not math.isnan(b) and v > b:
                best = e
        out.append(best)
        left.remove(best)
    return out


def brute_g(row, sel):
    """g_i = s_i / sum_{j in sel} s_j with s = softmax(row) over all experts, pure Python."""
    fin = [v for v in row if not math.isnan(v)]
    m = max(fin)
    z = [0.0 if math.isnan(v) else math.exp(v - m) for v in row]
    tot = sum(z)
    s = [v / tot for v in z]
    den = sum(s[j] for j in sel)
    return [s[i] / den for i in sel]


@pytest.mark.parametrize('seed', [0, 1, 2])
def test_topk_brute_force(seed):
    rng = np.random.default_rng(seed)
    T, E, K = 40, 11, 4
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[::3] = np.round(lg[::3] * 2) / 2            # many ties
    lg[5, :] = 0.0
    lg[5, 3] = -0.0                                  # -0.0 ties +0.0
    lg[7, 2] = np.nan
    lg[8, [1, 4]] = -np.inf
    idx = oracle.route_topk(lg, K)
    g = oracle.routing_weights(lg, idx)
    for t in range(T):
        row = [float(v) for v in lg[t]]
        want = brute_topk(row, K)
        assert list(idx[t]) == want, (t, row)
        np.testing.assert_allclose(g[t], brute_g(row, want), rtol=1e-13)
    assert list(idx[5]) == [0, 1, 2, 3]


def test_g_sums_to_one_and_full_softmax():
    cfg = synth.TINY
    lg = synth.router_logits_host(cfg, synth.host_normal(cfg.seed, synth.TID_X, (cfg.T, cfg.D), 1.0))
    idx = oracle.route_topk(lg, cfg.K)
    g = oracle.routing_weights(lg, idx)
    np.testing.assert_allclose(g.sum(1), 1.0, rtol=0, atol=1e-15)
    # K = E: g is the full softmax (library routine), in top-k order
    idxE = oracle.route_topk(lg, cfg.E)
    gE = oracle.routing_weights(lg, idxE)
    ref = scipy.special.softmax(lg.astype(np.float64), axis=1)
    np.testing.assert_allclose(gE, np.take_along_axis(ref, idxE.astype(np.int64), 1), rtol=1e-14)
    # descending order of the chosen logits
    ch = np.take_along_axis(lg, idx.astype(np.int64), 1)
    assert np.all(np.diff(ch, axis=1) <= 0)


def test_route_golden(golden_dir):
    """Hand-worked cases (closed forms) in tests/golden/route_cases.txt."""
    path = os.path.join(golden_dir, 'route_cases.txt')
    cases = []
    for line in open(path):
        line = line.split('#')[0].strip()
        if not line:
            continue
        lhs, idx_s, g_s = [p.strip() for p in line.split('|')]
        cases.append(([float(v) for v in lhs.split()], [int(v) for v in idx_s.split()],
                      [eval(v, {'__builtins__': {}}, {'e': math.e, 'exp': math.exp}) for v in g_s.split()]))
    assert len(cases) >= 4
    for row, want_idx, want_g in cases:
        lg = np.array([row], dtype=np.float32)
        idx = oracle.route_topk(lg, len(want_idx))
        assert list(idx[0]) == want_idx
        np.testing.assert_allclose(oracle.routing_weights(lg, idx)[0], want_g, rtol=1e-14)


def test_schedule_invariants_and_brute_force():
    rng = np.random.default_rng(7)
    for T, E, K in [(1, 1, 1), (3, 5, 2), (50, 8, 2), (200, 16, 4), (64, 64, 8)]:
        idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
        counts, offsets, perm, inv = oracle.schedule(idx, E)
        assert counts.sum() == T * K and offsets[0] == 0 and offsets[-1] == T * K
        assert sorted(perm.tolist()) == list(range(T * K))
        assert np.all(inv[perm] == np.arange(T * K))
        # brute force: route ids sorted by (expert, route id)
        flat = idx.ravel().tolist()
        want = sorted(range(T * K), key=lambda r: (flat[r], r))
        assert perm.tolist() == want
        for e in range(E):
            seg = perm[offsets[e]:offsets[e + 1]]
            assert np.all(idx.ravel()[seg] == e) and np.all(np.diff(seg) > 0)
            assert counts[e] == sum(1 for v in flat if v == e)


def position_formula(routing, rank, L):
    """The pages' two-pass counting construction of the pull schedule (Blog, "Scheduling"), with
    the garbled count term read as #{r' : r' < r and M[l, r'] > o}. Written independently of
    oracle.pull_schedule, which sorts by the key the Notes state."""
    R, N, K = routing.shape
    Tc = np.zeros(L, np.int64)
    M = np.zeros((L, R), np.int64)
    for r in range(R):
        for i in range(N):
            for k in range(K):
                e = routing[r, i, k]
                if e // L == rank:
                    Tc[e - rank * L] += 1
                    M[e - rank * L, r] += 1
    S = np.concatenate([[0], np.cumsum(Tc)[:-1]])
    C = np.zeros((L, R), np.int64)
    phi = -np.ones((Tc.sum(), 2), np.int64)
    for r in range(R):
        for i in range(N):
            for k in range(K):
                e = routing[r, i, k]
                if e // L != rank:
                    continue
                le = e - rank * L
                o = C[le, r]
                p = sum(min(M[le, q], o) for q in range(R)) + sum(1 for q in range(r) if M[le, q] > o)
                assert phi[S[le] + p, 0] == -1, 'position collision'
                phi[S[le] + p] = (r, i * K + k)
                C[le, r] += 1
    return Tc, M, S, phi


def test_pull_schedule_matches_position_formula():
    rng = np.random.default_rng(11)
    for trial in range(150):
        R = int(rng.integers(1, 6))
        L = int(rng.integers(1, 5))
        N = int(rng.integers(0, 10))
        K = int(rng.integers(1, 4))
        G = R * L
        K = min(K, G)
        routing = np.stack([[rng.permutation(G)[:K] for _ in range(N)] for _ in range(R)]).reshape(R, N, K)
        for c in range(R):
            a = oracle.pull_schedule(routing, c, L)
            b = position_formula(routing, c, L)
            for u, v in zip(a, b):
                assert np.array_equal(u, v), (trial, c)


def test_pull_schedule_r1_is_stable_sort():
    rng = np.random.default_rng(3)
    T, E, K = 30, 6, 3
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    Tc, M, S, phi = oracle.pull_schedule(idx[None], 0, E)
    counts, offsets, perm, _ = oracle.schedule(idx, E)
    assert np.array_equal(Tc, counts) and np.array_equal(S, offsets[:-1])
    assert np.all(phi[:, 0] == 0) and np.array_equal(phi[:, 1], perm)


def test_pull_schedule_printed_example(golden_dir):
    """The Blog's pull-schedule example rows (Scheduling section): consecutive rows cycle the
    source ranks 0, 1, 2, 3. The pages do not give the routing behind the table; the fixture
    holds a routing built so that these are the first routes to the local expert."""
    lines = [l.split('#')[0].strip() for l in open(os.path.join(golden_dir, 'pull_schedule_example.txt'))]
    lines = [l for l in lines if l]
    hdr = dict(kv.split('=') for kv in lines[0].split())
    R, N, K, L, c = (int(hdr[k]) for k in ('R', 'N', 'K', 'L', 'rank'))
    routing = np.array([[int(v) for v in l.split()] for l in lines[1:1 + R * N]]).reshape(R, N, K)
    table = [tuple(int(v) for v in l.split()) for l in lines[1 + R * N:]]
    _, _, _, phi = oracle.pull_schedule(routing, c, L)
    for row_idx, src_rank, src_idx in table:
        assert tuple(phi[row_idx]) == (src_rank, src_idx)
