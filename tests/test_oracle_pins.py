"""Pins for the CPU oracle: each check compares the oracle with something other than itself
(exact arithmetic, brute-force enumeration, closed forms, a textbook stable sort, invariants that
the definitions imply, a hand-worked example).  CPU only."""
import itertools
import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle
from expert_dispatch_layout_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_example.json")


# ---------------------------------------------------------------------------------------------
# Sigmoid: correctly rounded binary32 of 1/(1+exp(-x)), checked with 60-digit decimal arithmetic
# ---------------------------------------------------------------------------------------------

def _exact_sigmoid_f32(x: np.float32) -> np.float32:
    getcontext().prec = 60
    xd = Decimal(float(x))
    # Beyond |x| = 200 the value is within e^-200 of 1 (or of 0), far inside the rounding interval
    # of 1.0 (of 0.0: e^-200 < 2^-150), and the decimal exponential would overflow.
    if xd > 200:
        return np.float32(1.0)
    if xd < -200:
        return np.float32(0.0)
    d = Decimal(1) / (Decimal(1) + (-xd).exp())
    f = np.float32(float(d))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]

    def cost(c):
        return (abs(Decimal(float(c)) - d), int(np.array(c, np.float32).view(np.uint32)) & 1)

    return min(cands, key=cost)


def _bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def test_sigmoid_every_bf16_value():
    b = np.arange(1 << 16, dtype=np.uint32)
    finite = ((b >> 7) & 0xFF) != 0xFF
    x = (b[finite] << 16).view(np.float32)
    got = oracle.sigmoid(x)
    want = np.array([_exact_sigmoid_f32(v) for v in x], np.float32)
    bad = np.nonzero(_bits(got) != _bits(want))[0]
    assert bad.size == 0, (x[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_sigmoid_random_fp32_and_specials():
    rng = np.random.default_rng(7)
    x = rng.uniform(-110, 30, 4000).astype(np.float32)
    x = np.concatenate([x, np.array([0.0, -0.0, 1e-45, -1e-45, 17.5, 16.6, -87.0, -103.9, -104.0,
                                     -150.0, 3.0e38, -3.0e38, np.inf, -np.inf], np.float32)])
    got = oracle.sigmoid(x)
    want = np.array([_exact_sigmoid_f32(v) for v in x], np.float32)
    assert np.array_equal(_bits(got), _bits(want))
    assert got[4000] == np.float32(0.5) and got[4001] == np.float32(0.5)


def test_sigmoid_quad_fallback_cases_are_exact():
    # Inputs whose double-precision evaluation sits too close to a float midpoint take the
    # binary128 path; find some in [1, 4) and check them against decimal arithmetic.
    x = (np.uint32(0x3F800000) + np.arange(1 << 22, dtype=np.uint32)).view(np.float32)
    s, path = oracle.sigmoid(x, with_path=True)
    hard = x[path == 2]
    assert hard.size > 0
    want = np.array([_exact_sigmoid_f32(v) for v in hard], np.float32)
    assert np.array_equal(_bits(s[path == 2]), _bits(want))


# ---------------------------------------------------------------------------------------------
# Top-K selection: brute force over subsets
# ---------------------------------------------------------------------------------------------

def _beats(ka, ia, kb, ib):
    return ka > kb or (ka == kb and ia < ib)


def _brute_topk(keys, K, eligible):
    """The unique K-subset of eligible experts all of whose members beat every non-member."""
    cand = [e for e in range(len(keys)) if eligible[e]]
    winners = []
    for sub in itertools.combinations(cand, K):
        rest = [e for e in cand if e not in sub]
        if all(_beats(keys[a], a, keys[b], b) for a in sub for b in rest):
            winners.append(sub)
    assert len(winners) == 1
    return sorted(winners[0], key=lambda e: (-keys[e], e))


def _brute_groups(keys, n_group, topk_group, group_topn):
    gs = len(keys) // n_group
    scores = []
    for g in range(n_group):
        top = sorted(keys[g * gs:(g + 1) * gs], reverse=True)[:group_topn]
        acc = np.float32(top[0])
        for v in top[1:]:
            acc = np.float32(acc + np.float32(v))
        scores.append(acc)
    kept = _brute_topk(scores, topk_group, [True] * n_group)
    return [(e // gs) in kept for e in range(len(keys))]


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("E,K", [(6, 1), (6, 2), (8, 3), (10, 3)])
def test_softmax_topk_matches_brute_force(seed, E, K):
    rng = np.random.default_rng(100 * seed + E)
    # few distinct values -> many ties; ties must go to the lower expert index
    x = rng.integers(-2, 3, size=(12, E)).astype(np.float32) * np.float32(0.5)
    ids, _ = oracle.route(x, K)
    for t in range(x.shape[0]):
        assert list(ids[t]) == _brute_topk(list(x[t]), K, [True] * E)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("E,G,TG,K,topn", [(8, 4, 2, 2, 2), (12, 4, 2, 3, 2), (16, 4, 2, 4, 2),
                                           (12, 3, 1, 2, 1), (16, 8, 3, 3, 2)])
def test_sigmoid_group_topk_matches_brute_force(seed, E, G, TG, K, topn):
    rng = np.random.default_rng(1000 * seed + E + G)
    x = rng.standard_normal((10, E)).astype(np.float32)
    x[:, 1] = x[:, 0]                         # equal sigmoid values inside a row
    bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    if seed % 2 == 0:
        bias[:] = 0.0                          # zero bias keeps the equal keys equal
    ids, _ = oracle.route(x, K, bias=bias, score_fn=oracle.SIGMOID, n_group=G, topk_group=TG,
                          group_topn=topn, scale=2.5)
    s = oracle.sigmoid(x)
    keys = (s + bias[None, :]).astype(np.float32)   # one binary32 addition, as numpy does it
    for t in range(x.shape[0]):
        elig = _brute_groups(list(keys[t]), G, TG, topn)
        assert list(ids[t]) == _brute_topk(list(keys[t]), K, elig)


def test_sigmoid_without_groups_orders_like_logits():
    # sigmoid is monotone: with zero bias and no group limit the selection is the logit top-K
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 32)).astype(np.float32)
    a, _ = oracle.route(x, 6, bias=np.zeros(32, np.float32), score_fn=oracle.SIGMOID)
    b, _ = oracle.route(x, 6)
    assert np.array_equal(a, b)


def test_group_limit_with_all_groups_kept_is_plain_topk():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((64, 32)).astype(np.float32)
    bias = rng.uniform(-0.1, 0.1, 32).astype(np.float32)
    a, wa = oracle.route(x, 5, bias=bias, score_fn=oracle.SIGMOID, n_group=4, topk_group=4)
    b, wb = oracle.route(x, 5, bias=bias, score_fn=oracle.SIGMOID)
    assert np.array_equal(a, b) and np.array_equal(wa, wb)


# ---------------------------------------------------------------------------------------------
# Weights: closed forms
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("nthreads", [1, 3, 16])
def test_threaded_routing_equals_serial(nthreads):
    """The CPU baseline's threaded routing (contiguous token ranges on threads) returns the serial
    oracle's ids and weights bit for bit, for softmax and for group-limited sigmoid routing, with
    more threads than tokens too."""
    rng = np.random.default_rng(nthreads)
    x = rng.standard_normal((37, 64)).astype(np.float32)
    a = oracle.route(x, 4)
    b = oracle.route_threads(x, 4, nthreads)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    bias = rng.uniform(-0.1, 0.1, 64).astype(np.float32)
    kw = dict(bias=bias, score_fn=oracle.SIGMOID, n_group=2, topk_group=1, group_topn=2, scale=2.5)
    a = oracle.route(x, 4, **kw)
    b = oracle.route_threads(x, 4, nthreads, **kw)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    xs = x[:2]
    a = oracle.route(xs, 4, **kw)
    b = oracle.route_threads(xs, 4, 16, **kw)
    assert np.array_equal(a[0], b[0])


def test_weights_k1_equal_scale():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((50, 16)).astype(np.float32)
    _, w = oracle.route(x, 1, scale=1.0)
    assert np.all(w == 1.0)
    _, w = oracle.route(x, 1, bias=np.zeros(16, np.float32), score_fn=oracle.SIGMOID, scale=2.5)
    assert np.all(w == np.float32(2.5))


def test_weights_k2_softmax_is_logistic():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((200, 8)).astype(np.float32)
    ids, w = oracle.route(x, 2)
    for t in range(200):
        d = float(x[t, ids[t, 1]]) - float(x[t, ids[t, 0]])
        w0 = 1.0 / (1.0 + math.exp(d))
        assert abs(float(w[t, 0]) - w0) <= 1e-7 * w0
        assert abs(float(w[t, 1]) - (1.0 - w0)) <= 1e-7 * (1.0 - w0) + 1e-12


def test_weights_full_softmax_and_sums():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((100, 12)).astype(np.float32)
    ids, w = oracle.route(x, 3, renormalize=False)
    p = np.exp(x.astype(np.float64) - x.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    ref = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, ref, rtol=1e-7)
    ids, w = oracle.route(x, 3, renormalize=True, scale=2.5)
    np.testing.assert_allclose(w.astype(np.float64).sum(axis=1), 2.5, rtol=1e-6)


def test_weights_sigmoid_renorm_closed_form():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((100, 16)).astype(np.float32)
    bias = rng.uniform(-0.1, 0.1, 16).astype(np.float32)
    ids, w = oracle.route(x, 4, bias=bias, score_fn=oracle.SIGMOID, n_group=4, topk_group=2,
                          scale=2.5)
    s = oracle.sigmoid(x).astype(np.float64)
    sel = np.take_along_axis(s, ids.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, sel / sel.sum(axis=1, keepdims=True) * 2.5, rtol=1e-7)
    ids2, w2 = oracle.route(x, 4, bias=bias, score_fn=oracle.SIGMOID, renormalize=False, scale=2.5)
    assert np.array_equal(w2, (np.take_along_axis(oracle.sigmoid(x), ids2.astype(np.int64), axis=1)
                               * np.float32(2.5)).astype(np.float32))


# ---------------------------------------------------------------------------------------------
# Layout: equal to a textbook stable sort, with padding invariants
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("N,E,K,A", [(0, 4, 2, 3), (1, 8, 3, 1), (37, 8, 2, 128), (500, 16, 4, 3),
                                     (1000, 64, 8, 64), (333, 128, 8, 1), (200, 256, 8, 128)])
def test_layout_equals_stable_sort(N, E, K, A):
    ids = synth.random_ids(N, E, K, seed=N + E, hot=2)
    L = oracle.layout(ids, E, A)
    flat = ids.reshape(-1)
    cnt = np.bincount(flat, minlength=E)
    assert np.array_equal(L.tokens_per_expert, cnt)
    assert L.cu_seqlens[0] == 0 and np.all(L.cu_seqlens % A == 0)
    pad = np.diff(L.cu_seqlens)
    assert np.all((pad >= cnt) & (pad < cnt + A) & ((cnt > 0) | (pad == 0)))
    order = np.argsort(flat, kind="stable")           # slots grouped by expert, stable
    P = np.empty(N * K, np.int64)
    pos = 0
    for e in range(E):
        members = order[pos:pos + cnt[e]]
        P[members] = L.cu_seqlens[e] + np.arange(cnt[e])
        pos += cnt[e]
    assert np.array_equal(L.expanded_to_permuted, P)
    T = int(L.cu_seqlens[E])
    inv = np.full(T, -1, np.int64)
    inv[P] = np.arange(N * K)
    assert np.array_equal(L.permuted_to_expanded, inv)
    for e in range(E):
        extra = pad[e] - cnt[e]
        want = (L.cu_seqlens[e] + cnt[e], extra) if (cnt[e] > 0 and extra > 0) else (0, 0)
        assert tuple(L.zero_fill[e]) == tuple(want)


# ---------------------------------------------------------------------------------------------
# Plan: invariants implied by the definitions
# ---------------------------------------------------------------------------------------------

def _check_plan(ids, E, R, S, C, A):
    N, K = ids.shape
    epn = E // R
    L = oracle.layout(ids, E, A)
    NvS = N * min(K, epn) + epn * (A - 1)
    Pl = oracle.plan(ids, L.cu_seqlens, L.expanded_to_permuted, E, R, S, C, NvS)
    owner = ids // epn
    itr = np.zeros((N, R), np.uint8)
    for r in range(R):
        itr[:, r] = (owner == r).any(axis=1)
    assert np.array_equal(Pl.is_token_in_rank, itr)
    n = N // S if S else 0
    ntpr = itr.reshape(S, n, R).sum(axis=1) if N else np.zeros((S, R))
    assert np.array_equal(Pl.num_tokens_per_rank, ntpr)
    assert np.array_equal(Pl.rank_prefix_matrix, np.cumsum(ntpr, axis=0))
    assert np.array_equal(Pl.recv_tokens, Pl.rank_prefix_matrix[-1])
    ntpe = np.zeros((S, E), np.int64)
    for t in range(N):
        for k in range(K):
            ntpe[t // n, ids[t, k]] += 1
    assert np.array_equal(Pl.num_tokens_per_expert, ntpe)
    assert np.array_equal(Pl.num_tokens_per_expert.sum(axis=0), L.tokens_per_expert)
    cp = Pl.channel_prefix_matrix
    assert np.all(np.diff(cp, axis=2) >= 0) and np.array_equal(cp[:, :, -1], ntpr)
    q = -(-n // C) if n else 0
    for s in range(S):
        for c in range(C):
            end = min((c + 1) * q, n)
            assert np.array_equal(cp[s, :, c], itr[s * n:s * n + end].sum(axis=0))
    rc = Pl.recv_cu_seqlens
    cu = L.cu_seqlens
    for r in range(R):
        assert np.array_equal(rc[r], cu[r * epn:(r + 1) * epn + 1] - cu[r * epn])
    # dst decodes through the layout's inverse back to its own slot
    inv = L.permuted_to_expanded
    d = Pl.dst.astype(np.int64)
    raw = np.where(d >= 0, d, -d - 1)
    r_of = raw // NvS
    assert np.array_equal(r_of, owner.reshape(-1))
    slot = cu[r_of * epn] + raw % NvS
    assert np.array_equal(inv[slot], np.arange(N * K))
    # exactly the first slot of each (token, rank) is non-negative
    for t in range(N):
        seen = set()
        for k in range(K):
            r = owner[t, k]
            assert (d[t * K + k] >= 0) == (r not in seen)
            seen.add(r)
    # dedup counts: duplicates are the slots beyond one per (token, rank)
    slots_per_rank = np.bincount(owner.reshape(-1), minlength=R)
    assert np.array_equal(Pl.dup_counts[:, 1], slots_per_rank - Pl.recv_tokens)
    assert np.all(Pl.dup_counts[:, 0] <= Pl.recv_tokens)
    hits = np.stack([(owner == r).sum(axis=1) for r in range(R)], axis=1)   # [N,R]
    assert np.array_equal(Pl.dup_counts[:, 0], (hits >= 2).sum(axis=0))
    assert np.array_equal(Pl.dup_offsets[1:], np.cumsum(Pl.dup_counts, axis=0))
    assert np.array_equal(Pl.dup_offsets[0], [0, 0])
    if epn == 1:
        assert Pl.dup_offsets[R].tolist() == [0, 0]
    # every group decodes to (token, rank) in ascending token order and lists its duplicates
    for r in range(R):
        g0, g1 = Pl.dup_offsets[r, 0], Pl.dup_offsets[r + 1, 0]
        seg = Pl.dup_loffs[Pl.dup_offsets[r, 1]:Pl.dup_offsets[r + 1, 1]]
        prev_t = -1
        nxt = 0
        for g in range(g0, g1):
            ploff, begin, cnt = Pl.dup_groups[g]
            i = inv[cu[r * epn] + ploff]
            t = i // K
            assert t > prev_t and owner[t, i % K] == r
            prev_t = t
            ks = [k for k in range(K) if owner[t, k] == r]
            assert ks[0] == i % K and cnt == len(ks) - 1 and begin == nxt
            for j, k in enumerate(ks[1:]):
                assert inv[cu[r * epn] + seg[begin + j]] == t * K + k
            nxt += cnt
        assert nxt == len(seg)
    return Pl


@pytest.mark.parametrize("N,E,K,R,S,C,A", [(0, 8, 2, 2, 2, 4, 1), (128, 8, 2, 2, 2, 24, 1),
                                           (128, 8, 2, 2, 1, 24, 1), (96, 8, 2, 8, 8, 5, 128),
                                           (256, 64, 8, 8, 4, 24, 16), (240, 32, 6, 4, 3, 7, 3),
                                           (64, 16, 4, 16, 2, 3, 2), (200, 256, 8, 32, 8, 24, 128)])
def test_plan_invariants(N, E, K, R, S, C, A):
    ids = synth.random_ids(N, E, K, seed=7 * N + E, hot=3)
    _check_plan(ids, E, R, S, C, A)


def test_plan_shards_are_a_split_of_one_source():
    ids = synth.random_ids(512, 64, 8, seed=11, hot=4)
    L = oracle.layout(ids, 64, 16)
    NvS = 512 * 8 + 8 * 15
    many = oracle.plan(ids, L.cu_seqlens, L.expanded_to_permuted, 64, 8, 8, 24, NvS)
    one = oracle.plan(ids, L.cu_seqlens, L.expanded_to_permuted, 64, 8, 1, 24, NvS)
    assert np.array_equal(many.num_tokens_per_rank.sum(axis=0), one.num_tokens_per_rank[0])
    assert np.array_equal(many.num_tokens_per_expert.sum(axis=0), one.num_tokens_per_expert[0])
    for name in ("dst", "dup_counts", "dup_offsets", "dup_groups", "dup_loffs", "recv_tokens",
                 "is_token_in_rank", "recv_cu_seqlens", "recv_zero_fill"):
        assert np.array_equal(getattr(many, name), getattr(one, name)), name


# ---------------------------------------------------------------------------------------------
# Hand-worked example
# ---------------------------------------------------------------------------------------------

def test_hand_example():
    g = json.load(open(GOLDEN))
    rs = g["routing_softmax"]
    ids, w = oracle.route(np.array(rs["logits"], np.float32), rs["K"])
    assert ids.tolist() == rs["ids"]
    np.testing.assert_allclose(w, np.array(rs["weights"]), rtol=1e-7)

    rg = g["routing_sigmoid_group"]
    x = np.array(rg["logits"], np.float32)
    b = np.array(rg["bias"], np.float32)
    ids, w = oracle.route(x, rg["K"], bias=b, score_fn=oracle.SIGMOID, n_group=rg["n_group"],
                          topk_group=rg["topk_group"], group_topn=rg["group_topn"],
                          scale=rg["scale"])
    assert ids.tolist() == rg["ids"]
    ids2, _ = oracle.route(x, rg["K"], bias=b, score_fn=oracle.SIGMOID)
    assert ids2.tolist() == rg["ids_without_group_limit"]
    s = 1.0 / (1.0 + np.exp(-x.astype(np.float64)[0]))
    sel = s[[7, 4]]
    np.testing.assert_allclose(w[0], sel / sel.sum() * 2.5, rtol=1e-6)

    lp = g["layout_plan"]
    ids = np.array(lp["ids"], np.int32)
    L = oracle.layout(ids, lp["E"], lp["alignment"])
    for k in ("tokens_per_expert", "cu_seqlens", "expanded_to_permuted", "permuted_to_expanded",
              "zero_fill"):
        assert getattr(L, k).tolist() == lp[k], k
    Pl = oracle.plan(ids, L.cu_seqlens, L.expanded_to_permuted, lp["E"], lp["R"], lp["num_src"],
                     lp["num_channels"], lp["NvS"])
    for k in ("is_token_in_rank", "num_tokens_per_rank", "num_tokens_per_expert",
              "rank_prefix_matrix", "recv_tokens", "channel_prefix_matrix", "recv_cu_seqlens",
              "recv_zero_fill", "dst", "dup_counts", "dup_offsets", "dup_groups", "dup_loffs"):
        assert getattr(Pl, k).tolist() == lp[k], k


# ---------------------------------------------------------------------------------------------
# Workload generators feed the oracle end to end (small prefix of each workload)
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_prefix_end_to_end(name):
    wl = synth.WORKLOADS[name]
    n = min(wl.N, 64 * wl.R)
    inp = synth.make_inputs(wl, N=n)
    ids, w = oracle.route(inp.logits, wl.K, bias=inp.bias, score_fn=wl.score_fn,
                          renormalize=wl.renormalize, n_group=wl.n_group,
                          topk_group=wl.topk_group, group_topn=wl.group_topn, scale=wl.scale,
                          dtype=wl.dtype)
    assert np.all((ids >= 0) & (ids < wl.E))
    assert all(len(set(r)) == wl.K for r in ids.tolist())
    np.testing.assert_allclose(w.astype(np.float64).sum(axis=1), wl.scale, rtol=1e-6)
    _check_plan(ids, wl.E, wl.R, wl.S, wl.num_channels, wl.alignment)


# ---------------------------------------------------------------------------------------------
# Grouped-GEMM tile maps: a row-level enumeration and the layout's permuted rows
# ---------------------------------------------------------------------------------------------

def test_tile_map_hand_example():
    for c in json.load(open(GOLDEN))["tile_map"]["cases"]:
        tm = oracle.tile_map(np.array(c["counts"], np.int32), c["alignment"])
        assert tm.cta_to_expert.tolist() == c["cta_to_expert"]
        assert tm.mn_limit.tolist() == c["mn_limit"]
        assert (tm.permuted_idx_size, tm.num_ctas) == (c["permuted_idx_size"], c["num_ctas"])


def _rows_of(counts, A):
    """Permuted rows listed one by one: (owner, is_real) per row, experts back to back, each
    padded with dummy rows to a whole number of A-row tiles."""
    rows = []
    for e, c in enumerate(counts):
        real = [(e, True)] * int(c)
        while len(real) % A:
            real.append((e, False))
        rows += real
    return rows


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("E,A", [(1, 1), (5, 4), (16, 3), (64, 128), (33, 1)])
def test_tile_map_matches_row_enumeration(seed, E, A):
    rng = np.random.default_rng(1000 + seed)
    counts = rng.integers(0, 3 * A + 2, E).astype(np.int32)
    counts[rng.random(E) < 0.3] = 0
    counts[rng.random(E) < 0.2] = A * rng.integers(1, 3)
    tm = oracle.tile_map(counts, A)
    rows = _rows_of(counts, A)
    assert len(rows) % A == 0
    assert tm.num_ctas == len(rows) // A and tm.permuted_idx_size == len(rows)
    for j in range(tm.num_ctas):
        tile = rows[j * A:(j + 1) * A]
        assert len({o for o, _ in tile}) == 1  # a tile never straddles two experts
        assert tm.cta_to_expert[j] == tile[0][0]
        real = sum(r for _, r in tile)
        assert real >= 1 and tm.mn_limit[j] == j * A + real


def test_tile_map_alignment_one_is_repeat():
    counts = np.array([3, 0, 1, 7, 0, 2], np.int32)
    tm = oracle.tile_map(counts, 1)
    assert tm.cta_to_expert.tolist() == np.repeat(np.arange(6), counts).tolist()
    assert tm.mn_limit.tolist() == list(range(1, int(counts.sum()) + 1))


def test_tile_map_empty_and_invalid():
    tm = oracle.tile_map(np.zeros(7, np.int32), 5)
    assert tm.num_ctas == 0 and tm.permuted_idx_size == 0
    with pytest.raises(ValueError):
        oracle.tile_map(np.array([1, -1], np.int32), 2)


@pytest.mark.parametrize("N,E,K,A", [(37, 8, 2, 4), (300, 16, 4, 3), (129, 64, 8, 128)])
def test_tile_map_tiles_cover_layout_rows(N, E, K, A):
    """Tile j spans permuted rows [jA, (j+1)A) of the stable layout: rows below its limit hold
    slots of its expert, the rest are padding."""
    rng = np.random.default_rng(N)
    ids = np.stack([rng.permutation(E)[:K] for _ in range(N)]).astype(np.int32)
    L = oracle.layout(ids, E, A)
    tm = oracle.tile_map(L.tokens_per_expert, A)
    assert tm.permuted_idx_size == int(L.cu_seqlens[E])
    flat = ids.reshape(-1)
    for j in range(tm.num_ctas):
        lim = int(tm.mn_limit[j])
        assert j * A < lim <= (j + 1) * A
        real = L.permuted_to_expanded[j * A:lim]
        assert np.all(real >= 0) and np.all(flat[real] == tm.cta_to_expert[j])
        assert np.all(L.permuted_to_expanded[lim:(j + 1) * A] == -1)


# ---------------------------------------------------------------------------------------------
# Local permute / combine of hidden rows: round trips, exact small-integer sums, the binary32
# summation order and the bf16 rounding (checked against torch's CPU conversion)
# ---------------------------------------------------------------------------------------------

def _bf16_bits(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def _bf16_to_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _rand_layout(rng, N, E, K, A):
    ids = np.stack([rng.permutation(E)[:K] for _ in range(N)]).astype(np.int32)
    return ids, oracle.layout(ids, E, A)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N,E,K,A,H", [(1, 4, 1, 1, 8), (37, 8, 2, 4, 16), (64, 16, 4, 3, 24),
                                       (50, 32, 8, 8, 8)])
def test_permute_then_combine_round_trip(dtype, N, E, K, A, H):
    rng = np.random.default_rng(N * 31 + K)
    # values with at most 4 significant bits, so every partial sum j*x (j <= 8) is exact
    xf = (rng.integers(-15, 16, (N, H)) * np.exp2(rng.integers(-6, 7, (N, H)))).astype(np.float32)
    x = xf if dtype == "f32" else _bf16_bits(xf)
    ids, L = _rand_layout(rng, N, E, K, A)
    T = int(L.cu_seqlens[E])
    xp = oracle.permute_rows(x, L.expanded_to_permuted, L.zero_fill, T)
    # every row of [0, T) written: a slot's token row, or zeros on padding
    pad = np.ones(T, bool)
    pad[L.expanded_to_permuted] = False
    assert np.all(xp[pad].view(np.uint8) == 0)
    tok = L.permuted_to_expanded[~pad] // K
    assert np.array_equal(xp[~pad], x[tok])
    # K copies summed in order: exactly K * x
    y = oracle.combine_rows(xp, L.expanded_to_permuted, K)
    xv = xf if dtype == "f32" else _bf16_to_f32(x)
    got = y if dtype == "f32" else _bf16_to_f32(y)
    assert np.array_equal(got, xv * np.float32(K))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_combine_small_integers_exact(dtype):
    """Integer rows and power-of-two weights: every partial sum is exact, so the result is the
    exact weighted sum."""
    from fractions import Fraction
    rng = np.random.default_rng(3)
    N, E, K, A, H = 40, 16, 8, 4, 12
    ids, L = _rand_layout(rng, N, E, K, A)
    T = int(L.cu_seqlens[E])
    yv = rng.integers(-4, 5, (T, H)).astype(np.float32)
    w = rng.choice(np.array([0.25, 0.5, 1.0, 2.0, -1.0], np.float32), (N, K))
    y = yv if dtype == "f32" else _bf16_bits(yv)
    out = oracle.combine_rows(y, L.expanded_to_permuted, K, w)
    outv = out if dtype == "f32" else _bf16_to_f32(out)
    P = L.expanded_to_permuted.reshape(N, K)
    for t in range(N):
        for h in range(H):
            exact = sum(Fraction(float(w[t, k])) * Fraction(float(yv[P[t, k], h])) for k in range(K))
            assert Fraction(float(outv[t, h])) == exact


def test_combine_sums_in_slot_order():
    """1 + 2^-24 rounds back to 1 in binary32 (tie to even), so adding two 2^-24 terms after the
    1 leaves 1, while adding them first gives 1 + 2^-23: the order k = 0, 1, 2 is visible."""
    tiny = np.float32(2.0 ** -24)
    e2p = np.array([0, 1, 2], np.int32)
    y = np.array([[1.0], [tiny], [tiny]], np.float32)
    assert oracle.combine_rows(y, e2p, 3)[0, 0] == np.float32(1.0)
    y_rev = np.array([[tiny], [tiny], [1.0]], np.float32)
    assert oracle.combine_rows(y_rev, e2p, 3)[0, 0] == np.float32(1.0) + np.float32(2.0 ** -23)


def test_combine_bf16_rounding_matches_torch():
    """K = 1: out = bf16(w * y).  Compared bit for bit with torch's CPU binary32 product and its
    round-to-nearest-even conversion, over random values and hand-made ties, overflow and NaN."""
    import torch
    rng = np.random.default_rng(9)
    n = 4096
    yv = rng.standard_normal(n).astype(np.float32) * np.float32(3)
    w = rng.standard_normal(n).astype(np.float32)
    # ties at 1.0: 1 + 2^-8 rounds to 1 (even); 1 + 3*2^-8 rounds up to 1 + 2^-6
    yv[:4] = [1.0, 1.0, 3.0e38, 1.0]
    w[:4] = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 4.0, np.nan]
    y = _bf16_bits(yv)
    out = oracle.combine_rows(y.reshape(n, 1), np.arange(n, dtype=np.int32), 1, w.reshape(n, 1))
    ref = (torch.from_numpy(w) * torch.from_numpy(_bf16_to_f32(y))).to(torch.bfloat16)
    ref = ref.view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(_bf16_to_f32(ref))
    assert np.array_equal(out.reshape(-1)[~nan], ref[~nan])
    assert np.all(np.isnan(_bf16_to_f32(out.reshape(-1)[nan])))
    assert _bf16_to_f32(out[:2, 0]).tolist() == [1.0, 1.0 + 2.0 ** -6]


# ---------------------------------------------------------------------------------------------
# Capacity rebalancing: hand-worked cases, the no-move case against the plain plan, invariants
# ---------------------------------------------------------------------------------------------

def _balanced_from_counts(counts, R, B, tp, capacity, NvS):
    E = len(counts)
    ids = np.repeat(np.arange(E), counts).astype(np.int32).reshape(-1, 1)
    L = oracle.layout(ids, E, 1)
    return oracle.plan_balanced(ids, L.tokens_per_expert, L.cu_seqlens, L.expanded_to_permuted,
                                E, R, B, tp, capacity, NvS)


def test_balanced_hand_examples():
    for c in json.load(open(GOLDEN))["balanced_plan"]["cases"]:
        P = _balanced_from_counts(c["counts"], c["R"], c["B"], c["tp"], c["capacity"], c["NvS"])
        for k in ("group_tokens", "z", "alloc", "alloc_cumsum", "experts_to_copy", "remote_stats",
                  "cu_seqlens", "expert_offsets", "dst"):
            if k in c:
                assert getattr(P, k).tolist() == c[k], k
        if "zero_fill_nonzero" in c:
            nz = [[r, g] + P.zero_fill[r, g].tolist() for r in range(c["R"])
                  for g in range(P.zero_fill.shape[1]) if P.zero_fill[r, g, 1] != 0]
            assert nz == c["zero_fill_nonzero"]


@pytest.mark.parametrize("N,E,K,R,A", [(64, 8, 2, 2, 1), (200, 16, 4, 4, 3), (300, 32, 8, 8, 8)])
def test_balanced_without_moves_is_the_plain_plan(N, E, K, R, A):
    """A capacity above every rank's load moves nothing: every expert stays at its owner, the
    groups of a rank are its own experts' padded segments, and dst equals the plain plan's."""
    rng = np.random.default_rng(N + E)
    ids = np.stack([rng.permutation(E)[:K] for _ in range(N)]).astype(np.int32)
    L = oracle.layout(ids, E, A)
    epn = E // R
    NvS = N * min(K, epn) + (E + 2) * (A - 1)
    Pb = oracle.plan_balanced(ids, L.tokens_per_expert, L.cu_seqlens, L.expanded_to_permuted, E,
                              R, 2, A, N * K, NvS)
    Pp = oracle.plan(ids, L.cu_seqlens, L.expanded_to_permuted, E, R, 1, 1, NvS)
    assert not Pb.z.any() and np.all(Pb.experts_to_copy == -1) and not Pb.remote_stats.any()
    assert np.array_equal(Pb.dst, Pp.dst)
    for r in range(R):
        own = slice(r * epn, (r + 1) * epn)
        assert np.array_equal(Pb.alloc[r, own], L.tokens_per_expert[own])
        assert Pb.alloc[r].sum() == L.tokens_per_expert[own].sum()
        assert np.array_equal(Pb.cu_seqlens[r, own], Pp.recv_cu_seqlens[r, 1:])
        assert np.array_equal(Pb.zero_fill[r, own], Pp.recv_zero_fill[own])


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("E,K,R,B,tp", [(8, 2, 4, 1, 1), (16, 4, 4, 2, 3), (32, 6, 8, 3, 4),
                                        (64, 8, 8, 4, 1)])
def test_balanced_invariants(seed, E, K, R, B, tp):
    rng = np.random.default_rng(seed * 101 + E)
    N = 160
    # skewed routing: low experts are hot, so some ranks sit far above the capacity
    p = np.exp(-np.arange(E) / (E / 4))
    ids = np.stack([rng.choice(E, K, replace=False, p=p / p.sum()) for _ in range(N)]).astype(np.int32)
    L = oracle.layout(ids, E, 1)
    epn = E // R
    cap = N * K // R
    NvS = max(N * min(K, epn), cap) + (E + B) * tp
    P = oracle.plan_balanced(ids, L.tokens_per_expert, L.cu_seqlens, L.expanded_to_permuted, E,
                             R, B, tp, cap, NvS)
    tpe = L.tokens_per_expert.astype(np.int64)
    assert np.array_equal(P.group_tokens, tpe.reshape(R, epn).sum(axis=1))
    assert np.all(P.alloc >= 0) and np.array_equal(P.alloc.sum(axis=0), tpe)
    assert np.array_equal(P.alloc_cumsum, np.cumsum(P.alloc, axis=0).T)
    load = P.alloc.sum(axis=1)
    recv, sent = P.z.sum(axis=0), P.z.sum(axis=1)
    assert np.array_equal(load, P.group_tokens - sent + recv)       # every quota is handed out
    assert np.all(load[recv > 0] == cap)                            # receivers end at capacity
    assert not np.any((recv > 0) & (P.group_tokens > cap) & (sent == 0))
    for d in range(R):
        remote = [(int(P.alloc[d, e]), e) for e in range(E) if e // epn != d and P.alloc[d, e] > 0]
        assert P.remote_stats[d, 0] == len(remote)
        best = [e for _, e in sorted(remote, key=lambda ce: (-ce[0], -ce[1]))[:B]]
        assert P.experts_to_copy[d].tolist() == best + [-1] * (B - len(best))
    picks = P.experts_to_copy[P.experts_to_copy >= 0]
    assert np.array_equal(P.remote_stats[:, 1], np.bincount(picks // epn, minlength=R))
    # every slot decodes to a distinct row of its expert's group on the rank that computes it
    flat = ids.reshape(-1)
    raw = np.where(P.dst < 0, -P.dst - 1, P.dst)
    rank, loff = raw // NvS, raw % NvS
    q = L.expanded_to_permuted - L.cu_seqlens[flat]
    for i in range(N * K):
        e, r = flat[i], rank[i]
        lo_cum = P.alloc_cumsum[e, r - 1] if r > 0 else 0
        assert lo_cum <= q[i] < P.alloc_cumsum[e, r]
        assert loff[i] == P.expert_offsets[r, e] + (q[i] - lo_cum)
    assert len(set(raw.tolist())) == N * K
    for t in range(N):
        seen = set()
        for k in range(K):
            i = t * K + k
            assert (P.dst[i] < 0) == (rank[i] in seen)
            seen.add(rank[i])
    for r in range(R):
        ends = P.cu_seqlens[r]
        assert np.all(np.diff(ends) >= 0) and ends[-1] <= NvS
