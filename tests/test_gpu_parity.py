"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded inputs.

Integers (ids, counts, offsets, permutations, plan and dedup structures) must match bit for bit;
routing weights within 1e-6 relative for fp32 logits and 2e-3 for bf16 logits (the accuracy the
weights are specified to; both sides compute them in binary64 from identical binary32 inputs, so
the observed error is a few units in the last place).  Every workload runs at full size."""
import numpy as np
import pytest
import torch

import oracle
from expert_dispatch_layout_amd import _binding as B
from expert_dispatch_layout_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    B.lib()


def _note(msg):
    print(msg, flush=True)


def _to_dev_logits(logits, dtype):
    if dtype == synth.BF16:
        t = torch.from_numpy(logits.view(np.int16)).to(DEV)
        return t.view(torch.bfloat16)
    return torch.from_numpy(logits).to(DEV)


def gpu_route(logits, K, dtype, *, bias=None, score_fn=0, renormalize=True, n_group=1,
              topk_group=1, group_topn=2, scale=1.0):
    x = _to_dev_logits(logits, dtype)
    b = torch.from_numpy(bias).to(DEV) if bias is not None else None
    ids, w = B.route(x, K, bias=b, score_fn=score_fn, renormalize=renormalize, n_group=n_group,
                     topk_group=topk_group, group_topn=group_topn, scale=scale)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


def gpu_layout_plan(ids_np, E, A, R, S, C, NvS=None, combined=False, ws=None):
    """Layout and plan through the two calls, or through mep_layout_plan (`combined`); `ws` is an
    optional (layout, plan) workspace pair to reuse."""
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, np.int32)).to(DEV)
    if not combined:
        L = B.build_layout(ids, E, A, ws=ws[0] if ws else None)
        P = B.plan(ids, L.cu_seqlens, L.expanded_to_permuted, E, A, R, S, C, NvS=NvS,
                   ws=ws[1] if ws else None)
    else:
        N, K = ids.shape
        L = B.alloc_layout(N, E, K, A, DEV)
        P = B.alloc_plan(N, E, K, R, S, C, DEV)
        wp_ = ws[1] if ws else B.alloc_workspace(B.plan_workspace_size(N, E, K, R, S), DEV)
        nvs = NvS if NvS is not None else B.default_nvs(N, E, K, R, A)
        B.mep_layout_plan(ids, E, A, L, R, S, C, nvs, P, wp_)
    torch.cuda.synchronize()
    return L, P


def _np(t):
    return t.cpu().numpy()


def check_route(inp_logits, K, dtype, **kw):
    ids_g, w_g = gpu_route(inp_logits, K, dtype, **kw)
    ids_o, w_o = oracle.route(inp_logits, K, dtype=dtype, **kw)
    bad = np.nonzero((ids_g != ids_o).any(axis=1))[0]
    assert bad.size == 0, "ids differ on %d tokens, first %s: gpu %s oracle %s" % (
        bad.size, bad[:3], ids_g[bad[:3]], ids_o[bad[:3]])
    tol = 2e-3 if dtype == synth.BF16 else 1e-6
    err = np.abs(w_g.astype(np.float64) - w_o) / np.maximum(np.abs(w_o.astype(np.float64)), 1e-30)
    assert float(err.max(initial=0.0)) <= tol, "weight rel err %g" % err.max()
    return ids_o, float(err.max(initial=0.0))


def check_layout_plan(ids, E, A, R, S, C, NvS=None, combined=False, ws=None):
    N, K = ids.shape
    epn = E // R
    if NvS is None:
        NvS = N * min(K, epn) + epn * (A - 1)
    Lg, Pg = gpu_layout_plan(ids, E, A, R, S, C, NvS, combined=combined, ws=ws)
    Lo = oracle.layout(ids, E, A)
    T = int(Lo.cu_seqlens[E])
    assert np.array_equal(_np(Lg.tokens_per_expert), Lo.tokens_per_expert)
    assert np.array_equal(_np(Lg.cu_seqlens), Lo.cu_seqlens)
    assert np.array_equal(_np(Lg.expanded_to_permuted), Lo.expanded_to_permuted)
    assert np.array_equal(_np(Lg.permuted_to_expanded)[:T], Lo.permuted_to_expanded)
    assert np.array_equal(_np(Lg.zero_fill), Lo.zero_fill)
    Po = oracle.plan(ids, Lo.cu_seqlens, Lo.expanded_to_permuted, E, R, S, C, NvS)
    G, D = int(Po.dup_offsets[R, 0]), int(Po.dup_offsets[R, 1])
    for name in ("is_token_in_rank", "num_tokens_per_rank", "num_tokens_per_expert",
                 "rank_prefix_matrix", "channel_prefix_matrix", "recv_tokens", "recv_cu_seqlens",
                 "recv_zero_fill", "dst", "dup_counts", "dup_offsets"):
        g = _np(getattr(Pg, name))
        o = getattr(Po, name)
        assert g.shape == o.shape, name
        assert np.array_equal(g, o), name
    assert np.array_equal(_np(Pg.dup_groups)[:G], Po.dup_groups)
    assert np.array_equal(_np(Pg.dup_loffs)[:D], Po.dup_loffs)
    return Lo, Po


# -------------------------------------------------------------------------------------------
# the five workloads at full size, end to end
# -------------------------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_full_path(name):
    wl = synth.WORKLOADS[name]
    _note("workload %s N=%d E=%d K=%d" % (name, wl.N, wl.E, wl.K))
    inp = synth.make_inputs(wl)
    ids, err = check_route(inp.logits, wl.K, wl.dtype, bias=inp.bias, score_fn=wl.score_fn,
                           renormalize=wl.renormalize, n_group=wl.n_group,
                           topk_group=wl.topk_group, group_topn=wl.group_topn, scale=wl.scale)
    _note("  route ok, max weight rel err %.3g" % err)
    check_layout_plan(ids, wl.E, wl.alignment, wl.R, wl.S, wl.num_channels)
    _note("  layout + plan ok (S=%d)" % wl.S)
    check_layout_plan(ids, wl.E, wl.alignment, wl.R, 1, wl.num_channels)
    _note("  layout + plan ok (S=1)")
    check_layout_plan(ids, wl.E, wl.alignment, wl.R, wl.S, wl.num_channels, combined=True)
    _note("  combined layout + plan ok")


def test_layout_plan_combined_reuse_across_sizes():
    """mep_layout_plan on one workspace, sized for the largest call, over calls of shrinking and
    growing size, each checked against the oracle."""
    E, K, A, R, S, C = 256, 8, 128, 8, 8, 24
    big = 8192
    ws = (B.alloc_workspace(B.layout_workspace_size(big, E, K), DEV),
          B.alloc_workspace(B.plan_workspace_size(big, E, K, R, S), DEV))
    rng = np.random.default_rng(77)
    for N in (8192, 8, 4096, 1, 8192, 808):
        ids = np.argsort(rng.random((N, E)), axis=1)[:, :K].astype(np.int32)
        _note("combined N=%d" % N)
        check_layout_plan(ids, E, A, R, S if N % S == 0 else 1, C, combined=True, ws=ws)


# -------------------------------------------------------------------------------------------
# routing sweep: shapes, dtypes, modes, ragged E, K up to 32, ties
# -------------------------------------------------------------------------------------------

ROUTE_CASES = []
for E, K in [(3, 2), (8, 1), (8, 8), (12, 5), (16, 4), (64, 8), (100, 7), (128, 16), (200, 3),
             (256, 8), (256, 32), (512, 8), (1024, 8), (1024, 32)]:
    for dtype in (synth.F32, synth.BF16):
        ROUTE_CASES.append((E, K, dtype))


@pytest.mark.parametrize("E,K,dtype", ROUTE_CASES)
@pytest.mark.parametrize("mode", ["softmax", "softmax_full", "sigmoid", "sigmoid_group"])
def test_route_sweep(E, K, dtype, mode):
    rng = np.random.default_rng(E * 1000 + K * 10 + dtype)
    N = 333
    x = rng.standard_normal((N, E)).astype(np.float32)
    x[::7, 1::3] = x[::7, 0:1]          # equal logits inside rows -> ties
    x[5] = 0.0
    x[6, : E // 2] = -0.0               # signed zeros tie with +0
    logits = synth.f32_to_bf16_bits(x) if dtype == synth.BF16 else x
    bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    kw = {}
    if mode == "softmax_full":
        kw = dict(renormalize=False)
    elif mode == "sigmoid":
        kw = dict(score_fn=1, bias=np.zeros(E, np.float32) if K % 2 else bias, scale=2.5)
    elif mode == "sigmoid_group":
        G = next((g for g in (8, 4, 2) if E % g == 0 and (E // g) >= 2), 1)
        if G == 1:
            pytest.skip("no group split")
        TG = max(1, G // 2)
        if TG * (E // G) < K:
            TG = G
        kw = dict(score_fn=1, bias=bias, n_group=G, topk_group=TG, group_topn=1 + (K % 2),
                  scale=2.5, renormalize=bool(K % 3))
    check_route(logits, K, dtype, **kw)


# one expert group of 32 per lane (E = 32 * G), or no group limit, sigmoid scoring: the
# register-resident selection with certified margins; near ties, a group holding most of the top
# keys (list refill), equal logits (exact fallback) and a wide bias range (larger margins)
LANE_GROUP_CASES = []
for G in (2, 4, 8, 16):
    for K in (1, 2, 5, 8):
        for dtype in (synth.F32, synth.BF16):
            LANE_GROUP_CASES.append((G, K, dtype))


@pytest.mark.parametrize("G,K,dtype", LANE_GROUP_CASES)
def test_route_sigmoid_lane_groups(G, K, dtype):
    E = 32 * G
    rng = np.random.default_rng(G * 100 + K * 10 + dtype)
    N = 1000
    x = rng.standard_normal((N, E)).astype(np.float32)
    x[::11, :12] = 4.0 + rng.standard_normal((len(x[::11]), 12)).astype(np.float32) * 0.1  # one group wins
    x[3::13, 1::5] = x[3::13, 0:1]                 # equal logits
    x[7::17] = np.float32(0.5) + np.float32(2.0 ** -20) * rng.integers(0, 4, (len(x[7::17]), E))  # near ties
    logits = synth.f32_to_bf16_bits(x) if dtype == synth.BF16 else x
    # a bias beyond 2^20 in magnitude sends every token through the exact path (and makes keys
    # tie: the sigmoid is absorbed by the bias)
    for bias_scale in (0.1, 3.0, 2.0 ** 21):
        bias = rng.uniform(-bias_scale, bias_scale, E).astype(np.float32)
        for tg in sorted({1, max(1, G // 2), G}):
            if tg * 32 < K:
                continue
            _note("G=%d K=%d dtype=%d bias=%g tg=%d" % (G, K, dtype, bias_scale, tg))
            check_route(logits, K, dtype, score_fn=1, bias=bias, n_group=G, topk_group=tg,
                        group_topn=1 + (K % 2), scale=2.5, renormalize=K > 1)
        _note("G=%d K=%d dtype=%d bias=%g no group limit" % (G, K, dtype, bias_scale))
        check_route(logits, K, dtype, score_fn=1, bias=bias, scale=1.0, renormalize=False)


# long streams: workgroups of 96 sets or more take the sigmoid kernel with three waves per SIMD
# (every lane layout, with and without group limits, fp32 and bf16, a ragged last set); the oracle
# runs threaded (oracle.route_threads, pinned to oracle.route by the CPU tests)
LONG_CASES = [
    (100003, 512, 8, synth.F32, 0),    # 16 lanes per token, no group limit
    (400001, 128, 6, synth.BF16, 1),   # 4 lanes per token, groups of 32
    (800003, 64, 4, synth.F32, 1),     # 2 lanes per token
]


@pytest.mark.parametrize("N,E,K,dtype,grouped", LONG_CASES)
def test_route_sigmoid_long_streams(N, E, K, dtype, grouped):
    import os
    rng = np.random.default_rng(N + E)
    x = rng.standard_normal((N, E)).astype(np.float32)
    x[::97, 1::3] = x[::97, 0:1]       # equal logits: the exact path
    logits = synth.f32_to_bf16_bits(x) if dtype == synth.BF16 else x
    del x
    bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    kw = dict(score_fn=1, bias=bias, scale=2.5)
    if grouped:
        G = E // 32
        kw.update(n_group=G, topk_group=max(1, G // 2), group_topn=2)
    ids_g, w_g = gpu_route(logits, K, dtype, **kw)
    ids_o, w_o = oracle.route_threads(logits, K, max(1, min(16, os.cpu_count() or 1)), dtype=dtype, **kw)
    bad = np.nonzero((ids_g != ids_o).any(axis=1))[0]
    assert bad.size == 0, "ids differ on %d tokens, first %s" % (bad.size, bad[:3])
    tol = 2e-3 if dtype == synth.BF16 else 1e-6
    err = np.abs(w_g.astype(np.float64) - w_o) / np.maximum(np.abs(w_o.astype(np.float64)), 1e-30)
    assert float(err.max()) <= tol, err.max()


def test_route_tiny_batches():
    rng = np.random.default_rng(9)
    for N in (1, 2, 3, 63, 65, 257):
        x = rng.standard_normal((N, 256)).astype(np.float32)
        check_route(x, 8, synth.F32, score_fn=1, bias=np.zeros(256, np.float32), n_group=8,
                    topk_group=4, scale=2.5)


@pytest.mark.parametrize("score_fn,E,dtype", [(1, 256, synth.F32), (0, 128, synth.BF16),
                                               (0, 40, synth.F32)])
def test_route_timed_matches_untimed(score_fn, E, dtype):
    """mep_route_topk_timed writes the same bytes as mep_route_topk on the sigmoid, fast and
    generic routing paths, and its events bracket the kernel (positive elapsed time)."""
    rng = np.random.default_rng(11)
    N, K = 3000, 8
    x = _to_dev_logits(rng.standard_normal((N, E)).astype(np.float32), dtype)
    bias = torch.from_numpy(rng.uniform(-0.1, 0.1, E).astype(np.float32)).to(DEV)
    p = B.route_params(score_fn, 1, 8 if score_fn else 1, 4, 2, 2.5)
    outs = []
    timer = B.KernelTimer()
    for t in (None, timer):
        ids = torch.full((N, K), -7, dtype=torch.int32, device=DEV)
        w = torch.full((N, K), -7.0, dtype=torch.float32, device=DEV)
        B.bound_route_topk(x, K, bias, p, ids, w, timer=t)()
        torch.cuda.synchronize()
        outs.append((ids.cpu().numpy(), w.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1].view(np.int32), outs[1][1].view(np.int32))
    assert timer.elapsed_ms() > 0.0


# -------------------------------------------------------------------------------------------
# sigmoid: every bf16 value, hard fp32 cases, a dense fp32 range
# -------------------------------------------------------------------------------------------

def _sigmoid_via_route(xs):
    """sigmoid of each value, read back through routing with K = E = 32, no renormalisation and
    unit scale: the weight of a selected expert is then exactly its sigmoid."""
    n = -(-xs.size // 32) * 32
    pad = np.zeros(n, np.float32)
    pad[: xs.size] = xs
    x = pad.reshape(-1, 32)
    ids, w = gpu_route(x, 32, synth.F32, score_fn=1, bias=np.zeros(32, np.float32),
                       renormalize=False, scale=1.0)
    s = np.empty_like(x)
    np.put_along_axis(s, ids.astype(np.int64), w, axis=1)
    return s.reshape(-1)[: xs.size]


def test_sigmoid_every_bf16_value():
    b = np.arange(1 << 16, dtype=np.uint32)
    finite = ((b >> 7) & 0xFF) != 0xFF
    xs = (b[finite] << 16).view(np.float32)
    got = _sigmoid_via_route(xs)
    want = oracle.sigmoid(xs)
    bad = np.nonzero(got.view(np.uint32) != want.view(np.uint32))[0]
    assert bad.size == 0, (xs[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_sigmoid_fp32_range_and_hard_cases():
    xs = (np.uint32(0x3F800000) + np.arange(1 << 22, dtype=np.uint32)).view(np.float32)
    want, path = oracle.sigmoid(xs, with_path=True)
    assert (path == 2).sum() > 0        # includes inputs that sit near a rounding midpoint
    got = _sigmoid_via_route(xs)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    rng = np.random.default_rng(11)
    xs = np.concatenate([rng.uniform(-110, 30, 1 << 18).astype(np.float32),
                         np.array([0.0, -0.0, 1e-45, -1e-45, 17.5, -87.5, -103.9, -104.0, -150.0,
                                   3e38, -3e38], np.float32)])
    got = _sigmoid_via_route(xs)
    want = oracle.sigmoid(xs)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


# -------------------------------------------------------------------------------------------
# layout and plan sweeps on synthetic id rows
# -------------------------------------------------------------------------------------------

LAYOUT_CASES = [
    # N, E, K, A, R, S, C
    (0, 8, 2, 3, 2, 2, 4),
    (1, 8, 2, 1, 2, 1, 24),
    (1023, 8, 2, 128, 8, 1, 24),       # N*K = 2046: one ragged tile
    (1024, 8, 2, 128, 8, 8, 24),       # N*K = 2048: exactly one tile
    (1025, 8, 2, 128, 1, 5, 24),       # one slot into the second tile
    (777, 16, 4, 3, 4, 3, 7),
    (4096, 64, 8, 64, 8, 8, 24),
    (5000, 128, 8, 1, 16, 8, 1),
    (3000, 256, 8, 128, 32, 3, 1000),  # more channels than tokens per shard
    (2048, 256, 8, 2, 128, 4, 24),     # R = 128 (epn = 2)
    (999, 96, 6, 5, 12, 3, 10),
    (640, 512, 16, 8, 8, 2, 24),       # K > 8 path
    (300, 1024, 32, 16, 128, 3, 4),    # K = 32, E = 1024
    (2000, 8, 8, 4, 8, 4, 24),         # epn = 1, K = E
    (6000, 64, 4, 8, 8, 120, 3),       # 120 count tiles: plan prefixes through the look-back
    (9000, 32, 2, 4, 4, 300, 2),       # 300 count tiles: look-back in ticket order
]


@pytest.mark.parametrize("N,E,K,A,R,S,C", LAYOUT_CASES)
def test_layout_plan_sweep(N, E, K, A, R, S, C):
    _note("layout/plan N=%d E=%d K=%d A=%d R=%d S=%d C=%d" % (N, E, K, A, R, S, C))
    ids = synth.random_ids(N, E, K, seed=N + 31 * E + K, hot=min(4, E))
    check_layout_plan(ids, E, A, R, S, C)
    check_layout_plan(ids, E, A, R, S, C, combined=True)


def test_plan_larger_nvs_stride():
    ids = synth.random_ids(1000, 64, 8, seed=3, hot=4)
    check_layout_plan(ids, 64, 16, 8, 4, 24, NvS=1000 * 8 + 8 * 15 + 12345)


# -------------------------------------------------------------------------------------------
# determinism, workspace reuse, optional outputs
# -------------------------------------------------------------------------------------------

def test_run_twice_is_byte_identical():
    wl = synth.WORKLOADS["dsv3"]
    inp = synth.make_inputs(wl)
    outs = []
    for _ in range(2):
        ids, w = gpu_route(inp.logits, wl.K, wl.dtype, bias=inp.bias, score_fn=wl.score_fn,
                           n_group=wl.n_group, topk_group=wl.topk_group, scale=wl.scale)
        L, P = gpu_layout_plan(ids, wl.E, wl.alignment, wl.R, wl.S, wl.num_channels)
        T = int(L.cu_seqlens[wl.E].item())
        G, D = [int(v) for v in P.dup_offsets[wl.R].tolist()]
        # capacity-sized buffers: only their valid prefixes are defined
        outs.append([ids, w, _np(L.expanded_to_permuted), _np(L.permuted_to_expanded)[:T],
                     _np(P.dst), _np(P.dup_groups)[:G], _np(P.dup_loffs)[:D],
                     _np(P.channel_prefix_matrix), _np(P.is_token_in_rank)])
    for a, b in zip(outs[0], outs[1]):
        assert a.tobytes() == b.tobytes()


def test_workspace_reuse_across_sizes():
    E, K, A, R, S, C = 64, 8, 16, 8, 4, 24
    ws_l = B.alloc_workspace(B.layout_workspace_size(8000, E, K), DEV)
    ws_p = B.alloc_workspace(B.plan_workspace_size(8000, E, K, R, S), DEV)
    for N in (8000, 40, 4000, 0, 8000, 4):
        ids_np = synth.random_ids(N, E, K, seed=N, hot=2)
        ids = torch.from_numpy(ids_np).to(DEV)
        L = B.build_layout(ids, E, A, ws=ws_l)
        P = B.plan(ids, L.cu_seqlens, L.expanded_to_permuted, E, A, R, S, C, ws=ws_p)
        torch.cuda.synchronize()
        Lo = oracle.layout(ids_np, E, A)
        assert np.array_equal(_np(L.expanded_to_permuted), Lo.expanded_to_permuted)
        Po = oracle.plan(ids_np, Lo.cu_seqlens, Lo.expanded_to_permuted, E, R, S, C,
                         B.default_nvs(N, E, K, R, A))
        assert np.array_equal(_np(P.dst), Po.dst)
        assert np.array_equal(_np(P.channel_prefix_matrix), Po.channel_prefix_matrix)


def test_optional_outputs_may_be_null():
    E, K, A, R, S, C, N = 64, 8, 16, 8, 4, 24, 3000
    ids_np = synth.random_ids(N, E, K, seed=5, hot=2)
    ids = torch.from_numpy(ids_np).to(DEV)
    out = B.alloc_layout(N, E, K, A, DEV)
    ws = B.alloc_workspace(B.layout_workspace_size(N, E, K), DEV)
    B.mep_build_layout(ids, E, A, None, out.cu_seqlens, out.expanded_to_permuted, None, None, ws)
    Lo = oracle.layout(ids_np, E, A)
    torch.cuda.synchronize()
    assert np.array_equal(_np(out.expanded_to_permuted), Lo.expanded_to_permuted)
    P = B.alloc_plan(N, E, K, R, S, C, DEV)
    keep = B.PlanTensors(None, None, None, None, None, None, None, None, P.dst, None, None,
                         None, P.dup_loffs)
    wsp = B.alloc_workspace(B.plan_workspace_size(N, E, K, R, S), DEV)
    B.mep_plan(ids, out.cu_seqlens, out.expanded_to_permuted, E, A, R, S, C,
               B.default_nvs(N, E, K, R, A), keep, wsp)
    torch.cuda.synchronize()
    Po = oracle.plan(ids_np, Lo.cu_seqlens, Lo.expanded_to_permuted, E, R, S, C,
                     B.default_nvs(N, E, K, R, A))
    assert np.array_equal(_np(P.dst), Po.dst)
    assert np.array_equal(_np(P.dup_loffs)[: Po.dup_loffs.size], Po.dup_loffs)
    ids_o, w_o = oracle.route(np.zeros((4, 16), np.float32), 2)
    t = torch.zeros((4, 16), device=DEV)
    ids_g = torch.empty((4, 2), dtype=torch.int32, device=DEV)
    B.mep_route_topk(t, 2, None, B.route_params(), ids_g, None)
    torch.cuda.synchronize()
    assert np.array_equal(_np(ids_g), ids_o)


@pytest.mark.parametrize("E,K,dtype", [(128, 8, synth.BF16), (256, 8, synth.F32), (512, 4, synth.BF16)])
def test_route_candidate_overflow_takes_exact_path(E, K, dtype):
    """Rows with long runs of equal logits put every tied key above the threshold, so the
    candidate list overflows and those tokens are redone exactly; ties go to the lower index."""
    rng = np.random.default_rng(E + K)
    N = 300
    x = rng.standard_normal((N, E)).astype(np.float32)
    x[::3] = 0.5                                  # whole rows tied
    x[1::3, : E // 2] = 1.25                      # half rows tied at the top
    if dtype == synth.BF16:
        x = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    check_route(x, K, dtype)


def test_earlier_runtime_error_is_not_reported_as_this_calls():
    """An error that an unrelated HIP call left in the runtime's last-error slot is not returned
    as the status of a later, successful entry-point call: each call reports the return codes of
    its own launches."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipGetDeviceCount.argtypes = [ctypes.c_void_p]
    assert hip.hipGetDeviceCount(None) != 0          # invalid argument: leaves a last error
    rng = np.random.default_rng(3)
    x = rng.standard_normal((512, 64)).astype(np.float32)
    ids, w = gpu_route(x, 4, synth.F32)              # raises MepError if the call reports failure
    ids_o, _ = oracle.route(x, 4)
    assert np.array_equal(ids, ids_o)
    hip.hipGetLastError()
