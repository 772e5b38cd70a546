"""GPU parity of the fused path (mep_route_layout_plan above the one-workgroup size, and
mep_layout_plan) against the CPU oracle.

Where the sigmoid routing kernel covers the shape, it counts the plan tiles it routes and its
epilogue forms every prefix; otherwise the counting kernel does it after routing.  Either way the
plan-tile kernel writes the rest.  Integers must match bit for bit, weights within 1e-6 relative
(2e-3 for bf16 logits).  The workspace's error word (header word 3) must stay 0."""
import numpy as np
import pytest
import torch

import oracle
from expert_dispatch_layout_amd import _binding as B
from expert_dispatch_layout_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ERR_WORD = 3  # u32 index of the sticky error bits in the workspace header


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    B.lib()


def _np(t):
    return t.cpu().numpy()


def _dev_logits(x, dtype):
    xd = torch.from_numpy(x.view(np.int16) if dtype == synth.BF16 else x).to(DEV)
    return xd.view(torch.bfloat16) if dtype == synth.BF16 else xd


def ws_error(ws):
    return int(ws[:32].cpu().numpy().view(np.uint32)[ERR_WORD])


def run_fused(x, dtype, K, A, R, S, C, *, bias=None, score_fn=0, renormalize=1, n_group=1,
              topk_group=1, group_topn=2, scale=1.0, ws=None, timers=None):
    N, E = x.shape
    xd = _dev_logits(x, dtype)
    bd = torch.from_numpy(bias).to(DEV) if bias is not None else None
    params = B.route_params(score_fn, renormalize, n_group, topk_group, group_topn, scale)
    ids = torch.full((N, K), -9, dtype=torch.int32, device=DEV)
    w = torch.full((N, K), -9.0, dtype=torch.float32, device=DEV)
    L = B.alloc_layout(N, E, K, A, DEV)
    L.permuted_to_expanded.fill_(-7)
    P = B.alloc_plan(N, E, K, R, S, C, DEV)
    ws = ws if ws is not None else B.alloc_workspace(B.plan_workspace_size(N, E, K, R, S), DEV)
    nvs = B.default_nvs(N, E, K, R, A)
    if timers is None:
        B.mep_route_layout_plan(xd, K, bd, params, ids, w, A, L, R, S, C, nvs, P, ws)
    else:
        B.bound_route_layout_plan(xd, K, bd, params, ids, w, A, L, R, S, C, nvs, P, ws,
                                  route_timer=timers[0], plan_timer=timers[1])()
    torch.cuda.synchronize()
    return ids, w, L, P, ws, nvs


def check_fused(x, dtype, K, A, R, S, C, *, bias=None, score_fn=0, renormalize=1, n_group=1,
                topk_group=1, group_topn=2, scale=1.0, ws=None, label=""):
    N, E = x.shape
    print("fused %s N=%d E=%d K=%d A=%d R=%d S=%d C=%d dtype=%d fn=%d groups=%d" % (
        label, N, E, K, A, R, S, C, dtype, score_fn, n_group), flush=True)
    ids, w, L, P, ws, nvs = run_fused(x, dtype, K, A, R, S, C, bias=bias, score_fn=score_fn,
                                      renormalize=renormalize, n_group=n_group,
                                      topk_group=topk_group, group_topn=group_topn, scale=scale,
                                      ws=ws)
    ids_o, w_o = oracle.route(x, K, dtype=dtype, bias=bias, score_fn=score_fn,
                              renormalize=renormalize, n_group=n_group, topk_group=topk_group,
                              group_topn=group_topn, scale=scale)
    bad = np.nonzero((_np(ids) != ids_o).any(axis=1))[0]
    assert bad.size == 0, "ids differ on %d tokens, first %s" % (bad.size, bad[:3])
    tol = 2e-3 if dtype == synth.BF16 else 1e-6
    err = np.abs(_np(w).astype(np.float64) - w_o) / np.maximum(np.abs(w_o), 1e-30)
    assert float(err.max(initial=0.0)) <= tol
    Lo = oracle.layout(ids_o, E, A)
    T = int(Lo.cu_seqlens[E])
    for name in ("tokens_per_expert", "cu_seqlens", "expanded_to_permuted", "zero_fill"):
        assert np.array_equal(_np(getattr(L, name)), getattr(Lo, name)), name
    p2e = _np(L.permuted_to_expanded)
    assert np.array_equal(p2e[:T], Lo.permuted_to_expanded)
    assert (p2e[T:] == -7).all(), "rows past cu_seqlens[E] written"
    Po = oracle.plan(ids_o, Lo.cu_seqlens, Lo.expanded_to_permuted, E, R, S, C, nvs)
    for name in ("is_token_in_rank", "num_tokens_per_rank", "num_tokens_per_expert",
                 "rank_prefix_matrix", "channel_prefix_matrix", "recv_tokens", "recv_cu_seqlens",
                 "recv_zero_fill", "dst", "dup_counts", "dup_offsets"):
        g = _np(getattr(P, name))
        assert g.shape == getattr(Po, name).shape, name
        assert np.array_equal(g, getattr(Po, name)), name
    G, D = int(Po.dup_offsets[R, 0]), int(Po.dup_offsets[R, 1])
    assert np.array_equal(_np(P.dup_groups)[:G], Po.dup_groups)
    assert np.array_equal(_np(P.dup_loffs)[:D], Po.dup_loffs)
    assert ws_error(ws) == 0
    return ids_o


def _wl_kwargs(wl, inp):
    return dict(bias=inp.bias, score_fn=wl.score_fn, renormalize=wl.renormalize,
                n_group=wl.n_group, topk_group=wl.topk_group, group_topn=wl.group_topn,
                scale=wl.scale)


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_fused_workloads(name):
    wl = synth.WORKLOADS[name]
    inp = synth.make_inputs(wl)
    check_fused(inp.logits, wl.dtype, wl.K, wl.alignment, wl.R, wl.S, wl.num_channels,
                label=name, **_wl_kwargs(wl, inp))
    check_fused(inp.logits, wl.dtype, wl.K, wl.alignment, wl.R, 1, wl.num_channels,
                label=name + " S=1", **_wl_kwargs(wl, inp))


@pytest.mark.parametrize("name", ["dsv3", "dsv3big"])
def test_fused_timed_matches_untimed(name):
    wl = synth.WORKLOADS[name]
    inp = synth.make_inputs(wl)
    kw = _wl_kwargs(wl, inp)
    a = run_fused(inp.logits, wl.dtype, wl.K, wl.alignment, wl.R, wl.S, wl.num_channels, **kw)
    timers = (B.KernelTimer(), B.KernelTimer())
    b = run_fused(inp.logits, wl.dtype, wl.K, wl.alignment, wl.R, wl.S, wl.num_channels,
                  timers=timers, **kw)
    for ta, tb in zip(a[:2], b[:2]):
        assert torch.equal(ta, tb)
    for name_ in ("expanded_to_permuted", "cu_seqlens", "permuted_to_expanded"):
        assert torch.equal(getattr(a[2], name_), getattr(b[2], name_))
    for name_ in ("dst", "channel_prefix_matrix", "dup_offsets"):
        assert torch.equal(getattr(a[3], name_), getattr(b[3], name_))
    G, D = [int(v) for v in a[3].dup_offsets[wl.R].tolist()]
    assert torch.equal(a[3].dup_groups[:G], b[3].dup_groups[:G])
    assert torch.equal(a[3].dup_loffs[:D], b[3].dup_loffs[:D])
    assert timers[0].elapsed_ms() > 0 and timers[1].elapsed_ms() > 0


FUSED_CASES = [
    # N, E, K, dtype, routing, A, R, S, C
    (777, 256, 8, synth.F32, "sigmoid_group", 128, 8, 7, 24),
    (3000, 256, 8, synth.BF16, "sigmoid_group", 64, 32, 1, 5),
    (2600, 64, 8, synth.F32, "sigmoid_group", 16, 2, 2, 3),
    (5000, 128, 4, synth.BF16, "sigmoid_group", 1, 4, 5, 1000),
    (4100, 512, 8, synth.F32, "sigmoid_group", 128, 16, 4, 24),
    (4100, 512, 8, synth.BF16, "sigmoid", 32, 32, 2, 7),
    (2049, 256, 2, synth.F32, "sigmoid", 8, 8, 1, 24),
    (9001, 256, 1, synth.BF16, "sigmoid", 3, 1, 1, 24),
    (4097, 128, 8, synth.BF16, "softmax", 128, 8, 1, 24),
    (3333, 100, 7, synth.F32, "softmax", 5, 10, 3, 9),
    (6000, 8, 2, synth.BF16, "softmax_full", 128, 8, 8, 24),
    (40000, 256, 8, synth.F32, "sigmoid_group", 128, 8, 8, 24),
    (65536, 256, 8, synth.F32, "sigmoid_group", 128, 8, 1024, 4),  # 1024 tiles, 4 per counting workgroup
    # shapes of the generic routing kernel: with counting (2 to 8 lanes per token, tiles of 64
    # tokens with a ragged last one, experts per rank not a power of two) and, for 16 or more
    # lanes per token, followed by the counting kernel (sigmoid outside the sigmoid kernel's lane
    # layout, 64 lanes per token with two chunks each)
    (3000, 24, 5, synth.F32, "softmax", 16, 8, 3, 24),
    (1800, 16, 3, synth.BF16, "sigmoid", 4, 4, 2, 5),
    (700, 12, 8, synth.F32, "softmax_full", 2, 3, 1, 7),
    (2500, 96, 4, synth.F32, "sigmoid", 8, 6, 2, 11),
    (1500, 500, 8, synth.F32, "softmax", 4, 20, 2, 6),
    (3099, 300, 6, synth.BF16, "softmax_full", 16, 12, 3, 24),
]


@pytest.mark.parametrize("N,E,K,dtype,routing,A,R,S,C", FUSED_CASES)
def test_fused_sweep(N, E, K, dtype, routing, A, R, S, C):
    rng = np.random.default_rng(N + E * 7 + K * 131 + dtype)
    x = rng.standard_normal((N, E)).astype(np.float32)
    x[::11] = x[3]                     # repeated rows: equal keys across tokens
    x[::13, 1::3] = x[::13, 0:1]       # equal logits inside rows: ties to the lower index
    if dtype == synth.BF16:
        x = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))
    kw = {}
    if routing.startswith("sigmoid"):
        kw = dict(bias=rng.uniform(-0.1, 0.1, E).astype(np.float32), score_fn=1, scale=2.5)
        if routing == "sigmoid_group":
            G = E // 32
            kw.update(n_group=G, topk_group=max(1, G // 2), group_topn=2)
    elif routing == "softmax_full":
        kw = dict(renormalize=0)
    xin = synth.f32_to_bf16_bits(x) if dtype == synth.BF16 else x
    check_fused(xin, dtype, K, A, R, S, C, label=routing, **kw)


def test_fused_workspace_reuse_and_sharing():
    """One workspace across fused calls of shrinking and growing size, shared with mep_plan and
    mep_layout_plan calls on the same stream; every call checked against the oracle."""
    E, K, A, R, C = 256, 8, 128, 8, 24
    big = 20000
    ws = B.alloc_workspace(B.plan_workspace_size(big, E, K, R, 8), DEV)
    rng = np.random.default_rng(5)
    bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    kw = dict(bias=bias, score_fn=1, n_group=8, topk_group=4, group_topn=2, scale=2.5)
    for N in (20000, 4000, 19992, 2560, 20000):
        S = 8 if N % 8 == 0 else 1
        x = rng.standard_normal((N, E)).astype(np.float32)
        ids_o = check_fused(x, synth.F32, K, A, R, S, C, ws=ws, label="reuse", **kw)
        # the same workspace through mep_plan (count-tile kernels) and mep_layout_plan
        idt = torch.from_numpy(ids_o).to(DEV)
        L = B.build_layout(idt, E, A)
        P = B.plan(idt, L.cu_seqlens, L.expanded_to_permuted, E, A, R, S, C, ws=ws)
        L2 = B.alloc_layout(N, E, K, A, DEV)
        P2 = B.alloc_plan(N, E, K, R, S, C, DEV)
        B.mep_layout_plan(idt, E, A, L2, R, S, C, B.default_nvs(N, E, K, R, A), P2, ws)
        torch.cuda.synchronize()
        assert torch.equal(L.expanded_to_permuted, L2.expanded_to_permuted)
        for name in ("dst", "channel_prefix_matrix", "dup_offsets", "num_tokens_per_expert"):
            assert torch.equal(getattr(P, name), getattr(P2, name)), name
        assert ws_error(ws) == 0


def test_layout_plan_unaligned_buffers():
    """mep_layout_plan with ids 4- but not 16-byte aligned (the plan-tile kernel then loads them
    word by word) and is_token_in_rank 4- but not 16-byte aligned with R = 16 (its rows then go
    out as words instead of 16-byte stores): every output as the oracle's."""
    N, E, K, A, R, S, C = 3000, 64, 4, 16, 16, 4, 6
    print("layout+plan unaligned N=%d E=%d K=%d R=%d" % (N, E, K, R), flush=True)
    rng = np.random.default_rng(11)
    ids_o = np.argsort(rng.random((N, E)), axis=1)[:, :K].astype(np.int32)
    ids = torch.zeros(N * K + 1, dtype=torch.int32, device=DEV)[1:].view(N, K)
    ids.copy_(torch.from_numpy(ids_o))
    assert ids.data_ptr() % 16 == 4
    L = B.alloc_layout(N, E, K, A, DEV)
    P = B.alloc_plan(N, E, K, R, S, C, DEV)
    P.is_token_in_rank = torch.full((N * R + 4,), 7, dtype=torch.uint8, device=DEV)[4:].view(N, R)
    assert P.is_token_in_rank.data_ptr() % 16 == 4
    ws = B.alloc_workspace(B.plan_workspace_size(N, E, K, R, S), DEV)
    nvs = B.default_nvs(N, E, K, R, A)
    B.mep_layout_plan(ids, E, A, L, R, S, C, nvs, P, ws)
    torch.cuda.synchronize()
    Lo = oracle.layout(ids_o, E, A)
    T = int(Lo.cu_seqlens[E])
    for name in ("tokens_per_expert", "cu_seqlens", "expanded_to_permuted", "zero_fill"):
        assert np.array_equal(_np(getattr(L, name)), getattr(Lo, name)), name
    assert np.array_equal(_np(L.permuted_to_expanded)[:T], Lo.permuted_to_expanded)
    Po = oracle.plan(ids_o, Lo.cu_seqlens, Lo.expanded_to_permuted, E, R, S, C, nvs)
    for name in ("is_token_in_rank", "num_tokens_per_rank", "num_tokens_per_expert",
                 "rank_prefix_matrix", "channel_prefix_matrix", "recv_tokens", "recv_cu_seqlens",
                 "recv_zero_fill", "dst", "dup_counts", "dup_offsets"):
        assert np.array_equal(_np(getattr(P, name)), getattr(Po, name)), name
    G, D = int(Po.dup_offsets[R, 0]), int(Po.dup_offsets[R, 1])
    assert np.array_equal(_np(P.dup_groups)[:G], Po.dup_groups)
    assert np.array_equal(_np(P.dup_loffs)[:D], Po.dup_loffs)
    assert ws_error(ws) == 0


def test_fused_run_twice_identical():
    wl = synth.WORKLOADS["dsv3"]
    inp = synth.make_inputs(wl, N=16384)
    kw = _wl_kwargs(wl, inp)
    ws = B.alloc_workspace(B.plan_workspace_size(16384, wl.E, wl.K, wl.R, wl.S), DEV)
    a = run_fused(inp.logits, wl.dtype, wl.K, wl.alignment, wl.R, wl.S, wl.num_channels, ws=ws, **kw)
    b = run_fused(inp.logits, wl.dtype, wl.K, wl.alignment, wl.R, wl.S, wl.num_channels, ws=ws, **kw)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    for name in ("expanded_to_permuted", "permuted_to_expanded", "cu_seqlens", "zero_fill"):
        assert torch.equal(getattr(a[2], name), getattr(b[2], name)), name
    for name in ("dst", "dup_offsets", "channel_prefix_matrix", "is_token_in_rank"):
        assert torch.equal(getattr(a[3], name), getattr(b[3], name)), name
    G, D = [int(v) for v in a[3].dup_offsets[wl.R].tolist()]
    assert torch.equal(a[3].dup_groups[:G], b[3].dup_groups[:G])
    assert torch.equal(a[3].dup_loffs[:D], b[3].dup_loffs[:D])


def test_fused_graph_replay_matches_eager():
    """Three fused steps (different batches, one workspace) captured into a HIP graph and replayed
    three times, with eager calls and synchronisations between the replays: every replay writes
    the same bytes as the eager calls (the path records no memset node; the workspace's call
    counter advances on the device)."""
    wl = synth.WORKLOADS["dsv3"]
    inp = synth.make_inputs(wl)
    N, E, K, A, R, S, C = wl.N, wl.E, wl.K, wl.alignment, wl.R, wl.S, wl.num_channels
    params = B.route_params(wl.score_fn, wl.renormalize, wl.n_group, wl.topk_group, wl.group_topn, wl.scale)
    bias = torch.from_numpy(inp.bias).to(DEV)
    nvs = B.default_nvs(N, E, K, R, A)
    ws = B.alloc_workspace(B.plan_workspace_size(N, E, K, R, S), DEV)
    xs = [_dev_logits(np.roll(inp.logits, 97 * i, axis=0), wl.dtype) for i in range(3)]

    def outputs():
        ids = torch.full((N, K), -9, dtype=torch.int32, device=DEV)
        w = torch.full((N, K), -9.0, dtype=torch.float32, device=DEV)
        return ids, w, B.alloc_layout(N, E, K, A, DEV), B.alloc_plan(N, E, K, R, S, C, DEV)

    def snapshot(o):
        ids, w, L, P = o
        G, D = [int(v) for v in P.dup_offsets[R].tolist()]
        T = int(L.cu_seqlens[E].item())   # rows past T of permuted_to_expanded are not written
        return [ids.clone(), w.clone(), L.expanded_to_permuted.clone(), L.permuted_to_expanded[:T].clone(),
                L.cu_seqlens.clone(), L.zero_fill.clone(), P.dst.clone(), P.channel_prefix_matrix.clone(),
                P.is_token_in_rank.clone(), P.dup_offsets.clone(), P.dup_groups[:G].clone(),
                P.dup_loffs[:D].clone()]

    eager = []
    for x in xs:
        o = outputs()
        B.mep_route_layout_plan(x, K, bias, params, o[0], o[1], A, o[2], R, S, C, nvs, o[3], ws)
        torch.cuda.synchronize()
        eager.append(snapshot(o))

    gs = torch.cuda.Stream()
    gouts = [outputs() for _ in xs]
    calls = [B.bound_route_layout_plan(x, K, bias, params, o[0], o[1], A, o[2], R, S, C, nvs, o[3], ws, gs)
             for x, o in zip(xs, gouts)]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=gs):
        for c in calls:
            c()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in gouts:
            o[0].fill_(-9)
            o[2].expanded_to_permuted.fill_(-9)
            o[3].dst.fill_(-9)
        torch.cuda.synchronize()
        with torch.cuda.stream(gs):
            g.replay()
        gs.synchronize()
        for i, o in enumerate(gouts):
            got = snapshot(o)
            for k, (a, b) in enumerate(zip(eager[i], got)):
                assert torch.equal(a, b), "replay %d, batch %d, output %d" % (rep, i, k)
        # eager work on the same workspace between replays
        o = outputs()
        B.mep_route_layout_plan(xs[rep], K, bias, params, o[0], o[1], A, o[2], R, S, C, nvs, o[3], ws)
        torch.cuda.synchronize()
        assert torch.equal(o[0], eager[rep][0])
    assert ws_error(ws) == 0
