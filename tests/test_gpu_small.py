"""GPU parity of mep_route_layout_plan (one kernel for small batches, the three-kernel path
above that) against the CPU oracle: routing ids bit for bit and weights to 1e-6 (2e-3 for bf16
logits), every layout and plan output bit for bit."""
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


def _np(t):
    return t.cpu().numpy()


def run_and_check(x, dtype, K, A, R, S, C, *, bias=None, score_fn=0, renormalize=1, n_group=1,
                  topk_group=1, group_topn=2, scale=1.0):
    N, E = x.shape
    print("small path N=%d E=%d K=%d A=%d R=%d S=%d C=%d dtype=%d fn=%d" % (N, E, K, A, R, S, C,
                                                                         dtype, score_fn), flush=True)
    xd = torch.from_numpy(x.view(np.int16) if dtype == synth.BF16 else x).to(DEV)
    if dtype == synth.BF16:
        xd = xd.view(torch.bfloat16)
    bd = torch.from_numpy(bias).to(DEV) if bias is not None else None
    params = B.route_params(score_fn, renormalize, n_group, topk_group, group_topn, scale)
    ids = torch.full((N, K), -9, dtype=torch.int32, device=DEV)
    w = torch.full((N, K), -9.0, dtype=torch.float32, device=DEV)
    L = B.alloc_layout(N, E, K, A, DEV)
    P = B.alloc_plan(N, E, K, R, S, C, DEV)
    ws = B.alloc_workspace(B.plan_workspace_size(N, E, K, R, S), DEV)
    nvs = B.default_nvs(N, E, K, R, A)
    B.mep_route_layout_plan(xd, K, bd, params, ids, w, A, L, R, S, C, nvs, P, ws)
    torch.cuda.synchronize()

    ids_o, w_o = oracle.route(x, K, dtype=dtype, bias=bias, score_fn=score_fn,
                              renormalize=renormalize, n_group=n_group, topk_group=topk_group,
                              group_topn=group_topn, scale=scale)
    assert np.array_equal(_np(ids), ids_o)
    tol = 2e-3 if dtype == synth.BF16 else 1e-6
    err = np.abs(_np(w).astype(np.float64) - w_o) / np.maximum(np.abs(w_o), 1e-30)
    assert float(err.max(initial=0.0)) <= tol
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


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_small_workloads(name):
    wl = synth.WORKLOADS[name]
    inp = synth.make_inputs(wl)
    run_and_check(inp.logits, wl.dtype, wl.K, wl.alignment, wl.R, wl.S, wl.num_channels,
                  bias=inp.bias, score_fn=wl.score_fn, renormalize=wl.renormalize,
                  n_group=wl.n_group, topk_group=wl.topk_group, group_topn=wl.group_topn,
                  scale=wl.scale)


def _logits(rng, N, E, dtype, sd=1.0):
    x = (rng.standard_normal((N, E)) * sd).astype(np.float32)
    if dtype == synth.BF16:
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return x


CASES = [
    # N, E, K, A, R, S, C, dtype, routing
    (250, 64, 8, 16, 4, 5, 5, synth.F32, "sigmoid_group"),
    (1000, 64, 8, 16, 4, 4, 5, synth.F32, "sigmoid_group"),   # three-kernel path
    (300, 32, 4, 3, 8, 3, 7, synth.BF16, "softmax_full"),
    (256, 16, 8, 1, 2, 1, 24, synth.F32, "softmax"),           # 2048 slots, many duplicates
    (1024, 16, 8, 1, 2, 1, 24, synth.F32, "softmax"),          # three-kernel path, duplicates
    (1, 2, 1, 1, 1, 1, 1, synth.F32, "softmax"),
    (256, 256, 8, 128, 8, 1, 1, synth.F32, "sigmoid"),         # 2048 slots, E = 256
    (1500, 24, 1, 2, 4, 3, 4, synth.F32, "softmax"),           # K = 1, 1500 slots
    (777, 40, 3, 5, 4, 7, 9, synth.BF16, "sigmoid"),           # E not a multiple of 16 bytes of bf16
    (2000, 64, 8, 4, 4, 2, 3, synth.F32, "softmax"),           # above the one-kernel envelope
    (1000, 16, 2, 1, 2, 1, 24, synth.F32, "softmax"),          # duplicates over two 512-token chunks
    (700, 30, 2, 3, 3, 7, 5, synth.BF16, "softmax"),           # two chunks, 10 experts per rank
    (500, 512, 4, 2, 8, 5, 2, synth.BF16, "softmax"),          # E above the one-kernel envelope
]


@pytest.mark.parametrize("N,E,K,A,R,S,C,dtype,routing", CASES)
def test_small_sweep(N, E, K, A, R, S, C, dtype, routing):
    rng = np.random.default_rng(N * 13 + E + K)
    x = _logits(rng, N, E, dtype, sd=2.0 if routing == "softmax" else 1.0)
    kw = {}
    if routing.startswith("sigmoid"):
        kw = dict(score_fn=1, bias=(rng.random(E).astype(np.float32) - 0.5) * 0.2, scale=2.5)
        if routing == "sigmoid_group":
            kw.update(n_group=8, topk_group=4, group_topn=2)
    if routing == "softmax_full":
        kw = dict(renormalize=0)
    run_and_check(x, dtype, K, A, R, S, C, **kw)


def test_small_ties_go_to_lower_index():
    """Tied rows in bf16 (every logit equal): the lowest expert indices win."""
    x = np.full((64, 8), 0x3F80, np.uint16)  # bf16 1.0
    run_and_check(x, synth.BF16, 2, 1, 2, 2, 3)


def test_small_empty_batch():
    E, K, R = 8, 2, 2
    params = B.route_params(0, 1, 1, 1, 2, 1.0)
    x = torch.empty((0, E), dtype=torch.float32, device=DEV)
    ids = torch.empty((0, K), dtype=torch.int32, device=DEV)
    L = B.alloc_layout(0, E, K, 1, DEV)
    P = B.alloc_plan(0, E, K, R, 1, 4, DEV)
    ws = B.alloc_workspace(B.plan_workspace_size(0, E, K, R, 1), DEV)
    B.mep_route_layout_plan(x, K, None, params, ids, None, 1, L, R, 1, 4, 1, P, ws)
    torch.cuda.synchronize()
    assert _np(L.cu_seqlens).tolist() == [0] * (E + 1)
