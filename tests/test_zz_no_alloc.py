"""GPU: mep_route_layout_plan_noalloc (the library's own per-GPU workspace, no allocation) against
mep_route_layout_plan with a caller workspace.  Calls in a row, the second with a smaller input
than the first, then other shapes: ids, counts, offsets, permutations, plan and dedup structures
bit for bit, weights within 1e-6 relative (2e-3 for bf16 logits) -- the same kernels run, so they
are in fact identical."""
import numpy as np
import pytest
import torch

from expert_dispatch_layout_amd import _binding as B
from expert_dispatch_layout_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    B.lib()


def _outputs(N, E, K, A, R, S, C):
    ids = torch.full((N, K), -9, dtype=torch.int32, device=DEV)
    w = torch.full((N, K), -9.0, dtype=torch.float32, device=DEV)
    L = B.alloc_layout(N, E, K, A, DEV)
    L.permuted_to_expanded.fill_(-7)
    P = B.alloc_plan(N, E, K, R, S, C, DEV)
    return ids, w, L, P


def _case(wl, N):
    inp = synth.make_inputs(wl, N=N)
    x = torch.from_numpy(inp.logits.view(np.int16) if wl.dtype == synth.BF16 else inp.logits).to(DEV)
    if wl.dtype == synth.BF16:
        x = x.view(torch.bfloat16)
    b = torch.from_numpy(inp.bias).to(DEV) if inp.bias is not None else None
    params = B.route_params(wl.score_fn, wl.renormalize, wl.n_group, wl.topk_group, wl.group_topn,
                            wl.scale)
    return x, b, params


def _compare(wl, N, S):
    E, K, A, R, C = wl.E, wl.K, wl.alignment, wl.R, wl.num_channels
    print("noalloc %s N=%d S=%d" % (wl.name, N, S), flush=True)
    x, b, params = _case(wl, N)
    nvs = B.default_nvs(N, E, K, R, A)
    ref = _outputs(N, E, K, A, R, S, C)
    ws = B.alloc_workspace(B.plan_workspace_size(N, E, K, R, S), DEV)
    B.mep_route_layout_plan(x, K, b, params, ref[0], ref[1], A, ref[2], R, S, C, nvs, ref[3], ws)
    got = _outputs(N, E, K, A, R, S, C)
    B.mep_route_layout_plan_noalloc(x, K, b, params, got[0], got[1], A, got[2], R, S, C, nvs, got[3])
    torch.cuda.synchronize()
    assert torch.equal(ref[0], got[0]), "ids"
    tol = 2e-3 if wl.dtype == synth.BF16 else 1e-6
    rel = ((got[1].double() - ref[1].double()).abs() / ref[1].double().abs().clamp_min(1e-30)).max()
    assert float(rel) <= tol, "weights"
    T = int(ref[2].cu_seqlens[E].item())
    for name in ("tokens_per_expert", "cu_seqlens", "expanded_to_permuted", "zero_fill"):
        assert torch.equal(getattr(ref[2], name), getattr(got[2], name)), name
    assert torch.equal(ref[2].permuted_to_expanded[:T], got[2].permuted_to_expanded[:T])
    assert bool((got[2].permuted_to_expanded[T:] == -7).all()), "rows past cu_seqlens[E] written"
    for name in ("is_token_in_rank", "num_tokens_per_rank", "num_tokens_per_expert",
                 "rank_prefix_matrix", "channel_prefix_matrix", "recv_tokens", "recv_cu_seqlens",
                 "recv_zero_fill", "dst", "dup_counts", "dup_offsets"):
        assert torch.equal(getattr(ref[3], name), getattr(got[3], name)), name
    G, D = [int(v) for v in ref[3].dup_offsets[R].tolist()]
    assert torch.equal(ref[3].dup_groups[:G], got[3].dup_groups[:G])
    assert torch.equal(ref[3].dup_loffs[:D], got[3].dup_loffs[:D])


def test_noalloc_matches_workspace_call_in_a_row():
    dsv3 = synth.WORKLOADS["dsv3"]
    # two calls in a row, the second smaller, then a larger one again and other routing kernels
    _compare(dsv3, 65536, 8)
    _compare(dsv3, 12000, 8)
    _compare(dsv3, 40000, 1)
    _compare(synth.WORKLOADS["skewed"], 16384, 8)      # softmax routing, counting kernel
    _compare(synth.WORKLOADS["tiny"], 128, 2)          # one-workgroup kernel, no workspace use
    _compare(dsv3, 4096, 8)
