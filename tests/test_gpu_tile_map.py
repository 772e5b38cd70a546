"""GPU parity of mep_tile_map against the CPU oracle: the grouped-GEMM tile maps must match bit
for bit, and entries past the tile count must stay untouched."""
import numpy as np
import pytest
import torch

import oracle
from expert_dispatch_layout_amd import _binding as B
from expert_dispatch_layout_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
UNTOUCHED = -7


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    B.lib()


def gpu_tile_map(counts_dev, num_slots, A, with_arrays=(True, True), with_scalars=(True, True)):
    E = counts_dev.numel()
    cap = B.tile_map_capacity(num_slots, E, A)
    c2e = torch.full((max(cap, 1),), UNTOUCHED, dtype=torch.int32, device=DEV) if with_arrays[0] else None
    lim = torch.full((max(cap, 1),), UNTOUCHED, dtype=torch.int32, device=DEV) if with_arrays[1] else None
    pis = torch.full((1,), UNTOUCHED, dtype=torch.int32, device=DEV) if with_scalars[0] else None
    nct = torch.full((1,), UNTOUCHED, dtype=torch.int32, device=DEV) if with_scalars[1] else None
    B.mep_tile_map(counts_dev, num_slots, A, c2e, lim, pis, nct)
    torch.cuda.synchronize()
    out = [None if t is None else t.cpu().numpy() for t in (c2e, lim, pis, nct)]
    return out


def check_tile_map(counts, num_slots, A, counts_dev=None):
    counts = np.ascontiguousarray(counts, np.int32)
    if counts_dev is None:
        counts_dev = torch.from_numpy(counts).to(DEV)
    c2e, lim, pis, nct = gpu_tile_map(counts_dev, num_slots, A)
    o = oracle.tile_map(counts, A)
    T = o.num_ctas
    assert int(nct[0]) == T and int(pis[0]) == o.permuted_idx_size
    assert np.array_equal(c2e[:T], o.cta_to_expert)
    assert np.array_equal(lim[:T], o.mn_limit)
    if T < c2e.size:
        assert np.all(c2e[T:] == UNTOUCHED) and np.all(lim[T:] == UNTOUCHED)
    return o


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_tile_map_workloads(name):
    """Tile maps of each workload's routed histogram, for the whole layout and for every rank's
    experts (rank-local expert indices)."""
    wl = synth.WORKLOADS[name]
    print("workload %s N=%d E=%d K=%d A=%d" % (name, wl.N, wl.E, wl.K, wl.alignment), flush=True)
    inp = synth.make_inputs(wl)
    x = torch.from_numpy(inp.logits.view(np.int16) if wl.dtype == synth.BF16 else inp.logits).to(DEV)
    if wl.dtype == synth.BF16:
        x = x.view(torch.bfloat16)
    b = torch.from_numpy(inp.bias).to(DEV) if inp.bias is not None else None
    ids, _ = B.route(x, wl.K, bias=b, score_fn=wl.score_fn, renormalize=wl.renormalize,
                     n_group=wl.n_group, topk_group=wl.topk_group, group_topn=wl.group_topn,
                     scale=wl.scale)
    L = B.build_layout(ids, wl.E, wl.alignment)
    torch.cuda.synchronize()
    tpe = L.tokens_per_expert.cpu().numpy()
    cu = L.cu_seqlens.cpu().numpy()
    o = check_tile_map(tpe, wl.N * wl.K, wl.alignment, counts_dev=L.tokens_per_expert)
    assert o.permuted_idx_size == int(cu[wl.E])
    epn = wl.E // wl.R
    for r in range(wl.R):
        sl = slice(r * epn, (r + 1) * epn)
        o = check_tile_map(tpe[sl], wl.N * min(wl.K, epn), wl.alignment,
                           counts_dev=L.tokens_per_expert[sl])
        assert o.permuted_idx_size == int(cu[(r + 1) * epn] - cu[r * epn])


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("E,A", [(1, 1), (5, 3), (64, 128), (256, 64), (1000, 7), (1024, 1),
                                 (1024, 128)])
def test_tile_map_sweep(seed, E, A):
    rng = np.random.default_rng(seed * 7919 + E * 13 + A)
    counts = rng.integers(0, 4 * A + 3, E).astype(np.int32)
    counts[rng.random(E) < 0.25] = 0
    counts[rng.random(E) < 0.1] = A * rng.integers(1, 4)
    slack = int(rng.integers(0, 50))
    check_tile_map(counts, int(counts.sum()) + slack, A)


@pytest.mark.parametrize("E,A", [(256, 1), (256, 128), (1024, 3)])
def test_tile_map_one_hot_expert(E, A):
    """Every slot on one expert: its tiles are spread over all threads and workgroups."""
    counts = np.zeros(E, np.int32)
    counts[E // 3] = 300_000
    check_tile_map(counts, 300_000, A)


def test_tile_map_grid_stride_large():
    """Two million unit tiles: more tiles than the grid's threads, so each thread loops."""
    rng = np.random.default_rng(5)
    counts = rng.multinomial(2 ** 21, np.full(256, 1 / 256)).astype(np.int32)
    check_tile_map(counts, 2 ** 21, 1)


def test_tile_map_empty_histograms():
    check_tile_map(np.zeros(64, np.int32), 0, 16)
    check_tile_map(np.zeros(64, np.int32), 1000, 16)


def test_tile_map_optional_outputs():
    counts = np.array([5, 0, 3, 8, 1], np.int32)
    dev = torch.from_numpy(counts).to(DEV)
    o = oracle.tile_map(counts, 4)
    c2e, lim, pis, nct = gpu_tile_map(dev, 17, 4, with_arrays=(True, False), with_scalars=(False, False))
    assert lim is None and np.array_equal(c2e[:o.num_ctas], o.cta_to_expert)
    c2e, lim, pis, nct = gpu_tile_map(dev, 17, 4, with_arrays=(False, True), with_scalars=(False, True))
    assert np.array_equal(lim[:o.num_ctas], o.mn_limit) and int(nct[0]) == o.num_ctas
    c2e, lim, pis, nct = gpu_tile_map(dev, 17, 4, with_arrays=(False, False), with_scalars=(True, False))
    assert int(pis[0]) == o.permuted_idx_size


def test_tile_map_repeat_smaller_second_call():
    """Two calls into the same arrays, the second with fewer tiles: its entries replace the
    first call's and the rest keep the first call's values."""
    E, A = 128, 16
    rng = np.random.default_rng(11)
    big = rng.integers(0, 200, E).astype(np.int32)
    small = (big // 3).astype(np.int32)
    M = int(big.sum())
    cap = B.tile_map_capacity(M, E, A)
    c2e = torch.full((cap,), UNTOUCHED, dtype=torch.int32, device=DEV)
    lim = torch.full((cap,), UNTOUCHED, dtype=torch.int32, device=DEV)
    nct = torch.zeros(1, dtype=torch.int32, device=DEV)
    B.mep_tile_map(torch.from_numpy(big).to(DEV), M, A, c2e, lim, None, nct)
    B.mep_tile_map(torch.from_numpy(small).to(DEV), M, A, c2e, lim, None, nct)
    torch.cuda.synchronize()
    ob, os_ = oracle.tile_map(big, A), oracle.tile_map(small, A)
    g = c2e.cpu().numpy()
    assert int(nct.item()) == os_.num_ctas
    assert np.array_equal(g[:os_.num_ctas], os_.cta_to_expert)
    assert np.array_equal(g[os_.num_ctas:ob.num_ctas], ob.cta_to_expert[os_.num_ctas:])
    assert np.array_equal(lim.cpu().numpy()[:os_.num_ctas], os_.mn_limit)
