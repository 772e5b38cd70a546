"""GPU parity of mep_plan_balanced against the CPU oracle: every output bit for bit, on skewed
routing that forces moves and copies, on the corner cases of the envelope, and at the dsv3 batch
size.  The layout inputs come from the oracle and are uploaded, so both sides plan from the same
arrays."""
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import oracle
from expert_dispatch_layout_amd import _binding as B

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    B.lib()


def _skewed_ids(rng, N, E, K, hot):
    """Routing with experts 0.. favoured (hot = scale of the exponential preference)."""
    if N == 0:
        return np.zeros((0, K), np.int32)
    g = rng.gumbel(size=(N, E)) - np.arange(E) / hot
    return np.argsort(-g, axis=1)[:, :K].astype(np.int32)


def check_balanced(ids, E, R, nb, tp, cap, NvS=None, A=1):
    N, K = ids.shape
    if NvS is None:
        NvS = B.balanced_nvs(N, E, K, R, nb, tp, cap)
    L = oracle.layout(ids, E, A)
    want = oracle.plan_balanced(ids, L.tokens_per_expert, L.cu_seqlens, L.expanded_to_permuted,
                                E, R, nb, tp, cap, NvS)
    lay = SimpleNamespace(tokens_per_expert=torch.from_numpy(L.tokens_per_expert).to(DEV),
                          cu_seqlens=torch.from_numpy(L.cu_seqlens).to(DEV),
                          expanded_to_permuted=torch.from_numpy(L.expanded_to_permuted).to(DEV))
    out = B.alloc_balanced(N, E, K, R, nb, DEV)
    for f in B.BALANCED_FIELDS:
        getattr(out, f).fill_(-7)
    B.mep_plan_balanced(torch.from_numpy(ids).to(DEV), lay, E, R, nb, tp, cap, NvS, out)
    torch.cuda.synchronize()
    for f in B.BALANCED_FIELDS:
        g = getattr(out, f).cpu().numpy()
        w = getattr(want, f)
        assert g.shape == w.shape, f
        assert np.array_equal(g, w), "%s differs at %s" % (f, np.argwhere(g != w)[:4].tolist())
    return want


CASES = [
    # N, E, K, R, B, tp, cap as a fraction of the mean rank load, hot
    (256, 8, 2, 4, 1, 1, 1.0, 2.0),
    (500, 16, 4, 4, 2, 3, 0.8, 3.0),
    (777, 32, 6, 8, 3, 4, 1.0, 6.0),
    (1000, 64, 8, 8, 4, 1, 1.1, 8.0),
    (1000, 64, 8, 8, 4, 128, 0.5, 8.0),
    (300, 256, 8, 8, 8, 16, 1.0, 40.0),
    (200, 1024, 32, 128, 64, 2, 1.0, 200.0),
    (200, 1024, 8, 1, 5, 1, 0.5, 100.0),       # one rank: nothing to move or copy
    (400, 128, 4, 128, 2, 1, 1.0, 30.0),       # one expert per rank
    (128, 8, 2, 4, 0, 1, 1.0, 2.0),            # no copies
    (0, 16, 2, 4, 2, 4, 1.0, 2.0),             # empty batch
    (256, 8, 2, 4, 2, 1, 0.0, 2.0),            # capacity 0: no rank is short
    (256, 8, 2, 4, 2, 1, 100.0, 2.0),          # capacity above every load: no moves
    (256, 8, 2, 4, 2, 1, 20000.0, 2.0),        # balances beyond 2^21: the 64-bit keys
    (640, 96, 6, 16, 3, 2, 0.9, 12.0),         # R = 16: four 16-byte loads per allocation row
    (600, 48, 4, 12, 2, 1, 1.0, 8.0),          # R = 12: three
    (500, 36, 4, 6, 2, 1, 1.0, 6.0),           # R = 6: binary search
]


@pytest.mark.parametrize("N,E,K,R,nb,tp,capf,hot", CASES)
def test_balanced_parity(N, E, K, R, nb, tp, capf, hot):
    print("balanced case N=%d E=%d K=%d R=%d B=%d tp=%d cap=%.2f" % (N, E, K, R, nb, tp, capf),
          flush=True)
    rng = np.random.default_rng(N * 3 + E + R)
    ids = _skewed_ids(rng, N, E, K, hot)
    cap = int(capf * N * K / R)
    check_balanced(ids, E, R, nb, tp, cap)


def test_balanced_layout_alignment_does_not_matter():
    """The plan reads only positions within an expert, so any layout alignment gives the same
    result."""
    rng = np.random.default_rng(5)
    ids = _skewed_ids(rng, 600, 32, 4, 6.0)
    a = check_balanced(ids, 32, 8, 2, 4, 250, A=1)
    b = check_balanced(ids, 32, 8, 2, 4, 250, A=64)
    assert np.array_equal(a.dst, b.dst)


def test_balanced_larger_stride():
    rng = np.random.default_rng(6)
    ids = _skewed_ids(rng, 500, 16, 4, 3.0)
    nvs = B.balanced_nvs(500, 16, 4, 4, 2, 3, 400) + 1000
    check_balanced(ids, 16, 4, 2, 3, 400, NvS=nvs)


def test_balanced_dsv3_batch():
    """N = 65536, E = 256, K = 8 over 8 ranks, routing skewed so that ranks overflow a capacity
    of the mean load: every output compared."""
    rng = np.random.default_rng(7)
    N, E, K, R = 65536, 256, 8, 8
    print("balanced dsv3 batch", flush=True)
    ids = _skewed_ids(rng, N, E, K, 96.0)
    P = check_balanced(ids, E, R, 4, 128, N * K // R)
    assert P.z.any() and (P.experts_to_copy >= 0).any()


def test_balanced_unaligned_cumsum():
    """alloc_cumsum 4- but not 16-byte aligned: dst takes the binary search instead of the
    16-byte row loads, with the same result."""
    rng = np.random.default_rng(9)
    N, E, K, R, nb, tp = 1000, 64, 8, 8, 4, 1
    ids = _skewed_ids(rng, N, E, K, 8.0)
    cap = N * K // R
    NvS = B.balanced_nvs(N, E, K, R, nb, tp, cap)
    L = oracle.layout(ids, E, 1)
    want = oracle.plan_balanced(ids, L.tokens_per_expert, L.cu_seqlens, L.expanded_to_permuted,
                                E, R, nb, tp, cap, NvS)
    lay = SimpleNamespace(tokens_per_expert=torch.from_numpy(L.tokens_per_expert).to(DEV),
                          cu_seqlens=torch.from_numpy(L.cu_seqlens).to(DEV),
                          expanded_to_permuted=torch.from_numpy(L.expanded_to_permuted).to(DEV))
    out = B.alloc_balanced(N, E, K, R, nb, DEV)
    out.alloc_cumsum = torch.zeros(E * R + 1, dtype=torch.int32, device=DEV)[1:].view(E, R)
    assert out.alloc_cumsum.data_ptr() % 16 == 4
    B.mep_plan_balanced(torch.from_numpy(ids).to(DEV), lay, E, R, nb, tp, cap, NvS, out)
    torch.cuda.synchronize()
    for f in B.BALANCED_FIELDS:
        assert np.array_equal(getattr(out, f).cpu().numpy(), getattr(want, f)), f
    assert want.z.any()


def test_balanced_wide_keys_with_moves():
    """4.8 M one-slot tokens over two ranks of one expert each: the hot expert holds about 3.5 M
    slots, beyond the 2^21 range of the 32-bit arg-extremum keys, so the balancing, quota and
    copy loops run on 64-bit keys; one move and one copy."""
    rng = np.random.default_rng(8)
    N, E, K, R = 4_800_000, 2, 1, 2
    print("balanced wide keys N=%d" % N, flush=True)
    ids = _skewed_ids(rng, N, E, K, 1.0)
    assert np.count_nonzero(ids == 0) >= 1 << 21
    P = check_balanced(ids, E, R, 1, 1, N * K // R)
    assert P.z.any() and (P.experts_to_copy >= 0).any()
