"""GPU parity of mep_permute_rows / mep_combine_rows against the CPU oracle: bytes must match
exactly (permute is a copy; combine sums in binary32 in slot order on both sides and casts the
same way), rows outside what a call defines must stay untouched, and at the full dsv3 shape the
results are checked on all rows through torch gathers (permute) and on sampled tokens through
the oracle (combine)."""
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


def _rand_rows(rng, shape, dtype, specials=False):
    v = rng.standard_normal(shape).astype(np.float32) * np.float32(4)
    if specials:
        flat = v.reshape(-1)
        flat[rng.integers(0, flat.size, 8)] = np.inf
        flat[rng.integers(0, flat.size, 8)] = -np.inf
        flat[rng.integers(0, flat.size, 8)] = 0.0
        flat[rng.integers(0, flat.size, 8)] = -0.0
        flat[rng.integers(0, flat.size, 8)] = 3.3e38
    if dtype == "f32":
        return v
    return torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _to_dev(a):
    t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(DEV)
    return t.view(torch.bfloat16) if a.dtype == np.uint16 else t


def _to_host(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _same_rows(got, want):
    """Bit-equal outside NaNs; NaNs in the same places (a NaN's payload after arithmetic is the
    hardware's own, and x86 and gfx950 make different ones)."""
    gf = got if got.dtype == np.float32 else (got.astype(np.uint32) << 16).view(np.float32)
    wf = want if want.dtype == np.float32 else (want.astype(np.uint32) << 16).view(np.float32)
    gn, wn = np.isnan(gf), np.isnan(wf)
    return np.array_equal(gn, wn) and np.array_equal(got[~gn], want[~wn])


def _layout(rng, N, E, K, A):
    ids = np.stack([rng.permutation(E)[:K] for _ in range(N)]).astype(np.int32) if N else \
        np.zeros((0, K), np.int32)
    return ids, oracle.layout(ids, E, A)


CASES = [(0, 8, 2, 4, 8), (1, 4, 1, 1, 8), (37, 8, 2, 4, 16), (300, 16, 4, 3, 72),
         (1000, 64, 8, 128, 64), (513, 256, 8, 128, 200), (97, 32, 6, 5, 1032), (64, 128, 32, 2, 24)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N,E,K,A,H", CASES)
def test_permute_and_combine_parity(dtype, N, E, K, A, H):
    if dtype == "f32" and H % 4:
        pytest.skip("fp32 rows need H % 4 == 0")
    print("rows case dtype=%s N=%d E=%d K=%d A=%d H=%d" % (dtype, N, E, K, A, H), flush=True)
    rng = np.random.default_rng(N * 7 + E + K * 131 + H)
    x = _rand_rows(rng, (N, H), dtype, specials=N > 10)
    ids, L = _layout(rng, N, E, K, A)
    T = int(L.cu_seqlens[E])
    rows = T + 3                       # three rows past the layout must stay untouched
    e2p = torch.from_numpy(L.expanded_to_permuted).to(DEV)
    zf = torch.from_numpy(L.zero_fill).to(DEV)
    xd = _to_dev(x)
    xp = torch.empty((rows, H), dtype=xd.dtype, device=DEV)
    xp.view(torch.uint8).fill_(0xFF)
    B.mep_permute_rows(xd, e2p, K, zf, xp)
    torch.cuda.synchronize()
    want = oracle.permute_rows(x, L.expanded_to_permuted, L.zero_fill, rows)
    got = _to_host(xp)
    assert np.array_equal(got.view(np.uint8), want.view(np.uint8))

    w = rng.standard_normal((N, K)).astype(np.float32)
    y = _rand_rows(rng, (rows, H), dtype, specials=N > 10)
    yd = _to_dev(y)
    for weights in (w, None):
        out = torch.empty((N, H), dtype=xd.dtype, device=DEV)
        B.mep_combine_rows(yd, e2p, K, None if weights is None else torch.from_numpy(weights).to(DEV),
                           out)
        torch.cuda.synchronize()
        want = oracle.combine_rows(y, L.expanded_to_permuted, K, weights)
        assert _same_rows(_to_host(out), want), "combine differs (weights=%s)" % (weights is not None)


def test_permute_without_zero_fill_leaves_padding():
    rng = np.random.default_rng(1)
    N, E, K, A, H = 200, 16, 4, 16, 32
    x = _rand_rows(rng, (N, H), "bf16")
    ids, L = _layout(rng, N, E, K, A)
    T = int(L.cu_seqlens[E])
    xp = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    xp.view(torch.uint8).fill_(0x5A)
    B.mep_permute_rows(_to_dev(x), torch.from_numpy(L.expanded_to_permuted).to(DEV), K, None, xp)
    torch.cuda.synchronize()
    want = oracle.permute_rows(x, L.expanded_to_permuted, None, T, fill=0x5A)
    assert np.array_equal(_to_host(xp).view(np.uint8), want.view(np.uint8))


def test_combine_nan_positions_agree():
    """NaN payloads after arithmetic are the hardware's; only where NaNs land is compared."""
    rng = np.random.default_rng(2)
    N, K, H = 64, 4, 16
    y = rng.standard_normal((N * K, H)).astype(np.float32)
    y.reshape(-1)[rng.integers(0, y.size, 40)] = np.nan
    e2p = rng.permutation(N * K).astype(np.int32)
    w = rng.standard_normal((N, K)).astype(np.float32)
    for dtype in ("f32", "bf16"):
        yy = y if dtype == "f32" else torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        out = torch.empty((N, H), dtype=torch.float32 if dtype == "f32" else torch.bfloat16, device=DEV)
        B.mep_combine_rows(_to_dev(yy), torch.from_numpy(e2p).to(DEV), K, torch.from_numpy(w).to(DEV), out)
        torch.cuda.synchronize()
        want = oracle.combine_rows(yy, e2p, K, w)
        g = out.float().cpu().numpy()
        wv = want if dtype == "f32" else (want.astype(np.uint32) << 16).view(np.float32)
        assert np.array_equal(np.isnan(g), np.isnan(wv))
        assert np.array_equal(g[~np.isnan(g)], wv[~np.isnan(wv)])


def test_full_shape_dsv3():
    """N = 65536 tokens, E = 256, K = 8, A = 128, H = 7168 bf16 rows: every permuted row checked
    through a torch gather on the device, every padding row zero, combine checked on sampled
    tokens through the oracle."""
    N, E, K, A, H = 65536, 256, 8, 128, 7168
    print("rows full shape N=%d H=%d" % (N, H), flush=True)
    rng = np.random.default_rng(7)
    ids = np.argsort(rng.random((N, E)), axis=1)[:, :K].astype(np.int32)
    L = oracle.layout(ids, E, A)
    T = int(L.cu_seqlens[E])
    e2p = torch.from_numpy(L.expanded_to_permuted).to(DEV)
    zf = torch.from_numpy(L.zero_fill).to(DEV)
    g = torch.Generator(device=DEV).manual_seed(3)
    x = torch.randn((N, H), generator=g, device=DEV).to(torch.bfloat16)
    xp = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    xp.view(torch.uint8).fill_(0xFF)
    B.mep_permute_rows(x, e2p, K, zf, xp)
    torch.cuda.synchronize()
    xi, xpi = x.view(torch.int16), xp.view(torch.int16)
    tok = torch.arange(N, device=DEV).repeat_interleave(K)
    for c in range(0, N * K, 1 << 16):          # gather in chunks to bound the extra memory
        sl = slice(c, c + (1 << 16))
        assert torch.equal(xpi[e2p[sl].long()], xi[tok[sl]])
    pad = torch.ones(T, dtype=torch.bool, device=DEV)
    pad[e2p.long()] = False
    assert int(pad.sum()) == T - N * K
    assert int(xpi[pad].abs().sum()) == 0
    w = torch.rand((N, K), generator=g, device=DEV)
    out = torch.empty((N, H), dtype=torch.bfloat16, device=DEV)
    B.mep_combine_rows(xp, e2p, K, w, out)
    torch.cuda.synchronize()
    sample = np.sort(rng.choice(N, 48, replace=False))
    P = L.expanded_to_permuted.reshape(N, K)[sample]
    y_sub = _to_host(xp[torch.from_numpy(P.reshape(-1)).long().to(DEV)])
    want = oracle.combine_rows(y_sub, np.arange(P.size, dtype=np.int32), K, w.cpu().numpy()[sample])
    got = _to_host(out[torch.from_numpy(sample).to(DEV)])
    assert np.array_equal(got, want)
