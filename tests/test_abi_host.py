"""Host-side checks of libmep.so that need no GPU: the library loads, exports every entry point
include/mep.h declares, sizes its workspaces, and rejects bad arguments before touching memory.
The pointers passed here are fake (never dereferenced: validation returns first)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mep.h")

pytest.importorskip("torch")
from expert_dispatch_layout_amd import _binding as B  # noqa: E402


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(mep_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    assert _declared() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(B.LIB_PATH)
    for name in _declared():
        assert hasattr(L, name), name


def test_status_strings():
    assert B.status_string(0) == "MEP_OK"
    assert B.status_string(3) == "MEP_ERR_CAPACITY"
    assert B.status_string(99) == "MEP_UNKNOWN_STATUS"


def test_workspace_sizes():
    # layout: header, arrival counters of up to 4096 count tiles (fixed region), then 4096-slot
    # tiles grouped by 4 into 32 count tiles: one look-back word per (count tile, expert) and
    # one tagged count per (tile, expert), each region 256-byte aligned
    arrive = 4096 * 4
    assert B.layout_workspace_size(0, 8, 2) == 256 + arrive
    assert B.layout_workspace_size(65536, 256, 8) == 256 + arrive + 32 * 256 * 8 + 128 * 256 * 8
    assert B.layout_workspace_size(1, 8, 2) == 256 + arrive + 256 + 256
    # plan: write tiles of 4096 / K tokens that never cross a shard, halved to 2048 / K while
    # that still gives at most 256 tiles (one per compute unit); tiles grouped into about 32
    # count tiles; arrival counters (fixed region), look-back words for the 3R rank columns,
    # tagged expert aggregates per count tile, and tagged 3R+E column histograms per write tile
    # (each part 256-aligned)
    def a256(x):
        return (x + 255) // 256 * 256

    # every plan workspace first reserves the fused path's two buffers of group sums (64 groups
    # x (512 + 3 * 32) columns of u32 each) right after the header
    gsum = 2 * 64 * (512 + 96) * 4

    # 65536 tokens, K = 8: 256 tiles of 256 tokens (halved), 8 per count tile, 32 count tiles
    old = (256 + gsum + 2048 * 4 + a256(32 * 24 * 8) + a256(32 * 256 * 8)
           + a256(256 * (24 + 256) * 8))

    # the fused path's plan tiles (at most 4096 slots, at most ceil(N / 256) tokens rounded up
    # to a multiple of 64 but no fewer than 64, never crossing a shard), counting workgroups of
    # `sub` tiles (about 256 of them): header, group sums, the count-tile
    # counters of mep_plan, then the workgroup totals and the within-workgroup tile prefixes
    # (E + 3R columns, 256-aligned parts)
    def path(ntiles, sub, nc):
        nwg = -(-ntiles // sub)
        return 256 + gsum + 8192 + a256(nwg * nc * 4) + a256(ntiles * nc * 4)

    want = max(old, path(256, 1, 256 + 24))
    assert B.plan_workspace_size(65536, 256, 8, 8, 8) == want
    assert B.plan_workspace_size(65536, 256, 8, 8, 1) == want
    # 262144 tokens over 32 shards: halving would give 1024 tiles, so 512 tiles of 512 tokens
    # stay, 16 per count tile (one per shard), 32 count tiles; the fused path has 512 tiles of
    # 512 tokens (4096 slots), 2 per counting workgroup
    old = (256 + gsum + 2048 * 4 + a256(32 * 96 * 8) + a256(32 * 256 * 8)
           + a256(512 * (96 + 256) * 8))
    assert B.plan_workspace_size(262144, 256, 8, 32, 32) == max(old, path(512, 2, 256 + 96))


FAKE = 0x10000          # aligned, never dereferenced
MIS = 0x10004           # 4-aligned but not 16-aligned


def _route(logits=FAKE, dtype=0, N=16, E=8, K=2, bias=FAKE, score_fn=0, renorm=1, n_group=1,
           topk_group=1, group_topn=2, scale=1.0, ids=FAKE, w=FAKE):
    p = B.RouteParams(score_fn, renorm, n_group, topk_group, group_topn, scale)
    return B.lib().mep_route_topk(logits, dtype, N, E, K, bias, ctypes.byref(p), ids, w, None)


def test_route_validation():
    assert _route(N=0) == B.MEP_OK                       # nothing to do, nothing launched
    assert _route(logits=None) == B.MEP_ERR_INVALID_ARG
    assert _route(N=0, logits=None, ids=None, w=None) == B.MEP_OK
    assert _route(ids=None) == B.MEP_ERR_INVALID_ARG
    assert _route(logits=MIS) == B.MEP_ERR_INVALID_ARG
    assert _route(dtype=7) == B.MEP_ERR_INVALID_ARG
    assert _route(score_fn=5) == B.MEP_ERR_INVALID_ARG
    assert _route(score_fn=1, bias=None) == B.MEP_ERR_INVALID_ARG
    assert _route(N=-1) == B.MEP_ERR_INVALID_ARG
    assert _route(scale=float("nan")) == B.MEP_ERR_INVALID_ARG
    assert _route(E=1025, K=2) == B.MEP_ERR_UNSUPPORTED
    assert _route(E=64, K=33) == B.MEP_ERR_UNSUPPORTED
    assert _route(E=8, K=9) == B.MEP_ERR_UNSUPPORTED
    assert _route(E=12, n_group=5) == B.MEP_ERR_UNSUPPORTED          # E % n_group
    assert _route(E=64, n_group=64) == B.MEP_ERR_UNSUPPORTED         # > 32 groups
    assert _route(E=16, n_group=4, topk_group=0) == B.MEP_ERR_INVALID_ARG
    assert _route(E=16, n_group=4, topk_group=1, group_topn=3) == B.MEP_ERR_UNSUPPORTED
    assert _route(E=16, K=8, n_group=4, topk_group=1) == B.MEP_ERR_UNSUPPORTED  # 4 eligible < K
    assert _route(N=2 ** 28, E=64, K=16) == B.MEP_ERR_UNSUPPORTED    # N*K > INT32_MAX


def _layout(N=16, E=8, K=2, A=4, tpe=FAKE, cu=FAKE, e2p=FAKE, p2e=FAKE, cap=None, zf=FAKE,
            ws=FAKE, ws_bytes=1 << 20, ids=FAKE):
    if cap is None:
        cap = N * K + min(E, N * K) * (A - 1)
    return B.lib().mep_build_layout(ids, N, E, K, A, tpe, cu, e2p, p2e, cap, zf, ws, ws_bytes, None)


def test_layout_validation():
    assert _layout(ids=None) == B.MEP_ERR_INVALID_ARG
    assert _layout(N=0, ids=None, e2p=None, ws=None) == B.MEP_ERR_INVALID_ARG   # workspace needed
    assert _layout(cu=None) == B.MEP_ERR_INVALID_ARG
    assert _layout(e2p=None) == B.MEP_ERR_INVALID_ARG
    assert _layout(ws=None) == B.MEP_ERR_INVALID_ARG
    assert _layout(e2p=FAKE + 2) == B.MEP_ERR_INVALID_ARG
    assert _layout(ws=FAKE + 64) == B.MEP_ERR_INVALID_ARG             # workspace needs 256 B
    assert _layout(A=0) == B.MEP_ERR_INVALID_ARG
    assert _layout(E=2048) == B.MEP_ERR_UNSUPPORTED
    assert _layout(K=9, E=8) == B.MEP_ERR_UNSUPPORTED
    assert _layout(N=2 ** 28, K=8, E=64) == B.MEP_ERR_UNSUPPORTED
    assert _layout(cap=16 * 2 + 8 * 3 - 1) == B.MEP_ERR_CAPACITY
    assert _layout(ws_bytes=255) == B.MEP_ERR_CAPACITY


def _plan(N=64, E=16, K=4, A=2, R=4, S=2, C=3, NvS=None, ws_bytes=1 << 24, cap_g=None,
          cap_d=None, out_ptr=FAKE, **kw):
    epn = E // R
    if NvS is None:
        NvS = N * min(K, epn) + epn * (A - 1)
    g, d = B.dedup_capacity(N, E, K, R)
    po = B.PlanOutputs(*([FAKE] * 12), g if cap_g is None else cap_g, FAKE,
                       d if cap_d is None else cap_d)
    for k, v in kw.items():
        setattr(po, k, v)
    return B.lib().mep_plan(FAKE, FAKE, FAKE, N, E, K, A, R, S, C, NvS, ctypes.byref(po), FAKE,
                            ws_bytes, None)


def test_plan_validation():
    assert _plan(E=18, R=4) == B.MEP_ERR_UNSUPPORTED                  # E % R
    assert _plan(R=129, E=129 * 2) == B.MEP_ERR_UNSUPPORTED
    assert _plan(N=63, S=2) == B.MEP_ERR_INVALID_ARG                  # N % num_src
    assert _plan(C=0) == B.MEP_ERR_INVALID_ARG
    assert _plan(S=0) == B.MEP_ERR_INVALID_ARG
    assert _plan(dst=FAKE + 1) == B.MEP_ERR_INVALID_ARG
    assert _plan(NvS=64 * 4 + 4 * 1 - 1) == B.MEP_ERR_CAPACITY       # below the per-rank bound
    assert _plan(N=2 ** 20, E=16, K=4, R=4, NvS=2 ** 30) == B.MEP_ERR_CAPACITY  # R*NvS > INT32_MAX
    g, d = B.dedup_capacity(64, 16, 4, 4)
    assert g == 64 * 2 and d == 64 * 3
    assert _plan(cap_g=g - 1) == B.MEP_ERR_CAPACITY
    assert _plan(cap_d=d - 1) == B.MEP_ERR_CAPACITY
    assert _plan(ws_bytes=100) == B.MEP_ERR_CAPACITY
    # epn == 1: no duplicates are possible, zero capacity is enough for both lists
    assert B.dedup_capacity(64, 8, 2, 8) == (0, 0)


def _tile(E=8, M=64, A=4, tpe=FAKE, c2e=FAKE, lim=FAKE, cap=None, pis=FAKE, nct=FAKE):
    if cap is None:
        cap = B.tile_map_capacity(M, E, A) if A > 0 else 0
    return B.lib().mep_tile_map(tpe, E, M, A, c2e, lim, cap, pis, nct, None)


def test_tile_map_validation():
    assert B.tile_map_capacity(64, 8, 4) == (64 + 8 * 3) // 4
    assert B.tile_map_capacity(3, 8, 4) == (3 + 3 * 3) // 4      # at most 3 experts hold slots
    assert B.tile_map_capacity(0, 8, 4) == 0
    assert _tile(tpe=None) == B.MEP_ERR_INVALID_ARG
    assert _tile(E=0) == B.MEP_ERR_INVALID_ARG
    assert _tile(A=0) == B.MEP_ERR_INVALID_ARG
    assert _tile(M=-1, cap=0) == B.MEP_ERR_INVALID_ARG
    assert _tile(cap=-1) == B.MEP_ERR_INVALID_ARG
    assert _tile(lim=FAKE + 2) == B.MEP_ERR_INVALID_ARG
    assert _tile(E=1025) == B.MEP_ERR_UNSUPPORTED
    assert _tile(M=2 ** 31, A=1, cap=2 ** 31) == B.MEP_ERR_UNSUPPORTED
    assert _tile(cap=(64 + 8 * 3) // 4 - 1) == B.MEP_ERR_CAPACITY
    assert _tile(c2e=None, cap=(64 + 8 * 3) // 4 - 1) == B.MEP_ERR_CAPACITY  # either array
    # nothing to write: accepted without a launch
    assert _tile(c2e=None, lim=None, pis=None, nct=None, cap=0) == B.MEP_OK


def test_rows_validation():
    L = B.lib()
    perm = lambda x=FAKE, dt=1, N=16, H=64, K=2, e2p=FAKE, zf=FAKE, E=4, out=FAKE, T=64: \
        L.mep_permute_rows(x, dt, N, H, K, e2p, zf, E, out, T, None)
    comb = lambda y=FAKE, dt=1, N=16, H=64, K=2, e2p=FAKE, w=FAKE, T=64, out=FAKE: \
        L.mep_combine_rows(y, dt, N, H, K, e2p, w, T, out, None)
    for f in (perm, comb):
        assert f(dt=2) == B.MEP_ERR_INVALID_ARG
        assert f(N=-1) == B.MEP_ERR_INVALID_ARG
        assert f(H=0) == B.MEP_ERR_INVALID_ARG
        assert f(K=0) == B.MEP_ERR_INVALID_ARG
        assert f(e2p=None) == B.MEP_ERR_INVALID_ARG
        assert f(e2p=FAKE + 2) == B.MEP_ERR_INVALID_ARG
        assert f(H=12) == B.MEP_ERR_UNSUPPORTED           # 24-byte bf16 rows
        assert f(dt=0, H=6) == B.MEP_ERR_UNSUPPORTED      # 24-byte fp32 rows
        assert f(K=33) == B.MEP_ERR_UNSUPPORTED
        assert f(T=2 ** 31) == B.MEP_ERR_UNSUPPORTED
    assert perm(x=MIS) == B.MEP_ERR_INVALID_ARG
    assert perm(out=MIS) == B.MEP_ERR_INVALID_ARG
    assert perm(x=None) == B.MEP_ERR_INVALID_ARG
    assert perm(E=0) == B.MEP_ERR_INVALID_ARG
    assert perm(N=0, x=None, e2p=None, out=None) == B.MEP_ERR_INVALID_ARG  # zero_fill needs out
    assert perm(N=0, x=None, e2p=None, zf=None, out=None) == B.MEP_OK       # nothing to do
    assert comb(y=MIS) == B.MEP_ERR_INVALID_ARG
    assert comb(out=None) == B.MEP_ERR_INVALID_ARG
    assert comb(w=FAKE + 1) == B.MEP_ERR_INVALID_ARG
    assert comb(N=0, y=None, e2p=None, out=None) == B.MEP_OK


def test_balanced_validation():
    def call(N=64, E=16, K=4, R=4, nb=2, tp=2, cap=100, NvS=None, ptrs=FAKE, **kw):
        if NvS is None:
            NvS = B.balanced_nvs(N, E, K, R, nb, tp, cap)
        out = B.BalancedOutputs(*([FAKE] * len(B.BALANCED_FIELDS)))
        for k, v in kw.items():
            setattr(out, k, v)
        return B.lib().mep_plan_balanced(ptrs, FAKE, ptrs, ptrs, N, E, K, R, nb, tp, cap, NvS,
                                         ctypes.byref(out), None)
    assert B.balanced_nvs(64, 16, 4, 4, 2, 2, 100) == max(64 * 4, 100) + 18
    assert call(N=-1) == B.MEP_ERR_INVALID_ARG
    assert call(tp=0) == B.MEP_ERR_INVALID_ARG
    assert call(nb=-1) == B.MEP_ERR_INVALID_ARG
    assert call(cap=-1) == B.MEP_ERR_INVALID_ARG
    assert call(z=None) == B.MEP_ERR_INVALID_ARG
    assert call(dst=None) == B.MEP_ERR_INVALID_ARG
    assert call(experts_to_copy=None) == B.MEP_ERR_INVALID_ARG
    assert call(alloc=FAKE + 2) == B.MEP_ERR_INVALID_ARG
    assert call(ptrs=None) == B.MEP_ERR_INVALID_ARG
    assert call(E=18, R=4) == B.MEP_ERR_UNSUPPORTED
    assert call(R=256, E=512) == B.MEP_ERR_UNSUPPORTED
    assert call(E=2048, R=4) == B.MEP_ERR_UNSUPPORTED
    assert call(nb=65) == B.MEP_ERR_UNSUPPORTED
    assert call(K=33, E=64) == B.MEP_ERR_UNSUPPORTED
    assert call(cap=2 ** 31) == B.MEP_ERR_UNSUPPORTED
    assert call(NvS=B.balanced_nvs(64, 16, 4, 4, 2, 2, 100) - 1) == B.MEP_ERR_CAPACITY
    assert call(N=2 ** 20, NvS=2 ** 30) == B.MEP_ERR_CAPACITY          # R * NvS > INT32_MAX


def test_noalloc_rejects_sizes_beyond_its_array():
    """mep_route_layout_plan_noalloc returns MEP_ERR_CAPACITY, before touching anything, when the
    call's plan workspace would exceed the library's 8 MiB per-GPU array."""
    N, E, K, A, R, S, C = 1 << 22, 256, 8, 128, 8, 8, 24
    assert B.plan_workspace_size(N, E, K, R, S) > 8 << 20
    params = B.RouteParams(1, 1, 8, 4, 2, 2.5)
    po = B.PlanOutputs(*([FAKE] * 12), N * 4, FAKE, N * 7)
    rc = B.lib().mep_route_layout_plan_noalloc(
        FAKE, 0, N, E, K, FAKE, ctypes.byref(params), FAKE, FAKE, A, FAKE, FAKE, FAKE, FAKE,
        N * K + E * (A - 1), FAKE, R, S, C, B.default_nvs(N, E, K, R, A), ctypes.byref(po), None)
    assert rc == B.MEP_ERR_CAPACITY
    # a bad argument is reported the same way as by mep_route_layout_plan, nothing enqueued
    rc = B.lib().mep_route_layout_plan_noalloc(
        FAKE, 0, 64, E, K, FAKE, ctypes.byref(params), FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE,
        64 * K, FAKE, R, S, C, B.default_nvs(64, E, K, R, 1), ctypes.byref(po), None)
    assert rc == B.MEP_ERR_INVALID_ARG


def test_sigmoid_eval_validation():
    L = B.lib()
    assert L.mep_sigmoid_eval(FAKE, -1, FAKE, None, None, None) == B.MEP_ERR_INVALID_ARG
    assert L.mep_sigmoid_eval(None, 16, FAKE, None, None, None) == B.MEP_ERR_INVALID_ARG
    assert L.mep_sigmoid_eval(FAKE, 16, FAKE + 2, None, None, None) == B.MEP_ERR_INVALID_ARG
    assert L.mep_sigmoid_eval(FAKE, 16, None, None, FAKE + 4, None) == B.MEP_ERR_INVALID_ARG
    # nothing to do: no launch
    assert L.mep_sigmoid_eval(FAKE, 0, FAKE, FAKE, FAKE, None) == B.MEP_OK
    assert L.mep_sigmoid_eval(FAKE, 16, None, None, None, None) == B.MEP_OK
