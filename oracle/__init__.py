"""CPU oracle for MoE routing, dispatch layout and expert-parallel planning.

TEST INFRASTRUCTURE ONLY.  Tests, the smoke check and the CPU-baseline leg of
the benchmark may import this package; the product path (the HIP library and
its Python binding) never does, and this package never imports the product.

The arithmetic lives in ``mep_oracle.c`` (plain C, fp64 weights, correctly
rounded sigmoid with a binary128 fallback).  This module compiles it with gcc
and exposes numpy-level wrappers.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mep_oracle.c")
_LIB = os.path.join(_HERE, "libmep_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle shared library with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-fexcess-precision=standard", "-Wall", "-shared", "-fPIC",
               _SRC, "-o", tmp, "-lquadmath", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def load(path: str):
    """Load an oracle shared library from `path` and declare its C signatures."""
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i64, i32, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_float
    L.oracle_sigmoid.argtypes = [f32]
    L.oracle_sigmoid.restype = f32
    L.oracle_sigmoid_batch.argtypes = [P, i64, P, P]
    L.oracle_sigmoid_batch.restype = None
    L.oracle_route.argtypes = [P, i32, i64, i32, i32, P, i32, i32, i32, i32, i32, f32, P, P]
    L.oracle_route.restype = i32
    L.oracle_layout.argtypes = [P, i64, i32, i32, i32, P, P, P, P, i64, P]
    L.oracle_layout.restype = i32
    L.oracle_plan.argtypes = ([P, P, P, i64, i32, i32, i32, i32, i32, i64]
                              + [P] * 11 + [P, i64, P, i64])
    L.oracle_plan.restype = i32
    L.oracle_tile_map.argtypes = [P, i32, i32, P, P, i64, P, P]
    L.oracle_tile_map.restype = i32
    L.oracle_permute_rows.argtypes = [P, i32, i64, i64, i32, P, P, i32, P, i64]
    L.oracle_permute_rows.restype = i32
    L.oracle_combine_rows.argtypes = [P, i32, i64, i64, i32, P, P, P, i64]
    L.oracle_combine_rows.restype = i32
    L.oracle_plan_balanced.argtypes = ([P, P, P, P, i64, i32, i32, i32, i32, i32, i64, i64]
                                       + [P] * 10)
    L.oracle_plan_balanced.restype = i32
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = load(_LIB)
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def sigmoid(x: np.ndarray, with_path: bool = False):
    """Correctly rounded binary32 logistic sigmoid of float32 inputs."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty_like(x)
    path = np.empty(x.shape, dtype=np.int32) if with_path else None
    lib().oracle_sigmoid_batch(_p(x), x.size, _p(out), _p(path))
    return (out, path) if with_path else out


SOFTMAX, SIGMOID = 0, 1
F32, BF16 = 0, 1


def route(logits: np.ndarray, K: int, *, bias=None, score_fn=SOFTMAX, renormalize=True,
          n_group=1, topk_group=1, group_topn=2, scale=1.0, dtype=F32):
    """logits: float32 [N,E] (dtype=F32) or uint16 bf16 bit patterns [N,E] (dtype=BF16)."""
    logits = np.ascontiguousarray(logits)
    assert logits.dtype == (np.float32 if dtype == F32 else np.uint16)
    N, E = logits.shape
    ids = np.empty((N, K), dtype=np.int32)
    w = np.empty((N, K), dtype=np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    rc = lib().oracle_route(_p(logits), dtype, N, E, K, _p(b), score_fn, int(renormalize),
                            n_group, topk_group, group_topn, float(scale), _p(ids), _p(w))
    if rc != 0:
        raise ValueError("oracle_route rejected the arguments (code %d)" % rc)
    return ids, w


@dataclass
class Layout:
    tokens_per_expert: np.ndarray
    cu_seqlens: np.ndarray
    expanded_to_permuted: np.ndarray
    permuted_to_expanded: np.ndarray
    zero_fill: np.ndarray


def route_threads(logits: np.ndarray, K: int, nthreads: int, **kw):
    """route() with the tokens split into `nthreads` contiguous ranges, each routed by the same
    C routine on its own thread (ctypes releases the GIL during the call).  Tokens are
    independent, so the result equals route()'s."""
    from concurrent.futures import ThreadPoolExecutor

    dtype = kw.get("dtype", F32)
    logits = np.ascontiguousarray(logits)
    assert logits.dtype == (np.float32 if dtype == F32 else np.uint16)
    N, E = logits.shape
    ids = np.empty((N, K), dtype=np.int32)
    w = np.empty((N, K), dtype=np.float32)
    bias = kw.get("bias")
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    bounds = [N * i // nthreads for i in range(nthreads + 1)]

    def one(i):
        lo, hi = bounds[i], bounds[i + 1]
        if hi <= lo:
            return 0
        return lib().oracle_route(_p(logits[lo:hi]), dtype, hi - lo, E, K, _p(b),
                                  kw.get("score_fn", SOFTMAX), int(kw.get("renormalize", True)),
                                  kw.get("n_group", 1), kw.get("topk_group", 1),
                                  kw.get("group_topn", 2), float(kw.get("scale", 1.0)),
                                  _p(ids[lo:hi]), _p(w[lo:hi]))

    with ThreadPoolExecutor(max_workers=nthreads) as ex:
        rcs = list(ex.map(one, range(nthreads)))
    if any(rc != 0 for rc in rcs):
        raise ValueError("oracle_route rejected the arguments (codes %s)" % rcs)
    return ids, w


def layout(ids: np.ndarray, E: int, alignment: int) -> Layout:
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    N, K = ids.shape
    cap = N * K + min(E, N * K) * (alignment - 1)
    tpe = np.empty(E, np.int32)
    cu = np.empty(E + 1, np.int32)
    e2p = np.empty(N * K, np.int32)
    p2e = np.empty(max(cap, 1), np.int32)
    zf = np.empty((E, 2), np.int32)
    rc = lib().oracle_layout(_p(ids), N, E, K, alignment, _p(tpe), _p(cu), _p(e2p), _p(p2e),
                             cap, _p(zf))
    if rc != 0:
        raise ValueError("oracle_layout failed (code %d)" % rc)
    T = int(cu[E])
    return Layout(tpe, cu, e2p, p2e[:T].copy(), zf)


@dataclass
class TileMap:
    cta_to_expert: np.ndarray  # [num_ctas]
    mn_limit: np.ndarray       # [num_ctas]
    permuted_idx_size: int
    num_ctas: int


def tile_map(counts: np.ndarray, alignment: int) -> TileMap:
    """Grouped-GEMM tile maps of per-expert counts ([TRT] routingPermutation CTA maps)."""
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    E = counts.shape[0]
    cap = int(np.sum((counts.astype(np.int64) + alignment - 1) // alignment)) if E else 0
    c2e = np.empty(max(cap, 1), np.int32)
    lim = np.empty(max(cap, 1), np.int32)
    pis = np.zeros(1, np.int32)
    nc = np.zeros(1, np.int32)
    rc = lib().oracle_tile_map(_p(counts), E, alignment, _p(c2e), _p(lim), cap, _p(pis), _p(nc))
    if rc != 0:
        raise ValueError("oracle_tile_map failed (code %d)" % rc)
    n = int(nc[0])
    return TileMap(c2e[:n].copy(), lim[:n].copy(), int(pis[0]), n)


def _row_dtype(a: np.ndarray) -> int:
    """0 for fp32 rows, 1 for bf16 rows (held as uint16 bit patterns)."""
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:
        return 1
    raise ValueError("rows must be float32 or uint16 (bf16 bits)")


def permute_rows(x: np.ndarray, expanded_to_permuted: np.ndarray, zero_fill: np.ndarray,
                 T: int, fill=None) -> np.ndarray:
    """Rows of x [N, H] copied to their permuted rows [T, H]; padding ranges zeroed.  Rows that
    neither step writes keep `fill` (default: an all-ones bit pattern, so they stand out)."""
    x = np.ascontiguousarray(x)
    N, H = x.shape
    K = expanded_to_permuted.size // max(N, 1) if N else 1
    e2p = np.ascontiguousarray(expanded_to_permuted, np.int32)
    zf = None if zero_fill is None else np.ascontiguousarray(zero_fill, np.int32)
    out = np.empty((T, H), x.dtype)
    out.view(np.uint8)[...] = 0xFF if fill is None else fill
    E = 1 if zf is None else zf.shape[0]
    rc = lib().oracle_permute_rows(_p(x), _row_dtype(x), N, H, K, _p(e2p), _p(zf), E, _p(out), T)
    if rc != 0:
        raise ValueError("oracle_permute_rows failed (code %d)" % rc)
    return out


def combine_rows(y: np.ndarray, expanded_to_permuted: np.ndarray, K: int,
                 topk_weights: np.ndarray = None) -> np.ndarray:
    """out[t] = sum over k (in order, binary32) of w[t,k] * y[P[t,k]], cast to y's type."""
    y = np.ascontiguousarray(y)
    T, H = y.shape
    e2p = np.ascontiguousarray(expanded_to_permuted, np.int32).reshape(-1)
    N = e2p.size // K
    w = None if topk_weights is None else np.ascontiguousarray(topk_weights, np.float32)
    out = np.empty((N, H), y.dtype)
    rc = lib().oracle_combine_rows(_p(y), _row_dtype(y), N, H, K, _p(e2p), _p(w), _p(out), T)
    if rc != 0:
        raise ValueError("oracle_combine_rows failed (code %d)" % rc)
    return out


@dataclass
class BalancedPlan:
    group_tokens: np.ndarray     # [R]
    z: np.ndarray                # [R, R] slots moved from rank s to rank d
    alloc: np.ndarray            # [R, E] slots of expert e computed on rank r
    alloc_cumsum: np.ndarray     # [E, R]
    experts_to_copy: np.ndarray  # [R, B]
    remote_stats: np.ndarray     # [R, 2]
    cu_seqlens: np.ndarray       # [R, E+B] group ends
    zero_fill: np.ndarray        # [R, E+B, 2]
    expert_offsets: np.ndarray   # [R, E]
    dst: np.ndarray              # [N*K]


def plan_balanced(ids, tokens_per_expert, cu_seqlens, expanded_to_permuted, E, R, B, tp,
                  capacity, NvS) -> BalancedPlan:
    """MoonEP capacity rebalancing with redundant remote experts, for all R ranks."""
    ids = np.ascontiguousarray(ids, np.int32)
    N, K = ids.shape
    G = E + B
    out = BalancedPlan(np.empty(R, np.int32), np.empty((R, R), np.int32),
                       np.empty((R, E), np.int32), np.empty((E, R), np.int32),
                       np.empty((R, max(B, 0)), np.int32), np.empty((R, 2), np.int32),
                       np.empty((R, G), np.int32), np.empty((R, G, 2), np.int32),
                       np.empty((R, E), np.int32), np.empty(N * K, np.int32))
    rc = lib().oracle_plan_balanced(
        _p(ids), _p(np.ascontiguousarray(tokens_per_expert, np.int32)),
        _p(np.ascontiguousarray(cu_seqlens, np.int32)),
        _p(np.ascontiguousarray(expanded_to_permuted, np.int32)), N, E, K, R, B, tp, capacity,
        NvS, *[_p(getattr(out, f)) for f in ("group_tokens", "z", "alloc", "alloc_cumsum",
                                              "experts_to_copy", "remote_stats", "cu_seqlens",
                                              "zero_fill", "expert_offsets", "dst")])
    if rc != 0:
        raise ValueError("oracle_plan_balanced failed (code %d)" % rc)
    return out


@dataclass
class Plan:
    is_token_in_rank: np.ndarray
    num_tokens_per_rank: np.ndarray
    num_tokens_per_expert: np.ndarray
    rank_prefix_matrix: np.ndarray
    channel_prefix_matrix: np.ndarray
    recv_tokens: np.ndarray
    recv_cu_seqlens: np.ndarray
    recv_zero_fill: np.ndarray
    dst: np.ndarray
    dup_counts: np.ndarray
    dup_offsets: np.ndarray
    dup_groups: np.ndarray
    dup_loffs: np.ndarray


def plan(ids: np.ndarray, cu_seqlens: np.ndarray, expanded_to_permuted: np.ndarray, E: int,
         R: int, num_src: int, num_channels: int, NvS: int) -> Plan:
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    N, K = ids.shape
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    e2p = np.ascontiguousarray(expanded_to_permuted, dtype=np.int32)
    S, C = num_src, num_channels
    epn = E // R
    itr = np.empty((N, R), np.uint8)
    ntpr = np.empty((S, R), np.int32)
    ntpe = np.empty((S, E), np.int32)
    rpm = np.empty((S, R), np.int32)
    cpm = np.empty((S, R, C), np.int32)
    rt = np.empty(R, np.int32)
    rcu = np.empty((R, epn + 1), np.int32)
    rzf = np.empty((E, 2), np.int32)
    dst = np.empty(N * K, np.int32)
    dc = np.empty((R, 2), np.int32)
    do = np.empty((R + 1, 2), np.int32)
    cap_g = max(N * (K // 2), 1)
    cap_d = max(N * (K - 1), 1)
    dg = np.empty((cap_g, 3), np.int32)
    dl = np.empty(cap_d, np.int32)
    rc = lib().oracle_plan(_p(ids), _p(cu), _p(e2p), N, E, K, R, S, C, NvS,
                           _p(itr), _p(ntpr), _p(ntpe), _p(rpm), _p(cpm), _p(rt), _p(rcu),
                           _p(rzf), _p(dst), _p(dc), _p(do), _p(dg), cap_g, _p(dl), cap_d)
    if rc != 0:
        raise ValueError("oracle_plan failed (code %d)" % rc)
    G, D = int(do[R, 0]), int(do[R, 1])
    return Plan(itr, ntpr, ntpe, rpm, cpm, rt, rcu, rzf, dst, dc, do, dg[:G].copy(), dl[:D].copy())
