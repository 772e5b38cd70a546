// Plan tiles of the fused layout + plan path: geometry, workspace, and the counting epilogue.
//
// Columns of a histogram row (NC = E + 3R), per token of the tile:
//   [0, E)        slots routed to expert e                        (the layout's histogram:
//                                                                   TensorRT-LLM RoutingKernel.cuh
//                                                                   routingIndicesHistogramKernel)
//   E + r         1 if the token sends anything to rank r          (is_token_in_rank, counted and
//                                                                   prefixed by DeepEP intranode.cu
//                                                                   notify_dispatch)
//   E + R + r     1 if the token sends >= 2 slots to rank r        (one dedup group)
//   E + 2R + r    slots to rank r beyond the first                 (duplicates, which MoonEP
//                                                                   planning.py encodes as -dst-1)
//
// Geometry.  A shard of n tokens is cut into plan tiles of T tokens (T*K <= 4096 slots, and for
// small batches fewer tokens, so that there are about 256 tiles); a counting workgroup owns
// `sub` consecutive plan tiles, which are consecutive tokens.  Counting workgroups form groups
// of GW.
//
// Epilogue of a counting workgroup, once its LDS rows are complete (it waits for no other
// workgroup):
//   - the within-workgroup exclusive prefix of every tile row -> tpre, and the workgroup's total
//     row -> wrow (plain stores);
//   - the total row added to its group's sum row (relaxed device atomics that return nothing).
// The plan-tile kernel then forms, after the kernel boundary, the exclusive prefix of any column
// before plan tile j as (sum rows of the earlier groups) + (total rows of the earlier workgroups
// of its group) + tpre[j], and the totals as the sum of every group row.  That is a two-level
// version of the reduce-then-scan prefix (per-tile reduction, a scan of the reductions, per-tile
// offsets), with the scan redone by every plan tile from at most ng + GW rows instead of a
// serial pass.  The group sums alternate between two buffers by the parity of the workspace's
// call counter: the counting kernel adds into one and clears the other (the previous call's), so
// during the plan-tile kernel one buffer holds this call's sums and the other is zero, and their
// sum is read without knowing which is which; the plan-tile kernel advances the counter.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mep.h"
#include "calls.h"
#include "device_common.h"
#include "host_common.h"

namespace mep {

constexpr int kPathMaxE = 512;
constexpr int kPathMaxR = 32;
constexpr int kPathMaxK = 8;
constexpr int kPathMaxNC = kPathMaxE + 3 * kPathMaxR;
constexpr int kPathSlots = 4096;    // slots of a plan tile, at most
constexpr int kPathTokens = 1024;   // tokens of a plan tile, at most
constexpr int kPathMinTileTokens = 64;  // tokens of a plan tile, at least (unless a shard is smaller)
constexpr int kPathMaxSub = 8;      // plan tiles per counting workgroup, at most
constexpr int kPathUnits = 256;     // compute units of an MI355X: counting workgroups aimed at
constexpr int kPathMaxGroups = 64;  // groups of counting workgroups, at most
// One buffer of group sums (the largest geometry), two of them right after the workspace
// header; every plan workspace reserves them, so no other kernel ever writes there.
constexpr size_t kPathGsumWords = (size_t)kPathMaxGroups * kPathMaxNC;
constexpr size_t kPathGsumBytes = 2 * kPathGsumWords * sizeof(uint32_t);

struct PathGeom {
    int N, E, K, R, epn, S, n, C, A;
    int eshift;  // log2(epn) when epn is a power of two, else -1
    int ashift;  // log2(A) when A is a power of two, else -1
    int T;       // tokens per plan tile
    int tps;     // plan tiles per shard
    int ntiles;  // plan tiles
    int NC;      // histogram columns
    int NCs;     // row stride of the histogram rows in the workspace (NC rounded up to 4 words)
    int sub;     // plan tiles per counting workgroup
    int nwg;     // counting workgroups
    int GW;      // counting workgroups per group
    int ng;      // groups
    int64_t NvS;
};

__host__ __device__ __forceinline__ int path_col_c0(const PathGeom& g, int r) { return g.E + r; }
__host__ __device__ __forceinline__ int path_col_c1(const PathGeom& g, int r) { return g.E + g.R + r; }
__host__ __device__ __forceinline__ int path_col_c2(const PathGeom& g, int r) { return g.E + 2 * g.R + r; }

// Tokens [t0, t1) of plan tile j.
__host__ __device__ __forceinline__ void path_tile_tokens(const PathGeom& g, int j, int64_t& t0, int64_t& t1) {
    const int sh = j / g.tps;
    const int l = j - sh * g.tps;
    t0 = (int64_t)sh * g.n + (int64_t)l * g.T;
    const int64_t e = (int64_t)(l + 1) * g.T;
    t1 = (int64_t)sh * g.n + (e < g.n ? e : (int64_t)g.n);
}

// Workspace views.
struct PathWs {
    uint32_t* gsum;  // [2][kPathGsumWords]: group sum rows [ng][NCs] of the two parities
    uint32_t* wrow;  // [nwg][NCs] counting-workgroup totals
    uint32_t* tpre;  // [ntiles][NCs] exclusive prefix within the counting workgroup
};

// Outputs of the layout and the plan (device pointers; NULL skips an optional one).  For
// mep_plan, whose layout is an input, the layout outputs are NULL and cu_in / p_in point to
// the given cu_seqlens and expanded_to_permuted, which the plan then uses (NULL otherwise: the
// plan-tile kernel forms them itself).
struct PathOut {
    int32_t* tokens_per_expert;
    int32_t* cu_seqlens;
    int32_t* e2p;
    int32_t* p2e;
    int32_t* zero_fill;
    PlanOutDev p;
    const int32_t* cu_in;
    const int32_t* p_in;
};

// The counting kernel's view of the call counter: its parity names the buffer the group sums go
// to; the plan-tile kernel advances the counter.
__device__ __forceinline__ uint32_t path_count_begin(WsHeader* hdr) {
    return __hip_atomic_load(&gptr(hdr)->pcall, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Epilogue of counting workgroup blockIdx.x: s_row holds its nsub tile rows (c2 not yet
// formed).  Every thread calls it; nothing waits for another workgroup.
template <int NT>
__device__ __forceinline__ void path_epilogue(const PathGeom& g, const PathWs& w, uint32_t pcall, int* s_row) {
    const int tid = threadIdx.x;
    const int b = blockIdx.x;
    const int j0 = b * g.sub;
    const int nsub = min(g.sub, g.ntiles - j0);
    const int NC = g.NC, NCs = g.NCs, R = g.R;
    __syncthreads();
    // duplicates per rank = slots on the rank (its experts' counts) - tokens on the rank: a wave
    // per (tile, rank), a lane per expert, then a sum over the wave
    {
        const int wv = tid >> 6, lane = tid & 63;
        for (int p = wv; p < nsub * R; p += NT / 64) {
            const int i = p / R, r = p - (p / R) * R;
            int* row = s_row + i * NC;
            int s = 0;
            for (int e = r * g.epn + lane; e < (r + 1) * g.epn; e += 64) s += row[e];
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
            if (lane == 0) row[path_col_c2(g, r)] = s - row[path_col_c0(g, r)];
        }
    }
    __syncthreads();
    // this workgroup's share of clearing the other parity's buffer (the previous call's sums)
    {
        MEP_GLOBAL uint32_t* other = gptr(w.gsum) + ((pcall + 1u) & 1u) * kPathGsumWords;
        const size_t per = (kPathGsumWords + g.nwg - 1) / g.nwg;
        const size_t lo = (size_t)b * per;
        const size_t hi = lo + per < kPathGsumWords ? lo + per : kPathGsumWords;
        for (size_t i = lo + tid; i < hi; i += NT) other[i] = 0u;
    }
    MEP_GLOBAL uint32_t* gs = gptr(w.gsum) + (pcall & 1u) * kPathGsumWords + (size_t)(b / g.GW) * NCs;
    for (int c = tid; c < NC; c += NT) {
        uint32_t run = 0;
        for (int i = 0; i < nsub; ++i) {
            gptr(w.tpre)[(size_t)(j0 + i) * NCs + c] = run;
            run += (uint32_t)s_row[i * NC + c];
        }
        gptr(w.wrow)[(size_t)b * NCs + c] = run;
        if (run != 0u) __hip_atomic_fetch_add(gs + c, run, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Adds one token's rank columns to histogram row `row` (LDS) from its rank masks m1 (ranks
// reached) and m2 (ranks reached by >= 2 slots), combined over the token's lanes beforehand;
// `rank_lane` / `rank_lanes` split the rank bits between the token's lanes (each rank counted
// by one lane).
__device__ __forceinline__ void path_count_ranks(const PathGeom& g, int* row, uint32_t m1, uint32_t m2,
                                                 int rank_lane, int rank_lanes) {
    uint32_t mine = 0;
    for (int r = rank_lane; r < g.R; r += rank_lanes) mine |= 1u << r;
    uint32_t a = m1 & mine;
    while (a) {
        const int r = __builtin_ctz(a);
        a &= a - 1u;
        atomicAdd(&row[path_col_c0(g, r)], 1);
        if ((m2 >> r) & 1u) atomicAdd(&row[path_col_c1(g, r)], 1);
    }
}

// Counts one routed token into histogram row `row` (LDS): the token's slots are held by its
// segment of LPT lanes, KPL per lane (-1 where there is none); expert columns by LDS atomics,
// then the rank columns from the rank masks combined over the segment.
template <int LPT, int KPL>
__device__ __forceinline__ void path_count_token(const PathGeom& g, int* row, const int (&e)[KPL], int lseg) {
    uint32_t m1 = 0u, m2 = 0u;
#pragma unroll
    for (int q = 0; q < KPL; ++q) {
        if (e[q] >= 0) {
            atomicAdd(&row[e[q]], 1);
            const int r = g.eshift >= 0 ? e[q] >> g.eshift : e[q] / g.epn;
            const uint32_t bit = 1u << r;
            m2 |= m1 & bit;
            m1 |= bit;
        }
    }
    auto step = [&](auto partner) {
        const uint32_t b1 = partner(m1), b2 = partner(m2);
        m2 = m2 | b2 | (m1 & b1);
        m1 = m1 | b1;
    };
    if constexpr (LPT >= 2) step([](uint32_t u) { return seg_partner_u32<1>(u); });
    if constexpr (LPT >= 4) step([](uint32_t u) { return seg_partner_u32<2>(u); });
    if constexpr (LPT >= 8) step([](uint32_t u) { return seg_partner_u32<4>(u); });
    if constexpr (LPT >= 16) step([](uint32_t u) { return seg_partner_u32<8>(u); });
    if constexpr (LPT >= 32) step([](uint32_t u) { return seg_partner_u32<16>(u); });
    if constexpr (LPT >= 64) step([](uint32_t u) { return seg_partner_u32<32>(u); });
    path_count_ranks(g, row, m1, m2, lseg, LPT);
}

// (m1, m2) of two lane shares combined: ranks reached, and ranks reached twice or more.
__device__ __forceinline__ void path_mask_merge(uint32_t& m1, uint32_t& m2, uint32_t b1, uint32_t b2) {
    m2 = m2 | b2 | (m1 & b1);
    m1 = m1 | b1;
}

// Host: geometry of the path for a batch (sub chosen so that about kPathUnits counting
// workgroups exist).
PathGeom path_geom(int64_t N, int E, int K, int R, int S, int C, int A, int64_t NvS);

struct PathWsLayout {
    size_t gsum, wrow, tpre, bytes;
};
PathWsLayout path_ws_layout(const PathGeom& g);
PathWs path_ws_views(void* ws, const PathGeom& g);

// True when the fused path covers the shape (K <= 8, R <= 32, E <= 512, N > 0).
bool path_supported(int64_t N, int E, int K, int R);
// Workspace bytes of the fused path (0 when it does not cover the shape).
size_t path_workspace_bytes(int64_t N, int E, int K, int R, int S);

// One call of the fused path: geometry, workspace views, outputs, ids.
struct PathCall {
    PathGeom g;
    PathWs w;
    WsHeader* hdr;
    PathOut o;
    const int32_t* ids;
};
PathCall path_call(const LayoutCall& lc, const PlanCall& pc, void* ws);
// mep_plan on the plan-tile path: the layout comes in (cu_seqlens, expanded_to_permuted of
// alignment A), only the plan goes out.
PathCall path_call_plan(const PlanCall& pc, const int32_t* cu_seqlens, const int32_t* e2p, int A, void* ws);
// The counting kernel over the ids (when the routing kernel did not count), then the plan-tile
// kernel (optionally stamped with start / stop events by its launch).
void path_launch_count(const PathCall& c, hipStream_t st);
void path_launch_plan(const PathCall& c, hipStream_t st, hipEvent_t start, hipEvent_t stop);

}  // namespace mep
