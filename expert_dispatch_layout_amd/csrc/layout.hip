// mep_build_layout: per-expert histogram, padded exclusive scan and the stable
// expanded <-> permuted maps of the N*K routed slots.
//
// Two kernels.  Scatter tiles are 4096 consecutive slots; a count tile groups enough of them that
// at most about 32 count tiles exist:
//
//   count   LDS-privatised histograms (one LDS atomic per slot, no global atomics), one per
//           scatter tile, written to the workspace; the last tile of a count tile (at most 32
//           of them) to arrive sums them and stores the count tile's totals, and the last count
//           tile to do so turns every expert column into inclusive prefixes over count tiles.
//           No workgroup waits for another.
//   scatter every tile reads the per-expert totals (last tile's inclusive prefix), forms the
//           padded offsets cu_seqlens (ceil(count/A)*A, 0 for an empty expert: MoonEP
//           planning.py Phase B2 padded group scan), and ranks its slots stably: within a wave
//           the slots sharing an expert are found with one ballot per id bit (a wave64 stand-in
//           for a warp match), counted per (wave, expert) in LDS and prefixed across waves --
//           the same order MoonEP planning.py run_c1 passA produces, so the permutation is
//           deterministic and stable in slot order.  The inverse is staged in LDS in expert
//           order, so each expert's run of the tile is written as consecutive addresses.
//
// The inverse holds the slot index t*K+k; padding rows hold -1 (MoonEP's empty-slot sentinel).
#include <limits.h>

#include "device_common.h"
#include "host_common.h"
#include "calls.h"
#include "layout_scatter.h"

namespace mep {

constexpr int kCountBlock = 1024;
constexpr int kCountTiles = 32;                      // count tiles at most
constexpr int kMaxCountTiles = 4096;  // arrival counters kept in the workspace
static_assert(kCountTiles <= kDirectCountTiles, "the last layout count tile scans them all");

static LayGeom lay_geom(int64_t NK, int E) {
    LayGeom g;
    g.NK = (int)NK;
    g.E = E;
    g.nsub = (int)ceil_div64(NK, kLayTile);
    int sub = (int)ceil_div64(g.nsub, kCountTiles);
    if (sub < 1) sub = 1;
    g.sub = sub;
    g.nct = (int)ceil_div64(g.nsub, sub);  // <= kCountTiles
    return g;
}


// One tile per workgroup: LDS-privatised histogram (one LDS atomic per slot), written to the
// workspace; the last tile of a count tile to arrive sums the count tile's histograms and stores
// the count tile's totals; the last count tile to finish scans them.
__global__ __launch_bounds__(kCountBlock) void layout_count_kernel(const int32_t* __restrict__ ids,
                                                                   LayGeom g, LayWs w, WsHeader* hdr) {
    __shared__ int hist[kMaxExperts];
    __shared__ uint32_t s_arrived;
    const int tid = threadIdx.x;
    const int E = g.E;
    for (int i = tid; i < E; i += kCountBlock) hist[i] = 0;
    __syncthreads();
    const int tile = blockIdx.x;
    const uint32_t epoch = __hip_atomic_load(&gptr(hdr)->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    const int base = tile * kLayTile;
    const MEP_GLOBAL int32_t* gids = gptr(ids);
    constexpr int kPer = kLayTile / kCountBlock;
    int v[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int i = base + j * kCountBlock + tid;
        v[j] = i < g.NK ? gids[i] : -1;
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j)
        if ((unsigned)v[j] < (unsigned)E) atomicAdd(&hist[v[j]], 1);  // out-of-range ids are skipped
    __syncthreads();
    const uint32_t want = status_tag(epoch);
    for (int e = tid; e < E; e += kCountBlock)
        status_store(w.tilehist + (size_t)tile * E + e, status_make(epoch, false, (uint32_t)hist[e]));
    // ---- arrival at the count tile; the last arriver continues ------------------------------
    const int ct = tile / g.sub;
    const int t0 = ct * g.sub;
    const int nsub_here = min(g.sub, g.nsub - t0);
    __syncthreads();
    if (tid == 0)
        s_arrived = __hip_atomic_fetch_add(gptr(w.arrive) + ct, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_arrived != (uint32_t)(nsub_here - 1)) return;
    if (tid == 0) __hip_atomic_store(gptr(w.arrive) + ct, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int e = tid; e < E; e += kCountBlock) {
        uint32_t agg = 0;
        for (int b0 = 0; b0 < nsub_here; b0 += 8) {
            uint64_t x[8];
#pragma unroll
            for (int b = 0; b < 8; ++b)
                x[b] = b0 + b < nsub_here ? status_load(w.tilehist + (size_t)(t0 + b0 + b) * E + e) : 0;
#pragma unroll
            for (int b = 0; b < 8; ++b)
                if (b0 + b < nsub_here) agg += tagged_value(w.tilehist + (size_t)(t0 + b0 + b) * E + e, x[b], want, &hdr->err);
        }
        status_store(w.status + (size_t)ct * E + e, status_make(epoch, false, agg));
    }
    if (last_count_tile(hdr, g.nct, &s_arrived))
        for (int e = tid; e < E; e += kCountBlock) scan_count_column(w.status, g.nct, E, e, epoch, &hdr->err);
}


template <int NB>
__global__ __launch_bounds__(kScatBlock) void layout_scatter_kernel(const int32_t* __restrict__ ids, int E,
                                                                    int A, ScatterSrc src, WsHeader* hdr,
                                                                    LayoutOut out) {
    __shared__ int s_cu[kMaxExperts + 1];
    __shared__ int s_tot[kMaxExperts];
    __shared__ int s_base[kMaxExperts];
    __shared__ int s_loc[kMaxExperts];
    __shared__ int s_cnt[kScatWaves][kMaxExperts];
    __shared__ int s_tmp[kScatWaves];
    __shared__ int s_slot[kLayTile];
    __shared__ int s_pos[kLayTile];
    const ScatterLds L{s_cu, s_tot, s_base, s_loc, s_cnt, s_tmp, s_slot, s_pos};
    scatter_tile<NB>(ids, E, A, src, hdr, out, L, nullptr, nullptr);
}

}  // namespace mep

namespace mep {
// Workspace of mep_build_layout: header, arrival counters, look-back words, tile histograms.
struct LayWsLayout {
    size_t arrive, status, tilehist, bytes;
};
static LayWsLayout lay_ws_layout(const LayGeom& g) {
    LayWsLayout l;
    l.arrive = sizeof(WsHeader);
    l.status = l.arrive + align256((size_t)kMaxCountTiles * sizeof(uint32_t));
    l.tilehist = l.status + align256((size_t)g.nct * (size_t)g.E * sizeof(uint64_t));
    l.bytes = l.tilehist + align256((size_t)g.nsub * (size_t)g.E * sizeof(uint64_t));
    return l;
}
}  // namespace mep

extern "C" size_t mep_layout_workspace_size(int64_t N, int E, int K) {
    using namespace mep;
    if (N < 0 || E < 1 || K < 1 || E > kMaxExperts) return sizeof(WsHeader);
    return lay_ws_layout(lay_geom(N * (int64_t)K, E)).bytes;
}

namespace mep {

// Checks of mep_build_layout's ids and outputs, and the launch arguments that do not involve
// its workspace; MEP_OK or the error code.
int layout_prepare_outputs(const int32_t* topk_ids, int64_t N, int E, int K, int alignment,
                           int32_t* tokens_per_expert, int32_t* cu_seqlens, int32_t* expanded_to_permuted,
                           int32_t* permuted_to_expanded, int64_t permuted_cap, int32_t* zero_fill,
                           LayoutCall& c) {
    if (!cu_seqlens) return MEP_ERR_INVALID_ARG;
    if (N > 0 && (!topk_ids || !expanded_to_permuted)) return MEP_ERR_INVALID_ARG;  // N == 0 reads nothing
    if (N < 0 || E < 1 || K < 1 || alignment < 1) return MEP_ERR_INVALID_ARG;
    const void* ptrs[] = {topk_ids, tokens_per_expert, cu_seqlens, expanded_to_permuted,
                          permuted_to_expanded, zero_fill};
    for (const void* q : ptrs)
        if (q && !aligned(q, 4)) return MEP_ERR_INVALID_ARG;
    if (E > kMaxExperts || K > 32 || K > E) return MEP_ERR_UNSUPPORTED;
    const int64_t NK = N * (int64_t)K;
    const int64_t bound = NK + (NK < E ? NK : (int64_t)E) * (int64_t)(alignment - 1);
    if (bound > INT32_MAX - (1 << 16)) return MEP_ERR_UNSUPPORTED;
    if (permuted_to_expanded && permuted_cap < bound) return MEP_ERR_CAPACITY;
    c.g = lay_geom(NK, E);
    c.ids = topk_ids;
    c.A = alignment;
    c.hdr = nullptr;
    c.lw = LayWs{nullptr, nullptr, nullptr};
    c.out = LayoutOut{tokens_per_expert, cu_seqlens, expanded_to_permuted, permuted_to_expanded, zero_fill,
                      permuted_to_expanded ? (int)(permuted_cap < INT32_MAX ? permuted_cap : INT32_MAX) : 0};
    return MEP_OK;
}

// All checks of mep_build_layout and its launch arguments.
int layout_prepare(const int32_t* topk_ids, int64_t N, int E, int K, int alignment,
                   int32_t* tokens_per_expert, int32_t* cu_seqlens, int32_t* expanded_to_permuted,
                   int32_t* permuted_to_expanded, int64_t permuted_cap, int32_t* zero_fill, void* ws,
                   size_t ws_bytes, LayoutCall& c) {
    if (!ws) return MEP_ERR_INVALID_ARG;
    const int rc = layout_prepare_outputs(topk_ids, N, E, K, alignment, tokens_per_expert, cu_seqlens,
                                          expanded_to_permuted, permuted_to_expanded, permuted_cap, zero_fill, c);
    if (rc != MEP_OK) return rc;
    if (!aligned(ws, 256)) return MEP_ERR_INVALID_ARG;
    if (ws_bytes < mep_layout_workspace_size(N, E, K)) return MEP_ERR_CAPACITY;
    c.hdr = reinterpret_cast<WsHeader*>(ws);
    const LayWsLayout wl = lay_ws_layout(c.g);
    char* wb = reinterpret_cast<char*>(ws);
    c.lw = LayWs{reinterpret_cast<uint32_t*>(wb + wl.arrive), reinterpret_cast<uint64_t*>(wb + wl.status),
                 reinterpret_cast<uint64_t*>(wb + wl.tilehist)};
    return MEP_OK;
}

static void launch_scatter(const LayoutCall& c, const ScatterSrc& src, int ntiles, WsHeader* hdr,
                           hipStream_t st) {
    const dim3 sgrid(ntiles > 0 ? ntiles : 1), sblock(kScatBlock);
    const int E = c.g.E;
    if (E <= 16)
        launch_ggl(layout_scatter_kernel<4>, sgrid, sblock, 0, st, c.ids, E, c.A, src, hdr, c.out);
    else if (E <= 64)
        launch_ggl(layout_scatter_kernel<6>, sgrid, sblock, 0, st, c.ids, E, c.A, src, hdr, c.out);
    else if (E <= 256)
        launch_ggl(layout_scatter_kernel<8>, sgrid, sblock, 0, st, c.ids, E, c.A, src, hdr, c.out);
    else
        launch_ggl(layout_scatter_kernel<10>, sgrid, sblock, 0, st, c.ids, E, c.A, src, hdr, c.out);
}

void layout_launch(const LayoutCall& c, hipStream_t st) {
    const LayGeom& g = c.g;
    if (g.nsub > 0)
        launch_ggl(layout_count_kernel, dim3(g.nsub), dim3(kCountBlock), 0, st, c.ids, g, c.lw, c.hdr);
    ScatterSrc src{};
    src.plan = 0;
    src.lg = g;
    src.lw = c.lw;
    launch_scatter(c, src, g.nsub, c.hdr, st);
}

void layout_launch_scatter_from_plan(const LayoutCall& lc, const PlanCall& pc, hipStream_t st) {
    ScatterSrc src{};
    src.plan = 1;
    src.pg = pc.g;
    src.pw = pc.pw;
    launch_scatter(lc, src, pc.g.ntiles, pc.hdr, st);
}

}  // namespace mep

extern "C" int mep_build_layout(const int32_t* topk_ids, int64_t N, int E, int K, int alignment,
                                int32_t* tokens_per_expert, int32_t* cu_seqlens,
                                int32_t* expanded_to_permuted, int32_t* permuted_to_expanded,
                                int64_t permuted_cap, int32_t* zero_fill, void* ws, size_t ws_bytes,
                                void* stream) {
    mep::launch_begin();
    using namespace mep;
    LayoutCall c;
    const int rc = layout_prepare(topk_ids, N, E, K, alignment, tokens_per_expert, cu_seqlens,
                                  expanded_to_permuted, permuted_to_expanded, permuted_cap, zero_fill, ws,
                                  ws_bytes, c);
    if (rc != MEP_OK) return rc;
    layout_launch(c, reinterpret_cast<hipStream_t>(stream));
    return launch_status();
}
