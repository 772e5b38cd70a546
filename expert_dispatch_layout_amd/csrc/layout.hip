// mep_build_layout: per-expert histogram, padded exclusive scan and the stable
// expanded <-> permuted maps of the N*K routed slots.
//
// Two kernels over tiles of 2048 consecutive slots:
//
//   count   LDS-privatised per-tile histogram (one LDS atomic per slot, no global atomics), then
//           a single-pass decoupled look-back per expert column (Merrill & Garland 2016) that
//           publishes each tile's inclusive per-expert prefix.  Tiles take an atomic ticket so
//           every awaited predecessor is already running.
//   scatter every tile reads the per-expert totals (last tile's inclusive prefix), forms the
//           padded offsets cu_seqlens (ceil(count/A)*A, 0 for an empty expert: MoonEP
//           planning.py Phase B2 padded group scan), and ranks its slots stably: within a wave
//           the slots sharing an expert are found with one ballot per id bit (a wave64 stand-in
//           for a warp match), counted per (wave, expert) in LDS and prefixed across waves --
//           the same order MoonEP planning.py run_c1 passA produces, so the permutation is
//           deterministic and stable in slot order.
//
// The inverse holds the slot index t*K+k; padding rows hold -1 (MoonEP's empty-slot sentinel).
#include <limits.h>

#include "device_common.h"
#include "host_common.h"

namespace mep {

constexpr int kLayBlock = 256;
constexpr int kLayPerThread = 8;
constexpr int kLayTile = kLayBlock * kLayPerThread;  // slots per tile
constexpr int kLayWaves = kLayBlock / kWave;
constexpr int kLayPerWave = kLayTile / kLayWaves;    // 512
constexpr int kMaxExperts = 1024;

__global__ __launch_bounds__(kLayBlock) void layout_count_kernel(const int32_t* __restrict__ ids,
                                                                 int NK, int E, uint64_t* status,
                                                                 WsHeader* hdr) {
    __shared__ int hist[kMaxExperts];
    __shared__ int s_tile;
    for (int e = threadIdx.x; e < E; e += kLayBlock) hist[e] = 0;
    if (threadIdx.x == 0) s_tile = take_ticket(hdr, (int)gridDim.x);
    __syncthreads();
    const int tile = s_tile;
    const uint32_t epoch = __hip_atomic_load(&hdr->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    const int base = tile * kLayTile;
#pragma unroll
    for (int it = 0; it < kLayPerThread; ++it) {
        const int i = base + it * kLayBlock + threadIdx.x;
        if (i < NK) {
            const int id = ids[i];
            if ((unsigned)id < (unsigned)E) atomicAdd(&hist[id], 1);  // out-of-range ids are skipped
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kLayBlock)
        lookback_column(status, tile, E, e, epoch, (uint32_t)hist[e]);
}

struct LayoutOut {
    int32_t* tokens_per_expert;
    int32_t* cu_seqlens;
    int32_t* e2p;
    int32_t* p2e;
    int32_t* zero_fill;
    int p2e_cap;
};

__global__ __launch_bounds__(kLayBlock) void layout_scatter_kernel(const int32_t* __restrict__ ids,
                                                                   int NK, int E, int A, int ntiles,
                                                                   const uint64_t* status,
                                                                   WsHeader* hdr, LayoutOut out) {
    __shared__ int s_cu[kMaxExperts + 1];
    __shared__ int s_tot[kMaxExperts];
    __shared__ int s_base[kMaxExperts];
    __shared__ int s_cnt[kLayWaves][kMaxExperts];
    __shared__ int s_tmp[kLayWaves];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int tile = blockIdx.x;

    // ---- padded offsets from the per-expert totals (4 experts per thread) ----------------
    int pad[4];
    int mysum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = tid * 4 + q;
        int tot = 0;
        if (e < E && ntiles > 0) tot = (int)status_value(status, ntiles - 1, E, e);
        if (e < E) s_tot[e] = tot;
        pad[q] = tot > 0 ? ((tot + A - 1) / A) * A : 0;
        mysum += pad[q];
    }
    int total;
    int run = block_exclusive_scan<kLayBlock>(mysum, s_tmp, total);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = tid * 4 + q;
        if (e < E) s_cu[e] = run;
        run += pad[q];
    }
    if (tid == 0) s_cu[E] = total;
    for (int e = tid; e < E; e += kLayBlock)
#pragma unroll
        for (int ww = 0; ww < kLayWaves; ++ww) s_cnt[ww][e] = 0;
    __syncthreads();
    for (int e = tid; e < E; e += kLayBlock)
        s_base[e] = s_cu[e] + ((tile > 0 && tile < ntiles) ? (int)status_value(status, tile - 1, E, e) : 0);

    // ---- stable in-tile ranks: wave match + per-(wave, expert) counters -----------------
    const int nbits = bits_for(E);
    const int wbase = tile * kLayTile + w * kLayPerWave;
    int key[kLayPerWave / kWave];
    int rank[kLayPerWave / kWave];
    if (tile < ntiles) {
#pragma unroll
        for (int it = 0; it < kLayPerWave / kWave; ++it) {
            const int i = wbase + it * kWave + lane;
            int k = i < NK ? ids[i] : 0;
            const bool valid = i < NK && (unsigned)k < (unsigned)E;
            if (!valid) k = 0;
            const uint64_t active = __ballot(valid);
            const uint64_t peers = match_peers((uint32_t)k, nbits, active);
            key[it] = valid ? k : -1;
            rank[it] = 0;
            if (valid) {
                const uint64_t below = peers & lanes_below();
                const int b = s_cnt[w][k];
                rank[it] = b + popc64(below);
                if (below == 0) s_cnt[w][k] = b + popc64(peers);
            }
        }
    }
    __syncthreads();
    for (int e = tid; e < E; e += kLayBlock) {
        int r = 0;
#pragma unroll
        for (int ww = 0; ww < kLayWaves; ++ww) {
            const int c = s_cnt[ww][e];
            s_cnt[ww][e] = r;
            r += c;
        }
    }
    __syncthreads();
    if (tile < ntiles) {
#pragma unroll
        for (int it = 0; it < kLayPerWave / kWave; ++it) {
            const int i = wbase + it * kWave + lane;
            const int k = key[it];
            if (k >= 0) {
                const int P = s_base[k] + s_cnt[w][k] + rank[it];
                out.e2p[i] = P;
                if (out.p2e && P < out.p2e_cap) out.p2e[P] = i;
            }
        }
    }

    // ---- padding rows of the inverse ------------------------------------------------------
    if (out.p2e) {
        for (int e = blockIdx.x; e < E; e += gridDim.x) {
            const int start = s_cu[e] + s_tot[e];
            const int end = min(s_cu[e + 1], out.p2e_cap);
            for (int p = start + tid; p < end; p += kLayBlock) out.p2e[p] = -1;
        }
    }

    // ---- per-expert outputs and workspace reset ------------------------------------------
    if (blockIdx.x == 0) {
        for (int e = tid; e <= E; e += kLayBlock) out.cu_seqlens[e] = s_cu[e];
        for (int e = tid; e < E; e += kLayBlock) {
            const int cnt = s_tot[e];
            if (out.tokens_per_expert) out.tokens_per_expert[e] = cnt;
            if (out.zero_fill) {
                const int padded = s_cu[e + 1] - s_cu[e];
                const bool z = cnt > 0 && padded > cnt;
                out.zero_fill[2 * e] = z ? s_cu[e] + cnt : 0;
                out.zero_fill[2 * e + 1] = z ? padded - cnt : 0;
            }
        }
        if (tid == 0) {
            hdr->epoch = hdr->epoch + 1u;
            hdr->ticket = 0u;
        }
    }
}

static int64_t layout_tiles(int64_t NK) { return ceil_div64(NK, kLayTile); }

}  // namespace mep

extern "C" size_t mep_layout_workspace_size(int64_t N, int E, int K) {
    using namespace mep;
    if (N < 0 || E < 1 || K < 1) return sizeof(WsHeader);
    return sizeof(WsHeader) + (size_t)layout_tiles(N * (int64_t)K) * (size_t)E * sizeof(uint64_t);
}

extern "C" int mep_build_layout(const int32_t* topk_ids, int64_t N, int E, int K, int alignment,
                                int32_t* tokens_per_expert, int32_t* cu_seqlens,
                                int32_t* expanded_to_permuted, int32_t* permuted_to_expanded,
                                int64_t permuted_cap, int32_t* zero_fill, void* ws, size_t ws_bytes,
                                void* stream) {
    using namespace mep;
    if (!cu_seqlens || !ws) return MEP_ERR_INVALID_ARG;
    if (N > 0 && (!topk_ids || !expanded_to_permuted)) return MEP_ERR_INVALID_ARG;  // N == 0 reads nothing
    if (N < 0 || E < 1 || K < 1 || alignment < 1) return MEP_ERR_INVALID_ARG;
    const void* ptrs[] = {topk_ids, tokens_per_expert, cu_seqlens, expanded_to_permuted,
                          permuted_to_expanded, zero_fill};
    for (const void* q : ptrs)
        if (q && !aligned(q, 4)) return MEP_ERR_INVALID_ARG;
    if (!aligned(ws, 256)) return MEP_ERR_INVALID_ARG;
    if (E > kMaxExperts || K > 32 || K > E) return MEP_ERR_UNSUPPORTED;
    const int64_t NK = N * (int64_t)K;
    const int64_t bound = NK + (NK < E ? NK : (int64_t)E) * (int64_t)(alignment - 1);
    if (bound > INT32_MAX - (1 << 16)) return MEP_ERR_UNSUPPORTED;
    if (permuted_to_expanded && permuted_cap < bound) return MEP_ERR_CAPACITY;
    if (ws_bytes < mep_layout_workspace_size(N, E, K)) return MEP_ERR_CAPACITY;

    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    WsHeader* hdr = reinterpret_cast<WsHeader*>(ws);
    uint64_t* status = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(ws) + sizeof(WsHeader));
    const int ntiles = (int)layout_tiles(NK);
    if (ntiles > 0)
        hipLaunchKernelGGL(layout_count_kernel, dim3(ntiles), dim3(kLayBlock), 0, st, topk_ids,
                           (int)NK, E, status, hdr);
    LayoutOut out{tokens_per_expert, cu_seqlens, expanded_to_permuted, permuted_to_expanded, zero_fill,
                  permuted_to_expanded ? (int)(permuted_cap < INT32_MAX ? permuted_cap : INT32_MAX) : 0};
    hipLaunchKernelGGL(layout_scatter_kernel, dim3(ntiles > 0 ? ntiles : 1), dim3(kLayBlock), 0, st,
                       topk_ids, (int)NK, E, alignment, ntiles, status, hdr, out);
    return launch_status();
}
