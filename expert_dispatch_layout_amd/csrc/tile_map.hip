// mep_tile_map: the grouped-GEMM tile maps of a per-expert histogram -- for every A-row tile of
// the padded permuted rows, the expert it belongs to and the end of that expert's real rows
// inside it (TensorRT-LLM RoutingKernel.cuh, routingPermutation and routingIndicesOffsetsKernel:
// the per-expert CTA bookkeeping between the histogram and the permutation).
//
// One kernel.  Every workgroup rebuilds the tile offsets itself (E <= 1024 counts, read once per
// workgroup and served from L2 after the first): tiles per expert ceil(count/A) go through a
// workgroup-wide exclusive scan in LDS.  The tile entries are then written one thread per tile,
// grid-strided, so the stores of a wave cover consecutive addresses whatever the expert sizes;
// each thread finds its tile's expert by binary search over the LDS offsets.  The pages instead
// give each expert's tiles to the thread that owns the expert, which serialises a hot expert.
#include <limits.h>

#include "host_common.h"

namespace mep {

namespace {

constexpr int kTmBlock = 256;
constexpr int kTmWaves = kTmBlock / 64;
constexpr int kTmMaxExperts = 1024;
constexpr int kTmPerThread = kTmMaxExperts / kTmBlock;
constexpr int kTmMaxGrid = 1024;

__global__ __launch_bounds__(kTmBlock) void tile_map_kernel(const int32_t* __restrict__ counts, int E,
                                                           int A, int32_t* __restrict__ cta_to_expert,
                                                           int32_t* __restrict__ mn_limit, int cap,
                                                           int32_t* __restrict__ permuted_idx_size,
                                                           int32_t* __restrict__ num_ctas) {
    __shared__ int s_off[kTmMaxExperts + 1];  // exclusive tile offsets, then the total
    __shared__ int s_cnt[kTmMaxExperts];
    __shared__ int s_wave[kTmWaves];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;

    // tiles of each expert; a thread owns kTmPerThread consecutive experts for the scan
    int tiles[kTmPerThread];
    int mine = 0;
#pragma unroll
    for (int i = 0; i < kTmPerThread; ++i) {
        const int e = tid * kTmPerThread + i;
        int c = e < E ? counts[e] : 0;
        c = c > 0 ? c : 0;
        if (e < E) s_cnt[e] = c;
        tiles[i] = c / A + (c % A != 0 ? 1 : 0);
        mine += tiles[i];
    }
    // wave-inclusive scan of the per-thread sums, then across the waves
    int incl = mine;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d, 64);
        if (lane >= d) incl += y;
    }
    if (lane == 63) s_wave[wv] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kTmWaves; ++w) {
        const int s = s_wave[w];
        before += w < wv ? s : 0;
        total += s;
    }
    int run = before + incl - mine;
#pragma unroll
    for (int i = 0; i < kTmPerThread; ++i) {
        const int e = tid * kTmPerThread + i;
        if (e < E) s_off[e] = run;
        run += tiles[i];
    }
    if (tid == 0) s_off[E] = total;
    __syncthreads();

    if (blockIdx.x == 0 && tid == 0) {
        if (permuted_idx_size) permuted_idx_size[0] = total * A;
        if (num_ctas) num_ctas[0] = total;
    }
    const int n = total < cap ? total : cap;
    for (int j = blockIdx.x * kTmBlock + tid; j < n; j += gridDim.x * kTmBlock) {
        // s_off[lo] <= j < s_off[hi]; ends with hi == lo + 1, so expert lo owns tile j (an empty
        // expert never satisfies both bounds)
        int lo = 0, hi = E;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_off[mid] <= j) lo = mid;
            else hi = mid;
        }
        if (cta_to_expert) cta_to_expert[j] = lo;
        if (mn_limit) {
            const int lim1 = (j + 1) * A;
            const int lim2 = s_off[lo] * A + s_cnt[lo];
            mn_limit[j] = lim1 < lim2 ? lim1 : lim2;
        }
    }
}

}  // namespace

}  // namespace mep

extern "C" int mep_tile_map(const int32_t* tokens_per_expert, int E, int64_t num_slots, int tile,
                            int32_t* cta_to_expert, int32_t* cta_mn_limit, int64_t cap_ctas,
                            int32_t* permuted_idx_size, int32_t* num_ctas, void* stream) {
    mep::launch_begin();
    using namespace mep;
    if (!tokens_per_expert || E < 1 || tile < 1 || num_slots < 0 || cap_ctas < 0)
        return MEP_ERR_INVALID_ARG;
    const void* ptrs[] = {tokens_per_expert, cta_to_expert, cta_mn_limit, permuted_idx_size, num_ctas};
    for (const void* q : ptrs)
        if (q && !aligned(q, 4)) return MEP_ERR_INVALID_ARG;
    if (E > kTmMaxExperts) return MEP_ERR_UNSUPPORTED;
    const int64_t nz = num_slots < E ? num_slots : (int64_t)E;
    const int64_t rows = num_slots + nz * (int64_t)(tile - 1);  // padded rows, at most
    if (rows > INT32_MAX - (1 << 16)) return MEP_ERR_UNSUPPORTED;
    const int64_t bound = rows / tile;  // tiles, at most
    if ((cta_to_expert || cta_mn_limit) && cap_ctas < bound) return MEP_ERR_CAPACITY;
    if (!cta_to_expert && !cta_mn_limit && !permuted_idx_size && !num_ctas) return MEP_OK;
    const int64_t cap = (cta_to_expert || cta_mn_limit) ? bound : 0;
    int64_t grid = ceil_div64(cap, kTmBlock);
    if (grid > kTmMaxGrid) grid = kTmMaxGrid;
    if (grid < 1) grid = 1;
    launch_ggl(tile_map_kernel, dim3((unsigned)grid), dim3(kTmBlock), 0,
                       reinterpret_cast<hipStream_t>(stream), tokens_per_expert, E, tile, cta_to_expert,
                       cta_mn_limit, (int)cap, permuted_idx_size, num_ctas);
    return launch_status();
}
