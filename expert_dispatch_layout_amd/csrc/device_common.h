// Device-side helpers shared by the routing, layout and plan kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mep {

constexpr int kWave = 64;

// Order-preserving map from binary32 to uint32 (larger float -> larger integer).
// -0 is folded onto +0 so that a signed-zero pair compares equal and is decided by index.
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float order_key_inv(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

// Lanes below the calling lane in the wave.
__device__ __forceinline__ uint64_t lanes_below() { return (1ull << __lane_id()) - 1ull; }

__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

// Relaxed device-scope 64-bit status word access for cross-workgroup look-back.  The value is
// carried inside the word, so no other data needs release/acquire ordering.
__device__ __forceinline__ void status_store(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t status_load(const uint64_t* p) {
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr uint32_t kLookbackSpinLimit = 1u << 22;

// Status word: high 32 bits = (epoch << 1) | inclusive_flag, low 32 bits = value.
__device__ __forceinline__ uint64_t status_make(uint32_t epoch, bool inclusive, uint32_t value) {
    return ((uint64_t)((epoch << 1) | (inclusive ? 1u : 0u)) << 32) | (uint64_t)value;
}

// Decoupled look-back for one column: publish this tile's aggregate, walk predecessors until an
// inclusive prefix is found, then publish this tile's inclusive prefix.  Tiles are numbered in
// the order their workgroups started (atomic ticket), so every awaited predecessor is resident.
// Returns the exclusive prefix of the column before this tile.
__device__ __forceinline__ uint32_t lookback_column(uint64_t* status, int tile, int ncols, int col,
                                                    uint32_t epoch, uint32_t aggregate) {
    uint64_t* mine = status + (size_t)tile * ncols + col;
    if (tile == 0) {
        status_store(mine, status_make(epoch, true, aggregate));
        return 0u;
    }
    status_store(mine, status_make(epoch, false, aggregate));
    uint32_t excl = 0;
    int p = tile - 1;
    uint32_t spins = 0;
    while (p >= 0) {
        uint64_t w = status_load(status + (size_t)p * ncols + col);
        uint32_t hi = (uint32_t)(w >> 32);
        if ((hi >> 1) != (epoch & 0x7FFFFFFFu)) {
            // A predecessor always publishes; the bound only guarantees that a misused
            // workspace (two calls sharing it at once) ends in wrong values, never in a hang.
            if (++spins > kLookbackSpinLimit) break;
            __builtin_amdgcn_s_sleep(1);
            continue;
        }
        excl += (uint32_t)w;
        if (hi & 1u) break;
        --p;
    }
    status_store(mine, status_make(epoch, true, excl + aggregate));
    return excl;
}

__device__ __forceinline__ uint32_t status_value(const uint64_t* status, int tile, int ncols, int col) {
    return (uint32_t)(status[(size_t)tile * ncols + col]);
}

// Workspace header shared by the layout and plan calls (first 256 bytes of the workspace).
struct WsHeader {
    uint32_t epoch;   // epoch of the last completed call
    uint32_t ticket;  // tile ticket counter, reset to 0 by the consuming kernel
    uint32_t pad[62];
};
static_assert(sizeof(WsHeader) == 256, "header is 256 bytes");

// Tile number in start order.  The counter is zero at the first launch (zero-filled workspace)
// and is reset by the consuming kernel of every call; the modulo only keeps a misused workspace
// in bounds.
__device__ __forceinline__ int take_ticket(WsHeader* h, int ntiles) {
    const uint32_t t = __hip_atomic_fetch_add(&h->ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return (int)(t % (uint32_t)ntiles);
}

// Stable rank of each lane's key among the lanes of this wave that share it:
// returns the mask of lanes holding the same key (restricted to `active`).
__device__ __forceinline__ uint64_t match_peers(uint32_t key, int nbits, uint64_t active) {
    uint64_t peers = active;
    for (int b = 0; b < nbits; ++b) {
        uint64_t ones = __ballot((key >> b) & 1u);
        peers &= ((key >> b) & 1u) ? ones : ~ones;
    }
    return peers;
}

}  // namespace mep

namespace mep {

// Exclusive scan of one int per thread over a block of NT threads (NT a multiple of 64).
// `s_tmp` needs NT/64 ints of shared memory.  Ends with a barrier so `s_tmp` can be reused.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_tmp, int& total) {
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    if (lane == 63) s_tmp[w] = incl;
    __syncthreads();
    int off = 0;
    total = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
        const int x = s_tmp[i];
        if (i < w) off += x;
        total += x;
    }
    __syncthreads();
    return off + incl - v;
}

__host__ __device__ constexpr int bits_for(int n_keys) {
    int b = 0;
    while ((1 << b) < n_keys) ++b;
    return b;
}

}  // namespace mep
