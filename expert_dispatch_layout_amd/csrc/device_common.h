// Device-side helpers shared by the routing, layout and plan kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mep {

constexpr int kWave = 64;

// Global-memory views of generic pointers.  Pointers that reach a kernel inside a struct are
// generic to the compiler, which then emits flat instructions; those count against the LDS
// counter as well, so every LDS wait would also wait for outstanding HBM loads.
#define MEP_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ const MEP_GLOBAL T* gptr(const T* p) {
    return (const MEP_GLOBAL T*)p;
}
template <typename T>
__device__ __forceinline__ MEP_GLOBAL T* gptr(T* p) {
    return (MEP_GLOBAL T*)p;
}

// Native 4 x 32-bit vector for 16-byte accesses: it loads from any address space and keeps
// register buffers in registers (HIP's uint4 is a struct with unions, which can defeat the
// promotion of a local array to registers).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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
    __hip_atomic_store(gptr(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t status_load(const uint64_t* p) {
    return __hip_atomic_load(gptr(const_cast<uint64_t*>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr uint32_t kLookbackSpinLimit = 1u << 22;

// Sticky error bit of the workspace header's word 3: a bounded wait ran out (only a misused
// workspace -- two calls on it at once -- can cause it; the values of that call are then wrong).
constexpr uint32_t kErrWaitLimit = 1u;

__device__ __forceinline__ void ws_raise(uint32_t* err, uint32_t bits) {
    if (err) __hip_atomic_fetch_or(gptr(err), bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Status word: high 32 bits = tag | inclusive_flag, low 32 bits = value.  The tag has bit 31 set
// and carries the low 30 bits of the call's epoch, so neither a zero-filled workspace nor the
// 32-bit counts that other calls with a different geometry store in the same bytes (always below
// 2^31) can pass for a status word of the current call.
__device__ __forceinline__ uint32_t status_tag(uint32_t epoch) {
    return 0x80000000u | ((epoch & 0x3FFFFFFFu) << 1);
}
__device__ __forceinline__ uint64_t status_make(uint32_t epoch, bool inclusive, uint32_t value) {
    return ((uint64_t)(status_tag(epoch) | (inclusive ? 1u : 0u)) << 32) | (uint64_t)value;
}

// Decoupled look-back for one column (Merrill & Garland, "Single-pass Parallel Prefix Scan with
// Decoupled Look-back", 2016): publish this tile's aggregate, walk predecessors until an inclusive
// prefix is found, then publish this tile's inclusive prefix.  The walk reads a window of kLbWin
// predecessors at once (independent loads in flight), consumes them nearest first, and stops at
// the first inclusive one; a predecessor that has not published yet is re-read after a short
// sleep.  Tiles are numbered in the order their workgroups started (atomic ticket), so every
// awaited predecessor is resident.  Returns the exclusive prefix of the column before this tile.
constexpr int kLbWin = 32;

__device__ __forceinline__ uint32_t lookback_column(uint64_t* status, int tile, int ncols, int col,
                                                    uint32_t epoch, uint32_t aggregate, uint32_t* err) {
    uint64_t* mine = status + (size_t)tile * ncols + col;
    if (tile == 0) {
        status_store(mine, status_make(epoch, true, aggregate));
        return 0u;
    }
    status_store(mine, status_make(epoch, false, aggregate));
    const uint32_t want = status_tag(epoch);
    uint32_t excl = 0;
    int p = tile - 1;
    uint32_t spins = 0;
    while (p >= 0) {
        uint64_t w[kLbWin];
#pragma unroll
        for (int i = 0; i < kLbWin; ++i)
            w[i] = (p - i >= 0) ? status_load(status + (size_t)(p - i) * ncols + col)
                                : status_make(epoch, true, 0u);
        int consumed = 0;
        bool done = false, stall = false;
#pragma unroll
        for (int i = 0; i < kLbWin; ++i) {
            const uint32_t hi = (uint32_t)(w[i] >> 32);
            const bool ready = (hi & ~1u) == want;
            const bool take = !done && !stall && ready;
            stall = stall || (!done && !ready);
            if (take) {
                excl += (uint32_t)w[i];
                consumed = i + 1;
                done = (hi & 1u) != 0u;
            }
        }
        if (done) break;
        p -= consumed;
        if (stall) {
            // A predecessor always publishes; the bound only guarantees that a misused workspace
            // (two calls sharing it at once) ends in wrong values, never in a hang.
            if (++spins > kLookbackSpinLimit) {
                ws_raise(err, kErrWaitLimit);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    status_store(mine, status_make(epoch, true, excl + aggregate));
    return excl;
}

__device__ __forceinline__ uint32_t status_value(const uint64_t* status, int tile, int ncols, int col) {
    return (uint32_t)(status[(size_t)tile * ncols + col]);
}

// Value of a tagged word written in this call, re-read until its tag is current (bounded: when
// the bound runs out, the error bit is raised in *err and the stale value is returned).
__device__ __forceinline__ uint32_t tagged_value(const uint64_t* p, uint64_t v, uint32_t want, uint32_t* err) {
    uint32_t spins = 0;
    while (((uint32_t)(v >> 32) & ~1u) != want) {
        if (++spins >= kLookbackSpinLimit) {
            ws_raise(err, kErrWaitLimit);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
        v = status_load(p);
    }
    return (uint32_t)v;
}

// Workspace header shared by the layout and plan calls (first 256 bytes of the workspace).
struct WsHeader {
    uint32_t epoch;    // epoch of the last completed call
    uint32_t ticket;   // tile ticket counter, reset to 0 by the consuming kernel
    uint32_t ct_done;  // count tiles whose totals are stored; reset to 0 by the last of them
    uint32_t err;      // sticky error bits (word 3): a bounded wait ran out, which only a misused
                       // workspace (two calls on it at once) can cause
    uint32_t pcall;    // calls of the fused path so far (its counting sums alternate between two
                       // buffers by the parity); advanced by the plan-tile kernel
    uint32_t pad[59];
};
static_assert(sizeof(WsHeader) == 256, "header is 256 bytes");

// Tile number in start order.  The counter is zero at the first launch (zero-filled workspace)
// and is reset by the consuming kernel of every call; the modulo only keeps a misused workspace
// in bounds.
__device__ __forceinline__ int take_ticket(WsHeader* h, int ntiles) {
    const uint32_t t = __hip_atomic_fetch_add(&h->ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return (int)(t % (uint32_t)ntiles);
}

// When the counting kernel ends, word c of every column holds the inclusive prefix through count
// tile c.  It gets there in one of two ways.  With at most kDirectCountTiles count tiles, every
// count tile stores its own totals and counts itself done; the last one to do so (all others have
// then stored) scans every column in place -- no workgroup ever waits for another.  With more,
// the totals go through the decoupled look-back below.
constexpr int kDirectCountTiles = 64;

// Inclusive scan in place of one column over count tiles 0..nct-1 whose words hold tagged totals
// of this call (re-read until current: their stores may still be in flight from other dies).
__device__ __forceinline__ void scan_count_column(uint64_t* status, int nct, int ncols, int col,
                                                  uint32_t epoch, uint32_t* err) {
    const uint32_t want = status_tag(epoch);
    uint32_t run = 0;
    for (int j0 = 0; j0 < nct; j0 += 32) {  // 32 loads in flight (one round trip at <= 32 count tiles)
        uint64_t v[32];
#pragma unroll
        for (int j = 0; j < 32; ++j)
            v[j] = status_load(status + (size_t)min(j0 + j, nct - 1) * ncols + col);
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            if (j0 + j >= nct) break;
            uint64_t* p = status + (size_t)(j0 + j) * ncols + col;
            run += tagged_value(p, v[j], want, err);
            status_store(p, status_make(epoch, true, run));
        }
    }
}

// Counts the calling workgroup's count tile as done; true in the last of the nct count tiles,
// which then resets the counter.  Call from every thread after the tile's words are stored.
__device__ __forceinline__ bool last_count_tile(WsHeader* hdr, int nct, uint32_t* s_flag) {
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t d = __hip_atomic_fetch_add(&gptr(hdr)->ct_done, 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
        const bool last = d == (uint32_t)(nct - 1);
        if (last) __hip_atomic_store(&gptr(hdr)->ct_done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_flag = last ? 1u : 0u;
    }
    __syncthreads();
    return *s_flag != 0u;
}

// Index into an LDS array of per-slot values with one pad word after every 64: a lane writing
// slot (lane * K + k) of a token-per-lane layout and a lane reading slot (base + lane) then both
// hit 64 different banks.  Arrays need n + n / 64 words.
__device__ __forceinline__ int slot_pad(int i) { return i + (i >> 6); }

// Lanes of this wave (restricted to `active`) holding the same key as the calling lane: one wave
// ballot per key bit (a wave64 stand-in for a warp match).  NB = key bits, fixed at compile time
// so the loop unrolls.
// Per bit, the lanes that agree with the calling lane are ~(ballot ^ m) with m the lane's bit
// spread over a word, taken on the two 32-bit halves (one three-input bit operation each).
template <int NB>
__device__ __forceinline__ uint64_t match_peers(uint32_t key, uint64_t active) {
    uint32_t lo = (uint32_t)active, hi = (uint32_t)(active >> 32);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const uint32_t m = 0u - ((key >> b) & 1u);
        const uint64_t ones = __ballot(m != 0u);
        lo &= ~((uint32_t)ones ^ m);
        hi &= ~((uint32_t)(ones >> 32) ^ m);
    }
    return ((uint64_t)hi << 32) | lo;
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

// Sum over the 64 lanes of a wave (every lane gets the result).
__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__host__ __device__ constexpr int bits_for(int n_keys) {
    int b = 0;
    while ((1 << b) < n_keys) ++b;
    return b;
}

}  // namespace mep

namespace mep {

// ---- cross-lane exchange within aligned segments of S lanes (S a power of two <= 64) ----------
// Partners: S>=2 lane^1, S>=4 lane^2 (DPP quad permutes), S>=8 the mirror lane within 8
// (DPP row_half_mirror), S>=16 the mirror lane within 16 (DPP row_mirror), S>=32/64 lane^16 and
// lane^32 through ds_bpermute.  Each step pairs lanes symmetrically, so folding a commutative
// operation over the steps leaves every lane of the segment with the full result.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <int STEP>
__device__ __forceinline__ uint32_t seg_partner_u32(uint32_t v) {
    if constexpr (STEP == 1) return dpp_u32<0xB1>(v);   // quad_perm [1,0,3,2]
    else if constexpr (STEP == 2) return dpp_u32<0x4E>(v);  // quad_perm [2,3,0,1]
    else if constexpr (STEP == 4) return dpp_u32<0x141>(v); // row_half_mirror
    else if constexpr (STEP == 8) return dpp_u32<0x140>(v); // row_mirror
    else return (uint32_t)__shfl_xor((int)v, STEP);
}

template <int STEP>
__device__ __forceinline__ float seg_partner_f32(float v) {
    return __uint_as_float(seg_partner_u32<STEP>(__float_as_uint(v)));
}

template <int STEP>
__device__ __forceinline__ double seg_partner_f64(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = seg_partner_u32<STEP>((uint32_t)u);
    const uint32_t hi = seg_partner_u32<STEP>((uint32_t)(u >> 32));
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// All-reduce over segments of S lanes; S is a run-time power of two (uniform) up to SMAX.
template <int SMAX, typename T, typename Partner, typename Op>
__device__ __forceinline__ T seg_allreduce(T v, int S, Partner partner, Op op) {
    if constexpr (SMAX >= 2) if (S >= 2) v = op(v, partner(v, std::integral_constant<int, 1>{}));
    if constexpr (SMAX >= 4) if (S >= 4) v = op(v, partner(v, std::integral_constant<int, 2>{}));
    if constexpr (SMAX >= 8) if (S >= 8) v = op(v, partner(v, std::integral_constant<int, 4>{}));
    if constexpr (SMAX >= 16) if (S >= 16) v = op(v, partner(v, std::integral_constant<int, 8>{}));
    if constexpr (SMAX >= 32) if (S >= 32) v = op(v, partner(v, std::integral_constant<int, 16>{}));
    if constexpr (SMAX >= 64) if (S >= 64) v = op(v, partner(v, std::integral_constant<int, 32>{}));
    return v;
}

struct PartnerF32 {
    template <int STEP>
    __device__ __forceinline__ float operator()(float v, std::integral_constant<int, STEP>) const {
        return seg_partner_f32<STEP>(v);
    }
};
struct PartnerF64 {
    template <int STEP>
    __device__ __forceinline__ double operator()(double v, std::integral_constant<int, STEP>) const {
        return seg_partner_f64<STEP>(v);
    }
};
struct PartnerU32 {
    template <int STEP>
    __device__ __forceinline__ uint32_t operator()(uint32_t v, std::integral_constant<int, STEP>) const {
        return seg_partner_u32<STEP>(v);
    }
};

}  // namespace mep
