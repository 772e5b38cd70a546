// mep_plan_balanced: the expert-parallel plan with capacity rebalancing and redundant remote
// experts (MoonEP planning.py, PlanningKernel: the balancing loop over rank loads, the
// per-owner quota allocation, the per-destination choice of experts to copy with its padded
// group scan, and dst by binary search over each expert's cumulative allocation), for all R
// ranks of one GPU's batch.
//
// The page gathers every rank's expert counts and then takes a source slot's position among
// its expert's slots from a per-rank prefix plus a local stable rank.  On one GPU the stable
// layout already holds that position: q = expanded_to_permuted[i] - cu_seqlens[e], because
// source-then-token order is global slot order.  So only the E totals enter the planning
// steps, and no per-source counts are formed.
//
// Three kernels:
//   owner   one workgroup per owner rank.  Wave 0 runs the balancing loop itself (every
//           workgroup gets the same moves; workgroup 0 stores z, the group totals and clears
//           remote_stats) and then hands the owner's moves out to its experts; the owner's
//           columns of alloc and the rows of alloc_cumsum of its experts are written from LDS.
//   dest    one workgroup per destination rank: the B experts to copy (wave 0, B wave-wide
//           arg-max passes over the remote counts held in registers), then the E + B groups
//           scanned across the workgroup; remote_stats[owner][1] is counted with one global
//           atomic add per copy.
//   dst     one thread per token: each slot's rank by binary search over its expert's
//           cumulative allocation (L2-resident), its row from the group offsets, and the
//           duplicate encoding from a 128-bit mask of the ranks seen so far.
// The loops are the page's, so each stops: every balancing step zeroes one deficit for good
// and a rank turns from surplus to deficit at most once (at most 2R steps); every quota step
// zeroes a quota or an expert's remainder (at most R + epn steps).
#include <hip/hip_runtime.h>
#include <limits.h>

#include "host_common.h"

namespace mep {

namespace {

constexpr int kBalMaxRanks = 128;
constexpr int kBalMaxExperts = 1024;
constexpr int kBalMaxCopies = 64;
constexpr int kBalMaxK = 32;
constexpr int kBalBlock = 256;
constexpr int kBalTokBlock = 256;

struct BalArgs {
    const int32_t* tpe;  // [E] slots per expert
    int E, R, epn, B, tp;
    int64_t cap;
    int32_t* group_tokens;     // [R]
    int32_t* z;                // [R,R]
    int32_t* alloc;            // [R,E]
    int32_t* alloc_cumsum;     // [E,R]
    int32_t* experts_to_copy;  // [R,B]
    int32_t* remote_stats;     // [R,2]
    int32_t* cu;               // [R,E+B]
    int32_t* zero_fill;        // [R,E+B,2]
    int32_t* expert_offsets;   // [R,E]
};

__device__ __forceinline__ long long wave_max64(long long v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const long long o = __shfl_xor(v, m, 64);
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ long long wave_min64(long long v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const long long o = __shfl_xor(v, m, 64);
        v = o < v ? o : v;
    }
    return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Arg-extremum keys: the value in the high bits, the index tie-break in the low 11 bits.
constexpr long long kIdxSpan = 2048;
__device__ __forceinline__ long long key_max_low(long long v, int i) { return v * kIdxSpan + (kIdxSpan - 1 - i); }
__device__ __forceinline__ long long key_min_low(long long v, int i) { return v * kIdxSpan + i; }
__device__ __forceinline__ long long key_max_high(long long v, int i) { return v * kIdxSpan + i; }
__device__ __forceinline__ long long key_value(long long k) {
    // floor division: the index part is always in [0, kIdxSpan)
    return k >= 0 ? k / kIdxSpan : -((-k + kIdxSpan - 1) / kIdxSpan);
}
__device__ __forceinline__ int key_index_low(long long k) { return (int)(kIdxSpan - 1 - (k - key_value(k) * kIdxSpan)); }
__device__ __forceinline__ int key_index(long long k) { return (int)(k - key_value(k) * kIdxSpan); }

// ---------------------------------------------------------------------------------------------
// owner kernel
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kBalBlock) void balance_owner_kernel(BalArgs a) {
    __shared__ int s_zrow[kBalMaxRanks];          // moves from this owner to each rank
    __shared__ int s_alloc[kBalMaxExperts];       // [R][epn] of this owner's experts
    const int o = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int R = a.R, epn = a.epn, E = a.E;

    for (int i = tid; i < R; i += kBalBlock) s_zrow[i] = 0;
    for (int i = tid; i < R * epn; i += kBalBlock) s_alloc[i] = 0;
    if (o == 0) {
        for (int i = tid; i < R * R; i += kBalBlock) a.z[i] = 0;
        for (int i = tid; i < 2 * R; i += kBalBlock) a.remote_stats[i] = 0;
    }
    __syncthreads();

    if (tid < 64) {
        // group totals; lane holds ranks lane and lane + 64
        long long bal[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int r = lane + 64 * c;
            long long s = 0;
            if (r < R)
                for (int j = 0; j < epn; ++j) s += a.tpe[r * epn + j];
            if (r < R && o == 0) a.group_tokens[r] = (int32_t)s;
            bal[c] = s - a.cap;
        }
        // balancing loop
        for (;;) {
            long long kmax = LLONG_MIN, kmin = LLONG_MAX;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int r = lane + 64 * c;
                if (r < R) {
                    const long long k1 = key_max_low(bal[c], r), k2 = key_min_low(bal[c], r);
                    kmax = k1 > kmax ? k1 : kmax;
                    kmin = k2 < kmin ? k2 : kmin;
                }
            }
            kmax = wave_max64(kmax);
            kmin = wave_min64(kmin);
            const long long surplus = key_value(kmax), deficit = key_value(kmin);
            if (surplus <= 0 || deficit >= 0) break;
            const int sr = key_index_low(kmax), dr = key_index(kmin);
            const long long move = -deficit;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int r = lane + 64 * c;
                if (r == sr) bal[c] -= move;
                if (r == dr) bal[c] = 0;
            }
            if (lane == 0) {
                if (o == 0) a.z[sr * R + dr] = (int32_t)move;
                if (sr == o) s_zrow[dr] = (int32_t)move;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        // quota allocation of this owner's moves over its experts
        long long quota[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int r = lane + 64 * c;
            quota[c] = r < R ? s_zrow[r] : 0;
        }
        constexpr int kCh = kBalMaxExperts / 64;
        long long rem[kCh];
#pragma unroll
        for (int c = 0; c < kCh; ++c) {
            const int j = lane + 64 * c;
            rem[c] = j < epn ? a.tpe[o * epn + j] : 0;
        }
        for (;;) {
            long long kq = LLONG_MIN;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int r = lane + 64 * c;
                if (r < R) {
                    const long long k = key_max_low(quota[c], r);
                    kq = k > kq ? k : kq;
                }
            }
            kq = wave_max64(kq);
            const long long mq = key_value(kq);
            if (mq <= 0) break;
            long long kr = LLONG_MIN;
#pragma unroll
            for (int c = 0; c < kCh; ++c) {
                const int j = lane + 64 * c;
                if (j < epn) {
                    const long long k = key_max_low(rem[c], j);
                    kr = k > kr ? k : kr;
                }
            }
            kr = wave_max64(kr);
            const long long mr = key_value(kr);
            if (mr <= 0) break;
            const int tr = key_index_low(kq), sj = key_index_low(kr);
            const long long take = mr < mq ? mr : mq;
#pragma unroll
            for (int c = 0; c < 2; ++c)
                if (lane + 64 * c == tr) quota[c] -= take;
#pragma unroll
            for (int c = 0; c < kCh; ++c)
                if (lane + 64 * c == sj) rem[c] -= take;
            if (lane == 0) s_alloc[tr * epn + sj] = (int)take;
        }
#pragma unroll
        for (int c = 0; c < kCh; ++c) {
            const int j = lane + 64 * c;
            if (j < epn) s_alloc[o * epn + j] = (int)rem[c];
        }
    }
    __syncthreads();
    // this owner's columns of alloc, and its experts' rows of alloc_cumsum
    for (int i = tid; i < R * epn; i += kBalBlock) {
        const int r = i / epn, j = i - r * epn;
        a.alloc[r * E + o * epn + j] = s_alloc[i];
    }
    for (int j = tid; j < epn; j += kBalBlock) {
        int run = 0;
        int32_t* row = a.alloc_cumsum + (int64_t)(o * epn + j) * R;
        for (int r = 0; r < R; ++r) {
            run += s_alloc[r * epn + j];
            row[r] = run;
        }
    }
}

// ---------------------------------------------------------------------------------------------
// destination kernel
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kBalBlock) void balance_dest_kernel(BalArgs a) {
    __shared__ int s_cnt[kBalMaxExperts];
    __shared__ int s_eoff[kBalMaxExperts];
    __shared__ unsigned char s_picked[kBalMaxExperts];
    __shared__ int s_slot[kBalMaxCopies];
    __shared__ int s_wave[kBalBlock / 64];
    const int d = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int E = a.E, B = a.B, epn = a.epn, G = E + B;

    for (int e = tid; e < E; e += kBalBlock) {
        s_cnt[e] = a.alloc[d * E + e];
        s_eoff[e] = -1;
        s_picked[e] = 0;
    }
    __syncthreads();
    if (tid < 64) {
        constexpr int kCh = kBalMaxExperts / 64;
        long long remote[kCh];
        int n = 0;
#pragma unroll
        for (int c = 0; c < kCh; ++c) {
            const int e = lane + 64 * c;
            const int v = (e < E && e / epn != d) ? s_cnt[e] : 0;
            remote[c] = v;
            n += v > 0 ? 1 : 0;
        }
        n = wave_sum(n);
        if (lane == 0) a.remote_stats[2 * d] = n;
        for (int b = 0; b < B; ++b) {
            long long k = LLONG_MIN;
#pragma unroll
            for (int c = 0; c < kCh; ++c) {
                const int e = lane + 64 * c;
                if (e < E) {
                    const long long kk = key_max_high(remote[c], e);
                    k = kk > k ? kk : k;
                }
            }
            k = wave_max64(k);
            const int best = key_index(k);
            const int chosen = key_value(k) > 0 ? best : -1;
#pragma unroll
            for (int c = 0; c < kCh; ++c)
                if (lane + 64 * c == best) remote[c] = 0;
            if (lane == 0) {
                s_slot[b] = chosen;
                a.experts_to_copy[d * B + b] = chosen;
                if (chosen >= 0) {
                    s_picked[chosen] = 1;
                    atomicAdd(a.remote_stats + 2 * (chosen / epn) + 1, 1);
                }
            }
        }
    }
    __syncthreads();
    // E + B groups, a few consecutive per thread, scanned across the workgroup
    constexpr int kPer = (kBalMaxExperts + kBalMaxCopies + kBalBlock - 1) / kBalBlock;
    int cnt[kPer], pad[kPer], ex[kPer];
    int mine = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int g = tid * kPer + i;
        int c = 0, x = -1;
        if (g < E) {
            if (!s_picked[g]) { c = s_cnt[g]; x = g; }
        } else if (g < G) {
            x = s_slot[g - E];
            c = x >= 0 ? s_cnt[x] : 0;
        }
        cnt[i] = c;
        ex[i] = x;
        pad[i] = c > 0 ? (a.tp > 1 ? (c + a.tp - 1) / a.tp * a.tp : c) : 0;
        mine += pad[i];
    }
    int incl = mine;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
        const int y = __shfl_up(incl, s, 64);
        if (lane >= s) incl += y;
    }
    if (lane == 63) s_wave[wv] = incl;
    __syncthreads();
    int base = incl - mine;
    for (int w = 0; w < wv; ++w) base += s_wave[w];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int g = tid * kPer + i;
        if (g < G) {
            const int64_t at = (int64_t)d * G + g;
            a.cu[at] = base + pad[i];
            const bool zf = cnt[i] > 0 && pad[i] > cnt[i];
            a.zero_fill[2 * at] = zf ? base + cnt[i] : 0;
            a.zero_fill[2 * at + 1] = zf ? pad[i] - cnt[i] : 0;
            if (cnt[i] > 0) s_eoff[ex[i]] = base;
        }
        base += pad[i];
    }
    __syncthreads();
    for (int e = tid; e < E; e += kBalBlock) a.expert_offsets[d * E + e] = s_eoff[e];
}

// ---------------------------------------------------------------------------------------------
// dst kernel
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kBalTokBlock) void balance_dst_kernel(const int32_t* __restrict__ ids,
                                                                   const int32_t* __restrict__ cu_seqlens,
                                                                   const int32_t* __restrict__ e2p,
                                                                   const int32_t* __restrict__ alloc_cumsum,
                                                                   const int32_t* __restrict__ expert_offsets,
                                                                   int64_t N, int E, int K, int R, int64_t NvS,
                                                                   int32_t* __restrict__ dst) {
    const int64_t t = (int64_t)blockIdx.x * kBalTokBlock + threadIdx.x;
    if (t >= N) return;
    unsigned long long seen_lo = 0, seen_hi = 0;
    for (int k = 0; k < K; ++k) {
        const int64_t i = t * K + k;
        const int e = ids[i];
        const int q = e2p[i] - cu_seqlens[e];
        const int32_t* cum = alloc_cumsum + (int64_t)e * R;
        int lo = 0, hi = R, pc = 0;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            const int ac = cum[mid];
            if (ac > q) hi = mid;
            else { lo = mid + 1; pc = ac; }
        }
        if (lo >= R) lo = R - 1;  // only for inputs that break the layout's invariants
        const int64_t raw = (int64_t)lo * NvS + expert_offsets[(int64_t)lo * E + e] + (q - pc);
        bool dup;
        if (lo < 64) {
            const unsigned long long bit = 1ull << lo;
            dup = (seen_lo & bit) != 0;
            seen_lo |= bit;
        } else {
            const unsigned long long bit = 1ull << (lo - 64);
            dup = (seen_hi & bit) != 0;
            seen_hi |= bit;
        }
        dst[i] = (int32_t)(dup ? -raw - 1 : raw);
    }
}

}  // namespace

}  // namespace mep

extern "C" int mep_plan_balanced(const int32_t* topk_ids, const int32_t* tokens_per_expert,
                                 const int32_t* cu_seqlens, const int32_t* expanded_to_permuted,
                                 int64_t N, int E, int K, int R, int num_copies, int token_padding,
                                 int64_t capacity, int64_t NvS, const mep_balanced_outputs* out,
                                 void* stream) {
    using namespace mep;
    if (!out || !tokens_per_expert) return MEP_ERR_INVALID_ARG;
    if (N < 0 || E < 1 || K < 1 || R < 1 || num_copies < 0 || token_padding < 1 || capacity < 0 ||
        NvS < 1)
        return MEP_ERR_INVALID_ARG;
    if (N > 0 && (!topk_ids || !cu_seqlens || !expanded_to_permuted || !out->dst)) return MEP_ERR_INVALID_ARG;
    const void* req[] = {out->group_tokens, out->z, out->alloc, out->alloc_cumsum, out->remote_stats,
                         out->cu_seqlens, out->zero_fill, out->expert_offsets};
    for (const void* q : req)
        if (!q) return MEP_ERR_INVALID_ARG;
    if (num_copies > 0 && !out->experts_to_copy) return MEP_ERR_INVALID_ARG;
    const void* all[] = {topk_ids, tokens_per_expert, cu_seqlens, expanded_to_permuted, out->group_tokens,
                         out->z, out->alloc, out->alloc_cumsum, out->experts_to_copy, out->remote_stats,
                         out->cu_seqlens, out->zero_fill, out->expert_offsets, out->dst};
    for (const void* q : all)
        if (q && !aligned(q, 4)) return MEP_ERR_INVALID_ARG;
    if (E % R != 0) return MEP_ERR_UNSUPPORTED;
    if (R > kBalMaxRanks || E > kBalMaxExperts || num_copies > kBalMaxCopies || K > kBalMaxK || K > E)
        return MEP_ERR_UNSUPPORTED;
    if (capacity > INT32_MAX || N * (int64_t)K > INT32_MAX) return MEP_ERR_UNSUPPORTED;
    const int epn = E / R;
    const int64_t most = N * (int64_t)(K < epn ? K : epn);           // slots one rank can own
    const int64_t load = (most > capacity ? most : capacity) +          // a rank's slots after moves
                         (int64_t)(E + num_copies) * (token_padding - 1);  // and their padding
    if (NvS < load) return MEP_ERR_CAPACITY;
    if ((int64_t)R * NvS > INT32_MAX) return MEP_ERR_CAPACITY;

    BalArgs a;
    a.tpe = tokens_per_expert;
    a.E = E;
    a.R = R;
    a.epn = epn;
    a.B = num_copies;
    a.tp = token_padding;
    a.cap = capacity;
    a.group_tokens = out->group_tokens;
    a.z = out->z;
    a.alloc = out->alloc;
    a.alloc_cumsum = out->alloc_cumsum;
    a.experts_to_copy = out->experts_to_copy;
    a.remote_stats = out->remote_stats;
    a.cu = out->cu_seqlens;
    a.zero_fill = out->zero_fill;
    a.expert_offsets = out->expert_offsets;
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(balance_owner_kernel, dim3(R), dim3(kBalBlock), 0, st, a);
    hipLaunchKernelGGL(balance_dest_kernel, dim3(R), dim3(kBalBlock), 0, st, a);
    if (N > 0)
        hipLaunchKernelGGL(balance_dst_kernel, dim3((unsigned)ceil_div64(N, kBalTokBlock)), dim3(kBalTokBlock), 0, st,
                           topk_ids, cu_seqlens, expanded_to_permuted, out->alloc_cumsum, out->expert_offsets, N,
                           E, K, R, NvS, out->dst);
    return launch_status();
}
