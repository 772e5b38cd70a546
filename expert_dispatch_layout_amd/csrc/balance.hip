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
// Two kernels:
//   plan    one workgroup per destination rank d.  Wave 0 runs the balancing loop (every
//           workgroup gets the same moves; workgroup 0 stores z and the group totals); then
//           the waves run the owners' quota loops, owner o on wave o mod 8, each appending its
//           (destination, expert, slots) allocations to an LDS list and leaving each expert's
//           remainder with its owner; the owners' loops are short and run in every workgroup,
//           which is cheaper than a second launch.  From the list the workgroup forms row d of
//           alloc, the alloc_cumsum rows of d's own experts, and then, as destination: the B
//           experts to copy (B wave-wide arg-max passes over the remote counts held in
//           registers) and the E + B groups scanned across the workgroup.
//   dst     one lane per slot, whole tokens per wave: each slot's rank by binary search over
//           its expert's cumulative allocation (L2-resident), its row from the group offsets,
//           and the duplicate encoding from the ranks of the token's earlier slots (shuffles);
//           workgroup 0 also counts each owner's copies (remote_stats[o][1]) from
//           experts_to_copy.
#include <hip/hip_runtime.h>
#include <limits.h>

#include "host_common.h"

namespace mep {

namespace {

constexpr int kBalMaxRanks = 128;
constexpr int kBalMaxExperts = 1024;
constexpr int kBalMaxCopies = 64;
constexpr int kBalMaxK = 32;
constexpr int kBalBlock = 512;  // 8 waves: owners' quota loops on 8 waves at once
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

// Wave-wide 64-bit max / min through DPP lane moves (no LDS round trips): two quad
// permutations, the half-row and row mirrors leave every lane with its row's extremum, the two
// row broadcasts carry it into the last row, and lane 63 holds the result.  Lanes a move does
// not reach keep their own value, which leaves the extremum unchanged.
template <int CTRL, int ROWS>
__device__ __forceinline__ long long dpp64(long long v) {
    const int lo = (int)(unsigned long long)v, hi = (int)((unsigned long long)v >> 32);
    const int l2 = __builtin_amdgcn_update_dpp(lo, lo, CTRL, ROWS, 0xf, false);
    const int h2 = __builtin_amdgcn_update_dpp(hi, hi, CTRL, ROWS, 0xf, false);
    return (long long)(((unsigned long long)(unsigned)h2 << 32) | (unsigned)l2);
}

template <bool MAX>
__device__ __forceinline__ long long wave_ext64(long long v) {
    auto pick = [](long long a, long long b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
    v = pick(v, dpp64<0xB1, 0xf>(v));   // quad_perm 1,0,3,2
    v = pick(v, dpp64<0x4E, 0xf>(v));   // quad_perm 2,3,0,1
    v = pick(v, dpp64<0x141, 0xf>(v));  // row_half_mirror
    v = pick(v, dpp64<0x140, 0xf>(v));  // row_mirror
    v = pick(v, dpp64<0x142, 0xa>(v));  // row_bcast:15 into rows 1 and 3
    v = pick(v, dpp64<0x143, 0xc>(v));  // row_bcast:31 into rows 2 and 3
    const int lo = __builtin_amdgcn_readlane((int)(unsigned long long)v, 63);
    const int hi = __builtin_amdgcn_readlane((int)((unsigned long long)v >> 32), 63);
    return (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}


__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Barrier that orders LDS only: global stores issued before it are not waited for.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROWS, 0xf, false);
}

// Wave-wide 32-bit max / min: the lane moves of wave_ext64, one 32-bit operation each.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_ext32(uint32_t v) {
    auto pick = [](uint32_t p, uint32_t q) { return MAX ? (p > q ? p : q) : (p < q ? p : q); };
    v = pick(v, dpp32<0xB1, 0xf>(v));   // quad_perm 1,0,3,2
    v = pick(v, dpp32<0x4E, 0xf>(v));   // quad_perm 2,3,0,1
    v = pick(v, dpp32<0x141, 0xf>(v));  // row_half_mirror
    v = pick(v, dpp32<0x140, 0xf>(v));  // row_mirror
    v = pick(v, dpp32<0x142, 0xa>(v));  // row_bcast:15 into rows 1 and 3
    v = pick(v, dpp32<0x143, 0xc>(v));  // row_bcast:31 into rows 2 and 3
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Arg-extremum keys: the value in the high bits and an index tie-break in the low bits, so that
// one integer maximum (or minimum) over the wave gives both.  Wide keys (64-bit: the value times
// 2048 plus an 11-bit index) take any value the plan forms; narrow keys (32-bit: the value plus
// 2^21 in the high 22 bits, a 10-bit index below) take values in (-2^21, 2^21), and reduce with
// one 32-bit operation per lane move instead of a 64-bit compare and two selects.  max_low:
// largest value, ties to the lower index; min_low: smallest value, ties to the lower index;
// max_high: largest value, ties to the higher index.
template <bool N32>
struct BalKeys;

template <>
struct BalKeys<false> {
    using T = long long;
    static constexpr long long kSpan = 2048;
    static constexpr T kLow = LLONG_MIN, kHigh = LLONG_MAX;
    __device__ static T max_low(long long v, int i) { return v * kSpan + (kSpan - 1 - i); }
    __device__ static T min_low(long long v, int i) { return v * kSpan + i; }
    __device__ static T max_high(long long v, int i) { return v * kSpan + i; }
    // floor division: the index part is always in [0, kSpan)
    __device__ static long long value(T k) { return k >= 0 ? k / kSpan : -((-k + kSpan - 1) / kSpan); }
    __device__ static int index_low(T k) { return (int)(kSpan - 1 - (k - value(k) * kSpan)); }
    __device__ static int index(T k) { return (int)(k - value(k) * kSpan); }
    __device__ static T wave_max(T v) { return wave_ext64<true>(v); }
    __device__ static T wave_min(T v) { return wave_ext64<false>(v); }
};

template <>
struct BalKeys<true> {
    using T = uint32_t;
    static constexpr int kBits = 10;
    static constexpr long long kOff = 1ll << 21;
    static constexpr T kLow = 0u, kHigh = 0xFFFFFFFFu;
    __device__ static T pack(long long v, int i) { return ((T)(v + kOff) << kBits) | (T)i; }
    __device__ static T max_low(long long v, int i) { return pack(v, (1 << kBits) - 1 - i); }
    __device__ static T min_low(long long v, int i) { return pack(v, i); }
    __device__ static T max_high(long long v, int i) { return pack(v, i); }
    __device__ static long long value(T k) { return (long long)(k >> kBits) - kOff; }
    __device__ static int index_low(T k) { return (1 << kBits) - 1 - (int)(k & ((1u << kBits) - 1u)); }
    __device__ static int index(T k) { return (int)(k & ((1u << kBits) - 1u)); }
    __device__ static T wave_max(T v) { return wave_ext32<true>(v); }
    __device__ static T wave_min(T v) { return wave_ext32<false>(v); }
};
constexpr long long kNarrowLimit = 1ll << 21;  // narrow keys: every value of magnitude below this

// The balancing loop on one wave (lane holds ranks lane and lane + 64): while some rank has a
// surplus and some a deficit, the largest surplus (lowest rank on ties) fills the largest deficit
// (lowest rank on ties) completely; each move (from, to, slots) goes to `s_moves`.  Returns the
// number of moves.
template <bool N32>
__device__ __forceinline__ int balance_moves(long long (&bal)[2], int R, int lane, int* s_moves) {
    using Kt = BalKeys<N32>;
    int nmoves = 0;
    for (;;) {
        typename Kt::T kmax = Kt::kLow, kmin = Kt::kHigh;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int r = lane + 64 * c;
            if (r < R) {
                const typename Kt::T k1 = Kt::max_low(bal[c], r), k2 = Kt::min_low(bal[c], r);
                kmax = k1 > kmax ? k1 : kmax;
                kmin = k2 < kmin ? k2 : kmin;
            }
        }
        kmax = Kt::wave_max(kmax);
        kmin = Kt::wave_min(kmin);
        const long long surplus = Kt::value(kmax), deficit = Kt::value(kmin);
        if (surplus <= 0 || deficit >= 0) break;
        const int sr = Kt::index_low(kmax), dr = Kt::index(kmin);
        const long long move = -deficit;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int r = lane + 64 * c;
            if (r == sr) bal[c] -= move;
            if (r == dr) bal[c] = 0;
        }
        if (lane == 0) {
            s_moves[3 * nmoves] = sr;
            s_moves[3 * nmoves + 1] = dr;
            s_moves[3 * nmoves + 2] = (int)move;
        }
        ++nmoves;
    }
    return nmoves;
}

// Owner o's quota loop on one wave: while a destination's quota (the largest, lowest rank on
// ties) and an expert's remainder (the largest, lowest expert on ties) are both left, the smaller
// of the two moves; each allocation (destination, expert, slots) is appended to `s_ent`.
template <bool N32, int kCh>
__device__ __forceinline__ void owner_quotas(long long (&quota)[2], long long (&rem)[kCh], int o, int R, int epn,
                                             int lane, int* s_nent, int (*s_ent)[3]) {
    using Kt = BalKeys<N32>;
    for (;;) {
        typename Kt::T kq = Kt::kLow;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int r = lane + 64 * c;
            if (r < R) {
                const typename Kt::T k = Kt::max_low(quota[c], r);
                kq = k > kq ? k : kq;
            }
        }
        typename Kt::T kr = Kt::kLow;
#pragma unroll
        for (int c = 0; c < kCh; ++c) {
            const int jj = lane + 64 * c;
            if (jj < epn) {
                const typename Kt::T k = Kt::max_low(rem[c], jj);
                kr = k > kr ? k : kr;
            }
        }
        kq = Kt::wave_max(kq);
        kr = Kt::wave_max(kr);
        const long long mq = Kt::value(kq), mr = Kt::value(kr);
        if (mq <= 0 || mr <= 0) break;
        const int tr = Kt::index_low(kq), sj = Kt::index_low(kr);
        const long long take = mr < mq ? mr : mq;
#pragma unroll
        for (int c = 0; c < 2; ++c)
            if (lane + 64 * c == tr) quota[c] -= take;
#pragma unroll
        for (int c = 0; c < kCh; ++c)
            if (lane + 64 * c == sj) rem[c] -= take;
        if (lane == 0) {
            const int at = atomicAdd(s_nent, 1);
            s_ent[at][0] = tr;
            s_ent[at][1] = o * epn + sj;
            s_ent[at][2] = (int)take;
        }
    }
}

// Destination d's experts to copy, on one wave: B passes, each taking the largest remote count
// (the higher expert on ties; -1 once none is left) and clearing it.
template <bool N32, int kCh>
__device__ __forceinline__ void copy_choice(long long (&remote)[kCh], const BalArgs& a, int d, int lane, int* s_slot,
                                            unsigned char* s_picked) {
    using Kt = BalKeys<N32>;
    for (int b = 0; b < a.B; ++b) {
        typename Kt::T k = Kt::kLow;
#pragma unroll
        for (int c = 0; c < kCh; ++c) {
            const int e = lane + 64 * c;
            if (e < a.E) {
                const typename Kt::T kk = Kt::max_high(remote[c], e);
                k = kk > k ? kk : k;
            }
        }
        k = Kt::wave_max(k);
        const int best = Kt::index(k);
        const int chosen = Kt::value(k) > 0 ? best : -1;
#pragma unroll
        for (int c = 0; c < kCh; ++c)
            if (lane + 64 * c == best) remote[c] = 0;
        if (lane == 0) {
            s_slot[b] = chosen;
            a.experts_to_copy[d * a.B + b] = chosen;
            if (chosen >= 0) s_picked[chosen] = 1;
        }
    }
}

// ---------------------------------------------------------------------------------------------
// plan kernel (balancing, owners' quotas, destination groups)
// ---------------------------------------------------------------------------------------------
constexpr int kBalWaves = kBalBlock / 64;
// allocation entries: each quota step zeroes a quota or an expert's remainder, and the nonzero
// quotas are the moves (at most 2R + 1 of them), so all owners together make at most
// moves + E entries
constexpr int kBalMaxEntries = 2 * kBalMaxRanks + 1 + kBalMaxExperts;

template <int CH>
__global__ __launch_bounds__(kBalBlock) void balance_plan_kernel(BalArgs a) {
    __shared__ int s_group[kBalMaxRanks];         // slots per rank before moves
    __shared__ int s_tot[kBalMaxExperts];         // slots per expert
    __shared__ int s_moves[3 * (2 * kBalMaxRanks + 1)];  // (from, to, slots) of each move
    __shared__ int s_nmoves;
    __shared__ int s_ent[kBalMaxEntries][3];      // (destination, expert, slots) allocations
    __shared__ int s_nent;
    __shared__ int s_rem[kBalMaxExperts];         // each expert's slots left with its owner
    __shared__ int s_acol[kBalMaxExperts];        // [R][epn]: d's experts' slots per rank
    __shared__ int s_cnt[kBalMaxExperts];         // row d of alloc
    __shared__ int s_eoff[kBalMaxExperts];
    __shared__ unsigned char s_picked[kBalMaxExperts];
    __shared__ int s_slot[kBalMaxCopies];
    __shared__ int s_wave[kBalWaves];
    __shared__ int s_wide;    // some slot count or rank balance needs wide keys
    __shared__ int s_narrow;  // the keys the loops use (the same in every workgroup)
    const int d = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int R = a.R, epn = a.epn, E = a.E, B = a.B, G = E + B;
    constexpr int kPerT = kBalMaxExperts / kBalBlock;
    constexpr int kCh = CH;  // 64-wide chunks covering the experts

    int tot[kPerT];  // loads first, so their latency overlaps the clearing below
#pragma unroll
    for (int i = 0; i < kPerT; ++i) {
        const int e = tid + i * kBalBlock;
        tot[i] = e < E ? a.tpe[e] : 0;
    }
    for (int i = tid; i < R; i += kBalBlock) s_group[i] = 0;
    for (int i = tid; i < E; i += kBalBlock) {
        s_acol[i] = 0;
        s_eoff[i] = -1;
        s_picked[i] = 0;
    }
    if (tid == 0) {
        s_nent = 0;
        s_wide = 0;
    }
    if (d == 0)
        for (int i = tid; i < R * R; i += kBalBlock) a.z[i] = 0;
    lds_barrier();
#pragma unroll
    for (int i = 0; i < kPerT; ++i) {
        const int e = tid + i * kBalBlock;
        if (e < E) {
            s_tot[e] = tot[i];
            atomicAdd(&s_group[e / epn], tot[i]);
            if (tot[i] < 0 || tot[i] >= kNarrowLimit) s_wide = 1;
        }
    }
    lds_barrier();

    // ---- balancing loop (wave 0) ----------------------------------------------------------------
    if (wv == 0) {
        // lane holds ranks lane and lane + 64
        long long bal[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int r = lane + 64 * c;
            const long long s2 = r < R ? s_group[r] : 0;
            if (r < R && d == 0) a.group_tokens[r] = (int32_t)s2;
            bal[c] = s2 - a.cap;
        }
        // narrow keys when every balance is within their range (then so is every quota, and
        // every remainder is a slot count, checked above)
        bool wide = s_wide != 0;
#pragma unroll
        for (int c = 0; c < 2; ++c)
            if (lane + 64 * c < R && (bal[c] <= -kNarrowLimit || bal[c] >= kNarrowLimit)) wide = true;
        wide = __ballot(wide) != 0ull;
        const int nmoves = wide ? balance_moves<false>(bal, R, lane, s_moves) : balance_moves<true>(bal, R, lane, s_moves);
        if (lane == 0) {
            s_narrow = wide ? 0 : 1;
            s_nmoves = nmoves;
        }
    }
    lds_barrier();

    // ---- quota allocation of every owner's moves over its experts (owner o on wave o mod 8) ----
    const int nmoves = s_nmoves;
    const bool narrow = s_narrow != 0;
    for (int o = wv; o < R; o += kBalWaves) {
        long long quota[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) quota[c] = 0;
        for (int m = 0; m < nmoves; ++m) {  // a (from, to) pair occurs at most once
            if (s_moves[3 * m] != o) continue;
            const int to = s_moves[3 * m + 1];
#pragma unroll
            for (int c = 0; c < 2; ++c)
                if (lane + 64 * c == to) quota[c] = s_moves[3 * m + 2];
        }
        long long rem[kCh];
#pragma unroll
        for (int c = 0; c < kCh; ++c) {
            const int jj = lane + 64 * c;
            rem[c] = jj < epn ? s_tot[o * epn + jj] : 0;
        }
        if (narrow) owner_quotas<true, kCh>(quota, rem, o, R, epn, lane, &s_nent, s_ent);
        else owner_quotas<false, kCh>(quota, rem, o, R, epn, lane, &s_nent, s_ent);
#pragma unroll
        for (int c = 0; c < kCh; ++c) {
            const int jj = lane + 64 * c;
            if (jj < epn) s_rem[o * epn + jj] = (int)rem[c];
        }
    }
    lds_barrier();

    // ---- row d of alloc, and the alloc_cumsum rows of d's own experts ----------------------------
    for (int e = tid; e < E; e += kBalBlock) s_cnt[e] = e / epn == d ? s_rem[e] : 0;
    for (int j = tid; j < epn; j += kBalBlock) s_acol[d * epn + j] = s_rem[d * epn + j];
    lds_barrier();
    const int nent = s_nent;
    for (int i = tid; i < nent; i += kBalBlock) {
        const int to = s_ent[i][0], e = s_ent[i][1], take = s_ent[i][2];
        if (to == d) s_cnt[e] = take;                       // e's owner is not d (moves leave d)
        if (e / epn == d) s_acol[to * epn + (e - d * epn)] = take;
    }
    lds_barrier();
    for (int e = tid; e < E; e += kBalBlock) a.alloc[d * E + e] = s_cnt[e];
    for (int j = tid; j < epn; j += kBalBlock) {
        int run = 0;
        int32_t* row = a.alloc_cumsum + (int64_t)(d * epn + j) * R;
        for (int r = 0; r < R; ++r) {
            run += s_acol[r * epn + j];
            row[r] = run;
        }
    }
    if (d == 0) {
        // the moves go over the zeros stored at the start: a full barrier orders the two
        __syncthreads();
        for (int m = tid; m < nmoves; m += kBalBlock)
            a.z[s_moves[3 * m] * R + s_moves[3 * m + 1]] = s_moves[3 * m + 2];
    }

    // ---- destination d: experts to copy, then the E + B groups ----------------------------------
    if (wv == 0) {
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
        if (narrow) copy_choice<true, kCh>(remote, a, d, lane, s_slot, s_picked);
        else copy_choice<false, kCh>(remote, a, d, lane, s_slot, s_picked);
    }
    lds_barrier();
    // E + B groups, a few consecutive per thread, scanned across the workgroup
    constexpr int kPer = (kBalMaxExperts + kBalMaxCopies + kBalBlock - 1) / kBalBlock;
    int cnt[kPer], pad[kPer], ex[kPer];
    int mine = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int gi = tid * kPer + i;
        int c = 0, x = -1;
        if (gi < E) {
            if (!s_picked[gi]) { c = s_cnt[gi]; x = gi; }
        } else if (gi < G) {
            x = s_slot[gi - E];
            c = x >= 0 ? s_cnt[x] : 0;
        }
        cnt[i] = c;
        ex[i] = x;
        pad[i] = c > 0 ? (a.tp > 1 ? (c + a.tp - 1) / a.tp * a.tp : c) : 0;
        mine += pad[i];
    }
    int incl = mine;
#pragma unroll
    for (int st = 1; st < 64; st <<= 1) {
        const int y = __shfl_up(incl, st, 64);
        if (lane >= st) incl += y;
    }
    if (lane == 63) s_wave[wv] = incl;
    lds_barrier();
    int base = incl - mine;
    for (int w = 0; w < wv; ++w) base += s_wave[w];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int gi = tid * kPer + i;
        if (gi < G) {
            const int64_t at = (int64_t)d * G + gi;
            a.cu[at] = base + pad[i];
            const bool zf = cnt[i] > 0 && pad[i] > cnt[i];
            a.zero_fill[2 * at] = zf ? base + cnt[i] : 0;
            a.zero_fill[2 * at + 1] = zf ? pad[i] - cnt[i] : 0;
            if (cnt[i] > 0) s_eoff[ex[i]] = base;
        }
        base += pad[i];
    }
    lds_barrier();
    for (int e = tid; e < E; e += kBalBlock) a.expert_offsets[d * E + e] = s_eoff[e];
}

// ---------------------------------------------------------------------------------------------
// dst kernel
// ---------------------------------------------------------------------------------------------
// A wave holds 64 / K whole tokens, one slot per lane (lanes past the last whole token idle), so
// the dependent loads of the search run for every slot at once and a slot finds the ranks of
// its token's earlier slots in the lanes just below it.  With at most kBalRowRanks ranks, a
// multiple of 4, and a 16-byte aligned table, a slot reads its expert's whole cumulative row at
// once (16-byte loads) and searches it in registers; otherwise a binary search (a dependent load
// per step).
constexpr int kBalRowRanks = 16;

template <bool ROW>
__global__ __launch_bounds__(kBalTokBlock) void balance_dst_kernel(const int32_t* __restrict__ ids,
                                                                   const int32_t* __restrict__ cu_seqlens,
                                                                   const int32_t* __restrict__ e2p,
                                                                   const int32_t* __restrict__ alloc_cumsum,
                                                                   const int32_t* __restrict__ expert_offsets,
                                                                   const int32_t* __restrict__ experts_to_copy,
                                                                   int64_t N, int E, int K, int R, int B, int64_t NvS,
                                                                   int32_t* __restrict__ dst,
                                                                   int32_t* __restrict__ remote_stats) {
    __shared__ int s_copies[kBalMaxRanks];
    if (blockIdx.x == 0) {
        // copies of each owner's experts over all destinations (remote_stats[o][1])
        const int epn = E / R;
        for (int o = threadIdx.x; o < R; o += kBalTokBlock) s_copies[o] = 0;
        __syncthreads();
        if (experts_to_copy)
            for (int i = threadIdx.x; i < R * B; i += kBalTokBlock) {
                const int x = experts_to_copy[i];
                if (x >= 0) atomicAdd(&s_copies[x / epn], 1);
            }
        __syncthreads();
        for (int o = threadIdx.x; o < R; o += kBalTokBlock) remote_stats[2 * o + 1] = s_copies[o];
    }
    const int lane = threadIdx.x & 63;
    const int tpw = 64 / K;
    const int64_t wave = ((int64_t)blockIdx.x * kBalTokBlock + threadIdx.x) >> 6;
    const int tl = lane / K, k = lane - tl * K;
    const int64_t t = wave * tpw + tl;
    const bool active = tl < tpw && t < N;
    int rank = -1;
    int64_t raw = 0;
    if (active) {
        const int64_t i = t * K + k;
        const int e = ids[i];
        const int q = e2p[i] - cu_seqlens[e];
        const int32_t* cum = alloc_cumsum + (int64_t)e * R;
        // lo = the first rank whose cumulative allocation exceeds q, pc = the one before it (0)
        int lo = 0, pc = 0;
        if constexpr (ROW) {
            int cv[kBalRowRanks];
#pragma unroll
            for (int r4 = 0; r4 < kBalRowRanks; r4 += 4) {
                int4 v = {0, 0, 0, 0};
                if (r4 < R) v = *reinterpret_cast<const int4*>(cum + r4);
                cv[r4] = v.x;
                cv[r4 + 1] = v.y;
                cv[r4 + 2] = v.z;
                cv[r4 + 3] = v.w;
            }
            lo = R;
#pragma unroll
            for (int r = kBalRowRanks - 1; r >= 0; --r)
                if (r < R && cv[r] > q) lo = r;
#pragma unroll
            for (int r = 0; r < kBalRowRanks; ++r)
                if (r + 1 == lo) pc = cv[r];
        } else {
            int hi = R;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                const int ac = cum[mid];
                if (ac > q) hi = mid;
                else { lo = mid + 1; pc = ac; }
            }
        }
        if (lo >= R) lo = R - 1;  // only for inputs that break the layout's invariants
        rank = lo;
        raw = (int64_t)lo * NvS + expert_offsets[(int64_t)lo * E + e] + (q - pc);
    }
    bool dup = false;
    for (int k2 = 0; k2 + 1 < K; ++k2) {
        const int src = lane - k + k2;
        const int r2 = __shfl(rank, src < 0 ? 0 : src, 64);
        if (k2 < k && r2 == rank) dup = true;
    }
    if (active) dst[t * K + k] = (int32_t)(dup ? -raw - 1 : raw);
}

// 64-wide chunks covering n entries, rounded up to a compiled count (1, 2, 4 or 16)
int chunks64(int n) {
    const int c = (n + 63) / 64;
    return c <= 1 ? 1 : c <= 2 ? 2 : c <= 4 ? 4 : 16;
}

}  // namespace

}  // namespace mep

extern "C" int mep_plan_balanced(const int32_t* topk_ids, const int32_t* tokens_per_expert,
                                 const int32_t* cu_seqlens, const int32_t* expanded_to_permuted,
                                 int64_t N, int E, int K, int R, int num_copies, int token_padding,
                                 int64_t capacity, int64_t NvS, const mep_balanced_outputs* out,
                                 void* stream) {
    mep::launch_begin();
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
    const int ch = chunks64(E);  // covers the owners' epn experts too
    if (ch == 1) launch_ggl(balance_plan_kernel<1>, dim3(R), dim3(kBalBlock), 0, st, a);
    else if (ch == 2) launch_ggl(balance_plan_kernel<2>, dim3(R), dim3(kBalBlock), 0, st, a);
    else if (ch == 4) launch_ggl(balance_plan_kernel<4>, dim3(R), dim3(kBalBlock), 0, st, a);
    else launch_ggl(balance_plan_kernel<16>, dim3(R), dim3(kBalBlock), 0, st, a);
    // at least one workgroup: workgroup 0 also counts the copies per owner
    const int64_t waves = N > 0 ? ceil_div64(N, 64 / K) : 1;
    // the row search's 16-byte loads need 16-byte aligned rows: R a multiple of 4 and the table
    // itself aligned (outputs are only required to be 4-byte aligned)
    const bool row = R <= kBalRowRanks && R % 4 == 0 && aligned(out->alloc_cumsum, 16);
    auto dst_kernel = row ? balance_dst_kernel<true> : balance_dst_kernel<false>;
    launch_ggl(dst_kernel, dim3((unsigned)ceil_div64(waves, kBalTokBlock / 64)), dim3(kBalTokBlock), 0, st,
               topk_ids, cu_seqlens, expanded_to_permuted, out->alloc_cumsum, out->expert_offsets,
               num_copies > 0 ? out->experts_to_copy : nullptr, N, E, K, R, num_copies, NvS, out->dst,
               out->remote_stats);
    return launch_status();
}
