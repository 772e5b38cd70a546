// Sigmoid routing kernel for the shapes where each lane of a token's segment holds one expert
// group of 32 (DeepSeek-V3 style group-limited routing: sigmoid scores plus a per-expert bias,
// groups ranked by the sum of their top scores, top-K inside the kept groups), or where there is
// no group limit.  E = 32 * LPT, K <= 8.
//
// Per token set (64 / LPT tokens per wave) the logits arrive by coalesced 16-byte loads one set
// ahead (as in the binary32 filter kernel, route_fast.h) and are staged in the wave's LDS area,
// where the 32 experts of a lane are one run of CPL 16-byte chunks followed by one chunk of
// padding: the lanes of a token then start 4 banks apart, so their reads of chunk j never share a
// bank, and every address is a per-lane base plus a constant.  The selection is
// register-resident:
//   1. keys  k'' = s~(x) + (b - c): the binary32 sigmoid s~ of the filter kernel, shifted by a
//      constant c > 1 + max|b| so that every key is negative and the largest keys have the
//      smallest magnitude (hence the finest spacing); the expert's index within the lane (0..31)
//      replaces the 5 low significand bits, which makes the keys of a lane distinct and lets a
//      value name its expert.  Negative binary32 values compare like their bit patterns read as
//      signed integers, in reverse, and -inf is below every key in both readings, so the
//      selection below is integer min / float med3 on the same bits (a median is the same
//      element in either order) with -inf as the empty entry, and no NaN canonicalisation;
//   2. a sorted list of the lane's 6 largest keys, one med3 per entry and key;
//   3. group score = sum of the group's top keys (list entries 0 and 1), with the group index in
//      its 3 (4 for 16 groups) low significand bits so that a lower index wins a tie; the rank of
//      each group among the segment's groups from the other lanes' scores (DPP),
//      kept = rank < topk_group;
//   4. K + 1 extraction rounds over the kept lanes' list heads (segment max through DPP); the
//      winning lane pops its head (a lane whose list runs dry before the last round, i.e. a group
//      holding more than 6 of the top K + 1, about one token in 10^4, takes the exact path);
//   5. certification: the selection on the exact keys (correctly rounded sigmoid plus bias, both
//      binary32) is the same when the last kept and first dropped group scores, and each pair
//      of consecutive extracted keys, differ by more than the error bounds below, and every
//      round had exactly one winner.  A token that fails is recorded in LDS and redone after
//      the streaming loop by a whole wave, on exact keys, from its row read again from global
//      memory (exact_token_sig), so the loop itself holds no call.
// The K selected experts then get their sigmoid in binary64 (relative error below 2^-30) for the
// weights.
//
// Error bounds.  Let S = RN(sigma(x)) and k = RN(S + b) be the exact key, s~ the binary32
// sigmoid (|s~ - sigma| <= 3.23 * 2^-23, see route_fast.h), b' = RN(b - c), k'' = RN(s~ + b'),
// and H a power of two above c + max|b| (so |k''|, |b'|, |k| < H).  Then
//     |k'' - (k - c)| <= 3.23*2^-23 + 2^-25 + 3 * H * 2^-25 = (3.48 + 0.75 H) 2^-23 = D.
// Replacing the 5 low significand bits changes a key by less than 32 ulp <= 2^-18 |key|.  So two
// extracted values m1 > m2 come from exact keys in the same order when
//     m1 - m2 > 2 D + 2^-18 (|m1| + |m2|) (1 + 2^-17).
// The top-2 sum is 1-Lipschitz in each order statistic, so a group score g~ = RN(L0 + L1) is
// within Dg(g~) = 2 D + (2^-18 (1 + 2^-10) + 2^-24 + 2^-19) |g~| + H 2^-24 of (exact score - 2c)
// (the 2^-19 term covers the group index in the low bits); the kept set is certain when the
// lowest kept and highest dropped scores differ by more than the sum of their bounds.  The tests
// run in binary32 with every constant enlarged by 2^-19 relative, which covers the rounding of
// the test itself.
#pragma once

#include "path.h"
#include "route_fast.h"

namespace mep {

constexpr int kSigT = 6;                          // list depth per lane
constexpr int kSigEmpty = (int)0xFF800000u;       // -inf: below every key as float and as integer

// LDS row layout: lane group g of a token (its CPL chunks) starts at chunk g * (CPL + 1).
template <int LPT, bool BF16>
struct SigGeom {
    static constexpr int W = BF16 ? 8 : 4;        // experts per 16-byte chunk
    static constexpr int CPL = kFastEPL / W;      // chunks per lane
    static constexpr int CPR = LPT * CPL;         // chunks per row
    static constexpr int GS = CPL + 1;            // lane group stride in chunks
    static constexpr int RS = LPT * GS;           // row stride in chunks
    static constexpr int TPW = 64 / LPT;          // tokens per set
    // position in the row of chunk ch
    static __device__ __forceinline__ int pos(int ch) { return (ch / CPL) * GS + ch % CPL; }
};

// A volatile read of an LDS float, re-done wherever it stands (so the compiler does not keep the
// value in a register across a loop).  The pointer is cast to the LDS address space: a generic
// volatile access would become a flat load, which counts against the vector-memory counter and
// would make the wait for it also wait for every global load in flight.
__device__ __forceinline__ float lds_volatile_load(const float* p) {
    return *(volatile const __attribute__((address_space(3))) float*)p;
}

struct SigCfg {
    int64_t tokens_per_group;  // tokens of a workgroup when it does not count (a multiple of TPW)
    int tg;                    // groups kept (MODE 1)
};

// Value held by lane (lane ^ O) of the aligned segment (O < 16), through DPP: quad permutes for
// the low two bits, row_half_mirror (i -> 7 - i) and row_mirror (i -> 15 - i) for the high ones.
template <int O>
__device__ __forceinline__ uint32_t seg_xor_u32(uint32_t v) {
    static_assert(O >= 0 && O < 16, "segments of at most 16 lanes");
    if constexpr (O == 0) {
        return v;
    } else if constexpr (O < 4) {
        return dpp_u32<(O == 1) ? 0xB1 : (O == 2) ? 0x4E : 0x1B>(v);  // quad_perm xor O
    } else if constexpr (O < 8) {
        const uint32_t h = dpp_u32<0x141>(v);  // lane ^ 7
        return seg_xor_u32<O ^ 7>(h);
    } else {
        const uint32_t m = dpp_u32<0x140>(v);  // lane ^ 15
        return seg_xor_u32<O ^ 15>(m);
    }
}

template <int LPT>
__device__ __forceinline__ int seg_min_i32(int v) {
    return (int)seg_allreduce<LPT>((uint32_t)v, LPT, PartnerU32{},
                                   [](uint32_t p, uint32_t q) { return (uint32_t)min((int)p, (int)q); });
}
template <int LPT>
__device__ __forceinline__ int seg_max_i32(int v) {
    return (int)seg_allreduce<LPT>((uint32_t)v, LPT, PartnerU32{},
                                   [](uint32_t p, uint32_t q) { return (uint32_t)max((int)p, (int)q); });
}
template <int LPT>
__device__ __forceinline__ uint32_t seg_or_u32(uint32_t v) {
    return seg_allreduce<LPT>(v, LPT, PartnerU32{}, [](uint32_t p, uint32_t q) { return p | q; });
}
template <int LPT>
__device__ __forceinline__ uint32_t seg_add_u32(uint32_t v) {
    return seg_allreduce<LPT>(v, LPT, PartnerU32{}, [](uint32_t p, uint32_t q) { return p + q; });
}

// Sorted insertion (best first: ascending integers, descending keys): entry i becomes the median
// of (L[i-1], L[i], v); the median is taken as binary32 (v_med3_f32), which picks the same
// element as the integer median.
__device__ __forceinline__ void list_insert(int (&L)[kSigT], int v) {
#pragma unroll
    for (int i = kSigT - 1; i >= 1; --i)
        L[i] = __float_as_int(__builtin_amdgcn_fmed3f(__int_as_float(L[i - 1]), __int_as_float(L[i]),
                                                       __int_as_float(v)));
    L[0] = min(L[0], v);
}

// ---- exact selection of one token by the whole wave ----------------------------------------------

template <typename P>
__device__ __forceinline__ uint64_t partner_u64(uint64_t v, P partner) {
    return ((uint64_t)partner((uint32_t)(v >> 32)) << 32) | partner((uint32_t)v);
}

// Wave-wide maximum of a 64-bit value (uniform result): DPP butterflies within rows of 16 lanes,
// then the row broadcasts (lane 15 of a row into the next row, lane 31 into the upper two rows)
// leave the maximum in lane 63, which is read once.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp_keep_u64(uint64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)v, (int)(uint32_t)v, CTRL, ROWS, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)(v >> 32), (int)(uint32_t)(v >> 32), CTRL,
                                                              ROWS, 0xF, false);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    uint64_t w;
    w = partner_u64(v, [](uint32_t u) { return seg_partner_u32<1>(u); });
    v = w > v ? w : v;
    w = partner_u64(v, [](uint32_t u) { return seg_partner_u32<2>(u); });
    v = w > v ? w : v;
    w = partner_u64(v, [](uint32_t u) { return seg_partner_u32<4>(u); });
    v = w > v ? w : v;
    w = partner_u64(v, [](uint32_t u) { return seg_partner_u32<8>(u); });
    v = w > v ? w : v;
    w = dpp_keep_u64<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v = w > v ? w : v;
    w = dpp_keep_u64<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    v = w > v ? w : v;
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), 63) << 32) |
           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
}

// Exact routing of token `tok` by the whole wave, from its row in global memory: lane l takes
// experts [l*NPL, (l+1)*NPL); a key is the correctly rounded sigmoid plus the bias, ordered by
// (key desc, expert asc) as one 64-bit word; group scores (binary32 sums of the top keys) and
// ranks (score desc, group asc) as in the fast path but exact; then K rounds of a wave-wide
// arg-max over the heads of the lanes' sorted keys.  Writes the K ids and weights.  It runs after
// the streaming loop, so inlined there its registers do not add to the loop's.
template <int LPT, bool BF16, int MODE>
__device__ __forceinline__ void exact_token_sig(const void* logits, const float* bias, int32_t* ids,
                                             float* weights, int K, int group_topn, int renormalize,
                                             float scale, int64_t tok, int tg, int wl,
                                             const u32x4* lds_row, int (&sel)[1]) {
    constexpr int E = kFastEPL * LPT;
    constexpr int NPL = E / 64;    // 1, 2, 4 or 8 experts per lane
    constexpr int S = 32 / NPL;    // lanes per group of 32 experts
    // the token's row: a copy in LDS (`lds_row`, plain layout), else read again from global memory
    const MEP_GLOBAL char* rb = gptr(reinterpret_cast<const char*>(logits)) + tok * E * (BF16 ? 2 : 4);
    const char* lb = reinterpret_cast<const char*>(lds_row);
    auto logit = [&](int e) -> float {
        if (lb) {
            if constexpr (BF16)
                return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(lb)[e] << 16);
            else
                return reinterpret_cast<const float*>(lb)[e];
        }
        if constexpr (BF16)
            return __uint_as_float((uint32_t)reinterpret_cast<const MEP_GLOBAL uint16_t*>(rb)[e] << 16);
        else
            return reinterpret_cast<const MEP_GLOBAL float*>(rb)[e];
    };
    // every load first (the sigmoid's rare slow path is a call, which later loads could not pass)
    float xs[NPL], bs[NPL], sv[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        xs[i] = logit(wl * NPL + i);
        bs[i] = gptr(bias)[wl * NPL + i];
    }
    // the correctly rounded sigmoids: every fast path first (independent chains the compiler can
    // interleave), then the rare values the binary64 interval could not decide
    bool ok[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) sv[i] = sigmoid_cr_fast(xs[i], ok[i]);
#pragma unroll
    for (int i = 0; i < NPL; ++i)
        if (!ok[i]) sv[i] = sigmoid_cr_slow(xs[i]);
    uint64_t P[NPL];  // the lane's keys, sorted descending
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int e = wl * NPL + i;
        const float key = sv[i] + bs[i];
        uint64_t v = ((uint64_t)order_key(key) << 32) | (uint32_t)~(uint32_t)e;
#pragma unroll
        for (int j = 0; j < i; ++j) {  // insertion into the sorted prefix
            const uint64_t hi = P[j] > v ? P[j] : v;
            v = P[j] > v ? v : P[j];
            P[j] = hi;
        }
        P[i] = v;
    }
    bool kept = true;
    if constexpr (MODE == 1) {
        uint64_t t1 = P[0], t2 = NPL > 1 ? P[NPL > 1 ? 1 : 0] : 0;  // the group's two largest keys
        auto merge = [&](auto partner) {
            const uint64_t b1 = partner_u64(t1, partner), b2 = partner_u64(t2, partner);
            const uint64_t lo = t1 < b1 ? t1 : b1;
            const uint64_t hi2 = t2 > b2 ? t2 : b2;
            t2 = lo > hi2 ? lo : hi2;
            t1 = t1 > b1 ? t1 : b1;
        };
        if constexpr (S >= 2) merge([](uint32_t u) { return seg_partner_u32<1>(u); });
        if constexpr (S >= 4) merge([](uint32_t u) { return seg_partner_u32<2>(u); });
        if constexpr (S >= 8) merge([](uint32_t u) { return seg_partner_u32<4>(u); });
        if constexpr (S >= 16) merge([](uint32_t u) { return seg_partner_u32<8>(u); });
        if constexpr (S >= 32) merge([](uint32_t u) { return seg_partner_u32<16>(u); });
        const float f1 = order_key_inv((uint32_t)(t1 >> 32));
        const float score = group_topn >= 2 ? f1 + order_key_inv((uint32_t)(t2 >> 32)) : f1;
        const int g = wl / S;
        const uint64_t gk = ((uint64_t)order_key(score) << 32) | (uint32_t)~(uint32_t)g;
        int rank = 0;
#pragma unroll
        for (int h = 0; h < LPT; ++h) {
            const uint64_t gh = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(gk >> 32), h * S) << 32) |
                                (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)gk, h * S);
            rank += gh > gk ? 1 : 0;
        }
        kept = rank < tg;
    }
    if (!kept) {
#pragma unroll
        for (int i = 0; i < NPL; ++i) P[i] = 0;  // 0 is below every key
    }
    int my_e = 0;
    for (int r = 0; r < K; ++r) {
        const uint64_t mx = wave_max_u64(P[0]);
        const bool win = P[0] == mx;
#pragma unroll
        for (int i = 0; i < NPL - 1; ++i) P[i] = win ? P[i + 1] : P[i];
        P[NPL - 1] = win ? 0 : P[NPL - 1];
        if (wl == r) my_e = (int)~(uint32_t)mx;
    }
    // weights from the correctly rounded sigmoid of the selected experts (lanes 0..K-1), taken
    // from the lane that holds each
    float s_sel = 0.0f;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const float u = __shfl(sv[i], (my_e / NPL) & 63);
        s_sel = (my_e % NPL) == i ? u : s_sel;
    }
    const double v = wl < K ? (double)s_sel : 0.0;
    const double den = seg_allreduce<8>(v, 8, PartnerF64{}, [](double x, double y) { return x + y; });
    sel[0] = my_e;
    if (wl < K) {
        const double inv = renormalize ? (den > 0.0 ? recip_f64(den) : 0.0) : 1.0;
        gptr(ids)[tok * K + wl] = my_e;
        if (weights) gptr(weights)[tok * K + wl] = (float)((v * inv) * (double)scale);
    }
}

// ---- the kernel -----------------------------------------------------------------------------------

// Counting of a routed token set into the histogram rows of the fused layout + plan path
// (path.h): the segment's lanes hold the token's slots (KPL per lane, -1 where there is none).
template <int LPT, int KPL>
__device__ __forceinline__ void sig_count_token(const PathGeom& g, int eshift, int* row, const int (&e)[KPL],
                                                int lseg) {
    uint32_t m1 = 0u, m2 = 0u;
#pragma unroll
    for (int q = 0; q < KPL; ++q) {
        if (e[q] >= 0) {
            const uint32_t bit = 1u << (e[q] >> eshift);
            m2 |= m1 & bit;
            m1 |= bit;
        }
    }
#pragma unroll
    for (int q = 0; q < KPL; ++q)
        if (e[q] >= 0) atomicAdd(&row[e[q]], 1);
    if constexpr (LPT >= 2) {
        auto step = [&](auto partner) {
            const uint32_t b1 = partner(m1), b2 = partner(m2);
            path_mask_merge(m1, m2, b1, b2);
        };
        step([](uint32_t u) { return seg_partner_u32<1>(u); });
        if constexpr (LPT >= 4) step([](uint32_t u) { return seg_partner_u32<2>(u); });
        if constexpr (LPT >= 8) step([](uint32_t u) { return seg_partner_u32<4>(u); });
        if constexpr (LPT >= 16) step([](uint32_t u) { return seg_partner_u32<8>(u); });
    }
    path_count_ranks(g, row, m1, m2, lseg, LPT);
}

// Where the routing kernel counts: off (mep_route_topk), or into the rows of the plan tiles it
// owns, followed by the counting epilogue (the routing phase of the fused path).
struct SigEpi {
    int on;
    int eshift;  // log2(E / R): E = 32 * LPT is a power of two, hence so is every E / R
    PathGeom g;
    PathWs w;
    WsHeader* hdr;
};

// Dynamic LDS of the kernel: uncertified-token bits per set, then (counting) the tile rows.
__host__ __device__ constexpr size_t sig_dyn_lds(int64_t sets_per_group, int sub, int nc) {
    return (size_t)sets_per_group * 4 + (size_t)sub * nc * 4;
}

// MODE 0: no group limit; MODE 1: lane lseg of a segment is group lseg (n_group == LPT).
// NW waves per workgroup.  A workgroup owns the contiguous tokens [t0, t1) -- with counting on,
// the plan tiles [blockIdx * sub, ...) -- cut into sets of TPW tokens, and its waves take sets one
// at a time from an LDS counter: every wave requests its first set at once, and a wave whose data
// arrives early takes more sets, so the workgroup ends when its last set is routed rather than
// when its slowest wave is.  Uncertified tokens are redone after the loop, spread over all the
// waves.
template <int LPT, bool BF16, int MODE, int NW>
__global__ __launch_bounds__(64 * NW) void route_sig_kernel(RouteArgs a, SigCfg cfg, SigEpi ep) {
    using G = SigGeom<LPT, BF16>;
    constexpr int W = G::W;
    constexpr int CPL = G::CPL;
    constexpr int CPR = G::CPR;
    constexpr int RS = G::RS;
    constexpr int TPW = G::TPW;
    constexpr int NE = kFastEPL;
    constexpr int KMAX = 8;
    constexpr int KPL = (KMAX + LPT - 1) / LPT;
    static_assert(CPL * W == NE, "32 experts per lane");
    static_assert(FastGeom<LPT, BF16>::TPW == TPW && FastGeom<LPT, BF16>::CPL == CPL, "load geometry");

    constexpr int NT = 64 * NW;
    __shared__ u32x4 s_rows[NW][TPW * RS];
    __shared__ float4 s_bsh4[LPT * kFastEPL / 4];  // b - c
    __shared__ float s_bconst[2];                   // constant terms of the two margins
    __shared__ int s_next;                          // next unclaimed set of this workgroup
    __shared__ int s_tb[kPathMaxSub + 1];           // token boundaries of the owned plan tiles
    extern __shared__ uint32_t s_dyn[];

    const int tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the set loop is not divergent
    const int wl = tid & 63;
    const int tw = wl / LPT;
    const int lseg = wl % LPT;
    const int K = a.K;
    const bool epi = ep.on != 0;

    // ---- this workgroup's tokens (N * K < 2^31, so token indices fit 32 bits) --------------------
    int t0, t1;
    int nsub = 0;
    if (epi) {
        const int j0 = blockIdx.x * ep.g.sub;
        nsub = min(ep.g.sub, ep.g.ntiles - j0);
        int64_t a0, a1, b0, b1;
        path_tile_tokens(ep.g, j0, a0, a1);
        path_tile_tokens(ep.g, j0 + nsub - 1, b0, b1);
        t0 = (int)a0;
        t1 = (int)b1;
        if (tid <= nsub) {
            int64_t c0, c1;
            path_tile_tokens(ep.g, j0 + min(tid, nsub - 1), c0, c1);
            s_tb[tid] = (int)(tid < nsub ? c0 : c1);
        }
    } else {
        t0 = blockIdx.x * (int)cfg.tokens_per_group;
        t1 = (int)min((int64_t)t0 + cfg.tokens_per_group, a.N);
    }
    t0 = __builtin_amdgcn_readfirstlane(t0);
    t1 = __builtin_amdgcn_readfirstlane(t1);
    const int nsets = (t1 - t0 + TPW - 1) / TPW;
    uint32_t* s_fail = s_dyn;          // per set: tokens the filter could not certify (bit t)
    int* s_row = reinterpret_cast<int*>(s_dyn + nsets);  // counting: the tile rows
    for (int i = tid; i < nsets; i += NT) s_fail[i] = 0u;
    if (epi)
        for (int i = tid; i < nsub * ep.g.NC; i += NT) s_row[i] = 0;
    if (tid == 0) s_next = NW;
    const uint32_t pcall = epi ? path_count_begin(ep.hdr) : 0u;

    // the bias first (so that waiting for it does not also wait for the logits), then the first set
    constexpr int BPL = LPT * NE / 64;  // bias entries per lane
    const MEP_GLOBAL float* gb = gptr(a.bias);
    float bv[BPL];
#pragma unroll
    for (int i = 0; i < BPL; ++i) bv[i] = gb[i * 64 + wl];
    __builtin_amdgcn_sched_barrier(0);  // keep the bias loads ahead of the logits loads
    const MEP_GLOBAL u32x4* lbase = gptr(reinterpret_cast<const u32x4*>(a.logits));
    // the CPL coalesced 16-byte loads of the set starting at token ts (rows past t1 re-read row
    // t1 - 1); a wave without a set of its own loads set 0 again, unused, so that the loads in
    // flight are the same on every path into the loop
    auto load_set = [&](int set, u32x4 (&b)[CPL]) {
        const int ts = t0 + set * TPW;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int q = c * 64 + wl;
            const int r = q / CPR;
            const int t = min(ts + r, t1 - 1);
            b[c] = lbase[(int64_t)t * CPR + (q - r * CPR)];
        }
    };
    u32x4 buf[CPL];
    load_set(wv < nsets ? wv : 0, buf);

    // ---- shift c, the error-bound constants, and the shifted biases --------------------------------
    float mb = 0.0f;
#pragma unroll
    for (int i = 0; i < BPL; ++i) mb = fmaxf(mb, fabsf(bv[i]));
    const float maxb = wave_max_nonneg(mb);
    const bool finite = maxb < 0x1p20f;  // false for inf / NaN: every token takes the exact path
    const float c = 1.0f + maxb + 0x1p-10f;
    const float a_gap = (float)(0x1p-18 * (1.0 + 0x1p-17) * (1.0 + 0x1p-19));
    const float a_grp = (float)((0x1p-18 * (1.0 + 0x1p-10) + 0x1p-24 + 0x1p-19) * (1.0 + 0x1p-19));
    if (tid == 0) {
        double H = 1.0;
        for (int i = 0; i < 24 && H < (double)c + (double)maxb; ++i) H *= 2.0;
        const double D = (3.48 + 0.75 * H) * 0x1p-23;
        s_bconst[0] = (float)(2.0 * D * (1.0 + 0x1p-19));
        s_bconst[1] = (float)((4.0 * D + 2.0 * H * 0x1p-24) * (1.0 + 0x1p-19));
    }
    const int e0 = lseg * NE;
    if (wv == 0) {
#pragma unroll
        for (int i = 0; i < BPL; ++i) reinterpret_cast<float*>(s_bsh4)[i * 64 + wl] = bv[i] - c;
    }
    __syncthreads();

    u32x4* my_rows = s_rows[wv];
    const u32x4* my_row = &my_rows[tw * RS];
    const u32x4* my_chunks = &my_row[lseg * G::GS];
    auto row_logit = [&](int e) -> float {
        const char* p = reinterpret_cast<const char*>(&my_row[G::pos(e / W)]) + (e % W) * (BF16 ? 2 : 4);
        if constexpr (BF16)
            return __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t*>(p)) << 16);
        else
            return *reinterpret_cast<const float*>(p);
    };
    // tagged keys (bit patterns) of the lane's chunk j: experts e0 + j * W + i
    auto chunk_keys = [&](int j, int (&k)[W]) {
        const u32x4 v = my_chunks[j];
        float x[W];
        if constexpr (BF16) {
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                x[2 * q] = __uint_as_float(w4[q] << 16);
                x[2 * q + 1] = __uint_as_float(w4[q] & 0xFFFF0000u);
            }
        } else {
            x[0] = __uint_as_float(v.x);
            x[1] = __uint_as_float(v.y);
            x[2] = __uint_as_float(v.z);
            x[3] = __uint_as_float(v.w);
        }
#pragma unroll
        for (int h = 0; h < W / 4; ++h) {
            const float4 b = s_bsh4[(e0 + j * W) / 4 + h];
            const float bb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                k[4 * h + i] = (int)((__float_as_uint(sigmoid_fast(x[4 * h + i]) + bb[i]) & ~31u) |
                                     (uint32_t)(j * W + 4 * h + i));
        }
    };

    int next_set = wv;
    for (int set = wv; set < nsets; set = next_set) {
        // ---- registers -> this wave's LDS rows; refill with the next set --------------------------
        wave_lds_sync();
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            const int q = cc * 64 + wl;
            const int r = q / CPR;
            my_rows[r * RS + G::pos(q - r * CPR)] = buf[cc];
        }
        {
            int claimed = 0;
            if (wl == 0) claimed = atomicAdd(&s_next, 1);
            next_set = __builtin_amdgcn_readfirstlane(claimed);
        }
        if (next_set < nsets) load_set(next_set, buf);
        wave_lds_sync();

        const int tok_raw = t0 + set * TPW + tw;
        const bool live = tok_raw < t1;
        const int tok = live ? tok_raw : t1 - 1;
        const float b_gap = lds_volatile_load(&s_bconst[0]);
        const float b_grp = lds_volatile_load(&s_bconst[1]);

        // ---- keys and the lane's top list ------------------------------------------------------
        int L[kSigT];
#pragma unroll
        for (int i = 0; i < kSigT; ++i) L[i] = kSigEmpty;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            int k[W];
            chunk_keys(j, k);
#pragma unroll
            for (int i = 0; i < W; ++i) list_insert(L, k[i]);
        }
        bool fail = !finite;

        // ---- groups ----------------------------------------------------------------------------
        if constexpr (MODE == 1) {
            // group index in the low bits: a lower index is a smaller magnitude, a larger value
            constexpr uint32_t gmask = LPT > 8 ? 15u : 7u;
            const float s01 = a.group_topn >= 2 ? __int_as_float(L[0]) + __int_as_float(L[1]) : __int_as_float(L[0]);
            const int gs = (int)((__float_as_uint(s01) & ~gmask) | (uint32_t)lseg);
            int rank = 0;
            static_for<LPT>([&](auto oc) {
                constexpr int o = decltype(oc)::value;
                if constexpr (o > 0) rank += (int)seg_xor_u32<o>((uint32_t)gs) < gs ? 1 : 0;
            });
            const bool kept = rank < cfg.tg;
            if (cfg.tg < LPT) {
                const float lk = __int_as_float(seg_max_i32<LPT>(kept ? gs : INT_MIN));  // lowest kept
                const float hr = __int_as_float(seg_min_i32<LPT>(kept ? INT_MAX : gs));  // highest dropped
                fail = fail || !(lk - hr > fmaf(-(lk + hr), a_grp, b_grp));
            }
#pragma unroll
            for (int i = 0; i < kSigT; ++i) L[i] = kept ? L[i] : kSigEmpty;
        }

        // ---- K + 1 extraction rounds ---------------------------------------------------------------
        // All KMAX + 1 rounds run whatever K is (rounds past K only feed bits that are masked off),
        // so no round depends on a run-time condition.  `slot_bits` marks this lane's output slots;
        // it is derived from the set index (the shift is always 0) so that the compiler forms the
        // per-round lane tests inside the loop instead of hoisting them all into scalar registers.
        const uint32_t slot_bits = (1u << lseg) << (uint32_t)(set >> 30);
        uint32_t wm = 0;      // rounds this lane won
        uint32_t gapbad = 0;  // rounds whose value is too close to the previous one
        int myM[KPL];         // value extracted in round lseg + q * LPT
        int myW[KPL];         // lane (within the segment) that won that round
#pragma unroll
        for (int q = 0; q < KPL; ++q) {
            myM[q] = kSigEmpty;
            myW[q] = 0;
        }
        int prev = 0;
        static_for<KMAX + 1>([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            const int m = seg_min_i32<LPT>(L[0]);
            const bool win = L[0] == m;
            if constexpr (r < KMAX) {
                const int wr = seg_max_i32<LPT>(win ? lseg : 0);
                constexpr int q = r / LPT;
                const bool mine = (slot_bits >> (r - q * LPT)) & 1u;
                myM[q] = mine ? m : myM[q];
                myW[q] = mine ? wr : myW[q];
            }
            if constexpr (r > 0) {
                // certification of the order: consecutive extracted values far enough apart
                const float fp = __int_as_float(prev), fm = __int_as_float(m);
                gapbad |= (fp - fm > fmaf(-(fp + fm), a_gap, b_gap)) ? 0u : (1u << r);
            }
            prev = m;
#pragma unroll
            for (int i = 0; i < kSigT - 1; ++i) L[i] = win ? L[i + 1] : L[i];
            L[kSigT - 1] = win ? kSigEmpty : L[kSigT - 1];
            wm |= win ? (1u << r) : 0u;
        });
        // every round up to K had exactly one winner in the segment, consecutive values were far
        // enough apart, and no list ran dry before round K (a group holding more than kSigT of the
        // top K + 1 is left to the exact path)
        const uint32_t all = (2u << K) - 1u;
        wm &= all;
        const int nw = __popc(wm);
        if ((gapbad & all) != 0u) fail = true;
        if (nw >= kSigT && (wm >> K) == 0u) fail = true;
        if (seg_or_u32<LPT>(wm) != all || seg_add_u32<LPT>((uint32_t)nw) != (uint32_t)(K + 1)) fail = true;

        // ---- experts of this lane's output slots, weights ------------------------------------------
        int my_e[KPL];
        double my_v[KPL];
#pragma unroll
        for (int q = 0; q < KPL; ++q) {
            const int j = lseg + q * LPT;
            const int e = myW[q] * NE + (int)((uint32_t)myM[q] & 31u);
            my_e[q] = e;
            my_v[q] = j < K ? sigmoid_f64_weight(row_logit(e)) : 0.0;
        }
        fail = seg_or_u32<LPT>(fail ? 1u : 0u) != 0u;
        // (v / sum(v)) * scale (renormalised) or v * scale, in binary64, rounded once
        double den = 0.0;
#pragma unroll
        for (int q = 0; q < KPL; ++q) den += my_v[q];
        den = seg_allreduce<LPT>(den, LPT, PartnerF64{}, [](double u, double w) { return u + w; });
        const double inv = a.renormalize ? (den > 0.0 ? recip_f64(den) : 0.0) : 1.0;
        if (live && !fail) {
#pragma unroll
            for (int q = 0; q < KPL; ++q) {
                const int j = lseg + q * LPT;
                if (j < K) {
                    // streaming stores: nothing in this kernel reads them back
                    __builtin_nontemporal_store(my_e[q], gptr(a.ids) + tok * K + j);
                    if (a.weights)
                        __builtin_nontemporal_store((float)((my_v[q] * inv) * (double)a.scale), gptr(a.weights) + tok * K + j);
                }
            }
        }
        // ---- counting (fused path): certified live tokens now, the others after the exact pass ----
        if (epi) {
            int ce[KPL];
#pragma unroll
            for (int q = 0; q < KPL; ++q) ce[q] = (live && !fail && lseg + q * LPT < K) ? my_e[q] : -1;
            int ri = 0;
            while (ri + 1 < nsub && tok >= s_tb[ri + 1]) ++ri;
            sig_count_token<LPT, KPL>(ep.g, ep.eshift, s_row + ri * ep.g.NC, ce, lseg);
        }

        // ---- uncertified tokens: recorded for the exact pass after the loop ------------------------
        const uint64_t fm = __ballot(fail && live && lseg == 0);
        if (fm != 0ull && wl == 0) {
            uint32_t m = 0u;
#pragma unroll
            for (int t = 0; t < TPW; ++t) m |= (uint32_t)((fm >> (t * LPT)) & 1ull) << t;
            s_fail[set] = m;
        }
    }

    // ---- uncertified tokens of this workgroup's sets: exact, one token per wave in turn ----------
    // The sets' failure words are read 64 at a time, one per lane, and only the non-zero ones are
    // visited (a serial scan of the words would be a chain of LDS round trips).
    __syncthreads();
    int idx = 0;
    for (int i0 = 0; i0 < nsets; i0 += 64) {
        const uint32_t mine = i0 + wl < nsets ? s_fail[i0 + wl] : 0u;
        uint64_t any = __ballot(mine != 0u);
        while (any) {
            const int l = __builtin_ctzll(any);
            any &= any - 1ull;
            uint32_t m = (uint32_t)__builtin_amdgcn_readlane((int)mine, l);
            const int i = i0 + l;
            while (m) {
                const int t = __builtin_ctz(m);
                m &= m - 1u;
                if (idx % NW == wv) {
                    const int tok = t0 + i * TPW + t;
                    int sel[1];
                    exact_token_sig<LPT, BF16, MODE>(a.logits, a.bias, a.ids, a.weights, K, a.group_topn,
                                                     a.renormalize, a.scale, tok, cfg.tg, wl, nullptr, sel);
                    if (epi) {
                        int ri = 0;
                        while (ri + 1 < nsub && tok >= s_tb[ri + 1]) ++ri;
                        int ce[1] = {wl < K ? sel[0] : -1};
                        // the token's slots are on lanes 0..K-1 (K <= 8): an 8-lane segment
                        if (wl < 8) sig_count_token<8, 1>(ep.g, ep.eshift, s_row + ri * ep.g.NC, ce, wl);
                    }
                }
                ++idx;
            }
        }
    }
    if (epi) path_epilogue<NT>(ep.g, ep.w, pcall, s_row);
}

}  // namespace mep
