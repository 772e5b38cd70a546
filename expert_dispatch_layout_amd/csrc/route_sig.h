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
//   2. a sorted list of the lane's 5 largest keys, one med3 per entry and key;
//   3. group score = sum of the group's top keys (list entries 0 and 1), with the group index in
//      its 3 (4 for 16 groups) low significand bits so that a lower index wins a tie; the rank of
//      each group among the segment's groups from the other lanes' scores (DPP),
//      kept = rank < topk_group;
//   4. K + 1 extraction rounds over the kept lanes' list heads (segment max through DPP); the
//      winning lane pops its head; a lane that empties its list refills it from its keys below
//      the value it last gave up (rare: a group holding more than 5 of the top K + 1);
//   5. certification: the selection on the exact keys (correctly rounded sigmoid plus bias, both
//      binary32) is the same when the last kept and first dropped group scores, and each pair
//      of consecutive extracted keys, differ by more than the error bounds below, and every
//      round had exactly one winner.  A token that fails is redone at once by the whole wave
//      from the row still in LDS, on exact keys (exact_token_sig).
// The K selected experts then get the correctly rounded sigmoid in binary64 and the weights.
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

#include "route_fast.h"

namespace mep {

constexpr int kSigT = 5;                          // list depth per lane
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

struct SigCfg {
    int64_t nsets;  // token sets of 64 / LPT tokens
    int tg;         // groups kept (MODE 1)
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

// Wave-wide maximum of a 64-bit value (uniform result): DPP within rows of 16 lanes, then the
// four row maxima through lane reads.
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
    uint64_t r = 0;
#pragma unroll
    for (int row = 0; row < 4; ++row) {
        const uint64_t x = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), row * 16) << 32) |
                           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, row * 16);
        r = x > r ? x : r;
    }
    return r;
}

// Exact routing of token `tok` whose row is at `row` in LDS (SigGeom layout), by the whole wave:
// lane l takes experts [l*NPL, (l+1)*NPL); a key is the correctly rounded sigmoid plus the bias,
// ordered by (key desc, expert asc) as one 64-bit word; group scores (binary32 sums of the top
// keys) and ranks (score desc, group asc) as in the fast path but exact; then K rounds of a
// wave-wide arg-max.  Writes the K ids and weights.
template <int LPT, bool BF16, int MODE>
__device__ __forceinline__ void exact_token_sig(const RouteArgs& a, const u32x4* row, int64_t tok,
                                                int tg, int wl) {
    using G = SigGeom<LPT, BF16>;
    constexpr int W = G::W;
    constexpr int E = kFastEPL * LPT;
    constexpr int NPL = E / 64;    // 1, 2, 4 or 8 experts per lane
    constexpr int S = 32 / NPL;    // lanes per group of 32 experts
    const int K = a.K;
    const char* rb = reinterpret_cast<const char*>(row);
    uint64_t pk[NPL];
    float sg[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int e = wl * NPL + i;
        const char* p = rb + G::pos(e / W) * 16 + (e % W) * (BF16 ? 2 : 4);
        const float x = BF16 ? __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t*>(p)) << 16)
                             : *reinterpret_cast<const float*>(p);
        sg[i] = sigmoid_cr(x);
        const float key = sg[i] + gptr(a.bias)[e];
        pk[i] = ((uint64_t)order_key(key) << 32) | (uint32_t)~(uint32_t)e;
    }
    bool kept = true;
    if constexpr (MODE == 1) {
        uint64_t t1 = 0, t2 = 0;  // the group's two largest keys (0 is below every key)
#pragma unroll
        for (int i = 0; i < NPL; ++i) {
            const uint64_t v = pk[i];
            const uint64_t lo = v < t1 ? v : t1;
            t2 = lo > t2 ? lo : t2;
            t1 = v > t1 ? v : t1;
        }
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
        const float score = a.group_topn >= 2 ? f1 + order_key_inv((uint32_t)(t2 >> 32)) : f1;
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
    uint32_t taken = 0;
    int my_e = 0;
    float my_s = 0.0f;
    double den = 0.0;
    for (int r = 0; r < K; ++r) {
        uint64_t best = 0;
        int bi = -1;
        float bs = 0.0f;
#pragma unroll
        for (int i = 0; i < NPL; ++i) {
            if (kept && !((taken >> i) & 1u) && pk[i] > best) {
                best = pk[i];
                bi = i;
                bs = sg[i];
            }
        }
        const uint64_t mx = wave_max_u64(best);
        const bool win = bi >= 0 && best == mx;
        if (win) taken |= 1u << bi;
        const uint64_t wmask = __ballot(win);
        const int wlane = wmask ? __builtin_ctzll(wmask) : 0;
        const float s_r = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(bs), wlane));
        const int e_r = (int)~(uint32_t)mx;
        den += (double)s_r;
        if (wl == r) {
            my_e = e_r;
            my_s = s_r;
        }
    }
    if (wl < K) {
        const double inv = a.renormalize ? (den > 0.0 ? recip_f64(den) : 0.0) : 1.0;
        gptr(a.ids)[tok * K + wl] = my_e;
        if (a.weights) gptr(a.weights)[tok * K + wl] = (float)(((double)my_s * inv) * (double)a.scale);
    }
}

// ---- the kernel -----------------------------------------------------------------------------------

// MODE 0: no group limit; MODE 1: lane lseg of a segment is group lseg (n_group == LPT).
template <int LPT, bool BF16, int MODE>
__global__ __launch_bounds__(kFastBlock, BF16 ? 4 : 3) void route_sig_kernel(RouteArgs a, SigCfg cfg) {
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

    __shared__ u32x4 s_rows[kFastWaves][TPW * RS];
    __shared__ float4 s_bsh4[LPT * kFastEPL / 4];  // b - c
    __shared__ float s_bconst[2];                   // constant terms of the two margins

    const int tid = threadIdx.x;
    const int wv = tid >> 6;
    const int wl = tid & 63;
    const int tw = wl / LPT;
    const int lseg = wl % LPT;
    const int K = a.K;
    const int64_t waves = (int64_t)gridDim.x * kFastWaves;
    const int64_t first_set = (int64_t)blockIdx.x * kFastWaves + wv;

    u32x4 buf[CPL];
    if (first_set < cfg.nsets) fast_load_set<LPT, BF16>(a, first_set, wl, buf);

    // ---- shift c, the error-bound constants, and the shifted biases --------------------------------
    const MEP_GLOBAL float* gb = gptr(a.bias);
    float mb = 0.0f;
    for (int e = wl; e < LPT * NE; e += 64) mb = fmaxf(mb, fabsf(gb[e]));
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
    for (int e = tid; e < LPT * NE; e += kFastBlock) reinterpret_cast<float*>(s_bsh4)[e] = gb[e] - c;
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

    for (int64_t set = first_set; set < cfg.nsets; set += waves) {
        // ---- registers -> this wave's LDS rows; refill with the next set --------------------------
        wave_lds_sync();
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            const int q = cc * 64 + wl;
            const int r = q / CPR;
            my_rows[r * RS + G::pos(q - r * CPR)] = buf[cc];
        }
        if (set + waves < cfg.nsets) fast_load_set<LPT, BF16>(a, set + waves, wl, buf);
        wave_lds_sync();

        const int64_t tok_raw = set * TPW + tw;
        const bool live = tok_raw < a.N;
        const int64_t tok = live ? tok_raw : (a.N - 1);
        const float b_gap = *reinterpret_cast<volatile const float*>(&s_bconst[0]);
        const float b_grp = *reinterpret_cast<volatile const float*>(&s_bconst[1]);

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
        uint32_t wm = 0;  // rounds this lane won
        int wins = 0;
        int myM[KPL];     // extracted value of round lseg + q * LPT
#pragma unroll
        for (int q = 0; q < KPL; ++q) myM[q] = kSigEmpty;
        int prev = 0;
#pragma unroll 1
        for (int r = 0; r <= K; ++r) {
            const int m = seg_min_i32<LPT>(L[0]);
#pragma unroll
            for (int q = 0; q < KPL; ++q) myM[q] = (r == lseg + q * LPT) ? m : myM[q];
            if (r > 0) {
                const float fp = __int_as_float(prev), fm = __int_as_float(m);
                fail = fail || !(fp - fm > fmaf(-(fp + fm), a_gap, b_gap));
            }
            prev = m;
            const bool win = L[0] == m;
#pragma unroll
            for (int i = 0; i < kSigT - 1; ++i) L[i] = win ? L[i + 1] : L[i];
            L[kSigT - 1] = win ? kSigEmpty : L[kSigT - 1];
            wins += win ? 1 : 0;
            wm |= win ? (1u << r) : 0u;
            const bool empty = win && wins == kSigT && r < K;
            if (__ballot(empty) != 0ull) {
                if (empty) {
                    // the lane's keys below the value it just gave up
#pragma unroll 1
                    for (int j = 0; j < CPL; ++j) {
                        int k[W];
                        chunk_keys(j, k);
#pragma unroll
                        for (int i = 0; i < W; ++i)
                            if (k[i] > m) list_insert(L, k[i]);
                    }
                }
            }
        }
        // every round had exactly one winner in the segment
        const uint32_t all = (2u << K) - 1u;
        if (seg_or_u32<LPT>(wm) != all || seg_add_u32<LPT>((uint32_t)__popc(wm)) != (uint32_t)(K + 1))
            fail = true;

        // ---- experts of this lane's output slots, weights ------------------------------------------
        int wlane[KPL];
#pragma unroll
        for (int q = 0; q < KPL; ++q) wlane[q] = 0;
        static_for<LPT>([&](auto oc) {
            constexpr int o = decltype(oc)::value;
            const uint32_t wo = seg_xor_u32<o>(wm);
#pragma unroll
            for (int q = 0; q < KPL; ++q)
                if ((wo >> (lseg + q * LPT)) & 1u) wlane[q] = lseg ^ o;
        });
        int my_e[KPL];
        float my_v[KPL];
#pragma unroll
        for (int q = 0; q < KPL; ++q) {
            const int j = lseg + q * LPT;
            const int e = wlane[q] * NE + (int)((uint32_t)myM[q] & 31u);
            my_e[q] = e;
            float v = 0.0f;
            if (j < K) {
                bool ok;
                v = sigmoid_cr_fast(row_logit(e), ok);
                fail = fail || !ok;
            }
            my_v[q] = v;
        }
        fail = seg_or_u32<LPT>(fail ? 1u : 0u) != 0u;
        // (v / sum(v)) * scale (renormalised) or v * scale, in binary64, rounded once
        double den = 0.0;
#pragma unroll
        for (int q = 0; q < KPL; ++q) den += (double)my_v[q];
        den = seg_allreduce<LPT>(den, LPT, PartnerF64{}, [](double u, double w) { return u + w; });
        const double inv = a.renormalize ? (den > 0.0 ? recip_f64(den) : 0.0) : 1.0;
        if (live && !fail) {
#pragma unroll
            for (int q = 0; q < KPL; ++q) {
                const int j = lseg + q * LPT;
                if (j < K) {
                    gptr(a.ids)[tok * K + j] = my_e[q];
                    if (a.weights) gptr(a.weights)[tok * K + j] = (float)(((double)my_v[q] * inv) * (double)a.scale);
                }
            }
        }

        // ---- uncertified tokens: exact, by the whole wave, from the row in LDS ------------------------
        uint64_t fm = __ballot(fail && live && lseg == 0);
        while (fm) {
            const int t = __builtin_ctzll(fm) / LPT;
            fm &= fm - 1;
            exact_token_sig<LPT, BF16, MODE>(a, &my_rows[t * RS], set * TPW + t, cfg.tg, wl);
        }
    }
}

}  // namespace mep
