// Fast routing kernel: selection on binary32 keys with a certified error bound.
//
// Memory pipeline.  The grid is sized to the resident capacity of the GPU and every wave walks
// token sets s = wave, wave + waves, ...  A set is 64/LPT consecutive tokens, i.e. one contiguous
// run of the logits (8 KiB of fp32 or 4 KiB of bf16 rows), fetched with one 16-byte load per lane
// and instruction (1 KiB per instruction, fully coalesced) into registers.  Loads run one set
// ahead: the registers of a set are copied into the wave's private LDS row area, then
// immediately refilled with the wave's next set while the current set is computed.  No block
// barrier is taken after the prologue: all exchange between the lanes of a token stays inside
// one wave (DPP, or LDS written and read by the same wave in program order).
//
// Selection per token (E/32 lanes, lane g owns experts [32g, 32g + 32), read back from LDS in a
// bank-rotated order):
//   1. keys k (sigmoid scoring: s~ = 1/(1 + 2^(-x log2 e)) with v_exp_f32 / v_rcp_f32, plus
//      the bias; softmax scoring: the logit itself, which is exact);
//   2. per group (or per lane when there is no group limit) the M largest keys, combined
//      across the group's lanes with DPP; group score = sum of the top group_topn keys;
//   3. groups kept by (score desc, group index asc); threshold tau = the smallest M'-th best
//      key of a kept unit, M' = ceil(K / units), so at least K keys are >= tau;
//   4. keys >= tau (less the error margin) go to a per-token candidate list in LDS; each
//      candidate's rank is the number of candidates that beat it (key desc, expert asc),
//      which orders the top-K;
//   5. certification (sigmoid scoring): with delta a proven bound on |k~ - k|, the selection
//      on k~ equals the selection on the exact keys if the TG-th and (TG+1)-th group scores
//      differ by more than 2*delta_group and each of the first K ranked keys exceeds the next
//      one by more than 2*delta.
// Tokens that fail (near-ties, list overflow, non-finite logits) are redone by the whole wave
// with exact keys (correctly rounded sigmoid + bias) and K rounds of a segmented arg-max.
// Only the K selected experts then get the correctly rounded sigmoid in binary64 for the
// weights.
//
// Error bound of the binary32 sigmoid, absolute and independent of x.  t = fl(x * c) with
// c = fl(-log2 e) equals -x log2(e) (1 + eta), |eta| <= 2^-23 + 2^-48; so 2^t = e^-x e^(-x eta).
// With v_exp_f32 and v_rcp_f32 taken as <= 2^-22 relative (the ISA documents 1 ulp) and the
// add 1 + e rounded once, to first order
//     |s~ - sigma| <= sigma (1 - sigma) (|x| 2^-23 + 2^-22) + sigma (2^-24 + 2^-22)
// and sigma (1 - sigma) |x| <= 0.224 for every x, so |s~ - sigma| <= 3.23 * 2^-23 (the second
// order terms are below 2^-40 since |x eta| <= 89 * 2^-23 whenever 2^t is finite and normal;
// outside that range s~ and sigma are both within 2^-126 of 0 or of 1).  The exact key rounds
// RN(sigma) + b and the fast key rounds s~ + b, each to binary32: with |key| <= 1 + max|b|,
// |k~ - k| <= 3.23 * 2^-23 + 2^-25 + (1 + max|b|) 2^-23 < (4 + (1 + max|b|)) 2^-23 = delta.
// A group score is a binary32 sum of two order statistics (each 1-Lipschitz in the keys), so
// |g~ - g| <= 2 delta + 2 (1 + max|b|) 2^-23 (+1%) = delta_group.
#pragma once

#include "route_common.h"

namespace mep {

// Candidate list length per token: a token whose keys above the threshold do not fit is redone
// on the slow exact path, which costs its wave far more than the rest of its set, so wide tokens
// (32 experts per lane and at least 4 lanes) get 64 entries; with 2 lanes the list stays at 32
// to keep the LDS of a workgroup's 128 tokens within budget.
template <int LPT>
constexpr int cand_cap() { return LPT >= 4 ? 64 : 32; }
constexpr int kFastEPL = 32;    // experts per lane
constexpr int kFastBlock = 256;  // four waves, each independent after the prologue
constexpr int kFastWaves = kFastBlock / 64;

__device__ __forceinline__ float sigmoid_fast(float x) {
    const float t = x * -1.44269504088896340736f;
    const float e = __builtin_amdgcn_exp2f(t);
    return __builtin_amdgcn_rcpf(1.0f + e);
}

// top-M (descending) of the union of two descending lists: the k-th largest is the max over
// splits i + j = k of min(a_i, b_j), with a_0 = b_0 = +inf.
template <int M>
__device__ __forceinline__ void merge_top(float (&a)[M], const float (&b)[M]) {
    float c[M];
#pragma unroll
    for (int k = 1; k <= M; ++k) {
        float best = fmaxf(a[k - 1], b[k - 1]);
#pragma unroll
        for (int i = 1; i < k; ++i) best = fmaxf(best, fminf(a[i - 1], b[k - i - 1]));
        c[k - 1] = best;
    }
#pragma unroll
    for (int k = 0; k < M; ++k) a[k] = c[k];
}

template <int M>
__device__ __forceinline__ void insert_top(float (&a)[M], float v) {
#pragma unroll
    for (int k = M - 1; k >= 1; --k) a[k] = fmaxf(a[k], fminf(a[k - 1], v));
    a[0] = fmaxf(a[0], v);
}

template <int M, int STEP>
__device__ __forceinline__ void merge_partner(float (&a)[M]) {
    float b[M];
#pragma unroll
    for (int k = 0; k < M; ++k) b[k] = seg_partner_f32<STEP>(a[k]);
    merge_top<M>(a, b);
}

// All-reduce of a top-M list over aligned segments of S lanes (run-time S <= SMAX).
template <int SMAX, int M>
__device__ __forceinline__ void seg_top_allreduce(float (&a)[M], int S) {
    if constexpr (SMAX >= 2) if (S >= 2) merge_partner<M, 1>(a);
    if constexpr (SMAX >= 4) if (S >= 4) merge_partner<M, 2>(a);
    if constexpr (SMAX >= 8) if (S >= 8) merge_partner<M, 4>(a);
    if constexpr (SMAX >= 16) if (S >= 16) merge_partner<M, 8>(a);
}

// Orders LDS accesses of this wave around a point (lanes of a token are one wave).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct FastCfg {
    int mode;   // 0: no group limit, 1: a group spans S lanes
    int S;      // lanes per group
    int log2S;
    int mt;     // M' = ceil(K / units): the unit's M'-th best key bounds the threshold
    int64_t nsets;  // token sets of 64/LPT tokens
};

__device__ __forceinline__ uint32_t seg_max_u32_dpp(uint32_t v, int S) {
    return seg_allreduce<16>(v, S, PartnerU32{}, [](uint32_t u, uint32_t w) { return max(u, w); });
}
__device__ __forceinline__ uint32_t seg_min_u32_dpp(uint32_t v, int S) {
    return seg_allreduce<16>(v, S, PartnerU32{}, [](uint32_t u, uint32_t w) { return min(u, w); });
}
__device__ __forceinline__ uint32_t seg_or_u32_dpp(uint32_t v, int S) {
    return seg_allreduce<16>(v, S, PartnerU32{}, [](uint32_t u, uint32_t w) { return u | w; });
}

// Wave-wide maximum of a non-negative float (bit order = value order).
__device__ __forceinline__ float wave_max_nonneg(float v) {
    uint32_t u = __float_as_uint(v);
    u = seg_allreduce<16>(u, 16, PartnerU32{}, [](uint32_t p, uint32_t q) { return max(p, q); });
    u = max(u, (uint32_t)__shfl_xor((int)u, 16));
    u = max(u, (uint32_t)__shfl_xor((int)u, 32));
    return __uint_as_float(u);
}

template <int LPT, bool BF16>
struct FastGeom {
    static constexpr int W = BF16 ? 8 : 4;        // experts per 16-byte chunk
    static constexpr int CPL = kFastEPL / W;      // chunks per lane (and loads per lane per set)
    static constexpr int CPR = LPT * CPL;         // chunks per row
    static constexpr int RS = CPR + LPT;          // row stride in chunks (padding spreads banks)
    static constexpr int TPW = 64 / LPT;          // tokens per set (one set per wave step)
    static constexpr int TPB = kFastWaves * TPW;  // token slots per block
};

// Issue the CPL coalesced 16-byte loads of token set `set` (rows are CPR 16-byte chunks, so a
// complete set is one contiguous run).  Rows past the last token re-read row N - 1.  One
// straight-line path: the loads of the two cases never compete for registers, so waiting for
// them never has to wait for other loads in flight.
template <int LPT, bool BF16>
__device__ __forceinline__ void fast_load_set(const RouteArgs& a, int64_t set, int wl,
                                              u32x4 (&buf)[FastGeom<LPT, BF16>::CPL]) {
    using G = FastGeom<LPT, BF16>;
    const MEP_GLOBAL u32x4* base = gptr(reinterpret_cast<const u32x4*>(a.logits));
    const int64_t t0 = set * G::TPW;
    const int64_t last = a.N - 1;
#pragma unroll
    for (int c = 0; c < G::CPL; ++c) {
        const int q = c * 64 + wl;  // chunk of the set
        const int r = q / G::CPR;   // its row (a shift: CPR is a power of two)
        const int64_t t = min(t0 + r, last);
        buf[c] = base[t * G::CPR + (q - r * G::CPR)];
    }
}

// Everything for one token by a whole wave, exactly: keys from the correctly rounded sigmoid,
// group limit, K rounds of a segmented arg-max, weights in binary64.  It runs only for the few
// tokens the binary32 filter cannot certify, after the streaming loop; out of line so that its
// registers do not count against the loop (the arguments are passed by value: a reference to a
// kernel argument would put a copy of it in scratch memory).
template <int LPT, bool BF16, int KMAX, int SCORE>
__device__ __noinline__ void exact_token_full(const RouteArgs a, const float* s_bias, int wl,
                                              int64_t tok) {
    constexpr int W = BF16 ? 8 : 4;
    constexpr int NV64 = (LPT * kFastEPL + 64 * W - 1) / (64 * W);
    constexpr int NE64 = NV64 * W;
    constexpr int KPL64 = (KMAX + 63) / 64;
    float x[NE64];
    load_row<64, NV64, BF16>(a, tok, wl, x);
    int e64[KPL64];
    float key[KPL64];
#pragma unroll
    for (int m = 0; m < KPL64; ++m) {
        e64[m] = 0;
        key[m] = 0.0f;
    }
    float fx;
    exact_select_token<64, NV64, BF16, KMAX>(a, s_bias, wl, x, e64, key, fx);
    // softmax: the selected logits are the keys; sigmoid: the row is read again
    float v[KPL64];
#pragma unroll
    for (int m = 0; m < KPL64; ++m) {
        const int j = m * 64 + wl;
        float vv = 0.0f;
        if (j < a.K) vv = SCORE == 2 ? sigmoid_cr(load_logit(a, tok, e64[m], BF16)) : key[m];
        v[m] = vv;
    }
    double full_max = 0.0, full_den = 0.0;
    if constexpr (SCORE == 1) {
        float fm = -FLT_MAX;
#pragma unroll
        for (int q = 0; q < NE64; ++q)
            if (chunk_expert(q, W, 64, wl) < a.E) fm = fmaxf(fm, x[q]);
        full_max = (double)order_key_inv(seg_max_u32<64>(order_key(fm)));
#pragma unroll
        for (int q = 0; q < NE64; ++q)
            if (chunk_expert(q, W, 64, wl) < a.E) full_den += exp_neg_f64((double)x[q] - full_max);
        full_den = seg_sum_f64<64>(full_den);
    }
    write_weights<64, KPL64>(a, tok, wl, true, e64, v, (double)fx, full_max, full_den);
}

constexpr int kFailCap = 64;  // deferred tokens per wave

// MODE 0: no group limit (units = lanes); MODE 1: a group spans S = gsize/32 lanes (S >= 1).
// SCORE: 0 softmax with renormalisation, 1 softmax over all experts, 2 sigmoid.
template <int LPT, bool BF16, int KMAX, int M, int MODE, int SCORE>
__global__ __launch_bounds__(kFastBlock, 3) void route_fast_kernel(RouteArgs a, FastCfg cfg) {
    using G = FastGeom<LPT, BF16>;
    constexpr int W = G::W;
    constexpr int CPL = G::CPL;
    constexpr int CPR = G::CPR;
    constexpr int RS = G::RS;
    constexpr int TPW = G::TPW;
    constexpr int TPB = G::TPB;
    constexpr int NE = kFastEPL;
    constexpr int KPL = (KMAX + LPT - 1) / LPT;
    constexpr int MAXG = LPT;
    constexpr bool sig = SCORE == 2;

    __shared__ u32x4 s_rows[kFastWaves][TPW * RS];
    __shared__ float4 s_bias4[LPT * kFastEPL / 4];
    __shared__ float s_gscore[TPB][MAXG];
    __shared__ float s_gthr[TPB][MAXG];
    constexpr int kCandCap = cand_cap<LPT>();
    __shared__ uint64_t s_cand[TPB][kCandCap];
    __shared__ int s_ccount[TPB];
    __shared__ int s_sel[TPB][KMAX];
    __shared__ uint32_t s_skey[TPB][KMAX + 1];
    __shared__ int s_fail[kFastWaves][kFailCap];

    const int tid = threadIdx.x;
    const int wv = tid >> 6;
    const int wl = tid & 63;
    const int tw = wl / LPT;         // token slot within the set
    const int tloc = wv * TPW + tw;  // token slot within the block
    const int lseg = wl % LPT;
    const int K = a.K;
    const int e0 = lseg * NE;  // this lane's experts: [e0, e0 + 32)
    const float* s_bias = reinterpret_cast<const float*>(s_bias4);
    const int64_t waves = (int64_t)gridDim.x * kFastWaves;
    const int64_t first_set = (int64_t)blockIdx.x * kFastWaves + wv;

    // ---- prologue: bias into registers, the first set in flight, bias into LDS -----------------
    constexpr int BPT = (LPT * kFastEPL + kFastBlock - 1) / kFastBlock;
    float bias_r[BPT];
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        const int e = tid + i * kFastBlock;
        bias_r[i] = (sig && e < a.E) ? gptr(a.bias)[e] : 0.0f;
    }
    u32x4 buf[CPL];
    if (first_set < cfg.nsets) fast_load_set<LPT, BF16>(a, first_set, wl, buf);
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        const int e = tid + i * kFastBlock;
        if (e < a.E) reinterpret_cast<float*>(s_bias4)[e] = bias_r[i];
    }
    __syncthreads();
    float delta = 0.0f, delta_g = 0.0f;  // 2 * the bounds of the header, as binary32 upper bounds
    if constexpr (sig) {
        float mb = 0.0f;
        for (int e = wl; e < a.E; e += 64) mb = fmaxf(mb, fabsf(s_bias[e]));
        const double maxb = (double)wave_max_nonneg(mb);
        const double d = (4.0 + (1.0 + maxb)) * 0x1p-23;
        delta = (float)(2.0 * d * (1.0 + 0x1p-20));
        delta_g = (float)(2.0 * (2.0 * d + 2.02 * (1.0 + maxb) * 0x1p-23) * (1.0 + 0x1p-20));
    }
    const int mt = cfg.mt;
    const int rot = lseg + lseg / CPL;
    u32x4* my_rows = s_rows[wv];
    const u32x4* my_row = &my_rows[tw * RS];
    const char* my_row_bytes = reinterpret_cast<const char*>(my_row);
    int nfail = 0;  // wave-uniform length of s_fail[wv]

    auto row_logit = [&](int e) -> float {
        if constexpr (BF16)
            return __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t*>(my_row_bytes + 2 * e)) << 16);
        else
            return *reinterpret_cast<const float*>(my_row_bytes + 4 * e);
    };

    for (int64_t set = first_set; set < cfg.nsets; set += waves) {
        // ---- registers -> this wave's LDS rows; refill with the next set --------------------------
        wave_lds_sync();  // the previous set's LDS reads are done
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int q = c * 64 + wl;
            const int r = q / CPR;
            my_rows[r * RS + (q - r * CPR)] = buf[c];
        }
        if (set + waves < cfg.nsets) fast_load_set<LPT, BF16>(a, set + waves, wl, buf);

        const int64_t tok_raw = set * TPW + tw;
        const bool live = tok_raw < a.N;
        const int64_t tok = live ? tok_raw : (a.N - 1);

        // Pass 0 selects on binary32 keys and certifies; if any token of the set fails, pass 1
        // redoes the set on exact keys (correctly rounded sigmoid, no margins, nothing to certify).
        // A token that still fails (candidate list overflow, an undecided rounding) is deferred.
        bool fail = false;
        double full_max = 0.0, full_den = 0.0;
        for (int pass = 0; pass < 2; ++pass) {
            const bool exact = pass == 1;
            const float dlt = exact ? 0.0f : delta;
            const float dlt_g = exact ? 0.0f : delta_g;
            fail = false;
            if (lseg == 0) s_ccount[tloc] = 0;
            static_assert(kCandCap % LPT == 0, "whole rounds of the token's lanes");
#pragma unroll
            for (int j = 0; j < kCandCap / LPT; ++j) s_cand[tloc][j * LPT + lseg] = 0ull;
            wave_lds_sync();

            // ---- keys -----------------------------------------------------------------------------
            float k[NE];
            auto chunk_logits = [&](int j, float (&x)[W]) {
                const int cl = (j + rot) & (CPL - 1);
                const u32x4 v = my_row[lseg * CPL + cl];
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
                return cl;
            };
            if (!sig || !exact) {
#pragma unroll
                for (int j = 0; j < CPL; ++j) {
                    float x[W];
                    const int cl = chunk_logits(j, x);
                    if constexpr (sig) {
#pragma unroll
                        for (int h = 0; h < W / 4; ++h) {
                            const float4 b = s_bias4[(e0 + cl * W) / 4 + h];
                            const float bb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
                            for (int i = 0; i < 4; ++i) k[j * W + 4 * h + i] = sigmoid_fast(x[4 * h + i]) + bb[i];
                        }
                    } else {
#pragma unroll
                        for (int i = 0; i < W; ++i) k[j * W + i] = x[i];
                    }
                }
            } else {
                // exact keys, one chunk at a time (a rare path: few values in flight, few registers)
#pragma unroll 1
                for (int jj = 0; jj < CPL; ++jj) {
                    float x[W], kv[W];
                    const int cl = chunk_logits(jj, x);
#pragma unroll
                    for (int i = 0; i < W; ++i) {
                        bool ok;
                        kv[i] = sigmoid_cr_fast(x[i], ok) + s_bias[e0 + cl * W + i];
                        fail = fail || !ok;
                    }
#pragma unroll
                    for (int j = 0; j < CPL; ++j)
#pragma unroll
                        for (int i = 0; i < W; ++i) k[j * W + i] = j == jj ? kv[i] : k[j * W + i];
                }
            }
            if constexpr (SCORE == 1) {
                // softmax over all experts: the max and the sum of exp(x - max) of the full row
                float fmx = -FLT_MAX;
#pragma unroll
                for (int q = 0; q < NE; ++q) fmx = fmaxf(fmx, k[q]);
                full_max = (double)order_key_inv(seg_max_u32_dpp(order_key(fmx), LPT));
                full_den = 0.0;
#pragma unroll
                for (int q = 0; q < NE; ++q) full_den += exp_neg_f64((double)k[q] - full_max);
                full_den = seg_allreduce<LPT>(full_den, LPT, PartnerF64{}, [](double u, double v) { return u + v; });
            }

            // ---- units: top-M keys per lane, groups of S lanes ---------------------------------------
            float lt[M];
#pragma unroll
            for (int m = 0; m < M; ++m) lt[m] = -FLT_MAX;
#pragma unroll
            for (int q = 0; q < NE; ++q) insert_top<M>(lt, k[q]);
            bool elig = true;
            float tau;
            if constexpr (MODE == 0) {
                float th = lt[0];
#pragma unroll
                for (int m = 1; m < M; ++m)
                    if (m == mt - 1) th = lt[m];
                tau = order_key_inv(seg_min_u32_dpp(order_key(th), LPT));
            } else {
                seg_top_allreduce<LPT, M>(lt, cfg.S);
                float th = lt[0];
#pragma unroll
                for (int m = 1; m < M; ++m)
                    if (m == mt - 1) th = lt[m];
                const int g_mine = lseg >> cfg.log2S;
                if ((lseg & (cfg.S - 1)) == 0) {
                    s_gscore[tloc][g_mine] = a.group_topn >= 2 ? lt[0] + lt[1] : lt[0];
                    s_gthr[tloc][g_mine] = th;
                }
                wave_lds_sync();
                // groups kept by rank (score desc, index asc); certification gap; threshold
                const int NG = a.n_group;
                const int TG = a.topk_group;
                uint32_t kept = 0, thr_key = 0xFFFFFFFFu, k_tg = 0, k_tg1 = 0;
                if (lseg < NG) {
                    const int g = lseg;
                    const float sg = s_gscore[tloc][g];
                    int rank = 0;
                    for (int h = 0; h < NG; ++h) {
                        const float sh = s_gscore[tloc][h];
                        rank += (sh > sg) || (sh == sg && h < g);
                    }
                    if (rank < TG) {
                        kept = 1u << g;
                        thr_key = order_key(s_gthr[tloc][g]);
                    }
                    if (rank == TG - 1) k_tg = order_key(sg);
                    if (rank == TG) k_tg1 = order_key(sg);
                }
                kept = seg_or_u32_dpp(kept, LPT);
                tau = order_key_inv(seg_min_u32_dpp(thr_key, LPT));
                if (sig && !exact && TG < NG) {
                    const float at_tg = order_key_inv(seg_max_u32_dpp(k_tg, LPT));
                    const float at_tg1 = order_key_inv(seg_max_u32_dpp(k_tg1, LPT));
                    if (!((double)at_tg - (double)at_tg1 > (double)dlt_g)) fail = true;
                }
                elig = (kept >> g_mine) & 1u;
            }

            // ---- candidates: keys >= tau (less the margin); one slot reservation per lane -----------
            float tau_low = tau;
            if (sig && !exact) tau_low = tau - dlt - fabsf(tau) * 0x1p-22f;
            uint32_t cmask = 0;
#pragma unroll
            for (int q = 0; q < NE; ++q) cmask |= (k[q] >= tau_low ? 1u : 0u) << q;
            if (!elig) cmask = 0;
            int pos = cmask ? atomicAdd(&s_ccount[tloc], __popc(cmask)) : 0;
            while (cmask) {
                const int q = __builtin_ctz(cmask);
                cmask &= cmask - 1;
                const int e = e0 + ((q / W + rot) & (CPL - 1)) * W + (q % W);
                const float xe = row_logit(e);
                float key = xe;  // the same value as k[q]
                if constexpr (sig) {
                    bool ok;  // already tested when k[q] was formed
                    key = (exact ? sigmoid_cr_fast(xe, ok) : sigmoid_fast(xe)) + s_bias[e];
                }
                if (pos < kCandCap) s_cand[tloc][pos] = ((uint64_t)order_key(key) << 32) | (uint64_t)(uint32_t)~e;
                ++pos;
            }
            wave_lds_sync();

            // ---- rank the candidates (packed: larger = better); certify the order -------------------
            // rank = number of candidates that beat it; the list is zero past its end (zero is below
            // every packed candidate), so the scan reads whole 4-entry groups without bounds tests.
            const int cnt = s_ccount[tloc];
            const bool overflow = cnt > kCandCap || cnt < K;
            if (!overflow) {
                for (int i = lseg; i < cnt; i += LPT) {
                    const uint64_t ci = s_cand[tloc][i];
                    int rank = 0;
                    for (int jj = 0; jj < cnt; jj += 4) {
                        rank += (s_cand[tloc][jj] > ci) + (s_cand[tloc][jj + 1] > ci) +
                                (s_cand[tloc][jj + 2] > ci) + (s_cand[tloc][jj + 3] > ci);
                    }
                    if (rank <= K) s_skey[tloc][rank] = (uint32_t)(ci >> 32);
                    if (rank < K) s_sel[tloc][rank] = (int)~(uint32_t)ci;
                }
                if (sig && !exact) {
                    wave_lds_sync();
                    // consecutive ranked keys among the first K + 1 must differ by more than 2 delta
                    for (int r = lseg; r < K; r += LPT) {
                        if (r + 1 < cnt) {
                            const double gap = (double)order_key_inv(s_skey[tloc][r]) -
                                               (double)order_key_inv(s_skey[tloc][r + 1]);
                            if (!(gap > (double)dlt)) fail = true;
                        }
                    }
                }
            }
            fail = fail || overflow;
            wave_lds_sync();

            if (exact || __ballot(fail && live) == 0ull) break;
        }

        // ---- exact values of the selected experts (logits from the LDS row), weights ------------
        int my_e[KPL];
        float my_v[KPL];
#pragma unroll
        for (int m = 0; m < KPL; ++m) {
            const int j = m * LPT + lseg;
            my_e[m] = j < K ? s_sel[tloc][j] : 0;
            float v = 0.0f;
            if (j < K && !fail) {
                const float xe = row_logit(my_e[m]);
                if constexpr (sig) {
                    bool ok;
                    v = sigmoid_cr_fast(xe, ok);
                    fail = fail || !ok;
                } else {
                    v = xe;
                }
            }
            my_v[m] = v;
        }
        fail = seg_or_u32_dpp((uint32_t)fail, LPT) != 0u;
        float first_x = 0.0f;
        if (SCORE == 0 && !fail) first_x = row_logit(s_sel[tloc][0]);
        write_weights<LPT, KPL>(a, tok, lseg, live && !fail, my_e, my_v, (double)first_x, full_max, full_den);

        // ---- defer the uncertified tokens ---------------------------------------------------------
        // Up to kFailCap per wave wait in LDS; beyond that a token is marked in the output (first id
        // -1) and found again after the loop.  No work that needs calls runs inside this loop.
        const bool defer = fail && live && lseg == 0;
        const uint64_t fm = __ballot(defer);
        if (fm) {
            const int slot = nfail + __popcll(fm & lanes_below());
            if (defer) {
                if (slot < kFailCap) s_fail[wv][slot] = (int)tok;
                else gptr(a.ids)[tok * K] = -1;
            }
            nfail += __popcll(fm);
        }
    }
    wave_lds_sync();
    const int nlist = min(nfail, kFailCap);
    for (int i = 0; i < nlist; ++i)
        exact_token_full<LPT, BF16, KMAX, SCORE>(a, s_bias, wl, (int64_t)s_fail[wv][i]);
    if (nfail > kFailCap) {
        // the marked tokens: every token of this wave's sets whose first id is -1
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "agent");
        for (int64_t set = first_set; set < cfg.nsets; set += waves) {
            const int64_t t = set * TPW + (wl % TPW);
            const bool marked = wl < TPW && t < a.N && gptr(a.ids)[t * K] == -1;
            uint64_t mm = __ballot(marked);
            while (mm) {
                const int l = __ffsll((long long)mm) - 1;
                mm &= mm - 1;
                exact_token_full<LPT, BF16, KMAX, SCORE>(a, s_bias, wl, set * TPW + l);
            }
        }
    }
}

// Blocks of `kernel` that fit on the current device at once (cached per device and kernel).
int resident_blocks(const void* kernel, int block_threads);

template <int LPT, bool BF16, int MODE, int SCORE>
void launch_fast_mode(const RouteArgs& a, const FastCfg& cfg_in, int M, const Launch& st) {
    FastCfg cfg = cfg_in;
    cfg.nsets = ceil_div64(a.N, FastGeom<LPT, BF16>::TPW);
    auto launch = [&](auto kernel) {
        const int64_t need = ceil_div64(cfg.nsets, kFastWaves);
        int64_t grid = resident_blocks(reinterpret_cast<const void*>(kernel), kFastBlock);
        if (grid > need) grid = need;
        if (grid < 1) grid = 1;
        launch_kernel(kernel, dim3((unsigned)grid), dim3(kFastBlock), 0, st, a, cfg);
    };
    if (a.K <= 8) {
        if (M <= 2) launch(route_fast_kernel<LPT, BF16, 8, 2, MODE, SCORE>);
        else launch(route_fast_kernel<LPT, BF16, 8, 4, MODE, SCORE>);
    } else {
        if (M <= 2) launch(route_fast_kernel<LPT, BF16, 32, 2, MODE, SCORE>);
        else launch(route_fast_kernel<LPT, BF16, 32, 4, MODE, SCORE>);
    }
}

template <int LPT, bool BF16>
void launch_fast_shape(const RouteArgs& a, const FastCfg& cfg, int M, const Launch& st) {
    if (a.score_fn == MEP_SIGMOID) {
        if (cfg.mode == 0) launch_fast_mode<LPT, BF16, 0, 2>(a, cfg, M, st);
        else launch_fast_mode<LPT, BF16, 1, 2>(a, cfg, M, st);
    } else if (a.renormalize) {
        if (cfg.mode == 0) launch_fast_mode<LPT, BF16, 0, 0>(a, cfg, M, st);
        else launch_fast_mode<LPT, BF16, 1, 0>(a, cfg, M, st);
    } else {
        if (cfg.mode == 0) launch_fast_mode<LPT, BF16, 0, 1>(a, cfg, M, st);
        else launch_fast_mode<LPT, BF16, 1, 1>(a, cfg, M, st);
    }
}

void launch_fast_f32(int LPT, const RouteArgs& a, const FastCfg& cfg, int M, const Launch& st);
void launch_fast_bf16(int LPT, const RouteArgs& a, const FastCfg& cfg, int M, const Launch& st);

}  // namespace mep
