// Fast routing kernel: selection on binary32 keys with a certified error bound.
//
// Every lane holds 32 experts of its token (E/32 lanes per token, chunk layout of
// route_common.h).  Per token, one selection pass:
//   1. keys k (pass 0, sigmoid scoring: s~ = 1/(1 + 2^(-x log2 e)) with v_exp_f32 / v_rcp_f32,
//      plus the bias; softmax scoring: the logit itself, which is exact);
//   2. per group (or per lane when there is no group limit) the M largest keys, combined
//      across the group's lanes with DPP; group score = sum of the top group_topn keys;
//   3. groups kept by (score desc, group index asc); threshold tau = the smallest M'-th best
//      key of a kept unit, M' = ceil(K / units), so at least K keys are >= tau;
//   4. keys >= tau (less the error margin) go to a per-token candidate list in LDS; each
//      candidate's rank is the number of candidates that beat it (key desc, expert asc),
//      which orders the top-K;
//   5. certification (pass 0, sigmoid scoring): with delta a proven bound on |k~ - k|, the
//      selection on k~ equals the selection on the exact keys if the TG-th and (TG+1)-th group
//      scores differ by more than 2*delta_group and each of the first K ranked keys exceeds the
//      next one by more than 2*delta.
// Tokens that fail (near-ties, list overflow, huge logits) run the pass again with exact keys
// (correctly rounded sigmoid + bias, delta = 0); a list overflow there falls back to K rounds of
// a segmented arg-max.  Only the K selected experts then get the correctly rounded sigmoid in
// binary64 for the weights.
//
// All exchange between the lanes of a token stays inside one wave (DPP, or LDS written and read
// by the same wave in program order), so the per-token second pass needs no block barrier.
//
// Error bound of s~ (relative): the binary32 product x * (-log2 e) perturbs the exponent by at
// most |x| log2(e) 2^-23 (constant and product rounding), i.e. |x| 2^-23 relative in 2^t;
// v_exp_f32 and v_rcp_f32 are taken as <= 2 ulp (the ISA documents 1 ulp); 1 + e adds 2^-24.
// Total eps_s <= (2|x| + 9) 2^-24 and |s~ - s| <= eps_s.  Rounding s + b costs at most one ulp
// of a key, <= (1 + max|b|) 2^-23 for keys below 1 + max|b|.
#pragma once

#include "route_common.h"

namespace mep {

constexpr int kCandCap = 32;
constexpr int kFastEPL = 32;  // experts per lane

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

template <int S>
__device__ __forceinline__ float seg_max_f32(float v) {
    return seg_allreduce<S>(v, S, PartnerF32{}, [](float u, float w) { return fmaxf(u, w); });
}
template <int S>
__device__ __forceinline__ float seg_min_f32(float v) {
    return seg_allreduce<S>(v, S, PartnerF32{}, [](float u, float w) { return fminf(u, w); });
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
};

// Threads per block: 256 for 8+ lanes per token, 128 below (keeps the per-token LDS small).
template <int LPT>
constexpr int fast_block() { return LPT >= 8 ? 256 : 128; }

#ifndef MEP_FAST_WAVES_PER_SIMD
#define MEP_FAST_WAVES_PER_SIMD 4
#endif

__device__ __forceinline__ uint32_t seg_max_u32_dpp(uint32_t v, int S) {
    return seg_allreduce<16>(v, S, PartnerU32{}, [](uint32_t u, uint32_t w) { return max(u, w); });
}
__device__ __forceinline__ uint32_t seg_min_u32_dpp(uint32_t v, int S) {
    return seg_allreduce<16>(v, S, PartnerU32{}, [](uint32_t u, uint32_t w) { return min(u, w); });
}
__device__ __forceinline__ uint32_t seg_or_u32_dpp(uint32_t v, int S) {
    return seg_allreduce<16>(v, S, PartnerU32{}, [](uint32_t u, uint32_t w) { return u | w; });
}

// MODE 0: no group limit (units = lanes); MODE 1: a group spans S = gsize/32 lanes (S >= 1).
//
// Row staging: each wave copies the rows of its 64/LPT tokens from HBM into LDS with
// global_load_lds_dwordx4 (one coalesced 16-byte chunk per lane and instruction), then lane
// `g` of a token reads its 32 experts [32g, 32g + 32) back as CPL 16-byte chunks.  Rows are
// padded by LPT chunks and lane g visits its chunks in the rotated order (j + g + g/CPL) mod CPL,
// which puts the 16 lanes of every LDS pass on 16 different bank groups.  Register slot q holds
// expert 32g + chunk(q / W) * W + q % W.  The row stays in LDS for the candidate pass (keys are
// recomputed from it by expert index) and for the exact values of the selected experts.
template <int LPT, bool BF16, int KMAX, int M, int MODE>
__global__ __launch_bounds__(fast_block<LPT>(), MEP_FAST_WAVES_PER_SIMD) void route_fast_kernel(RouteArgs a,
                                                                                               FastCfg cfg) {
    constexpr int kBlock = fast_block<LPT>();
    constexpr int kWaves = kBlock / 64;
    constexpr int W = BF16 ? 8 : 4;          // experts per 16-byte chunk
    constexpr int CPL = kFastEPL / W;        // chunks per lane
    constexpr int CPR = LPT * CPL;           // chunks per row
    constexpr int RS = CPR + LPT;            // row stride in chunks (padding spreads banks)
    constexpr int TPW = 64 / LPT;            // tokens per wave
    constexpr int NE = kFastEPL;
    constexpr int TPB = kBlock / LPT;
    constexpr int KPL = (KMAX + LPT - 1) / LPT;
    constexpr int MAXG = LPT;

    __shared__ uint4 s_rows[kWaves][TPW * RS];
    __shared__ float4 s_bias4[LPT * kFastEPL / 4];
    __shared__ float s_gscore[TPB][MAXG];
    __shared__ float s_gthr[TPB][MAXG];
    __shared__ uint64_t s_cand[TPB][kCandCap];
    __shared__ int s_ccount[TPB];
    __shared__ int s_sel[TPB][KMAX];
    __shared__ uint32_t s_maxb;

    const int tid = threadIdx.x;
    const int wv = tid >> 6;
    const int wl = tid & 63;
    const int tloc = tid / LPT;
    const int tw = wl / LPT;  // token slot within the wave
    const int lseg = tid % LPT;
    const int64_t tok_raw = (int64_t)blockIdx.x * TPB + tloc;
    const bool live = tok_raw < a.N;
    const int64_t tok = live ? tok_raw : (a.N - 1);
    const int K = a.K;
    const bool sig = a.score_fn == MEP_SIGMOID;
    const int e0 = lseg * NE;  // this lane's experts: [e0, e0 + 32)
    const float* s_bias = reinterpret_cast<const float*>(s_bias4);

    // ---- stage this wave's rows into LDS (coalesced DMA) ----------------------------------------
    {
        const int64_t first = (int64_t)blockIdx.x * TPB + wv * TPW;
#pragma unroll
        for (int r = 0; r < TPW; ++r) {
            const int64_t t = min(first + r, a.N - 1);
            const char* row = reinterpret_cast<const char*>(a.logits) + t * (int64_t)a.E * (BF16 ? 2 : 4);
#pragma unroll
            for (int c0 = 0; c0 < CPR; c0 += 64) {
                if (c0 + wl < CPR)
                    __builtin_amdgcn_global_load_lds(
                        row + (int64_t)(c0 + wl) * 16,
                        (__attribute__((address_space(3))) void*)&s_rows[wv][r * RS + c0], 16, 0, 0);
            }
        }
    }
    if (tid == 0) s_maxb = 0u;
    if (lseg == 0) s_ccount[tloc] = 0;
    __syncthreads();
    if (sig) {
        for (int e = tid; e < a.E; e += kBlock) {
            const float b = a.bias[e];
            reinterpret_cast<float*>(s_bias4)[e] = b;
            atomicMax(&s_maxb, __float_as_uint(fabsf(b)));  // |b| >= 0: bit order = value order
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's row copies have landed
    __syncthreads();                // bias, maxb

    // ---- keys -------------------------------------------------------------------------------------
    const uint4* my_row = &s_rows[wv][tw * RS];
    const int rot = lseg + lseg / CPL;
    float k[NE];
    float maxabs = 0.0f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int cl = (j + rot) & (CPL - 1);
        const uint4 v = my_row[lseg * CPL + cl];
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
        if (sig) {
#pragma unroll
            for (int h = 0; h < W / 4; ++h) {
                const float4 b = s_bias4[(e0 + cl * W) / 4 + h];
                const float bb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float xi = x[4 * h + i];
                    maxabs = fmaxf(maxabs, fabsf(xi));
                    k[j * W + 4 * h + i] = sigmoid_fast(xi) + bb[i];
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < W; ++i) k[j * W + i] = x[i];
        }
    }
    // softmax without renormalisation needs the full row: max and sum of exp(x - max)
    double full_max = 0.0, full_den = 0.0;
    if (!sig && !a.renormalize) {
        float fm = -FLT_MAX;
#pragma unroll
        for (int q = 0; q < NE; ++q) fm = fmaxf(fm, k[q]);
        full_max = (double)order_key_inv(seg_max_u32_dpp(order_key(fm), LPT));
#pragma unroll
        for (int q = 0; q < NE; ++q) full_den += exp_f64_call((double)k[q] - full_max);
        full_den = seg_allreduce<LPT>(full_den, LPT, PartnerF64{}, [](double u, double v) { return u + v; });
    }
    double delta = 0.0, delta_g = 0.0;
    bool fail = false;
    if (sig) {
        maxabs = __uint_as_float(seg_max_u32_dpp(__float_as_uint(maxabs), LPT));  // maxabs >= 0
        const double maxb = (double)__uint_as_float(s_maxb);
        delta = (2.0 * (double)maxabs + 9.0) * 0x1p-24 + (1.01 + maxb) * 0x1p-23;
        delta_g = 2.0 * delta + (2.02 + 2.0 * maxb) * 0x1p-23;
        fail = !(maxabs <= 64.0f);  // outside the range the error bound is written for
    }

    // ---- units: top-M keys per lane, groups of S lanes -----------------------------------------
    const int mt = cfg.mt;
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
        const int G = a.n_group;
        const int TG = a.topk_group;
        uint32_t kept = 0, thr_key = 0xFFFFFFFFu, k_tg = 0, k_tg1 = 0;
        if (lseg < G) {
            const int g = lseg;
            const float sg = s_gscore[tloc][g];
            int rank = 0;
            for (int h = 0; h < G; ++h) {
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
        if (sig && TG < G) {
            const float at_tg = order_key_inv(seg_max_u32_dpp(k_tg, LPT));
            const float at_tg1 = order_key_inv(seg_max_u32_dpp(k_tg1, LPT));
            if (!((double)at_tg - (double)at_tg1 > 2.0 * delta_g)) fail = true;
        }
        elig = (kept >> g_mine) & 1u;
    }

    // ---- candidates: keys >= tau (less the margin); one slot reservation per lane -------------
    float tau_low = tau;
    if (sig) tau_low = tau - (float)(2.0 * delta) - fabsf(tau) * 0x1p-22f;
    uint32_t cmask = 0;
#pragma unroll
    for (int q = 0; q < NE; ++q) cmask |= (k[q] >= tau_low ? 1u : 0u) << q;
    if (!elig) cmask = 0;
    int pos = cmask ? atomicAdd(&s_ccount[tloc], __popc(cmask)) : 0;
    const char* my_row_bytes = reinterpret_cast<const char*>(my_row);
    while (cmask) {
        const int q = __builtin_ctz(cmask);
        cmask &= cmask - 1;
        const int e = e0 + ((q / W + rot) & (CPL - 1)) * W + (q % W);
        float xe;
        if constexpr (BF16)
            xe = __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t*>(my_row_bytes + 2 * e)) << 16);
        else
            xe = *reinterpret_cast<const float*>(my_row_bytes + 4 * e);
        const float key = sig ? sigmoid_fast(xe) + s_bias[e] : xe;  // the same value as k[q]
        if (pos < kCandCap)
            s_cand[tloc][pos] = ((uint64_t)order_key(key) << 32) | (uint64_t)(uint32_t)~e;
        ++pos;
    }
    wave_lds_sync();

    // ---- rank the candidates (packed: larger = better); certify the order ---------------------
    const int cnt = s_ccount[tloc];
    const bool overflow = cnt > kCandCap || cnt < K;
    if (!overflow) {
        bool gap_fail = false;
        for (int i = lseg; i < cnt; i += LPT) {
            const uint64_t ci = s_cand[tloc][i];
            int rank = 0;
            uint32_t below = 0;  // order key of the best candidate below ci (0: none)
            for (int jj = 0; jj < cnt; ++jj) {
                const uint64_t cj = s_cand[tloc][jj];
                rank += cj > ci;
                if (cj < ci) below = max(below, (uint32_t)(cj >> 32));
            }
            if (rank < K) {
                s_sel[tloc][rank] = (int)~(uint32_t)ci;
                if (sig && below != 0u) {
                    const double gap = (double)order_key_inv((uint32_t)(ci >> 32)) - (double)order_key_inv(below);
                    if (!(gap > 2.0 * delta)) gap_fail = true;
                }
            }
        }
        fail = fail || gap_fail;
    }
    fail = seg_or_u32_dpp((uint32_t)(fail || overflow), LPT) != 0u;
    wave_lds_sync();

    // ---- tokens the filter could not certify: exact selection by the whole wave ---------------
    uint64_t todo = __ballot(fail && lseg == 0);
    while (todo) {
        const int lane0 = __ffsll((long long)todo) - 1;
        todo &= todo - 1;
        const int t_in_block = (tid - wl + lane0) / LPT;
        const int64_t ft = min((int64_t)blockIdx.x * TPB + t_in_block, a.N - 1);
        constexpr int NV64 = (LPT * kFastEPL + 64 * W - 1) / (64 * W);
        constexpr int KPL64 = (KMAX + 63) / 64;
        float x[NV64 * W];
        load_row<64, NV64, BF16>(a, ft, wl, x);
        int e64[KPL64];
        float fx;
        exact_select_token<64, NV64, BF16, KMAX>(a, s_bias, wl, x, e64, fx);
#pragma unroll
        for (int m = 0; m < KPL64; ++m) {
            const int j = m * 64 + wl;
            if (j < K) s_sel[t_in_block][j] = e64[m];
        }
        wave_lds_sync();
    }

    // ---- exact values of the selected experts (logits from the LDS row), weights --------------
    auto row_logit = [&](int e) -> float {
        if constexpr (BF16)
            return __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t*>(my_row_bytes + 2 * e)) << 16);
        else
            return *reinterpret_cast<const float*>(my_row_bytes + 4 * e);
    };
    int my_e[KPL];
    float my_v[KPL];
#pragma unroll
    for (int m = 0; m < KPL; ++m) {
        const int j = m * LPT + lseg;
        my_e[m] = j < K ? s_sel[tloc][j] : 0;
        float v = 0.0f;
        if (j < K) {
            const float xe = row_logit(my_e[m]);
            v = sig ? sigmoid_cr_call(xe) : xe;
        }
        my_v[m] = v;
    }
    float first_x = 0.0f;
    if (!sig && a.renormalize) first_x = row_logit(s_sel[tloc][0]);
    write_weights<LPT, KPL>(a, tok, lseg, live, my_e, my_v, (double)first_x, full_max, full_den);
}

template <int LPT, bool BF16, int MODE>
void launch_fast_mode(const RouteArgs& a, const FastCfg& cfg, int M, hipStream_t st) {
    const int64_t blocks = ceil_div64(a.N, fast_block<LPT>() / LPT);
    const dim3 grid((unsigned)blocks), block(fast_block<LPT>());
    if (a.K <= 8) {
        if (M <= 2) hipLaunchKernelGGL((route_fast_kernel<LPT, BF16, 8, 2, MODE>), grid, block, 0, st, a, cfg);
        else hipLaunchKernelGGL((route_fast_kernel<LPT, BF16, 8, 4, MODE>), grid, block, 0, st, a, cfg);
    } else {
        if (M <= 2) hipLaunchKernelGGL((route_fast_kernel<LPT, BF16, 32, 2, MODE>), grid, block, 0, st, a, cfg);
        else hipLaunchKernelGGL((route_fast_kernel<LPT, BF16, 32, 4, MODE>), grid, block, 0, st, a, cfg);
    }
}

template <int LPT, bool BF16>
void launch_fast_shape(const RouteArgs& a, const FastCfg& cfg, int M, hipStream_t st) {
    if (cfg.mode == 0) launch_fast_mode<LPT, BF16, 0>(a, cfg, M, st);
    else launch_fast_mode<LPT, BF16, 1>(a, cfg, M, st);
}

void launch_fast_f32(int LPT, const RouteArgs& a, const FastCfg& cfg, int M, hipStream_t st);
void launch_fast_bf16(int LPT, const RouteArgs& a, const FastCfg& cfg, int M, hipStream_t st);

}  // namespace mep
