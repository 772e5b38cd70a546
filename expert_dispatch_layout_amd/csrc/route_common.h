// Pieces shared by the routing kernels: arguments, the exact per-token selection (used by the
// generic kernel for every token and by the fast kernel for tokens its filter cannot certify),
// and the binary64 weight computation.
//
// Element layout used by both kernels: a token is handled by a segment of LPT lanes of one
// wave64.  Lane `lseg` of the segment loads NV 16-byte chunks; chunk j holds experts
// [(j*LPT + lseg)*W, +W) with W = 4 (fp32) or 8 (bf16), so each load instruction of a segment
// reads one contiguous run of the row ("line" j = experts [j*LPT*W, (j+1)*LPT*W)).
#pragma once

#include <float.h>
#include <hip/hip_ext.h>
#include <limits.h>

#include <type_traits>
#include <utility>

#include "device_common.h"
#include "host_common.h"
#include "sigmoid_cr.h"

namespace mep {

struct RouteArgs {
    const void* logits;
    const float* bias;
    int64_t N;
    int E;
    int K;
    int score_fn;
    int renormalize;
    int n_group;
    int topk_group;
    int group_topn;
    float scale;
    float inv_gsize;  // 1 / (E / n_group)
    int32_t* ids;
    float* weights;
    int vec;          // rows are 16-byte aligned and E is a multiple of the chunk width
};

// Where a routing kernel is launched: the caller's stream and two optional events that the
// launch itself updates with the kernel's start and end times (hipExtLaunchKernel), so the
// kernel can be timed without marker packets between it and its neighbours on the stream.
// Every routing path launches exactly one kernel.
struct Launch {
    hipStream_t st;
    hipEvent_t start;  // may be null
    hipEvent_t stop;   // may be null
};

template <typename F, typename... Args>
inline void launch_kernel(F kernel, dim3 grid, dim3 block, uint32_t shmem, const Launch& l,
                          Args... args) {
    launch_ext(kernel, grid, block, shmem, l.st, l.start, l.stop, 0, args...);
}

constexpr int kRouteBlock = 256;
constexpr int kMaxGroups = 32;

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0..N-1.
template <int N, typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

// Reductions over a token's segment of LPT lanes (all of them active): DPP lane moves for the
// partners within 16 lanes, ds_bpermute beyond (seg_partner_u32); every lane gets the result.
template <int LPT>
__device__ __forceinline__ uint32_t seg_max_u32(uint32_t v) {
    return seg_allreduce<LPT>(v, LPT, PartnerU32{}, [](uint32_t p, uint32_t q) { return max(p, q); });
}

template <int LPT>
__device__ __forceinline__ uint32_t seg_min_u32(uint32_t v) {
    return seg_allreduce<LPT>(v, LPT, PartnerU32{}, [](uint32_t p, uint32_t q) { return min(p, q); });
}

template <int LPT>
__device__ __forceinline__ double seg_sum_f64(double v) {
    return seg_allreduce<LPT>(v, LPT, PartnerF64{}, [](double p, double q) { return p + q; });
}

// keep the two largest of (t1 >= t2) and the partner lane's pair
template <int LPT>
__device__ __forceinline__ void seg_top2_u32(uint32_t& t1, uint32_t& t2) {
    auto step = [&](auto partner) {
        const uint32_t b1 = partner(t1), b2 = partner(t2);
        const uint32_t n2 = max(min(t1, b1), max(t2, b2));
        t1 = max(t1, b1);
        t2 = n2;
    };
    if constexpr (LPT >= 2) step([](uint32_t u) { return seg_partner_u32<1>(u); });
    if constexpr (LPT >= 4) step([](uint32_t u) { return seg_partner_u32<2>(u); });
    if constexpr (LPT >= 8) step([](uint32_t u) { return seg_partner_u32<4>(u); });
    if constexpr (LPT >= 16) step([](uint32_t u) { return seg_partner_u32<8>(u); });
    if constexpr (LPT >= 32) step([](uint32_t u) { return seg_partner_u32<16>(u); });
    if constexpr (LPT >= 64) step([](uint32_t u) { return seg_partner_u32<32>(u); });
}

__device__ __forceinline__ int chunk_expert(int q, int W, int LPT, int lseg) {
    return ((q / W) * LPT + lseg) * W + (q % W);
}

// Load the lane's NE = NV*W logits of token `tok` (as binary32; bf16 widening is exact).
template <int LPT, int NV, bool BF16>
__device__ __forceinline__ void load_row(const RouteArgs& a, int64_t tok, int lseg,
                                         float (&x)[NV * (BF16 ? 8 : 4)]) {
    constexpr int W = BF16 ? 8 : 4;
    const int E = a.E;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int e0 = (j * LPT + lseg) * W;
        if (a.vec && e0 < E) {
            if constexpr (BF16) {
                const u32x4 v = *reinterpret_cast<const MEP_GLOBAL u32x4*>(
                    gptr(reinterpret_cast<const uint16_t*>(a.logits)) + tok * E + e0);
                const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    x[j * W + 2 * q] = __uint_as_float(w4[q] << 16);
                    x[j * W + 2 * q + 1] = __uint_as_float(w4[q] & 0xFFFF0000u);
                }
            } else {
                const u32x4 v = *reinterpret_cast<const MEP_GLOBAL u32x4*>(
                    gptr(reinterpret_cast<const float*>(a.logits)) + tok * E + e0);
                x[j * W + 0] = __uint_as_float(v.x);
                x[j * W + 1] = __uint_as_float(v.y);
                x[j * W + 2] = __uint_as_float(v.z);
                x[j * W + 3] = __uint_as_float(v.w);
            }
        } else {
#pragma unroll
            for (int i = 0; i < W; ++i) {
                const int e = e0 + i;
                float v = 0.0f;
                if (e < E) {
                    if constexpr (BF16)
                        v = __uint_as_float(
                            (uint32_t)(gptr(reinterpret_cast<const uint16_t*>(a.logits))[tok * E + e]) << 16);
                    else
                        v = gptr(reinterpret_cast<const float*>(a.logits))[tok * E + e];
                }
                x[j * W + i] = v;
            }
        }
    }
}

__device__ __forceinline__ float load_logit(const RouteArgs& a, int64_t tok, int e, bool bf16) {
    if (bf16)
        return __uint_as_float((uint32_t)(gptr(reinterpret_cast<const uint16_t*>(a.logits))[tok * a.E + e])
                               << 16);
    return gptr(reinterpret_cast<const float*>(a.logits))[tok * a.E + e];
}

// Exact selection for one token by the LPT lanes of its segment: exact keys (logit, or
// correctly rounded sigmoid + bias), exact group limit, then K rounds of a segmented arg-max
// (max of the order-preserving key, then min expert index among the maxima).  On return the
// lane owning output slot k (k % LPT == lseg) holds its expert in my_e[k / LPT] and the slot's
// key in my_key[k / LPT] (for softmax the selected logit itself: the order key maps back to the
// value, a -0 logit coming back as +0, which no softmax weight tells apart); every lane holds the
// first selected logit in first_x (used by the softmax weights).
template <int LPT, int NV, bool BF16, int KMAX>
__device__ __forceinline__ void exact_select_token(const RouteArgs& a, const float* bias, int lseg,
                                                   const float (&x)[NV * (BF16 ? 8 : 4)],
                                                   int (&my_e)[(KMAX + LPT - 1) / LPT],
                                                   float (&my_key)[(KMAX + LPT - 1) / LPT], float& first_x) {
    constexpr int W = BF16 ? 8 : 4;
    constexpr int NE = NV * W;
    const int E = a.E;
    const int K = a.K;
    const bool sig = a.score_fn == MEP_SIGMOID;
    uint32_t ok[NE];
    uint32_t valid = 0;
#pragma unroll
    for (int q = 0; q < NE; ++q) {
        const int e = chunk_expert(q, W, LPT, lseg);
        const bool v = e < E;
        valid |= (v ? 1u : 0u) << q;
        float key = x[q];
        if (sig) key = (v ? sigmoid_cr(x[q]) : 0.0f) + (v ? bias[e] : 0.0f);
        ok[q] = v ? order_key(key) : 0u;
    }
    uint32_t eligible = valid;
    if (a.n_group > 1) {
        int grp[NE];
#pragma unroll
        for (int q = 0; q < NE; ++q)
            grp[q] = (int)(((float)chunk_expert(q, W, LPT, lseg) + 0.5f) * a.inv_gsize);
        uint32_t score[kMaxGroups];
#pragma unroll
        for (int g = 0; g < kMaxGroups; ++g) {
            score[g] = 0;
            if (g < a.n_group) {
                uint32_t t1 = 0, t2 = 0;
#pragma unroll
                for (int q = 0; q < NE; ++q) {
                    if (((valid >> q) & 1u) && grp[q] == g) {
                        t2 = max(t2, min(t1, ok[q]));
                        t1 = max(t1, ok[q]);
                    }
                }
                seg_top2_u32<LPT>(t1, t2);
                const float f1 = order_key_inv(t1);
                score[g] = order_key((a.group_topn >= 2) ? (f1 + order_key_inv(t2)) : f1);
            }
        }
        // keep topk_group groups by repeated extraction (score desc, group index asc)
        uint32_t kept = 0;
        for (int r = 0; r < a.topk_group; ++r) {
            uint32_t bs = 0;
            int bg = -1;
#pragma unroll
            for (int g = 0; g < kMaxGroups; ++g) {
                if (g < a.n_group && !((kept >> g) & 1u) && (bg < 0 || score[g] > bs)) {
                    bs = score[g];
                    bg = g;
                }
            }
            kept |= 1u << bg;
        }
        uint32_t el = 0;
#pragma unroll
        for (int q = 0; q < NE; ++q) el |= (((kept >> grp[q]) & 1u) ? 1u : 0u) << q;
        eligible &= el;
    }
    uint32_t taken = 0;
    first_x = 0.0f;
    static_for<KMAX>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        if (k >= K) return;
        uint32_t best = 0;
        int best_q = -1;
#pragma unroll
        for (int q = 0; q < NE; ++q) {
            // slots are visited in increasing expert index, so '>' keeps the lower index on ties
            if ((((eligible & ~taken) >> q) & 1u) && (best_q < 0 || ok[q] > best)) {
                best = ok[q];
                best_q = q;
            }
        }
        const int best_e = best_q < 0 ? INT_MAX : chunk_expert(best_q, W, LPT, lseg);
        const uint32_t m = seg_max_u32<LPT>(best_q < 0 ? 0u : best);
        const uint32_t cand = (best_q >= 0 && best == m) ? (uint32_t)best_e : 0xFFFFFFFFu;
        const int e_sel = (int)seg_min_u32<LPT>(cand);
        if (best_q >= 0 && best_e == e_sel) taken |= 1u << best_q;
        if (k == 0) first_x = order_key_inv(m);  // softmax: the first selected logit
        if ((k % LPT) == lseg) {
            my_e[k / LPT] = e_sel;
            my_key[k / LPT] = order_key_inv(m);
        }
    });
}

// Weights from the selected experts of a token.  The lane owning output slot j (j % LPT == lseg)
// holds v_j: the logit (softmax) or the correctly rounded sigmoid (sigmoid).  All arithmetic is
// binary64 (to within a few units of 2^-52), rounded once to binary32 (TensorRT-LLM
// RoutingKernel.cuh calcSoftmax, over the
// selected lanes or over the full score vector; sigmoid weights renormalised and scaled).
// For softmax without renormalisation `full_max`/`full_den` carry the max and the sum of
// exp(x - max) over all E logits of the token.
template <int LPT, int KPL>
__device__ __forceinline__ void write_weights(const RouteArgs& a, int64_t tok, int lseg, bool live,
                                              const int (&my_e)[KPL], const float (&my_v)[KPL],
                                              double first_x, double full_max, double full_den) {
    const bool sig = a.score_fn == MEP_SIGMOID;
    const int K = a.K;
    double term[KPL];
    double den = 0.0;
#pragma unroll
    for (int m = 0; m < KPL; ++m) {
        const int j = m * LPT + lseg;
        double t = 0.0;
        if (j < K) {
            if (sig)
                t = (double)my_v[m];
            else if (a.renormalize)
                t = exp_neg_f64((double)my_v[m] - first_x);
            else
                t = exp_neg_f64((double)my_v[m] - full_max);
        }
        term[m] = t;
        den += t;
    }
    if (sig) {
        if (a.renormalize) den = seg_sum_f64<LPT>(den);
    } else if (a.renormalize) {
        den = seg_sum_f64<LPT>(den);
    } else {
        den = full_den;
    }
    if (!live) return;
    // w = term / den to within a few units of 2^-52 (a reciprocal refined twice, then a product)
    const double inv_den = den > 0.0 ? recip_f64(den) : 0.0;
#pragma unroll
    for (int m = 0; m < KPL; ++m) {
        const int j = m * LPT + lseg;
        if (j < K) {
            gptr(a.ids)[tok * K + j] = my_e[m];
            if (a.weights) {
                double w;
                if (sig && !a.renormalize)
                    w = term[m];
                else
                    w = den > 0.0 ? term[m] * inv_den : 0.0;
                gptr(a.weights)[tok * K + j] = (float)(w * (double)a.scale);
            }
        }
    }
}

// Fast-kernel launcher (route_fast.hip).  Returns false when the shape is not covered.
// One token on LPT lanes, exactly: keys for every expert, K rounds of a segmented arg-max, and the
// weights (the generic routing kernel's whole body; also the routing phase of the one-workgroup
// small-batch kernel).  Token `tok_raw` past the batch computes on the last token and writes
// nothing.  On return, lane lseg holds the experts of output slots k = m*LPT + lseg in my_e[m].
template <int LPT, int NV, bool BF16, int KMAX>
__device__ __forceinline__ void route_generic_token(const RouteArgs& a, int64_t tok_raw, int lseg,
                                                    int (&my_e)[(KMAX + LPT - 1) / LPT]) {
    constexpr int W = BF16 ? 8 : 4;
    constexpr int NE = NV * W;
    constexpr int KPL = (KMAX + LPT - 1) / LPT;
    const bool live = tok_raw < a.N;
    const int64_t tok = live ? tok_raw : (a.N - 1);

    float x[NE];
    load_row<LPT, NV, BF16>(a, tok, lseg, x);
    float key[KPL];
#pragma unroll
    for (int m = 0; m < KPL; ++m) {
        my_e[m] = 0;
        key[m] = 0.0f;
    }
    float first_x;
    exact_select_token<LPT, NV, BF16, KMAX>(a, a.bias, lseg, x, my_e, key, first_x);

    // the weights' values: for softmax the selected logits (the keys), for sigmoid the correctly
    // rounded sigmoid of the selected logit, read again from the row
    const bool sig = a.score_fn == MEP_SIGMOID;
    float my_v[KPL];
#pragma unroll
    for (int m = 0; m < KPL; ++m) {
        const int j = m * LPT + lseg;
        float v = 0.0f;
        if (j < a.K) v = sig ? sigmoid_cr(load_logit(a, tok, my_e[m], BF16)) : key[m];
        my_v[m] = v;
    }
    double full_max = 0.0, full_den = 0.0;
    if (!sig && !a.renormalize) {
        float fm = -FLT_MAX;
#pragma unroll
        for (int q = 0; q < NE; ++q)
            if (chunk_expert(q, W, LPT, lseg) < a.E) fm = fmaxf(fm, x[q]);
        full_max = (double)order_key_inv(seg_max_u32<LPT>(order_key(fm)));
#pragma unroll
        for (int q = 0; q < NE; ++q)
            if (chunk_expert(q, W, LPT, lseg) < a.E) full_den += exp_neg_f64((double)x[q] - full_max);
        full_den = seg_sum_f64<LPT>(full_den);
    }
    write_weights<LPT, KPL>(a, tok, lseg, live, my_e, my_v, (double)first_x, full_max, full_den);
}

// Checks of mep_route_topk's arguments; on MEP_OK `a` holds the launch arguments (a.N == 0: nothing
// to launch).
int route_prepare(const void* logits, int dtype, int64_t N, int E, int K, const float* bias,
                  const mep_route_params* p, int32_t* topk_ids, float* topk_weights, RouteArgs& a);

bool launch_route_fast(const RouteArgs& a, int dtype, const Launch& st);
// Whether the fast kernel, or the sigmoid kernel, covers a routing call (route_launch then takes it).
bool route_fast_covers(const RouteArgs& a);
bool route_sig_covers(const RouteArgs& a);

// Enqueue the routing kernel that covers the shape (sigmoid, fast, or generic); MEP_OK or
// MEP_ERR_UNSUPPORTED.
int route_launch(const RouteArgs& a, int dtype, const Launch& st);

// Sigmoid routing kernel launcher (route_sig.hip).  Returns false when the shape is not covered.
bool launch_route_sig(const RouteArgs& a, int dtype, const Launch& st);
// The same kernel also counting the plan tiles of the fused path (path.h) it owns, with the
// counting epilogue; false when the shape is not covered (nothing is launched then).
struct PathCall;
bool launch_route_sig_counting(const RouteArgs& a, int dtype, const Launch& st, const PathCall& pc);
// The generic kernel counting the plan tiles it owns, for calls neither the sigmoid nor the fast
// kernel covers; false (nothing launched) otherwise or when K > 8.
bool launch_route_generic_counting(const RouteArgs& a, int dtype, const Launch& st, const PathCall& pc);

}  // namespace mep
