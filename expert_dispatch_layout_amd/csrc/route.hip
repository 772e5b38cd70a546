// mep_route_topk: router logits [N,E] -> top-K expert ids and routing weights.
//
// Mapping: a token is handled by a segment of LPT lanes of one wave64 (64/LPT tokens per wave).
// Each lane loads NV 16-byte chunks of the token's row; chunk c = j*LPT + lane covers experts
// [c*W, c*W+W) with W = 4 (fp32) or 8 (bf16), so every load instruction of a segment reads one
// contiguous run of the row.  Keys stay in registers; selection is K rounds of a segmented
// arg-max (max of an order-preserving integer key, then min expert index among the maxima),
// which realises the "key descending, expert index ascending" order.
//
// Weights: the lane that owns output slot j evaluates its term in binary64; a segmented sum
// gives the denominator (TensorRT-LLM RoutingKernel.cuh calcSoftmax, over the selected lanes or
// over the whole score vector).
#include <float.h>
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

constexpr int kRouteBlock = 256;
constexpr int kMaxGroups = 32;

template <int LPT>
__device__ __forceinline__ uint32_t seg_max_u32(uint32_t v) {
#pragma unroll
    for (int o = LPT / 2; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, LPT));
    return v;
}

template <int LPT>
__device__ __forceinline__ uint32_t seg_min_u32(uint32_t v) {
#pragma unroll
    for (int o = LPT / 2; o >= 1; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, LPT));
    return v;
}

template <int LPT>
__device__ __forceinline__ double seg_sum_f64(double v) {
#pragma unroll
    for (int o = LPT / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, LPT);
    return v;
}

// merge (a1 >= a2) with the partner lane's (b1 >= b2), keeping the two largest values
template <int LPT>
__device__ __forceinline__ void seg_top2_u32(uint32_t& t1, uint32_t& t2) {
#pragma unroll
    for (int o = LPT / 2; o >= 1; o >>= 1) {
        uint32_t b1 = (uint32_t)__shfl_xor((int)t1, o, LPT);
        uint32_t b2 = (uint32_t)__shfl_xor((int)t2, o, LPT);
        uint32_t n2 = max(min(t1, b1), max(t2, b2));
        t1 = max(t1, b1);
        t2 = n2;
    }
}

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0..N-1.
template <int N, typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

template <int LPT, int NV, bool BF16, int KMAX>
__global__ __launch_bounds__(kRouteBlock) void route_kernel(RouteArgs a) {
    constexpr int W = BF16 ? 8 : 4;
    constexpr int NE = NV * W;              // experts per lane
    constexpr int KPL = (KMAX + LPT - 1) / LPT;  // output slots per lane
    constexpr int TPB = kRouteBlock / LPT;

    const int lseg = threadIdx.x % LPT;
    const int64_t tok_raw = (int64_t)blockIdx.x * TPB + threadIdx.x / LPT;
    const bool live = tok_raw < a.N;
    const int64_t tok = live ? tok_raw : (a.N - 1);
    const int E = a.E;
    const int K = a.K;

    // ---- load the row ------------------------------------------------------------------
    float x[NE];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int c = j * LPT + lseg;
        const int e0 = c * W;
        if (a.vec && e0 < E) {
            if (BF16) {
                const uint4 v = *reinterpret_cast<const uint4*>(
                    reinterpret_cast<const uint16_t*>(a.logits) + tok * E + e0);
                const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    x[j * W + 2 * q] = __uint_as_float(w4[q] << 16);
                    x[j * W + 2 * q + 1] = __uint_as_float(w4[q] & 0xFFFF0000u);
                }
            } else {
                const float4 v = *reinterpret_cast<const float4*>(
                    reinterpret_cast<const float*>(a.logits) + tok * E + e0);
                x[j * W + 0] = v.x;
                x[j * W + 1] = v.y;
                x[j * W + 2] = v.z;
                x[j * W + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < W; ++i) {
                const int e = e0 + i;
                float v = 0.0f;
                if (e < E) {
                    if (BF16)
                        v = __uint_as_float(
                            (uint32_t)(reinterpret_cast<const uint16_t*>(a.logits)[tok * E + e]) << 16);
                    else
                        v = reinterpret_cast<const float*>(a.logits)[tok * E + e];
                }
                x[j * W + i] = v;
            }
        }
    }

    // ---- keys ---------------------------------------------------------------------------
    const bool sig = a.score_fn == MEP_SIGMOID;
    float s[NE];
    uint32_t ok[NE];
    uint32_t valid = 0;
#pragma unroll
    for (int q = 0; q < NE; ++q) {
        const int e = ((q / W) * LPT + lseg) * W + (q % W);
        const bool v = e < E;
        valid |= (v ? 1u : 0u) << q;
        float key = x[q];
        if (sig) {
            s[q] = v ? sigmoid_cr(x[q]) : 0.0f;
            key = s[q] + (v ? a.bias[e] : 0.0f);
        } else {
            s[q] = 0.0f;
        }
        ok[q] = v ? order_key(key) : 0u;
    }

    // ---- group limit ----------------------------------------------------------------------
    uint32_t eligible = valid;
    if (a.n_group > 1) {
        int grp[NE];
#pragma unroll
        for (int q = 0; q < NE; ++q) {
            const int e = ((q / W) * LPT + lseg) * W + (q % W);
            grp[q] = (int)(((float)e + 0.5f) * a.inv_gsize);
        }
        uint32_t score[kMaxGroups];
#pragma unroll
        for (int g = 0; g < kMaxGroups; ++g) {
            score[g] = 0;
            if (g < a.n_group) {
                uint32_t t1 = 0, t2 = 0;
#pragma unroll
                for (int q = 0; q < NE; ++q) {
                    if (((valid >> q) & 1u) && grp[q] == g) {
                        const uint32_t v = ok[q];
                        t2 = max(t2, min(t1, v));
                        t1 = max(t1, v);
                    }
                }
                seg_top2_u32<LPT>(t1, t2);
                const float f1 = order_key_inv(t1);
                const float sc = (a.group_topn >= 2) ? (f1 + order_key_inv(t2)) : f1;
                score[g] = order_key(sc);
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

    // ---- top-K by K rounds of segmented arg-max ---------------------------------------
    int my_e[KPL];
    float my_v[KPL];
#pragma unroll
    for (int m = 0; m < KPL; ++m) {
        my_e[m] = 0;
        my_v[m] = 0.0f;
    }
    float first_x = 0.0f;
    uint32_t taken = 0;
    static_for<KMAX>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        if (k >= K) return;
        uint32_t best = 0;
        int best_q = -1;
#pragma unroll
        for (int q = 0; q < NE; ++q) {
            // slots are visited in increasing expert index, so '>' keeps the lower index on ties
            if (((eligible & ~taken) >> q) & 1u) {
                if (best_q < 0 || ok[q] > best) {
                    best = ok[q];
                    best_q = q;
                }
            }
        }
        const int best_e = best_q < 0 ? INT_MAX
                                      : ((best_q / W) * LPT + lseg) * W + (best_q % W);
        const uint32_t m = seg_max_u32<LPT>(best_q < 0 ? 0u : best);
        const uint32_t cand = (best_q >= 0 && best == m) ? (uint32_t)best_e : 0xFFFFFFFFu;
        const int e_sel = (int)seg_min_u32<LPT>(cand);
        float own_v = 0.0f;
        if (best_q >= 0 && best_e == e_sel) taken |= 1u << best_q;
#pragma unroll
        for (int q = 0; q < NE; ++q)
            if (q == best_q) own_v = sig ? s[q] : x[q];
        float v;
        if (sig) {
            const int owner_lane = (e_sel / W) % LPT;
            v = __shfl(own_v, owner_lane, LPT);
        } else {
            v = order_key_inv(m);  // the logit itself (-0 read back as +0)
        }
        if (k == 0) first_x = v;
        if ((k % LPT) == lseg) {
            my_e[k / LPT] = e_sel;
            my_v[k / LPT] = v;
        }
    });

    // ---- weights ------------------------------------------------------------------------
    double term[KPL];
    double den = 0.0;
    if (!sig) {
        double mx;
        if (a.renormalize) {
            mx = (double)first_x;
#pragma unroll
            for (int m = 0; m < KPL; ++m) {
                const int j = m * LPT + lseg;
                term[m] = (j < K) ? exp((double)my_v[m] - mx) : 0.0;
                den += term[m];
            }
            den = seg_sum_f64<LPT>(den);
        } else {
            float fm = -FLT_MAX;
#pragma unroll
            for (int q = 0; q < NE; ++q)
                if ((valid >> q) & 1u) fm = fmaxf(fm, x[q]);
            mx = (double)order_key_inv(seg_max_u32<LPT>(order_key(fm)));
#pragma unroll
            for (int q = 0; q < NE; ++q)
                if ((valid >> q) & 1u) den += exp((double)x[q] - mx);
            den = seg_sum_f64<LPT>(den);
#pragma unroll
            for (int m = 0; m < KPL; ++m) {
                const int j = m * LPT + lseg;
                term[m] = (j < K) ? exp((double)my_v[m] - mx) : 0.0;
            }
        }
    } else {
#pragma unroll
        for (int m = 0; m < KPL; ++m) {
            const int j = m * LPT + lseg;
            term[m] = (j < K) ? (double)my_v[m] : 0.0;
            den += term[m];
        }
        if (a.renormalize) den = seg_sum_f64<LPT>(den);
    }

    if (live) {
#pragma unroll
        for (int m = 0; m < KPL; ++m) {
            const int j = m * LPT + lseg;
            if (j < K) {
                a.ids[tok * K + j] = my_e[m];
                if (a.weights) {
                    double w;
                    if (sig && !a.renormalize)
                        w = term[m];
                    else
                        w = den > 0.0 ? term[m] / den : 0.0;
                    a.weights[tok * K + j] = (float)(w * (double)a.scale);
                }
            }
        }
    }
}

template <int LPT, int NV, bool BF16>
static void launch_k(const RouteArgs& a, hipStream_t st) {
    const int tpb = kRouteBlock / LPT;
    const int64_t blocks = ceil_div64(a.N, tpb);
    if (a.K <= 8)
        hipLaunchKernelGGL((route_kernel<LPT, NV, BF16, 8>), dim3((unsigned)blocks), dim3(kRouteBlock),
                           0, st, a);
    else
        hipLaunchKernelGGL((route_kernel<LPT, NV, BF16, 32>), dim3((unsigned)blocks), dim3(kRouteBlock),
                           0, st, a);
}

template <bool BF16>
static int dispatch_shape(const RouteArgs& a, hipStream_t st) {
    constexpr int W = BF16 ? 8 : 4;
    const int nchunks = (a.E + W - 1) / W;
    if (nchunks <= 1) launch_k<1, 1, BF16>(a, st);
    else if (nchunks <= 2) launch_k<2, 1, BF16>(a, st);
    else if (nchunks <= 4) launch_k<4, 1, BF16>(a, st);
    else if (nchunks <= 8) launch_k<8, 1, BF16>(a, st);
    else if (nchunks <= 16) launch_k<16, 1, BF16>(a, st);
    else if (nchunks <= 32) launch_k<32, 1, BF16>(a, st);
    else if (nchunks <= 64) launch_k<64, 1, BF16>(a, st);
    else if (nchunks <= 128) launch_k<64, 2, BF16>(a, st);
    else if (nchunks <= 256) launch_k<64, 4, BF16>(a, st);
    else return MEP_ERR_UNSUPPORTED;
    return launch_status();
}

}  // namespace mep

extern "C" int mep_route_topk(const void* logits, int dtype, int64_t N, int E, int K,
                              const float* bias, const mep_route_params* p, int32_t* topk_ids,
                              float* topk_weights, void* stream) {
    using namespace mep;
    if (!p) return MEP_ERR_INVALID_ARG;
    if (N > 0 && (!logits || !topk_ids)) return MEP_ERR_INVALID_ARG;  // N == 0 reads nothing
    if (dtype != MEP_F32 && dtype != MEP_BF16) return MEP_ERR_INVALID_ARG;
    if (p->score_fn != MEP_SOFTMAX && p->score_fn != MEP_SIGMOID) return MEP_ERR_INVALID_ARG;
    if (N < 0 || E < 1 || K < 1) return MEP_ERR_INVALID_ARG;
    if (!aligned(logits, 16) || !aligned(topk_ids, 4) || (topk_weights && !aligned(topk_weights, 4)))
        return MEP_ERR_INVALID_ARG;
    if (p->score_fn == MEP_SIGMOID && ((N > 0 && !bias) || !aligned(bias, 4))) return MEP_ERR_INVALID_ARG;
    if (!(p->scale == p->scale) || p->scale > FLT_MAX || p->scale < -FLT_MAX) return MEP_ERR_INVALID_ARG;
    if (p->n_group < 1 || p->renormalize < 0 || p->renormalize > 1) return MEP_ERR_INVALID_ARG;
    if (E > 1024 || K > 32 || K > E) return MEP_ERR_UNSUPPORTED;
    if (N > 0 && (int64_t)N * K > INT32_MAX) return MEP_ERR_UNSUPPORTED;
    if (p->n_group > 1) {
        if (p->n_group > kMaxGroups || E % p->n_group != 0) return MEP_ERR_UNSUPPORTED;
        const int gsize = E / p->n_group;
        if (p->topk_group < 1 || p->topk_group > p->n_group) return MEP_ERR_INVALID_ARG;
        if (p->group_topn < 1 || p->group_topn > 2 || p->group_topn > gsize) return MEP_ERR_UNSUPPORTED;
        if ((int64_t)p->topk_group * gsize < K) return MEP_ERR_UNSUPPORTED;
    }
    if (N == 0) return MEP_OK;

    RouteArgs a;
    a.logits = logits;
    a.bias = bias;
    a.N = N;
    a.E = E;
    a.K = K;
    a.score_fn = p->score_fn;
    a.renormalize = p->renormalize;
    a.n_group = p->n_group;
    a.topk_group = p->n_group > 1 ? p->topk_group : 1;
    a.group_topn = p->group_topn;
    a.scale = p->scale;
    a.inv_gsize = 1.0f / (float)(E / p->n_group);
    a.ids = topk_ids;
    a.weights = topk_weights;
    const int W = dtype == MEP_BF16 ? 8 : 4;
    a.vec = (E % W) == 0;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    return dtype == MEP_BF16 ? dispatch_shape<true>(a, st) : dispatch_shape<false>(a, st);
}
