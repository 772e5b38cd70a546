// mep_route_topk: router logits [N,E] -> top-K expert ids and routing weights.
//
// Two kernels share one element layout (route_common.h):
//   route_fast_kernel     (route_fast.hip) binary32 keys with a certified error bound, group
//                         limit and top-K through a thresholded candidate list in LDS, exact
//                         binary64 work only for the K selected experts; covers the common
//                         shapes (E = 64..512 with full 16-byte chunks, group sizes aligned to
//                         the chunk layout).
//   route_generic_kernel  (this file) exact keys for every expert and K rounds of a segmented
//                         arg-max; covers every shape the ABI accepts.
#include "route_common.h"

namespace mep {

template <int LPT, int NV, bool BF16, int KMAX>
__global__ __launch_bounds__(kRouteBlock) void route_generic_kernel(RouteArgs a) {
    constexpr int KPL = (KMAX + LPT - 1) / LPT;
    constexpr int TPB = kRouteBlock / LPT;
    const int lseg = threadIdx.x % LPT;
    const int64_t tok_raw = (int64_t)blockIdx.x * TPB + threadIdx.x / LPT;
    int my_e[KPL];
    route_generic_token<LPT, NV, BF16, KMAX>(a, tok_raw, lseg, my_e);
}

template <int LPT, int NV, bool BF16>
static void launch_generic(const RouteArgs& a, const Launch& st) {
    const int tpb = kRouteBlock / LPT;
    const int64_t blocks = ceil_div64(a.N, tpb);
    if (a.K <= 8)
        launch_kernel((route_generic_kernel<LPT, NV, BF16, 8>), dim3((unsigned)blocks),
                           dim3(kRouteBlock), 0, st, a);
    else
        launch_kernel((route_generic_kernel<LPT, NV, BF16, 32>), dim3((unsigned)blocks),
                           dim3(kRouteBlock), 0, st, a);
}

template <bool BF16>
static int dispatch_generic(const RouteArgs& a, const Launch& st) {
    constexpr int W = BF16 ? 8 : 4;
    const int nchunks = (a.E + W - 1) / W;
    if (nchunks <= 1) launch_generic<1, 1, BF16>(a, st);
    else if (nchunks <= 2) launch_generic<2, 1, BF16>(a, st);
    else if (nchunks <= 4) launch_generic<4, 1, BF16>(a, st);
    else if (nchunks <= 8) launch_generic<8, 1, BF16>(a, st);
    else if (nchunks <= 16) launch_generic<16, 1, BF16>(a, st);
    else if (nchunks <= 32) launch_generic<32, 1, BF16>(a, st);
    else if (nchunks <= 64) launch_generic<64, 1, BF16>(a, st);
    else if (nchunks <= 128) launch_generic<64, 2, BF16>(a, st);
    else if (nchunks <= 256) launch_generic<64, 4, BF16>(a, st);
    else return MEP_ERR_UNSUPPORTED;
    return MEP_OK;
}

}  // namespace mep

namespace mep {

int route_prepare(const void* logits, int dtype, int64_t N, int E, int K, const float* bias,
                  const mep_route_params* p, int32_t* topk_ids, float* topk_weights, RouteArgs& a) {
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
    a.N = 0;
    if (N == 0) return MEP_OK;

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
    return MEP_OK;
}

int route_launch(const RouteArgs& a, int dtype, const Launch& st) {
    if (launch_route_sig(a, dtype, st)) return MEP_OK;
    if (launch_route_fast(a, dtype, st)) return MEP_OK;
    return dtype == MEP_BF16 ? dispatch_generic<true>(a, st) : dispatch_generic<false>(a, st);
}

static int route_topk(const void* logits, int dtype, int64_t N, int E, int K, const float* bias,
                      const mep_route_params* p, int32_t* topk_ids, float* topk_weights,
                      const Launch& st) {
    RouteArgs a;
    const int rc = route_prepare(logits, dtype, N, E, K, bias, p, topk_ids, topk_weights, a);
    if (rc != MEP_OK || a.N == 0) return rc;
    const int lr = route_launch(a, dtype, st);
    return lr != MEP_OK ? lr : launch_status();
}

}  // namespace mep

extern "C" int mep_route_topk(const void* logits, int dtype, int64_t N, int E, int K,
                              const float* bias, const mep_route_params* p, int32_t* topk_ids,
                              float* topk_weights, void* stream) {
    mep::launch_begin();
    const mep::Launch l{reinterpret_cast<hipStream_t>(stream), nullptr, nullptr};
    return mep::route_topk(logits, dtype, N, E, K, bias, p, topk_ids, topk_weights, l);
}

extern "C" int mep_route_topk_timed(const void* logits, int dtype, int64_t N, int E, int K,
                                    const float* bias, const mep_route_params* p,
                                    int32_t* topk_ids, float* topk_weights, void* stream,
                                    void* start_event, void* stop_event) {
    mep::launch_begin();
    const mep::Launch l{reinterpret_cast<hipStream_t>(stream),
                        reinterpret_cast<hipEvent_t>(start_event),
                        reinterpret_cast<hipEvent_t>(stop_event)};
    return mep::route_topk(logits, dtype, N, E, K, bias, p, topk_ids, topk_weights, l);
}
