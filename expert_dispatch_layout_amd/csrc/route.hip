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
#include "path.h"
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

// The generic kernel as the routing phase of the fused layout + plan path (path.h), for
// workgroups whose tokens fit one pass (small batches): workgroup b routes the tokens of plan
// tiles [b * sub, b * sub + nsub), keeping their experts in LDS, then counts each token into its
// tile's histogram row (LDS) and ends with the counting epilogue.  Routing first and counting
// after keeps the plan geometry out of the routing code's registers; a loop over several passes
// would make the routing code's live values spill, so larger batches take the routing kernel
// and then the counting kernel instead.
constexpr int kRouteCountBlock = 512;

template <int LPT, int NV, bool BF16>
__global__ __launch_bounds__(kRouteCountBlock) void route_generic_count_kernel(RouteArgs a, PathGeom g, PathWs w,
                                                                               WsHeader* hdr) {
    constexpr int NT = kRouteCountBlock;
    constexpr int KMAX = kPathMaxK;
    constexpr int KPL = (KMAX + LPT - 1) / LPT;
    constexpr int TPB = NT / LPT;
    __shared__ int s_e[TPB * kPathMaxK];  // experts of the workgroup's slots
    __shared__ int s_row[kPathMaxSub * kPathMaxNC];
    __shared__ int s_tb[kPathMaxSub + 1];
    const int tid = threadIdx.x;
    const int lseg = tid % LPT;
    const int j0 = blockIdx.x * g.sub;
    const int nsub = min(g.sub, g.ntiles - j0);
    for (int i = tid; i < nsub * g.NC; i += NT) s_row[i] = 0;
    if (tid <= nsub) {
        int64_t c0, c1;
        path_tile_tokens(g, j0 + min(tid, nsub - 1), c0, c1);
        s_tb[tid] = (int)(tid < nsub ? c0 : c1);
    }
    const uint32_t pcall = path_count_begin(hdr);
    __syncthreads();
    const int t0 = s_tb[0], t1 = s_tb[nsub];  // t1 - t0 <= TPB
    const int K = a.K;
    // ---- routing (a wave whose tokens all lie past the tiles skips it; a token past the tiles
    // computes on the batch's last token and writes nothing)
    if (t0 + __builtin_amdgcn_readfirstlane((tid & ~63) / LPT) < t1) {
        const int tok = t0 + tid / LPT;
        const bool mine = tok < t1;
        int my_e[KPL];
        route_generic_token<LPT, NV, BF16, KMAX>(a, mine ? (int64_t)tok : a.N, lseg, my_e);
#pragma unroll
        for (int m = 0; m < KPL; ++m) {
            const int j = m * LPT + lseg;
            if (mine && j < K) s_e[(tok - t0) * K + j] = my_e[m];
        }
    }
    __syncthreads();
    // ---- counting: one token per thread
    for (int t = t0 + tid; t < t1; t += NT) {
        int i = 0;
        while (i + 1 < nsub && t >= s_tb[i + 1]) ++i;
        int e[kPathMaxK];
#pragma unroll
        for (int k = 0; k < kPathMaxK; ++k) e[k] = k < K ? s_e[(t - t0) * K + k] : -1;
        path_count_token<1, kPathMaxK>(g, s_row + i * g.NC, e, 0);
    }
    path_epilogue<NT>(g, w, pcall, s_row);
}

template <int LPT, int NV, bool BF16>
static bool launch_generic_count(const RouteArgs& a, const Launch& st, const PathCall& pc) {
    if ((int64_t)pc.g.sub * pc.g.T > kRouteCountBlock / LPT) return false;  // more than one pass
    launch_kernel((route_generic_count_kernel<LPT, NV, BF16>), dim3((unsigned)pc.g.nwg), dim3(kRouteCountBlock), 0,
                  st, a, pc.g, pc.w, pc.hdr);
    return true;
}

template <bool BF16>
static bool dispatch_generic_count(const RouteArgs& a, const Launch& st, const PathCall& pc) {
    constexpr int W = BF16 ? 8 : 4;
    const int nchunks = (a.E + W - 1) / W;
    if (nchunks <= 1) return launch_generic_count<1, 1, BF16>(a, st, pc);
    if (nchunks <= 2) return launch_generic_count<2, 1, BF16>(a, st, pc);
    if (nchunks <= 4) return launch_generic_count<4, 1, BF16>(a, st, pc);
    if (nchunks <= 8) return launch_generic_count<8, 1, BF16>(a, st, pc);
    return false;  // 16 or more lanes per token: fewer than the 64 tokens of a tile per pass
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

bool launch_route_generic_counting(const RouteArgs& a, int dtype, const Launch& st, const PathCall& pc) {
    if (a.K > kPathMaxK || route_sig_covers(a) || route_fast_covers(a)) return false;
    return dtype == MEP_BF16 ? dispatch_generic_count<true>(a, st, pc) : dispatch_generic_count<false>(a, st, pc);
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
