// Shape dispatch of the sigmoid routing kernel (route_sig.h): plain routing (mep_route_topk) and
// routing that also counts the plan tiles it owns (the routing phase of the fused path).
#include "route_sig.h"

namespace mep {

namespace {

constexpr int kSigWaves = 8;          // one workgroup per compute unit: two waves per SIMD
constexpr int kSigWavesBig = 12;      // three per SIMD, where a workgroup has many sets
constexpr int64_t kSigBigSets = 96;   // sets per workgroup from which the third wave pays
constexpr size_t kLdsLimit = 160 * 1024;

// Static LDS of a kernel (bytes).
size_t static_lds(const void* kernel) {
    hipFuncAttributes attr;
    if (hipFuncGetAttributes(&attr, kernel) != hipSuccess) return kLdsLimit;
    return attr.sharedSizeBytes;
}

template <int LPT, bool BF16, int MODE>
bool launch_sig(const RouteArgs& a, const Launch& st, const PathCall* pc) {
    constexpr int TPW = SigGeom<LPT, BF16>::TPW;
    SigCfg cfg;
    cfg.tg = MODE == 1 ? a.topk_group : LPT;
    SigEpi ep{};
    int64_t grid, sets;
    size_t dyn;
    if (pc) {
        const PathGeom& g = pc->g;
        // sets of the largest workgroup: sub tiles of at most T tokens each
        sets = ceil_div64((int64_t)g.sub * g.T, TPW);
        dyn = sig_dyn_lds(sets, g.sub, g.NC);
        grid = g.nwg;
        ep.on = 1;
        ep.eshift = 0;
        while ((1 << ep.eshift) < g.epn) ++ep.eshift;
        ep.g = g;
        ep.w = pc->w;
        ep.hdr = pc->hdr;
        cfg.tokens_per_group = 0;
    } else {
        const int64_t nsets = ceil_div64(a.N, TPW);
        grid = device_units();
        if (grid > nsets) grid = nsets;
        sets = ceil_div64(nsets, grid);
        cfg.tokens_per_group = sets * TPW;
        grid = ceil_div64(a.N, cfg.tokens_per_group);
        dyn = sig_dyn_lds(sets, 0, 0);
        ep.on = 0;
    }
    // long streams (a decode-size workgroup has few sets) take a third wave per SIMD to hide
    // more of the loop's latencies, if its LDS fits
    auto fits = [&](const void* kernel) { return static_lds(kernel) + dyn <= kLdsLimit; };
    auto big = route_sig_kernel<LPT, BF16, MODE, kSigWavesBig>;
    auto base = route_sig_kernel<LPT, BF16, MODE, kSigWaves>;
    if (sets >= kSigBigSets && fits(reinterpret_cast<const void*>(big))) {
        launch_kernel(big, dim3((unsigned)grid), dim3(64 * kSigWavesBig), (uint32_t)dyn, st, a, cfg, ep);
        return true;
    }
    if (!fits(reinterpret_cast<const void*>(base))) return false;
    launch_kernel(base, dim3((unsigned)grid), dim3(64 * kSigWaves), (uint32_t)dyn, st, a, cfg, ep);
    return true;
}

template <bool BF16, int MODE>
bool launch_sig_lpt(int LPT, const RouteArgs& a, const Launch& st, const PathCall* pc) {
    switch (LPT) {
        case 2: return launch_sig<2, BF16, MODE>(a, st, pc);
        case 4: return launch_sig<4, BF16, MODE>(a, st, pc);
        case 8: return launch_sig<8, BF16, MODE>(a, st, pc);
        default: return launch_sig<16, BF16, MODE>(a, st, pc);
    }
}

// The kernel's lanes per token and group mode for a routing call; false when it does not cover it.
bool sig_plan(const RouteArgs& a, int& LPT, int& mode) {
    if (a.score_fn != MEP_SIGMOID || !a.vec || a.K > 8 || a.E % kFastEPL != 0) return false;
    LPT = a.E / kFastEPL;
    if (LPT != 2 && LPT != 4 && LPT != 8 && LPT != 16) return false;
    if (a.n_group <= 1) mode = 0;
    else if (a.n_group == LPT) mode = 1;
    else return false;
    return true;
}

bool route_sig_dispatch(const RouteArgs& a, int dtype, const Launch& st, const PathCall* pc) {
    int LPT, mode;
    if (!sig_plan(a, LPT, mode)) return false;
    const bool bf16 = dtype == MEP_BF16;
    if (bf16) return mode == 0 ? launch_sig_lpt<true, 0>(LPT, a, st, pc) : launch_sig_lpt<true, 1>(LPT, a, st, pc);
    return mode == 0 ? launch_sig_lpt<false, 0>(LPT, a, st, pc) : launch_sig_lpt<false, 1>(LPT, a, st, pc);
}

}  // namespace

bool route_sig_covers(const RouteArgs& a) {
    int LPT, mode;
    return sig_plan(a, LPT, mode);
}

bool launch_route_sig(const RouteArgs& a, int dtype, const Launch& st) {
    return route_sig_dispatch(a, dtype, st, nullptr);
}

bool launch_route_sig_counting(const RouteArgs& a, int dtype, const Launch& st, const PathCall& pc) {
    return route_sig_dispatch(a, dtype, st, &pc);
}

}  // namespace mep
