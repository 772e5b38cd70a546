// Shape dispatch of the sigmoid routing kernel (route_sig.h).
#include "route_sig.h"

namespace mep {

template <int LPT, bool BF16, int MODE>
static void launch_sig(const RouteArgs& a, const Launch& st) {
    SigCfg cfg;
    cfg.nsets = ceil_div64(a.N, FastGeom<LPT, BF16>::TPW);
    cfg.tg = MODE == 1 ? a.topk_group : LPT;
    constexpr int NW = 2;  // waves per workgroup: 2 measured ahead of 4 and 8 at the dsv3 batch
    auto kernel = route_sig_kernel<LPT, BF16, MODE, NW>;
    const int64_t need = ceil_div64(cfg.nsets, NW);
    int64_t grid = resident_blocks(reinterpret_cast<const void*>(kernel), 64 * NW);
    // more workgroups than fit at once when a workgroup would own more sets than its LDS list of
    // uncertified tokens holds
    if (grid < ceil_div64(cfg.nsets, kSigMaxSetsPerGroup)) grid = ceil_div64(cfg.nsets, kSigMaxSetsPerGroup);
    if (grid > need) grid = need;
    if (grid < 1) grid = 1;
    const int64_t spb = ceil_div64(cfg.nsets, grid);  // sets per workgroup (as the kernel computes)
    launch_kernel(kernel, dim3((unsigned)grid), dim3(64 * NW), (uint32_t)(spb * sizeof(uint32_t)), st, a, cfg);
}

template <bool BF16, int MODE>
static void launch_sig_lpt(int LPT, const RouteArgs& a, const Launch& st) {
    switch (LPT) {
        case 2: launch_sig<2, BF16, MODE>(a, st); break;
        case 4: launch_sig<4, BF16, MODE>(a, st); break;
        case 8: launch_sig<8, BF16, MODE>(a, st); break;
        default: launch_sig<16, BF16, MODE>(a, st); break;
    }
}

bool launch_route_sig(const RouteArgs& a, int dtype, const Launch& st) {
    if (a.score_fn != MEP_SIGMOID || !a.vec || a.K > 8 || a.E % kFastEPL != 0) return false;
    const int LPT = a.E / kFastEPL;
    if (LPT != 2 && LPT != 4 && LPT != 8 && LPT != 16) return false;
    int mode;
    if (a.n_group <= 1) mode = 0;
    else if (a.n_group == LPT) mode = 1;
    else return false;
    const bool bf16 = dtype == MEP_BF16;
    if (bf16) {
        if (mode == 0) launch_sig_lpt<true, 0>(LPT, a, st);
        else launch_sig_lpt<true, 1>(LPT, a, st);
    } else {
        if (mode == 0) launch_sig_lpt<false, 0>(LPT, a, st);
        else launch_sig_lpt<false, 1>(LPT, a, st);
    }
    return true;
}

}  // namespace mep
