// Shape dispatch of the fast routing kernel (route_fast.h): decides whether a routing call is
// covered and with which group mapping and list depth.
#include <mutex>

#include "route_fast.h"

namespace mep {

int resident_blocks(const void* kernel, int block_threads) {
    struct Entry {
        int device;
        const void* kernel;
        int blocks;
    };
    static std::mutex mu;
    static Entry cache[64];
    static int used = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    {
        std::lock_guard<std::mutex> lock(mu);
        for (int i = 0; i < used; ++i)
            if (cache[i].device == dev && cache[i].kernel == kernel) return cache[i].blocks;
    }
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block_threads, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    const int blocks = per_cu * cus;
    std::lock_guard<std::mutex> lock(mu);
    if (used < 64) cache[used++] = Entry{dev, kernel, blocks};
    return blocks;
}

static int ilog2(int v) {
    int l = 0;
    while ((1 << l) < v) ++l;
    return l;
}

// The fast kernel's configuration for a routing call; false when the kernel does not cover it.
static bool fast_plan(const RouteArgs& a, int& LPT, FastCfg& cfg, int& M) {
    if (a.E % kFastEPL != 0 || !a.vec) return false;
    LPT = a.E / kFastEPL;
    if (LPT != 2 && LPT != 4 && LPT != 8 && LPT != 16) return false;
    cfg = FastCfg{};
    int units;
    if (a.n_group <= 1) {
        cfg.mode = 0;
        units = LPT;
    } else {
        const int gsize = a.E / a.n_group;
        if (gsize % kFastEPL == 0) {
            cfg.mode = 1;  // a group spans gsize/32 lanes
            cfg.S = gsize / kFastEPL;
        } else {
            return false;
        }
        cfg.log2S = ilog2(cfg.S);
        if ((1 << cfg.log2S) != cfg.S) return false;
        units = a.topk_group;
    }
    cfg.mt = (a.K + units - 1) / units;
    M = (cfg.mode != 0 && cfg.mt < 2) ? 2 : cfg.mt;  // group scores need the top two
    return M <= 4;
}

bool route_fast_covers(const RouteArgs& a) {
    int LPT, M;
    FastCfg cfg;
    return fast_plan(a, LPT, cfg, M);
}

bool launch_route_fast(const RouteArgs& a, int dtype, const Launch& st) {
    int LPT, M;
    FastCfg cfg;
    if (!fast_plan(a, LPT, cfg, M)) return false;
    if (dtype == MEP_BF16)
        launch_fast_bf16(LPT, a, cfg, M, st);
    else
        launch_fast_f32(LPT, a, cfg, M, st);
    return true;
}

}  // namespace mep
