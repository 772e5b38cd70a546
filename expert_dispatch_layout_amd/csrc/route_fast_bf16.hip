// Instantiations of the fast routing kernel for bfloat16 logits.
#include "route_fast.h"

namespace mep {

void launch_fast_bf16(int LPT, const RouteArgs& a, const FastCfg& cfg, int M, const Launch& st) {
    switch (LPT) {
        case 2: launch_fast_shape<2, true>(a, cfg, M, st); break;
        case 4: launch_fast_shape<4, true>(a, cfg, M, st); break;
        case 8: launch_fast_shape<8, true>(a, cfg, M, st); break;
        default: launch_fast_shape<16, true>(a, cfg, M, st); break;
    }
}

}  // namespace mep
