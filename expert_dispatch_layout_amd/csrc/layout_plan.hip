// mep_layout_plan: the layout and the plan of one batch in one call, two kernels instead of
// four.  Where the fused path covers the shape (path.h: K <= 8, R <= 32, E <= 512), its counting
// kernel takes every histogram row and prefix (including the layout's totals and cu_seqlens) in
// one launch and the plan-tile kernel writes the rest; otherwise the plan's counting pass also
// takes the per-expert counts of its tiles and one kernel scatters each of the plan's tiles (the
// layout) and writes that tile's part of the plan.  The results are those of mep_build_layout
// followed by mep_plan.
#include "calls.h"
#include "host_common.h"
#include "path.h"

extern "C" int mep_layout_plan(const int32_t* topk_ids, int64_t N, int E, int K, int alignment,
                               int32_t* tokens_per_expert, int32_t* cu_seqlens, int32_t* expanded_to_permuted,
                               int32_t* permuted_to_expanded, int64_t permuted_cap, int32_t* zero_fill, int R,
                               int num_src, int num_channels, int64_t NvS, const mep_plan_outputs* out, void* ws,
                               size_t ws_bytes, void* stream) {
    mep::launch_begin();
    using namespace mep;
    PlanCall pc;
    int rc = plan_prepare(topk_ids, cu_seqlens, expanded_to_permuted, N, E, K, alignment, R, num_src, num_channels,
                          NvS, out, ws, ws_bytes, pc);
    if (rc != MEP_OK) return rc;
    // the layout's checks and outputs; its workspace is not used (the plan's serves both)
    LayoutCall lc;
    rc = layout_prepare_outputs(topk_ids, N, E, K, alignment, tokens_per_expert, cu_seqlens, expanded_to_permuted,
                                permuted_to_expanded, permuted_cap, zero_fill, lc);
    if (rc != MEP_OK) return rc;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (path_supported(N, E, K, R)) {
        const PathCall c = path_call(lc, pc, ws);
        path_launch_count(c, st);
        path_launch_plan(c, st, nullptr, nullptr);
        return launch_status();
    }
    plan_launch_count(pc, st);
    plan_launch_scatter_write(lc, pc, st);
    return launch_status();
}
