// Launch descriptions of the layout and plan calls, shared by their entry points and by the
// combined entry point mep_layout_plan (layout_plan.hip): geometry, workspace views, output
// pointers, and the host functions that check the arguments and enqueue the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mep.h"
#include "device_common.h"

namespace mep {

// Geometry: tiles of kLayTile slots (one workgroup each in both kernels); a count tile groups
// `sub` consecutive tiles so that at most kCountTiles count tiles exist.
struct LayGeom {
    int NK, E, nsub, sub, nct;
};

// Workspace of mep_build_layout after the header: arrival counters of count tiles (fixed place,
// always left at zero), look-back words [nct][E], and the tagged histogram of every tile
// [nsub][E].  Tagged words are written with single atomic stores and carry the call's epoch, so
// a reader on another compute die needs no cache write-back fence: it re-reads until the tag is
// current.
struct LayWs {
    uint32_t* arrive;
    uint64_t* status;
    uint64_t* tilehist;
};

struct LayoutOut {
    int32_t* tokens_per_expert;
    int32_t* cu_seqlens;
    int32_t* e2p;
    int32_t* p2e;
    int32_t* zero_fill;
    int p2e_cap;
};

struct LayoutCall {
    LayGeom g;
    LayWs lw;
    WsHeader* hdr;
    LayoutOut out;
    const int32_t* ids;
    int A;
};

// Write tiles: TT tokens, never crossing a shard (tps per shard, ntiles in all).  Count tiles:
// `sub` consecutive write tiles of one shard (ctps per shard, nct in all).
struct PlanGeom {
    int N, E, K, R, epn, S, n, tps, ntiles, TT, ncols, C;
    int sub, ctps, nct;
    int ticketed;  // write tiles in ticket order (when count tiles could outnumber resident groups)
    int direct;    // count-tile prefixes by the last count tile's scan (nct <= kDirectCountTiles),
                   // else by the decoupled look-back
    int64_t NvS;
};

// count tile of write tile wt, and the first write tile of that count tile
__device__ __forceinline__ int ct_of(const PlanGeom& g, int wt) {
    const int sh = wt / g.tps;
    return sh * g.ctps + (wt - sh * g.tps) / g.sub;
}
__device__ __forceinline__ int ct_first_wt(const PlanGeom& g, int ct) {
    const int sh = ct / g.ctps;
    return sh * g.tps + (ct - sh * g.ctps) * g.sub;
}

// Workspace of mep_plan after the header: arrival counters of count tiles (fixed place, always
// left at zero), look-back words of the rank columns [nct][3R] and of the expert columns
// [nct][E], and the tagged histograms of every write tile [ntiles][3R+E].
// Tagged words are written with single atomic stores and carry the call's epoch, so a reader on
// another compute die needs no cache write-back fence: it re-reads until the tag is current.
struct PlanWs {
    uint32_t* arrive;
    uint64_t* status3;
    uint64_t* statusE;
    uint64_t* tilehist;
};

struct PlanOutDev {
    uint8_t* itr;
    int32_t* ntpr;
    int32_t* ntpe;
    int32_t* rank_prefix;
    int32_t* chan;
    int32_t* recv_tokens;
    int32_t* recv_cu;
    int32_t* recv_zf;
    int32_t* dst;
    int32_t* dup_counts;
    int32_t* dup_offsets;
    int32_t* dup_groups;
    int64_t cap_g;
    int32_t* dup_loffs;
    int64_t cap_d;
};

// Where the scatter kernel of the layout takes its tiles and prefix data from: the layout's own
// counting pass (tiles of 4096 slots, look-back words [nct][E], histograms [nsub][E]), or, in
// mep_layout_plan, the plan's counting pass (write tiles of TT tokens that never cross a shard,
// expert look-back words [nct][E], expert counts at column 3R of each tile histogram).
struct ScatterSrc {
    int plan;  // 0: layout geometry, 1: plan geometry
    LayGeom lg;
    LayWs lw;
    PlanGeom pg;
    PlanWs pw;
};

struct PlanCall {
    PlanGeom g;
    PlanWs pw;
    WsHeader* hdr;
    PlanOutDev o;
    const int32_t* ids;
    const int32_t* cu;
    const int32_t* e2p;
};

// Argument checks of mep_build_layout / mep_plan (MEP_OK or the error code, nothing enqueued on
// error) and the launch descriptions.
int layout_prepare_outputs(const int32_t* topk_ids, int64_t N, int E, int K, int alignment,
                           int32_t* tokens_per_expert, int32_t* cu_seqlens, int32_t* expanded_to_permuted,
                           int32_t* permuted_to_expanded, int64_t permuted_cap, int32_t* zero_fill,
                           LayoutCall& c);
int layout_prepare(const int32_t* topk_ids, int64_t N, int E, int K, int alignment,
                   int32_t* tokens_per_expert, int32_t* cu_seqlens, int32_t* expanded_to_permuted,
                   int32_t* permuted_to_expanded, int64_t permuted_cap, int32_t* zero_fill, void* ws,
                   size_t ws_bytes, LayoutCall& c);
int plan_prepare(const int32_t* topk_ids, const int32_t* cu_seqlens, const int32_t* expanded_to_permuted,
                 int64_t N, int E, int K, int alignment, int R, int num_src, int num_channels, int64_t NvS,
                 const mep_plan_outputs* out, void* ws, size_t ws_bytes, PlanCall& c);

// Enqueue the layout kernels; the plan's counting and writing passes.
void layout_launch(const LayoutCall& c, hipStream_t st);
// The layout's scatter pass over the plan's tiles, from the plan's counting pass (mep_layout_plan).
void layout_launch_scatter_from_plan(const LayoutCall& lc, const PlanCall& pc, hipStream_t st);
void plan_launch_count(const PlanCall& c, hipStream_t st);
// The scatter and write passes of mep_layout_plan in one kernel (after plan_launch_count); two
// kernels for K > 8.
void plan_launch_scatter_write(const LayoutCall& lc, const PlanCall& pc, hipStream_t st);
void plan_launch_write(const PlanCall& c, hipStream_t st);

// Optional events stamped by the launches of mep_route_layout_plan_timed: the routing kernel (or
// the one small-batch kernel) and the plan-tile kernel.
struct StepEvents {
    hipEvent_t route_start = nullptr, route_stop = nullptr, plan_start = nullptr, plan_stop = nullptr;
};

}  // namespace mep
