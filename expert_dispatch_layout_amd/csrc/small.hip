// mep_route_layout_plan: routing, layout and plan of one batch in one call.  Small batches
// (decode sizes) run as one kernel of one workgroup, in the spirit of TensorRT-LLM
// RoutingKernel.cuh's routingPermutation (the whole routing permutation of a small batch inside
// one cluster, without a second launch); larger batches take the plan-tile path (path.h): the
// routing kernel, which also counts the plan tiles it routes (the sigmoid kernel, and the
// generic kernel for the shapes neither specialised kernel covers; after the fast kernel the
// counting kernel does), then the plan-tile kernel.  Results are identical to
// mep_route_topk followed by mep_build_layout and mep_plan either way.
//
// The one-workgroup kernel (512 threads) keeps every slot's expert and permuted position in
// LDS and walks the phases with barriers in between:
//   route    tokens on LPT lanes each, 512 / LPT at a time, with the generic routing code
//            (exact keys, K rounds of a segmented arg-max, binary64 weights); the experts also
//            go to LDS
//   layout   histogram by LDS atomics, padded exclusive scan, then the slots in order, 512 at
//            a time: a slot's rank among its wave's slots of the same expert from one ballot per
//            id bit, per-(wave, expert) counts prefixed across the waves, plus the running
//            count of the earlier chunks -- the stable order
//   plan     per token: membership mask, per-shard counts and channel counts by LDS atomics,
//            dst with the duplicate encoding; then the prefix matrices, the receive layout, and
//            per rank two token-order scans (totals, then positions) for the dedup lists
// Nothing crosses workgroups, so the kernel needs no workspace and has no look-back.
#include <float.h>
#include <limits.h>

#include "calls.h"
#include "host_common.h"
#include "path.h"
#include "route_common.h"

namespace mep {

namespace {

constexpr int kSmBlock = 512;
constexpr int kSmWaves = kSmBlock / 64;
constexpr int kSmMaxSlots = 2048;  // above this the three-kernel path is faster
constexpr int kSmMaxE = 256;
constexpr int kSmMaxR = 8;
constexpr int kSmMaxShardE = 4096;   // num_src * E
constexpr int kSmMaxChan = 4096;     // num_src * R * num_channels
constexpr int kSmKMax = 8;

// Barrier that orders LDS only.  Every phase below reads what other threads wrote in LDS, never
// in global memory, so no barrier needs to wait for the global stores still in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Exclusive scan over the 64 lanes of a wave (all active); `total` gets the sum.  DPP row
// shifts give the inclusive scan within rows of 16 lanes, the row broadcasts carry it across.
__device__ __forceinline__ int sm_wave_excl_scan(int v, int& total) {
    int x = v;
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    total = __builtin_amdgcn_readlane(x, 63);
    return x - v;
}

// Exclusive scan of one int per thread over the workgroup, with LDS-only barriers.
__device__ __forceinline__ int lds_block_scan(int v, int* s_tmp, int& total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    if (lane == 63) s_tmp[w] = incl;
    lds_barrier();
    int off = 0;
    total = 0;
    for (int i = 0; i < kSmWaves; ++i) {
        const int x = s_tmp[i];
        off += i < w ? x : 0;
        total += x;
    }
    lds_barrier();
    return off + incl - v;
}

struct SmallArgs {
    RouteArgs ra;
    int A;
    LayoutOut lo;
    PlanGeom g;
    PlanOutDev po;
};

template <int LPT, int NV, bool BF16>
__global__ __launch_bounds__(kSmBlock) void small_path_kernel(SmallArgs sa) {
    __shared__ int s_ids[kSmMaxSlots];
    __shared__ int s_P[kSmMaxSlots];
    __shared__ int s_cnt[kSmMaxE];
    __shared__ int s_cu[kSmMaxE + 1];
    __shared__ int s_run[kSmMaxE];
    __shared__ int s_chunk[kSmMaxE];
    __shared__ int s_wc[kSmWaves][kSmMaxE];
    __shared__ int s_ntpe[kSmMaxShardE];
    __shared__ int s_ntpr[kSmMaxShardE];
    __shared__ int s_chan[kSmMaxChan];
    __shared__ int s_tmp[kSmWaves];
    __shared__ int s_dtot[2 * kSmMaxR];
    __shared__ int s_wsum[kSmMaxSlots / kSmBlock][kSmWaves][kSmMaxR];
    __shared__ int s_goff[kSmMaxR];
    __shared__ int s_doff[kSmMaxR];
    __shared__ uint32_t s_hc[kSmMaxSlots];  // per token: slots on each rank, 4-bit fields

    const RouteArgs& a = sa.ra;
    const PlanGeom& g = sa.g;
    const int tid = threadIdx.x;
    const int wv = tid >> 6;
    const int N = (int)a.N, E = a.E, K = a.K, NK = N * K;
    const int R = g.R, epn = g.epn, S = g.S, C = g.C, n = g.n;
    // owner rank of an expert: a shift when epn is a power of two
    const int esh = (epn & (epn - 1)) == 0 ? __builtin_ctz((unsigned)epn) : -1;
    auto owner = [&](int e) { return esh >= 0 ? e >> esh : e / epn; };

    // ---- route -----------------------------------------------------------------------------------
    {
        constexpr int KPL = (kSmKMax + LPT - 1) / LPT;
        constexpr int TPI = kSmBlock / LPT;
        const int lseg = tid % LPT;
        for (int base = 0; base < N; base += TPI) {
            const int tok = base + tid / LPT;
            int my_e[KPL];
            route_generic_token<LPT, NV, BF16, kSmKMax>(a, tok, lseg, my_e);
            if (tok < N) {
#pragma unroll
                for (int m = 0; m < KPL; ++m) {
                    const int j = m * LPT + lseg;
                    if (j < K) s_ids[tok * K + j] = my_e[m];
                }
            }
        }
    }
    for (int e = tid; e < E; e += kSmBlock) {
        s_cnt[e] = 0;
        s_run[e] = 0;
    }
    for (int i = tid; i < S * E; i += kSmBlock) s_ntpe[i] = 0;
    for (int i = tid; i < S * R; i += kSmBlock) s_ntpr[i] = 0;
    for (int i = tid; i < S * R * C; i += kSmBlock) s_chan[i] = 0;
    lds_barrier();

    // ---- layout: histogram, padded scan ----------------------------------------------------------
    for (int i = tid; i < NK; i += kSmBlock) atomicAdd(&s_cnt[s_ids[i]], 1);
    lds_barrier();
    {
        const int c = tid < E ? s_cnt[tid] : 0;
        const int padded = c > 0 ? (c + sa.A - 1) / sa.A * sa.A : 0;
        int total;
        const int excl = lds_block_scan(padded, s_tmp, total);
        if (tid < E) {
            s_cu[tid] = excl;
            if (sa.lo.tokens_per_expert) sa.lo.tokens_per_expert[tid] = c;
            sa.lo.cu_seqlens[tid] = excl;
            if (sa.lo.zero_fill) {
                const bool zf = c > 0 && padded > c;
                sa.lo.zero_fill[2 * tid] = zf ? excl + c : 0;
                sa.lo.zero_fill[2 * tid + 1] = zf ? padded - c : 0;
            }
        }
        if (tid == 0) {
            s_cu[E] = total;
            sa.lo.cu_seqlens[E] = total;
        }
    }
    lds_barrier();

    // ---- layout: stable positions, 512 slots at a time ------------------------------------------
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    for (int c0 = 0; c0 < NK; c0 += kSmBlock) {
        for (int i = tid; i < kSmWaves * E; i += kSmBlock) s_wc[i / E][i % E] = 0;
        lds_barrier();
        const int i = c0 + tid;
        const bool valid = i < NK;
        const int e = valid ? s_ids[i] : 0;
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const uint64_t ones = __ballot(valid && ((e >> b) & 1));
            peers &= ((e >> b) & 1) ? ones : ~ones;
        }
        const int rank = __popcll(peers & lanes_below());
        if (valid && rank == 0) s_wc[wv][e] = __popcll(peers);
        lds_barrier();
        if (tid < E) {
            int run = 0;
            for (int w = 0; w < kSmWaves; ++w) {
                const int t = s_wc[w][tid];
                s_wc[w][tid] = run;
                run += t;
            }
            s_chunk[tid] = run;
        }
        lds_barrier();
        if (valid) {
            const int P = s_cu[e] + s_run[e] + s_wc[wv][e] + rank;
            s_P[i] = P;
            sa.lo.e2p[i] = P;
            if (sa.lo.p2e) sa.lo.p2e[P] = i;
        }
        lds_barrier();
        if (tid < E) s_run[tid] += s_chunk[tid];  // the earlier chunks' slots of each expert
        lds_barrier();
    }
    if (sa.lo.p2e) {
        for (int e = 0; e < E; ++e) {
            const int start = s_cu[e] + s_cnt[e], end = s_cu[e + 1];
            for (int p = start + tid; p < end; p += kSmBlock) sa.lo.p2e[p] = -1;
        }
    }

    // ---- plan: per token ---------------------------------------------------------------------------
    const int q = (n + C - 1) / C;
    for (int t = tid; t < N; t += kSmBlock) {
        const int s = t / n;
        const int ch = (t - s * n) / q;
        uint32_t mask = 0, hc = 0;
        for (int k = 0; k < K; ++k) {
            const int e = s_ids[t * K + k];
            const int r = owner(e);
            atomicAdd(&s_ntpe[s * E + e], 1);
            const int raw = (int)((int64_t)r * g.NvS + (s_P[t * K + k] - s_cu[r * epn]));
            const bool dup = (mask >> r) & 1u;
            if (sa.po.dst) sa.po.dst[t * K + k] = dup ? -raw - 1 : raw;
            mask |= 1u << r;
            hc += 1u << (4 * r);  // R <= 8 ranks, at most K <= 8 slots on one
        }
        s_hc[t] = hc;
        for (int r = 0; r < R; ++r) {
            const bool in = (mask >> r) & 1u;
            if (sa.po.itr) sa.po.itr[(int64_t)t * R + r] = in ? 1 : 0;
            if (in) {
                atomicAdd(&s_ntpr[s * R + r], 1);
                atomicAdd(&s_chan[(s * R + r) * C + ch], 1);
            }
        }
    }
    lds_barrier();

    // ---- plan: matrices and receive layout -----------------------------------------------------------
    for (int i = tid; i < S * E; i += kSmBlock)
        if (sa.po.ntpe) sa.po.ntpe[i] = s_ntpe[i];
    for (int r = tid; r < R; r += kSmBlock) {
        int run = 0;
        for (int s = 0; s < S; ++s) {
            const int v = s_ntpr[s * R + r];
            run += v;
            if (sa.po.ntpr) sa.po.ntpr[s * R + r] = v;
            if (sa.po.rank_prefix) sa.po.rank_prefix[s * R + r] = run;
        }
        if (sa.po.recv_tokens) sa.po.recv_tokens[r] = run;
    }
    if (sa.po.chan) {
        for (int sr = tid; sr < S * R; sr += kSmBlock) {
            int run = 0;
            for (int c = 0; c < C; ++c) {
                run += s_chan[sr * C + c];
                sa.po.chan[sr * C + c] = run;
            }
        }
    }
    if (sa.po.recv_cu) {
        for (int i = tid; i < R * (epn + 1); i += kSmBlock) {
            const int r = i / (epn + 1), j = i - r * (epn + 1);
            sa.po.recv_cu[i] = s_cu[r * epn + j] - s_cu[r * epn];
        }
    }
    if (sa.po.recv_zf) {
        for (int e = tid; e < E; e += kSmBlock) {
            const int c = s_cnt[e], padded = s_cu[e + 1] - s_cu[e], r = e / epn;
            const bool zf = c > 0 && padded > c;
            sa.po.recv_zf[2 * e] = zf ? s_cu[e] + c - s_cu[r * epn] : 0;
            sa.po.recv_zf[2 * e + 1] = zf ? padded - c : 0;
        }
    }

    // ---- plan: dedup lists in token order, all ranks at once ----------------------------------------
    // Per rank r and token t: a group when t has >= 2 slots on r, with hits - 1 duplicates (the
    // slots per rank come from the plan pass as 4-bit fields).  Every rank's (group, duplicates)
    // pair, packed 16:16 (at most 2048 of each in a batch), is scanned per wave with DPP; the wave
    // totals, prefixed over chunks and waves per rank, give the totals and the rank offsets, and
    // a second round of the same scans places every record.  Three barriers in all.
    if (epn == 1) {
        // distinct experts on distinct ranks: no token has two slots on one rank
        for (int i = tid; i < 2 * R; i += kSmBlock)
            if (sa.po.dup_counts) sa.po.dup_counts[i] = 0;
        for (int i = tid; i < 2 * (R + 1); i += kSmBlock)
            if (sa.po.dup_offsets) sa.po.dup_offsets[i] = 0;
        return;
    }
    const int lane = tid & 63;
    const int nch = (N + kSmBlock - 1) / kSmBlock;  // chunks of 512 tokens, at most 4
    // the packed pair of token t on rank r: (1 group, h - 1 duplicates) when it has h >= 2 slots
    auto pair_of = [&](uint32_t hc, int r) {
        const int h = (int)((hc >> (4 * r)) & 15u);
        return h >= 2 ? (1 << 16) | (h - 1) : 0;
    };
    // pass 1: every rank's wave totals of the pairs, per chunk
    for (int c = 0; c < nch; ++c) {
        const int t = c * kSmBlock + tid;
        const uint32_t hc = t < N ? s_hc[t] : 0u;
#pragma unroll
        for (int r = 0; r < kSmMaxR; ++r) {
            if (r >= R) continue;  // uniform: ranks past R cost nothing
            int wt;
            sm_wave_excl_scan(pair_of(hc, r), wt);
            if (lane == 0) s_wsum[c][wv][r] = wt;
        }
    }
    lds_barrier();
    // per rank (one thread each): the wave totals become exclusive prefixes over chunks and
    // waves; the rank's total
    if (tid < R) {
        int run = 0;
        for (int c = 0; c < nch; ++c)
            for (int w = 0; w < kSmWaves; ++w) {
                const int x = s_wsum[c][w][tid];
                s_wsum[c][w][tid] = run;
                run += x;
            }
        s_dtot[tid] = run;
    }
    lds_barrier();
    // rank offsets (exclusive scans over the ranks of the group and duplicate totals), counts
    if (wv == 0) {
        const int packed = lane < R ? s_dtot[lane] : 0;
        const int gt = packed >> 16, dt = packed & 0xFFFF;
        int gall, dall;
        const int go = sm_wave_excl_scan(gt, gall), dof = sm_wave_excl_scan(dt, dall);
        if (lane < R) {
            s_goff[lane] = go;
            s_doff[lane] = dof;
            if (sa.po.dup_counts) {
                sa.po.dup_counts[2 * lane] = gt;
                sa.po.dup_counts[2 * lane + 1] = dt;
            }
            if (sa.po.dup_offsets) {
                sa.po.dup_offsets[2 * lane] = go;
                sa.po.dup_offsets[2 * lane + 1] = dof;
            }
        }
        if (lane == 0 && sa.po.dup_offsets) {
            sa.po.dup_offsets[2 * R] = gall;
            sa.po.dup_offsets[2 * R + 1] = dall;
        }
    }
    lds_barrier();
    // pass 2: the same wave scans again plus the prefixes give each token's group and duplicate
    // indices on each rank; the records
    for (int c = 0; c < nch; ++c) {
        const int t = c * kSmBlock + tid;
        const uint32_t hc = t < N ? s_hc[t] : 0u;
#pragma unroll
        for (int r = 0; r < kSmMaxR; ++r) {
            if (r >= R) continue;
            int wt;
            const int x = pair_of(hc, r);
            const int ex = sm_wave_excl_scan(x, wt) + s_wsum[c][wv][r];
            if (x != 0) {
                const int h = (x & 0xFFFF) + 1;
                const int gi = ex >> 16, di = ex & 0xFFFF;
                const int dbase = s_doff[r] + di;
                int first = -1, j = 0;
                for (int k = 0; k < K; ++k) {
                    const int e = s_ids[t * K + k];
                    if (owner(e) != r) continue;
                    const int loff = s_P[t * K + k] - s_cu[r * epn];
                    if (first < 0) {
                        first = loff;
                    } else {
                        if (sa.po.dup_loffs) sa.po.dup_loffs[dbase + j] = loff;
                        ++j;
                    }
                }
                if (sa.po.dup_groups) {
                    int32_t* grp = sa.po.dup_groups + 3 * (int64_t)(s_goff[r] + gi);
                    grp[0] = first;
                    grp[1] = di;
                    grp[2] = h - 1;
                }
            }
        }
    }
}

}  // namespace

}  // namespace mep

namespace mep {

namespace {

template <int LPT, int NV, bool BF16>
void launch_small(const SmallArgs& sa, const Launch& st) {
    launch_kernel(small_path_kernel<LPT, NV, BF16>, dim3(1), dim3(kSmBlock), 0, st, sa);
}

template <bool BF16>
bool dispatch_small(const SmallArgs& sa, const Launch& st) {
    constexpr int W = BF16 ? 8 : 4;
    const int nchunks = (sa.ra.E + W - 1) / W;
    if (nchunks <= 1) launch_small<1, 1, BF16>(sa, st);
    else if (nchunks <= 2) launch_small<2, 1, BF16>(sa, st);
    else if (nchunks <= 4) launch_small<4, 1, BF16>(sa, st);
    else if (nchunks <= 8) launch_small<8, 1, BF16>(sa, st);
    else if (nchunks <= 16) launch_small<16, 1, BF16>(sa, st);
    else if (nchunks <= 32) launch_small<32, 1, BF16>(sa, st);
    else if (nchunks <= 64) launch_small<64, 1, BF16>(sa, st);
    else return false;
    return true;
}

}  // namespace

}  // namespace mep

namespace mep {

// The whole path in one call: the one-workgroup kernel for small batches, else the routing kernel
// (counting the plan tiles itself where it can), then the plan-tile kernel of the fused path; or
// the routing kernel followed by mep_layout_plan's kernels where the fused path does not cover
// the shape.  `ev` optionally stamps the routing kernel (or the single small kernel) and the
// plan-tile kernel with their start and end times.  With `validate_only` every check runs and
// nothing is enqueued (the workspace pointer is checked, never dereferenced).
int route_layout_plan(const void* logits, int dtype, int64_t N, int E, int K, const float* bias,
                      const mep_route_params* p, int32_t* topk_ids, float* topk_weights, int alignment,
                      int32_t* tokens_per_expert, int32_t* cu_seqlens, int32_t* expanded_to_permuted,
                      int32_t* permuted_to_expanded, int64_t permuted_cap, int32_t* zero_fill, int R, int num_src,
                      int num_channels, int64_t NvS, const mep_plan_outputs* out, void* ws, size_t ws_bytes,
                      void* stream, const StepEvents& ev, bool validate_only) {
    if (N > 0 && !topk_ids) return MEP_ERR_INVALID_ARG;
    SmallArgs sa;
    int rc = route_prepare(logits, dtype, N, E, K, bias, p, topk_ids, topk_weights, sa.ra);
    if (rc != MEP_OK) return rc;
    PlanCall pc;
    rc = plan_prepare(topk_ids, cu_seqlens, expanded_to_permuted, N, E, K, alignment, R, num_src, num_channels,
                      NvS, out, ws, ws_bytes, pc);
    if (rc != MEP_OK) return rc;
    LayoutCall lc;
    rc = layout_prepare_outputs(topk_ids, N, E, K, alignment, tokens_per_expert, cu_seqlens, expanded_to_permuted,
                                permuted_to_expanded, permuted_cap, zero_fill, lc);
    if (rc != MEP_OK || validate_only) return rc;
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int64_t NK = N * (int64_t)K;
    const bool small = N > 0 && NK <= kSmMaxSlots && E <= kSmMaxE && K <= kSmKMax && R <= kSmMaxR &&
                       (int64_t)num_src * E <= kSmMaxShardE &&
                       (int64_t)num_src * R * num_channels <= kSmMaxChan;
    if (small) {
        sa.A = alignment;
        sa.lo = lc.out;
        sa.g = pc.g;
        sa.po = pc.o;
        const Launch sl{st, ev.route_start, ev.route_stop};
        const bool ok = dtype == MEP_BF16 ? dispatch_small<true>(sa, sl) : dispatch_small<false>(sa, sl);
        if (ok) return launch_status();
    }
    const Launch rl{st, ev.route_start, ev.route_stop};
    if (path_supported(N, E, K, R)) {
        const PathCall c = path_call(lc, pc, ws);
        if (!launch_route_sig_counting(sa.ra, dtype, rl, c) && !launch_route_generic_counting(sa.ra, dtype, rl, c)) {
            rc = route_launch(sa.ra, dtype, rl);
            if (rc != MEP_OK) return rc;
            path_launch_count(c, st);
        }
        path_launch_plan(c, st, ev.plan_start, ev.plan_stop);
        return launch_status();
    }
    // shapes outside the fused path: the routing kernel, then the layout and plan kernels
    if (N > 0) {
        rc = route_launch(sa.ra, dtype, rl);
        if (rc != MEP_OK) return rc;
    }
    plan_launch_count(pc, st);
    plan_launch_scatter_write(lc, pc, st);
    return launch_status();
}

}  // namespace mep

extern "C" int mep_route_layout_plan(const void* logits, int dtype, int64_t N, int E, int K, const float* bias,
                                     const mep_route_params* p, int32_t* topk_ids, float* topk_weights,
                                     int alignment, int32_t* tokens_per_expert, int32_t* cu_seqlens,
                                     int32_t* expanded_to_permuted, int32_t* permuted_to_expanded,
                                     int64_t permuted_cap, int32_t* zero_fill, int R, int num_src,
                                     int num_channels, int64_t NvS, const mep_plan_outputs* out, void* ws,
                                     size_t ws_bytes, void* stream) {
    mep::launch_begin();
    return mep::route_layout_plan(logits, dtype, N, E, K, bias, p, topk_ids, topk_weights, alignment,
                                  tokens_per_expert, cu_seqlens, expanded_to_permuted, permuted_to_expanded,
                                  permuted_cap, zero_fill, R, num_src, num_channels, NvS, out, ws, ws_bytes, stream,
                                  mep::StepEvents{}, false);
}

extern "C" int mep_route_layout_plan_timed(const void* logits, int dtype, int64_t N, int E, int K,
                                           const float* bias, const mep_route_params* p, int32_t* topk_ids,
                                           float* topk_weights, int alignment, int32_t* tokens_per_expert,
                                           int32_t* cu_seqlens, int32_t* expanded_to_permuted,
                                           int32_t* permuted_to_expanded, int64_t permuted_cap, int32_t* zero_fill,
                                           int R, int num_src, int num_channels, int64_t NvS,
                                           const mep_plan_outputs* out, void* ws, size_t ws_bytes, void* stream,
                                           void* route_start, void* route_stop, void* plan_start,
                                           void* plan_stop) {
    mep::launch_begin();
    const mep::StepEvents ev{reinterpret_cast<hipEvent_t>(route_start), reinterpret_cast<hipEvent_t>(route_stop),
                             reinterpret_cast<hipEvent_t>(plan_start), reinterpret_cast<hipEvent_t>(plan_stop)};
    return mep::route_layout_plan(logits, dtype, N, E, K, bias, p, topk_ids, topk_weights, alignment,
                                  tokens_per_expert, cu_seqlens, expanded_to_permuted, permuted_to_expanded,
                                  permuted_cap, zero_fill, R, num_src, num_channels, NvS, out, ws, ws_bytes, stream,
                                  ev, false);
}
