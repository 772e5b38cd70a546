// One tile of the layout's scatter kernel, shared by mep_build_layout (layout.hip) and the
// combined layout + plan kernel of mep_layout_plan (plan.hip).  See layout.hip for the method.
#pragma once

#include "calls.h"
#include "device_common.h"
#include "host_common.h"

namespace mep {

constexpr int kLayTile = 4096;                       // slots per scatter tile
constexpr int kScatBlock = 1024;
constexpr int kScatWaves = kScatBlock / kWave;
constexpr int kScatPerWave = kLayTile / kScatWaves;  // 256
constexpr int kMaxExperts = 1024;

// LDS of one scatter tile.
struct ScatterLds {
    int* cu;                      // [kMaxExperts + 1] padded offsets (cu_seqlens)
    int* tot;                     // [kMaxExperts] slots per expert
    int* base;                    // [kMaxExperts] cu[e] + slots of e in earlier tiles
    int* loc;                     // [kMaxExperts] start of e in this tile's expert-ordered staging
    int (*cnt)[kMaxExperts];      // [kScatWaves][kMaxExperts] per-(wave, expert) counters
    int* tmp;                     // [kScatWaves]
    int* slot;                    // [kLayTile] staging of the inverse in expert order
    int* pos;                     // [kLayTile]
};

// One scatter tile (one workgroup of kScatBlock threads): the padded scan of the expert totals,
// stable in-tile ranks, the tile's expanded_to_permuted and permuted_to_expanded entries, a
// slice of the padding rows, and (workgroup 0) the per-expert outputs.  With `keep_ids` and
// `keep_pos` (kLayTile + kLayTile / 64 ints each in LDS), it leaves the tile's ids and permuted
// positions there by slot, at slot_pad(slot) (-1 / 0 where there is no valid slot), for a later
// phase of the same workgroup; their storage may be L.slot and L.pos, which are free by then.
template <int NB>
__device__ __forceinline__ void scatter_tile(const int32_t* __restrict__ ids, int E, int A,
                                             const ScatterSrc& src, WsHeader* hdr,
                                             const LayoutOut& out, const ScatterLds& L,
                                             int* keep_ids, int* keep_pos) {
    constexpr int EPT = kMaxExperts / kScatBlock;  // experts per thread in the per-expert passes
    int* s_cu = L.cu;
    int* s_tot = L.tot;
    int* s_base = L.base;
    int* s_loc = L.loc;
    int (*s_cnt)[kMaxExperts] = L.cnt;
    int* s_tmp = L.tmp;
    int* s_slot = L.slot;
    int* s_pos = L.pos;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int tile = blockIdx.x;
    // the tile's slots [s_beg, s_end), its count tile and the source of the prefix data
    int ntiles, s_beg, s_end, ct, first, nct, th_stride, th_off;
    const uint64_t *status, *th;
    if (!src.plan) {
        const LayGeom& g = src.lg;
        ntiles = g.nsub;
        s_beg = tile * kLayTile;
        s_end = min(s_beg + kLayTile, g.NK);
        ct = tile / g.sub;
        first = ct * g.sub;
        nct = g.nct;
        status = src.lw.status;
        th = src.lw.tilehist;
        th_stride = E;
        th_off = 0;
    } else {
        const PlanGeom& g = src.pg;
        ntiles = g.ntiles;
        const int sh = tile / g.tps;
        const int64_t t0 = (int64_t)sh * g.n + (int64_t)(tile - sh * g.tps) * g.TT;
        const int64_t t1 = min(t0 + g.TT, (int64_t)(sh + 1) * g.n);
        s_beg = (int)(t0 * g.K);
        s_end = (int)(t1 * g.K);
        ct = tile < ntiles ? ct_of(g, tile) : 0;
        first = tile < ntiles ? ct_first_wt(g, ct) : 0;
        nct = g.nct;
        status = src.pw.statusE;
        th = src.pw.tilehist;
        th_stride = g.ncols;
        th_off = 3 * g.R;
    }
    if (tile >= ntiles) s_end = s_beg;  // the single workgroup of an empty call
    const MEP_GLOBAL int32_t* gids = gptr(ids);
    MEP_GLOBAL int32_t* g_e2p = gptr(out.e2p);
    MEP_GLOBAL int32_t* g_p2e = gptr(out.p2e);
    const int wbase = s_beg + w * kScatPerWave;
    int idv[kScatPerWave / kWave];  // this lane's ids, loaded first so the loads overlap the scan
#pragma unroll
    for (int it = 0; it < kScatPerWave / kWave; ++it) {
        const int i = wbase + it * kWave + lane;
        idv[it] = i < s_end ? gids[i] : 0;
    }

    // ---- per-expert totals (the last count tile's inclusive prefix) and the slots of each expert
    // before this tile (the inclusive prefix of the count tile before this one plus the
    // histograms of the earlier tiles of this count tile), all loads issued together
    int tot[EPT], pre[EPT];
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
        const int e = tid * EPT + q;
        tot[q] = 0;
        pre[q] = 0;
        if (e >= E || tile >= ntiles) continue;
        const MEP_GLOBAL uint64_t* gs = gptr(status) + e;
        const MEP_GLOBAL uint64_t* gt = gptr(th) + (size_t)first * th_stride + th_off + e;
        const int nwt = tile - first;  // earlier tiles of this count tile
        tot[q] = (int)(uint32_t)gs[(size_t)(nct - 1) * E];
        pre[q] = (int)(uint32_t)gs[(size_t)(ct > 0 ? ct - 1 : 0) * E];
        if (ct == 0) pre[q] = 0;
        int v[8];
        for (int j0 = 0; j0 < nwt; j0 += 8) {  // rows past the end re-read the last one, counted 0
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = (int)(uint32_t)gt[(size_t)min(j0 + j, nwt - 1) * th_stride];
#pragma unroll
            for (int j = 0; j < 8; ++j) pre[q] += j0 + j < nwt ? v[j] : 0;
        }
    }
    int pad[EPT];
    int mysum = 0;
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
        const int e = tid * EPT + q;
        if (e < E) s_tot[e] = tot[q];
        pad[q] = tot[q] > 0 ? ((tot[q] + A - 1) / A) * A : 0;
        mysum += pad[q];
    }
    int total;
    int run = block_exclusive_scan<kScatBlock>(mysum, s_tmp, total);
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
        const int e = tid * EPT + q;
        if (e < E) {
            s_cu[e] = run;
            s_base[e] = run + pre[q];
        }
        run += pad[q];
    }
    if (tid == 0) s_cu[E] = total;
    for (int e = tid; e < E; e += kScatBlock)
#pragma unroll
        for (int ww = 0; ww < kScatWaves; ++ww) s_cnt[ww][e] = 0;
    __syncthreads();

    // ---- stable in-tile ranks: wave match + per-(wave, expert) counters -----------------
    int key[kScatPerWave / kWave];
    int rank[kScatPerWave / kWave];
    if (tile < ntiles) {
#pragma unroll
        for (int it = 0; it < kScatPerWave / kWave; ++it) {
            const int i = wbase + it * kWave + lane;
            int k = idv[it];
            const bool valid = i < s_end && (unsigned)k < (unsigned)E;
            if (!valid) k = 0;
            const uint64_t active = __ballot(valid);
            const uint64_t peers = match_peers<NB>((uint32_t)k, active);
            key[it] = valid ? k : -1;
            rank[it] = 0;
            if (valid) {
                const uint64_t below = peers & lanes_below();
                const int b = s_cnt[w][k];
                rank[it] = b + popc64(below);
                if (below == 0) s_cnt[w][k] = b + popc64(peers);
            }
        }
    }
    __syncthreads();
    // per expert: exclusive prefix over waves, and the tile's expert-ordered staging offsets
    int my_tile_cnt[EPT];
    int cnt_sum = 0;
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
        const int e = tid * EPT + q;
        int r = 0;
        if (e < E) {
#pragma unroll
            for (int ww = 0; ww < kScatWaves; ++ww) {
                const int c = s_cnt[ww][e];
                s_cnt[ww][e] = r;
                r += c;
            }
        }
        my_tile_cnt[q] = r;
        cnt_sum += r;
    }
    int tile_slots;
    int loc = block_exclusive_scan<kScatBlock>(cnt_sum, s_tmp, tile_slots);
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
        const int e = tid * EPT + q;
        if (e < E) s_loc[e] = loc;
        loc += my_tile_cnt[q];
    }
    __syncthreads();
    int Pv[kScatPerWave / kWave];
    if (tile < ntiles) {
#pragma unroll
        for (int it = 0; it < kScatPerWave / kWave; ++it) {
            const int i = wbase + it * kWave + lane;
            const int k = key[it];
            Pv[it] = 0;
            if (k >= 0) {
                const int within = s_cnt[w][k] + rank[it];
                const int P = s_base[k] + within;
                Pv[it] = P;
                g_e2p[i] = P;
                const int j = s_loc[k] + within;
                s_slot[j] = i;
                s_pos[j] = P;
            }
        }
    }
    __syncthreads();
    if (out.p2e && tile < ntiles) {
        for (int j = tid; j < tile_slots; j += kScatBlock) {
            const int P = s_pos[j];
            if (P < out.p2e_cap) g_p2e[P] = s_slot[j];
        }
    }
    if (keep_ids) {  // ids and positions by slot, for a later phase of this workgroup
        __syncthreads();
        if (tile < ntiles) {
#pragma unroll
            for (int it = 0; it < kScatPerWave / kWave; ++it) {
                const int li = w * kScatPerWave + it * kWave + lane;  // slot - s_beg
                keep_ids[slot_pad(li)] = key[it];
                keep_pos[slot_pad(li)] = Pv[it];
            }
        }
    }

    // ---- padding rows of the inverse ------------------------------------------------------
    if (out.p2e) {
        for (int e = blockIdx.x; e < E; e += gridDim.x) {
            const int start = s_cu[e] + s_tot[e];
            const int end = min(s_cu[e + 1], out.p2e_cap);
            for (int p = start + tid; p < end; p += kScatBlock) g_p2e[p] = -1;
        }
    }

    // ---- per-expert outputs and workspace reset ------------------------------------------
    if (blockIdx.x == 0) {
        MEP_GLOBAL int32_t* g_cu = gptr(out.cu_seqlens);
        for (int e = tid; e <= E; e += kScatBlock) g_cu[e] = s_cu[e];
        for (int e = tid; e < E; e += kScatBlock) {
            const int cnt = s_tot[e];
            if (out.tokens_per_expert) gptr(out.tokens_per_expert)[e] = cnt;
            if (out.zero_fill) {
                const int padded = s_cu[e + 1] - s_cu[e];
                const bool z = cnt > 0 && padded > cnt;
                gptr(out.zero_fill)[2 * e] = z ? s_cu[e] + cnt : 0;
                gptr(out.zero_fill)[2 * e + 1] = z ? padded - cnt : 0;
            }
        }
        if (tid == 0 && !src.plan) {  // (the plan's writing pass resets its own workspace)
            MEP_GLOBAL WsHeader* h = gptr(hdr);
            h->epoch = h->epoch + 1u;
            h->ticket = 0u;
        }
    }
}

}  // namespace mep
