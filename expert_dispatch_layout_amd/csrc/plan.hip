// mep_plan: expert-parallel dispatch plan over R virtual ranks, computed on one GPU's batch.
//
// Tokens are cut into tiles that never cross a source shard (TT tokens, TT*K <= 4096 slots;
// 2048 when that still gives at most one tile per compute unit).
// Per token, with owner(e) = e / epn:
//   c0[r]  1 if the token sends anything to r       (is_token_in_rank; DeepEP intranode.cu
//                                                     notify_dispatch counts and prefixes these)
//   c1[r]  1 if the token sends >= 2 slots to r     (one dedup group)
//   c2[r]  slots to r beyond the first              (duplicates: MoonEP planning.py duplicate
//                                                     canonicalisation encodes them as -dst-1)
//   cE[e]  1 if the token is routed to e            (per-shard expert counts)
//
//   count kernel  one write tile per workgroup: LDS histograms of the 3R+E columns, stored to
//                 the workspace; the last write tile of a count tile (a few consecutive write
//                 tiles of one shard) to arrive sums them.  With at most kDirectCountTiles count
//                 tiles (about 32 are aimed at) it stores that count tile's totals, and the last
//                 count tile to do so scans every column into inclusive prefixes (no workgroup
//                 ever waits); with more, the sums go through a decoupled look-back across count
//                 tiles.  Either way the prefix of a column at any write-tile boundary is a
//                 count-tile inclusive prefix plus a few write-tile histograms; the expert
//                 columns also give the layout's totals and prefixes in mep_layout_plan.  Also
//                 writes is_token_in_rank.
//   write kernel  dst with the duplicate encoding; dedup groups and duplicate offsets in a stable
//                 (rank, token, k) order -- each slot is ranked among same-rank slots of its
//                 wave by ballot-matching and per-(wave, rank) LDS counters, then offset by the
//                 tile prefix and the rank's segment start; channel prefix matrix from wave
//                 ballots of c0 at channel boundaries; per-shard matrices from tile prefixes at
//                 shard boundaries; small per-rank outputs from the totals.
#include <limits.h>

#include "device_common.h"
#include "host_common.h"
#include "calls.h"
#include "layout_scatter.h"
#include "path.h"

namespace mep {

constexpr int kPlanBlock = 512;
constexpr int kPlanWaves = kPlanBlock / kWave;
constexpr int kPlanSlots = 4096;  // slots per tile, at most (LDS arrays are sized for it)
// Compute units of an MI355X: tiles are halved (to 2048 slots) while that still leaves at most
// one tile per unit -- a fused scatter + write workgroup needs most of a unit's LDS, so tiles
// beyond the unit count only add rounds, and below it half the units would sit idle.
constexpr int kTileUnits = 256;
constexpr int kMaxRanks = 128;
constexpr int kMaxE = 1024;
constexpr int kMaxCols = 3 * kMaxRanks + kMaxE;

constexpr int kMaxSources = 1024;   // virtual source shards (keeps count tiles <= kMaxCountTiles)
// Only the last arriving workgroup of a count tile ever waits (on earlier count tiles).  With at
// most this many count tiles, waiting workgroups can never fill the GPU, so every awaited one
// gets to run and write tiles can follow the workgroup index; beyond it they take a ticket.
constexpr int kUnticketedCountTiles = 128;
constexpr int kCountTilesP = 32;    // count tiles aimed at (parallelism vs look-back length)

static int plan_tile_tokens(int K) {
    int kp = 1;
    while (kp < K) kp <<= 1;
    int tt = kPlanSlots / kp;
    return tt > kPlanBlock ? kPlanBlock : tt;
}



// Per-token view: owner ranks, hit counts and first-occurrence flags of its K slots.
template <int KMAX>
struct TokenSlots {
    int id[KMAX];
    int r[KMAX];
    int h[KMAX];
    bool first[KMAX];
    bool ok[KMAX];
};

template <int KMAX>
__device__ __forceinline__ void token_slots(TokenSlots<KMAX>& ts, const int (&idk)[KMAX], int K, int E,
                                            int R, const int* s_owner) {
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        if (k < K) {
            const int id = idk[k];
            ts.ok[k] = (unsigned)id < (unsigned)E;
            ts.id[k] = ts.ok[k] ? id : 0;
            ts.r[k] = ts.ok[k] ? s_owner[ts.id[k]] : -1;
        } else {
            ts.ok[k] = false;
            ts.id[k] = 0;
            ts.r[k] = -1;
        }
    }
    if (KMAX <= 8 && R <= 16) {
        // slots per rank as 4-bit counters packed in one word; first slot per rank from a mask
        uint64_t packed = 0;
        uint32_t seen = 0;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const int r = ts.ok[k] ? ts.r[k] : 0;
            ts.first[k] = ts.ok[k] && !((seen >> r) & 1u);
            if (ts.ok[k]) {
                packed += 1ull << (4 * r);
                seen |= 1u << r;
            }
        }
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            ts.h[k] = ts.ok[k] ? (int)((packed >> (4 * ts.r[k])) & 15u) : 0;
    } else {
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            int h = 0;
            bool first = true;
#pragma unroll
            for (int k2 = 0; k2 < KMAX; ++k2) {
                const bool same = ts.ok[k] && ts.ok[k2] && ts.r[k2] == ts.r[k];
                h += same;
                if (k2 < k && same) first = false;
            }
            ts.h[k] = h;
            ts.first[k] = first;
        }
    }
}

// The K entries of token t's row (ids or permuted positions): two 16-byte loads when `vec8`
// (K == 8 and 16-byte aligned rows), else K 4-byte loads; `fill` where there is no token.
template <int KMAX>
__device__ __forceinline__ void load_token_row(int (&v)[KMAX], const int32_t* p, int64_t t, int K,
                                               bool live, bool vec8, int fill) {
    const MEP_GLOBAL int32_t* gp = gptr(p);
    if constexpr (KMAX == 8) {
        if (vec8) {
            if (live) {
                const MEP_GLOBAL u32x4* q = reinterpret_cast<const MEP_GLOBAL u32x4*>(gp + t * 8);
                const u32x4 a = q[0], b = q[1];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    v[k] = (int)a[k];
                    v[4 + k] = (int)b[k];
                }
            } else {
#pragma unroll
                for (int k = 0; k < 8; ++k) v[k] = fill;
            }
            return;
        }
    }
#pragma unroll
    for (int k = 0; k < KMAX; ++k) v[k] = (live && k < K) ? gp[t * K + k] : fill;
}

// Rank sets of a token as bit masks: RW 32-bit words (1 word when R <= 32, else 4).
template <int RW>
struct RankMask {
    uint32_t w[RW];
    __device__ __forceinline__ void clear() {
#pragma unroll
        for (int q = 0; q < RW; ++q) w[q] = 0u;
    }
    __device__ __forceinline__ bool test(int r) const {
        if constexpr (RW == 1) return (w[0] >> r) & 1u;
        uint32_t v = 0;
#pragma unroll
        for (int q = 0; q < RW; ++q) v |= ((r >> 5) == q) ? w[q] : 0u;
        return (v >> (r & 31)) & 1u;
    }
    __device__ __forceinline__ void set(int r) {
        if constexpr (RW == 1) {
            w[0] |= 1u << r;
        } else {
#pragma unroll
            for (int q = 0; q < RW; ++q) w[q] |= ((r >> 5) == q) ? (1u << (r & 31)) : 0u;
        }
    }
};


constexpr int kMaxCountTiles = 2048;

// One write tile per workgroup.  Each writes its histograms; the last of the write tiles of a
// count tile to arrive sums them and takes the rank columns and the expert columns through the
// look-back (the expert prefixes also serve the layout in mep_layout_plan).
template <int KMAX, int RW>
__global__ __launch_bounds__(kPlanBlock) void plan_count_kernel(const int32_t* __restrict__ ids,
                                                                PlanGeom g, PlanWs w, WsHeader* hdr,
                                                                uint8_t* itr) {
    __shared__ int s_cnt[kMaxCols];
    __shared__ int s_owner[kMaxE];
    __shared__ int s_tile;
    __shared__ uint32_t s_arrived;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int nc = g.ncols;
    const int R = g.R;
    const int E = g.E;
    const int K = g.K;
    const int n3 = 3 * R;
    for (int c = tid; c < nc; c += kPlanBlock) s_cnt[c] = 0;
    for (int e = tid; e < E; e += kPlanBlock) s_owner[e] = e / g.epn;
    if (tid == 0) s_tile = g.ticketed ? take_ticket(hdr, (int)gridDim.x) : (int)blockIdx.x;
    __syncthreads();
    const int wt = s_tile;
    const uint32_t epoch = __hip_atomic_load(&gptr(hdr)->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    const int sh = wt / g.tps;
    const int64_t t = (int64_t)sh * g.n + (int64_t)(wt - sh * g.tps) * g.TT + tid;
    const bool live = tid < g.TT && t < (int64_t)(sh + 1) * g.n;
    int idk[KMAX];
    load_token_row<KMAX>(idk, ids, t, K, live, K == 8 && (((uintptr_t)ids) & 15u) == 0, -1);
    {
        RankMask<RW> seen, multi;  // ranks reached; ranks reached by >= 2 slots
        seen.clear();
        multi.clear();
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const int id = idk[k];
            if (k < K && (unsigned)id < (unsigned)E) {  // false for a lane without a token
                atomicAdd(&s_cnt[n3 + id], 1);
                const int r = s_owner[id];
                if (seen.test(r)) multi.set(r);
                seen.set(r);
            }
        }
        if (live && itr) {
            MEP_GLOBAL uint8_t* row = gptr(itr) + t * R;
            if ((R & 3) == 0) {
                for (int bb = 0; bb < R; bb += 4) {
                    const uint32_t word = (seen.test(bb) ? 1u : 0u) | (seen.test(bb + 1) ? 1u << 8 : 0u) |
                                          (seen.test(bb + 2) ? 1u << 16 : 0u) | (seen.test(bb + 3) ? 1u << 24 : 0u);
                    *reinterpret_cast<MEP_GLOBAL uint32_t*>(row + bb) = word;
                }
            } else {
                for (int bb = 0; bb < R; ++bb) row[bb] = seen.test(bb) ? 1 : 0;
            }
        }
        // tokens per rank (c0) and tokens with >= 2 slots per rank (c1): wave ballots; lane r
        // collects rank r's counts (one pass per 64 ranks), then one LDS add per lane
        for (int r0 = 0; r0 < R; r0 += 64) {
            int n0 = 0, n1 = 0;
            const int rmax = min(64, R - r0);
            for (int j = 0; j < rmax; ++j) {
                const int c0 = popc64(__ballot(seen.test(r0 + j)));
                const int c1 = popc64(__ballot(multi.test(r0 + j)));
                n0 = lane == j ? c0 : n0;
                n1 = lane == j ? c1 : n1;
            }
            if (lane < rmax) {
                if (n0) atomicAdd(&s_cnt[r0 + lane], n0);
                if (n1) atomicAdd(&s_cnt[R + r0 + lane], n1);
            }
        }
    }
    __syncthreads();
    // duplicates per rank (c2) = slots on the rank (its experts' counts) - tokens on the rank
    for (int e = tid; e < E; e += kPlanBlock) {
        const int c = s_cnt[n3 + e];
        if (c) atomicAdd(&s_cnt[2 * R + s_owner[e]], c);
    }
    __syncthreads();
    for (int r = tid; r < R; r += kPlanBlock) s_cnt[2 * R + r] -= s_cnt[r];
    __syncthreads();
    const uint32_t want = status_tag(epoch);
    for (int c = tid; c < nc; c += kPlanBlock)
        status_store(w.tilehist + (size_t)wt * nc + c, status_make(epoch, false, (uint32_t)s_cnt[c]));
    // ---- arrival at the count tile; the last arriver continues ------------------------------
    const int ct = ct_of(g, wt);
    const int wt0 = ct_first_wt(g, ct);
    const int nsub_here = min(g.sub, (ct / g.ctps + 1) * g.tps - wt0);
    __syncthreads();
    if (tid == 0)
        s_arrived = __hip_atomic_fetch_add(gptr(w.arrive) + ct, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_arrived != (uint32_t)(nsub_here - 1)) return;
    if (tid == 0) __hip_atomic_store(gptr(w.arrive) + ct, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int c = tid; c < nc; c += kPlanBlock) {
        uint32_t agg = 0;
        for (int b0 = 0; b0 < nsub_here; b0 += 8) {
            uint64_t v[8];
#pragma unroll
            for (int b = 0; b < 8; ++b)
                v[b] = b0 + b < nsub_here ? status_load(w.tilehist + (size_t)(wt0 + b0 + b) * nc + c) : 0;
#pragma unroll
            for (int b = 0; b < 8; ++b)
                if (b0 + b < nsub_here) agg += tagged_value(w.tilehist + (size_t)(wt0 + b0 + b) * nc + c, v[b], want, &hdr->err);
        }
        if (g.direct) {
            uint64_t* word = c < n3 ? w.status3 + (size_t)ct * n3 + c : w.statusE + (size_t)ct * E + (c - n3);
            status_store(word, status_make(epoch, false, agg));
        } else if (c < n3) {
            lookback_column(w.status3, ct, n3, c, epoch, agg, &hdr->err);
        } else {
            lookback_column(w.statusE, ct, E, c - n3, epoch, agg, &hdr->err);
        }
    }
    if (g.direct && last_count_tile(hdr, g.nct, &s_arrived)) {
        for (int c = tid; c < nc; c += kPlanBlock) {
            if (c < n3) scan_count_column(w.status3, g.nct, n3, c, epoch, &hdr->err);
            else scan_count_column(w.statusE, g.nct, E, c - n3, epoch, &hdr->err);
        }
    }
}


enum : uint32_t { kNone = 0, kHead = 1, kDup = 2 };

// LDS of one write tile.
struct WriteLds {
    int* owner;                   // [kMaxE] owner rank of each expert
    int* cu_r;                    // [kMaxRanks + 1] cu_seqlens at each rank's first expert
    int* excl;                    // [3 * kMaxRanks] rank-column prefixes before this write tile
    int (*ctp)[3 * kMaxRanks];    // [3] count-tile prefixes of the rank columns (kCt*)
    int (*doff)[kMaxRanks + 1];   // [2] segment starts of the groups / duplicates per rank
    uint32_t* code;               // [kPlanSlots + kPlanSlots / 64] slot codes, at slot_pad(slot)
    int* loff;                    // [kPlanSlots + kPlanSlots / 64] rank-local offsets, likewise
    int (*hc)[kMaxRanks];         // [waves] per-(wave, rank) head counters
    int (*dc)[kMaxRanks];         // [waves] per-(wave, rank) duplicate counters
    uint64_t (*mask)[kMaxRanks];  // [waves] per-(wave, rank) token ballots
    int* tmp;                     // [waves]
};

// Where a write tile takes its tokens' ids and permuted positions and the cu_seqlens entries:
// global memory (mep_plan), or the LDS that the scatter phase of the same workgroup left them in
// (the fused kernel of mep_layout_plan: ids and positions by slot of the tile, cu_seqlens whole).
struct WriteSrcGlobal {
    const int32_t* ids;
    const int32_t* pos;
    const int32_t* cu;
    template <int KMAX>
    __device__ __forceinline__ void token(int (&idk)[KMAX], int (&pk)[KMAX], int64_t t, int /*li*/, int K,
                                          bool live) const {
        const bool vec8 = K == 8 && ((((uintptr_t)ids) | ((uintptr_t)pos)) & 15u) == 0;
        load_token_row<KMAX>(idk, ids, t, K, live, vec8, -1);
        load_token_row<KMAX>(pk, pos, t, K, live, vec8, 0);
    }
    __device__ __forceinline__ int cuv(int i) const { return gptr(cu)[i]; }
};
struct WriteSrcLds {
    const int* ids;  // by slot of the tile, at slot_pad(slot)
    const int* pos;
    const int* cu;   // [E + 1]
    template <int KMAX>
    __device__ __forceinline__ void token(int (&idk)[KMAX], int (&pk)[KMAX], int64_t /*t*/, int li, int K,
                                          bool live) const {
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            idk[k] = (live && k < K) ? ids[slot_pad(li * K + k)] : -1;
            pk[k] = (live && k < K) ? pos[slot_pad(li * K + k)] : 0;
        }
    }
    __device__ __forceinline__ int cuv(int i) const { return cu[i]; }
};

// One write tile by a workgroup of NT threads (NT / 64 waves, one thread per token of the tile).
template <int KMAX, int NB, int NT, class Src>
__device__ __forceinline__ void plan_write_tile(const Src& src, const PlanGeom& g, const PlanWs& pw,
                                                WsHeader* hdr, const PlanOutDev& o, const WriteLds& L) {
    constexpr int kWTWaves = NT / kWave;
    static_assert(NT >= kPlanBlock, "a thread per token");
    int* s_owner = L.owner;
    int* s_cu_r = L.cu_r;
    int* s_excl = L.excl;
    int (*s_ctp)[3 * kMaxRanks] = L.ctp;
    int (*s_doff)[kMaxRanks + 1] = L.doff;
    uint32_t* s_code = L.code;
    int* s_loff = L.loff;
    int (*s_hc)[kMaxRanks] = L.hc;
    int (*s_dc)[kMaxRanks] = L.dc;
    uint64_t (*s_mask)[kMaxRanks] = L.mask;
    int* s_tmp = L.tmp;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int R = g.R;
    const int tile = g.ntiles > 0 ? (int)blockIdx.x : -1;
    const int sh = tile >= 0 ? tile / g.tps : 0;
    const int ct = tile >= 0 ? tile - sh * g.tps : 0;
    const int64_t t0 = (int64_t)sh * g.n + (int64_t)ct * g.TT;
    const int64_t t1 = tile >= 0 ? min(t0 + g.TT, (int64_t)(sh + 1) * g.n) : t0;
    const int ctile = tile >= 0 ? ct_of(g, tile) : 0;     // count tile of this write tile
    const int ct_shard0 = sh * g.ctps;                      // first count tile of the shard
    const int n3 = 3 * g.R;  // rank columns: look-back words and write-tile histograms
    const uint64_t* status = pw.status3;

    // ---- prologue: every load the tile needs before its per-token pass, issued together ------
    // Prefixes of the 3R rank columns: s_excl = before this write tile (the count tiles before
    // its count tile plus the earlier write tiles of its count tile), and three count-tile
    // prefixes (before the shard's first count tile, through this count tile, all).
    enum { kCtShard0 = 0, kCtIncl = 1, kCtTotal = 2 };
    for (int e = tid; e < g.E; e += NT) s_owner[e] = e / g.epn;
    for (int r = tid; r < R; r += NT)
#pragma unroll
        for (int ww = 0; ww < kWTWaves; ++ww) {
            s_hc[ww][r] = 0;
            s_dc[ww][r] = 0;
            s_mask[ww][r] = 0ull;
        }

    // this thread's token: ids and permuted positions
    const int64_t my_t = t0 + tid;
    const bool my_live = tile >= 0 && tid < g.TT && my_t < t1;
    int idk[KMAX], pk[KMAX];
    src.template token<KMAX>(idk, pk, my_t, tid, g.K, my_live);
    const int cu_r = tid <= R ? src.cuv(tid * g.epn) : 0;
    // the per-expert tail's first expert of this wave: its inclusive prefixes at the shards' last
    // count tiles (lane s2 < S) and at the last count tile, and its cu_seqlens entries
    const int e_first = (int)blockIdx.x + w * (int)gridDim.x;
    const bool tail_pref = g.ntiles > 0 && e_first < g.E && g.S <= 64;
    int tail_hi = 0, tail_lo = 0, tail_tot = 0, tail_cu0 = 0, tail_cu1 = 0, tail_cuo = 0;
    if (tail_pref) {
        if (lane < g.S) {
            tail_hi = (int)status_value(pw.statusE, (lane + 1) * g.ctps - 1, g.E, e_first);
            tail_lo = lane > 0 ? (int)status_value(pw.statusE, lane * g.ctps - 1, g.E, e_first) : 0;
        }
        if (lane == 0) {
            tail_tot = (int)status_value(pw.statusE, g.nct - 1, g.E, e_first);
            tail_cu0 = src.cuv(e_first);
            tail_cu1 = src.cuv(e_first + 1);
            tail_cuo = src.cuv((e_first / g.epn) * g.epn);
        }
    }
    // the earlier write tiles of this count tile
    const int first_wt = tile >= 0 ? ct_first_wt(g, ctile) : 0;
    const int nwt = tile >= 0 ? tile - first_wt : 0;
    for (int c = tid; c < n3; c += NT) {
        // inclusive count-tile prefixes at the four count tiles, plus the earlier write tiles
        int sx = 0, s0 = 0, si = 0, stt = 0;
        if (tile >= 0) {
            const MEP_GLOBAL uint64_t* gs = gptr(status) + c;
            const MEP_GLOBAL uint64_t* gt = gptr(pw.tilehist) + (size_t)first_wt * g.ncols + c;
            sx = (int)(uint32_t)gs[(size_t)(ctile > 0 ? ctile - 1 : 0) * n3];
            s0 = (int)(uint32_t)gs[(size_t)(ct_shard0 > 0 ? ct_shard0 - 1 : 0) * n3];
            si = (int)(uint32_t)gs[(size_t)ctile * n3];
            stt = (int)(uint32_t)gs[(size_t)(g.nct - 1) * n3];
            if (ctile == 0) sx = 0;
            if (ct_shard0 == 0) s0 = 0;
            int v[8];
            for (int j0 = 0; j0 < nwt; j0 += 8) {  // rows past the end re-read the last one
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] = (int)(uint32_t)gt[(size_t)min(j0 + j, nwt - 1) * g.ncols];
#pragma unroll
                for (int j = 0; j < 8; ++j) sx += j0 + j < nwt ? v[j] : 0;
            }
        }
        s_excl[c] = sx;
        s_ctp[kCtShard0][c] = s0;
        s_ctp[kCtIncl][c] = si;
        s_ctp[kCtTotal][c] = stt;
    }
    if (tid <= R) s_cu_r[tid] = cu_r;
    __syncthreads();
    {
        // segment starts of every rank's groups and duplicates (exclusive prefix over ranks)
        const int ng = tid < R ? s_ctp[kCtTotal][R + tid] : 0;
        const int nd = tid < R ? s_ctp[kCtTotal][2 * R + tid] : 0;
        int tg, td;
        const int eg = block_exclusive_scan<NT>(ng, s_tmp, tg);
        const int ed = block_exclusive_scan<NT>(nd, s_tmp, td);
        if (tid < R) {
            s_doff[0][tid] = eg;
            s_doff[1][tid] = ed;
        }
        if (tid == 0) {
            s_doff[0][R] = tg;
            s_doff[1][R] = td;
        }
    }
    __syncthreads();

    // ---- per-token pass: dst, slot codes, is_token_in_rank ballots ------------------------
    const int nslots = (int)(t1 - t0) * g.K;
    if (tile >= 0 && tid < g.TT) {
        const int64_t t = my_t;
        const bool live = my_live;
        uint32_t m[kMaxRanks / 32] = {0u, 0u, 0u, 0u};
        if (live) {
            TokenSlots<KMAX> ts;
            token_slots<KMAX>(ts, idk, g.K, g.E, R, s_owner);
            // branch-free over the slots (k < K is uniform): every LDS read first, then the codes
            int32_t dv[KMAX];
            int cr[KMAX];
            bool all_ok = true;
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                const bool v = k < g.K && ts.ok[k];
                cr[k] = s_cu_r[v ? ts.r[k] : 0];
                all_ok = all_ok && (k >= g.K || ts.ok[k]);
            }
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                dv[k] = 0;
                if (k >= g.K) continue;
                const bool v = ts.ok[k];
                const int si = tid * g.K + k;
                const int r = v ? ts.r[k] : 0;
                const int loff = pk[k] - cr[k];
                const int64_t raw = (int64_t)r * g.NvS + loff;
                dv[k] = (int32_t)(ts.first[k] ? raw : -raw - 1);
                const uint32_t type = ts.first[k] ? (ts.h[k] >= 2 ? kHead : kNone) : kDup;
                s_code[slot_pad(si)] = v ? (type | ((uint32_t)r << 2) | ((uint32_t)ts.h[k] << 10)) : kNone;
                s_loff[slot_pad(si)] = loff;
                const bool mark = v && ts.first[k];
#pragma unroll
                for (int q = 0; q < kMaxRanks / 32; ++q) m[q] |= (mark && (r >> 5) == q) ? (1u << (r & 31)) : 0u;
            }
            if (o.dst) {  // the token's K entries: two 16-byte stores when K == 8 and all are valid
                MEP_GLOBAL int32_t* drow = gptr(o.dst) + t * g.K;
                if (KMAX == 8 && g.K == 8 && all_ok && (((uintptr_t)o.dst) & 15u) == 0) {
                    MEP_GLOBAL u32x4* d4 = reinterpret_cast<MEP_GLOBAL u32x4*>(drow);
                    d4[0] = u32x4{(uint32_t)dv[0], (uint32_t)dv[1], (uint32_t)dv[2], (uint32_t)dv[3]};
                    d4[1] = u32x4{(uint32_t)dv[4 % KMAX], (uint32_t)dv[5 % KMAX], (uint32_t)dv[6 % KMAX], (uint32_t)dv[7 % KMAX]};
                } else {
#pragma unroll
                    for (int k = 0; k < KMAX; ++k)
                        if (k < g.K && ts.ok[k]) drow[k] = dv[k];
                }
            }
        }
        if (o.chan) {
            for (int r = 0; r < R; ++r) {
                const uint64_t b = __ballot(live && ((m[r >> 5] >> (r & 31)) & 1u));
                if (lane == 0) s_mask[w][r] = b;
            }
        }
    }
    __syncthreads();

    // ---- slot pass 1: stable ranks among same-rank heads / duplicates of this wave --------
    constexpr int kIters = kPlanSlots / kWTWaves / kWave;
    const int per_wave = (nslots + kWTWaves - 1) / kWTWaves;
    const int wbeg = w * per_wave;
    const int wend = min(nslots, wbeg + per_wave);
    int hrank[kIters];
    int drank[kIters];
    if (tile >= 0) {
#pragma unroll
        for (int it = 0; it < kIters; ++it) {
            const int si = wbeg + it * kWave + lane;
            const bool inb = si < wend;
            const uint32_t code = inb ? s_code[slot_pad(si)] : kNone;
            const uint32_t type = code & 3u;
            const bool valid = type != kNone;
            const int r = valid ? (int)((code >> 2) & 0xFFu) : 0;
            const uint64_t act = __ballot(valid);
            const uint64_t hm = __ballot(valid && type == kHead);
            const uint64_t dm = __ballot(valid && type == kDup);
            const uint64_t peers = match_peers<NB>((uint32_t)r, act);
            hrank[it] = 0;
            drank[it] = 0;
            if (valid) {
                const uint64_t below = peers & lanes_below();
                const int hb = s_hc[w][r];
                const int db = s_dc[w][r];
                hrank[it] = hb + popc64(below & hm);
                drank[it] = db + popc64(below & dm);
                if (below == 0) {
                    s_hc[w][r] = hb + popc64(peers & hm);
                    s_dc[w][r] = db + popc64(peers & dm);
                }
            }
        }
    }
    __syncthreads();
    for (int r = tid; r < R; r += NT) {
        int hr = 0, dr = 0;
#pragma unroll
        for (int ww = 0; ww < kWTWaves; ++ww) {
            const int hc = s_hc[ww][r], dc = s_dc[ww][r];
            s_hc[ww][r] = hr;
            s_dc[ww][r] = dr;
            hr += hc;
            dr += dc;
        }
    }
    __syncthreads();

    // ---- slot pass 2: write groups and duplicate offsets ----------------------------------
    if (tile >= 0 && (o.dup_groups || o.dup_loffs)) {
#pragma unroll
        for (int it = 0; it < kIters; ++it) {
            const int si = wbeg + it * kWave + lane;
            if (si >= wend) continue;
            const uint32_t code = s_code[slot_pad(si)];
            const uint32_t type = code & 3u;
            if (type == kNone) continue;
            const int r = (int)((code >> 2) & 0xFFu);
            const int dup_local = s_excl[2 * R + r] + s_dc[w][r] + drank[it];  // within r's segment
            if (type == kHead) {
                const int64_t gpos = (int64_t)s_doff[0][r] + s_excl[R + r] + s_hc[w][r] + hrank[it];
                if (o.dup_groups && gpos < o.cap_g) {
                    const int h = (int)(code >> 10);
                    gptr(o.dup_groups)[3 * gpos + 0] = s_loff[slot_pad(si)];
                    gptr(o.dup_groups)[3 * gpos + 1] = dup_local;
                    gptr(o.dup_groups)[3 * gpos + 2] = h - 1;
                }
            } else {
                const int64_t dpos = (int64_t)s_doff[1][r] + dup_local;
                if (o.dup_loffs && dpos < o.cap_d) gptr(o.dup_loffs)[dpos] = s_loff[slot_pad(si)];
            }
        }
    }

    // ---- channel prefix at channel boundaries inside this tile ----------------------------
    if (tile >= 0 && o.chan) {
        const int64_t q = (g.n + g.C - 1) / g.C;
        const int64_t tl0 = t0 - (int64_t)sh * g.n;
        const int64_t tl1 = t1 - (int64_t)sh * g.n;
        const int c_lo = (int)(tl0 / q);
        // channels c_lo.. whose end min((c+1)q, n) lies in (tl0, tl1]
        int c_hi = c_lo;
        while (c_hi < g.C && min((int64_t)(c_hi + 1) * q, (int64_t)g.n) <= tl1) ++c_hi;
        const int npairs = (c_hi - c_lo) * R;
        for (int p = tid; p < npairs; p += NT) {
            const int c = c_lo + p / R;
            const int r = p - (p / R) * R;
            const int L = (int)(min((int64_t)(c + 1) * q, (int64_t)g.n) - tl0);  // tokens before the end
            int cnt = 0;
            const int wf = L >> 6;
            for (int ww = 0; ww < wf; ++ww) cnt += popc64(s_mask[ww][r]);
            const int rem = L & 63;
            if (rem) cnt += popc64(s_mask[wf][r] & ((1ull << rem) - 1ull));
            gptr(o.chan)[((int64_t)sh * R + r) * g.C + c] = s_excl[r] + cnt - s_ctp[kCtShard0][r];
        }
    }

    // ---- per-shard matrices from the last tile of each shard -----------------------------
    if (tile >= 0 && ct == g.tps - 1) {
        // the count tile of a shard's last write tile ends at the shard's end
        for (int r = tid; r < R; r += NT) {
            const int incl = s_ctp[kCtIncl][r];
            if (o.rank_prefix) gptr(o.rank_prefix)[(int64_t)sh * R + r] = incl;
            if (o.ntpr) gptr(o.ntpr)[(int64_t)sh * R + r] = incl - s_ctp[kCtShard0][r];
        }
    }

    // ---- per-shard expert counts and expert totals, one wave per expert, a slice of the
    // experts per workgroup: differences of the inclusive prefixes at the shards' last count tiles
    if (g.ntiles > 0) {
        for (int e = e_first; e < g.E; e += gridDim.x * kWTWaves) {
            const bool pref = tail_pref && e == e_first;
            for (int s2 = lane; s2 < g.S; s2 += 64) {
                const int hi = pref ? tail_hi : (int)status_value(pw.statusE, (s2 + 1) * g.ctps - 1, g.E, e);
                const int lo = pref ? tail_lo : s2 > 0 ? (int)status_value(pw.statusE, s2 * g.ctps - 1, g.E, e) : 0;
                if (o.ntpe) gptr(o.ntpe)[(int64_t)s2 * g.E + e] = hi - lo;
            }
            if (o.recv_zf && lane == 0) {
                const int total = pref ? tail_tot : (int)status_value(pw.statusE, g.nct - 1, g.E, e);
                const int cu0 = pref ? tail_cu0 : src.cuv(e);
                const int cu1 = pref ? tail_cu1 : src.cuv(e + 1);
                const int cuo = pref ? tail_cuo : src.cuv(s_owner[e] * g.epn);
                const int padded = cu1 - cu0;
                const bool z = total > 0 && padded > total;
                gptr(o.recv_zf)[2 * e] = z ? cu0 + total - cuo : 0;
                gptr(o.recv_zf)[2 * e + 1] = z ? padded - total : 0;
            }
        }
    }

    // ---- block 0: per-rank outputs, empty-shard case, workspace reset ---------------------
    if (blockIdx.x == 0) {
        for (int r = tid; r < R; r += NT) {
            if (o.recv_tokens) gptr(o.recv_tokens)[r] = s_ctp[kCtTotal][r];
            if (o.dup_counts) {
                gptr(o.dup_counts)[2 * r] = s_doff[0][r + 1] - s_doff[0][r];
                gptr(o.dup_counts)[2 * r + 1] = s_doff[1][r + 1] - s_doff[1][r];
            }
        }
        if (o.dup_offsets)
            for (int r = tid; r <= R; r += NT) {
                gptr(o.dup_offsets)[2 * r] = s_doff[0][r];
                gptr(o.dup_offsets)[2 * r + 1] = s_doff[1][r];
            }
        if (o.recv_cu)
            for (int p = tid; p < R * (g.epn + 1); p += NT) {
                const int r = p / (g.epn + 1);
                const int j = p - r * (g.epn + 1);
                gptr(o.recv_cu)[p] = src.cuv(r * g.epn + j) - s_cu_r[r];
            }

        if (g.ntiles == 0) {  // no tokens: every per-shard matrix is zero
            for (int p = tid; p < g.S * R; p += NT) {
                if (o.rank_prefix) gptr(o.rank_prefix)[p] = 0;
                if (o.ntpr) gptr(o.ntpr)[p] = 0;
            }
            if (o.ntpe)
                for (int p = tid; p < g.S * g.E; p += NT) gptr(o.ntpe)[p] = 0;
            if (o.recv_zf)
                for (int p = tid; p < 2 * g.E; p += NT) gptr(o.recv_zf)[p] = 0;
            if (o.chan)
                for (int64_t p = tid; p < (int64_t)g.S * R * g.C; p += NT) gptr(o.chan)[p] = 0;
        }
        if (tid == 0) {
            gptr(hdr)->epoch = gptr(hdr)->epoch + 1u;
            gptr(hdr)->ticket = 0u;
        }
    }
}


template <int KMAX, int NB>
__global__ __launch_bounds__(kPlanBlock) void plan_write_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ e2p, PlanGeom g, PlanWs pw, WsHeader* hdr, PlanOutDev o) {
    __shared__ int s_owner[kMaxE];
    __shared__ int s_cu_r[kMaxRanks + 1];
    __shared__ int s_excl[3 * kMaxRanks];
    __shared__ int s_ctp[3][3 * kMaxRanks];
    __shared__ int s_doff[2][kMaxRanks + 1];
    __shared__ uint32_t s_code[kPlanSlots + kPlanSlots / 64];
    __shared__ int s_loff[kPlanSlots + kPlanSlots / 64];
    __shared__ int s_hc[kPlanWaves][kMaxRanks];
    __shared__ int s_dc[kPlanWaves][kMaxRanks];
    __shared__ uint64_t s_mask[kPlanWaves][kMaxRanks];
    __shared__ int s_tmp[kPlanWaves];
    const WriteLds L{s_owner, s_cu_r, s_excl, s_ctp, s_doff, s_code, s_loff, s_hc, s_dc, s_mask, s_tmp};
    plan_write_tile<KMAX, NB, kPlanBlock>(WriteSrcGlobal{ids, e2p, cu_seqlens}, g, pw, hdr, o, L);
}

// The scatter and write passes of mep_layout_plan in one kernel: a workgroup scatters its plan
// tile (layout_scatter.h), keeps the tile's ids and permuted positions in LDS, and writes its
// part of the plan from them (cu_seqlens from its own padded scan).  The write phase's large LDS
// arrays reuse the scatter phase's per-(wave, expert) counters, free by then.
template <int NBE, int KMAX, int NB>
__global__ __launch_bounds__(kScatBlock) void plan_scatter_write_kernel(const int32_t* __restrict__ ids, int A,
                                                                        ScatterSrc src, WsHeader* hdr,
                                                                        LayoutOut lout, PlanOutDev o) {
    constexpr int kW = kScatBlock / kWave;
    constexpr int kPadSlots = kPlanSlots + kPlanSlots / 64;
    // one region for the scatter phase's per-(wave, expert) counters and, later, the write
    // phase's slot codes, offsets and per-wave counters
    constexpr int kWriteBytes = 8 * kPadSlots + (4 + 4 + 8) * kW * kMaxRanks;
    constexpr int kScatBytes = 4 * kScatWaves * kMaxExperts;
    constexpr int kBigBytes = kWriteBytes > kScatBytes ? kWriteBytes : kScatBytes;
    static_assert(kLayTile >= kPlanSlots, "a plan tile fits a scatter tile");
    __shared__ __align__(16) char s_big[kBigBytes];
    __shared__ int s_cu[kMaxExperts + 1];
    __shared__ int s_tot[kMaxExperts];
    __shared__ int s_base[kMaxExperts];
    __shared__ int s_loc[kMaxExperts];
    __shared__ int s_tmp[kScatWaves];
    __shared__ int s_slot[kLayTile + kLayTile / 64];
    __shared__ int s_pos[kLayTile + kLayTile / 64];
    __shared__ int s_owner[kMaxE];
    __shared__ int s_cu_r[kMaxRanks + 1];
    __shared__ int s_excl[3 * kMaxRanks];
    __shared__ int s_ctp[3][3 * kMaxRanks];
    __shared__ int s_doff[2][kMaxRanks + 1];
    __shared__ int s_wtmp[kW];
    int (*s_cnt)[kMaxExperts] = reinterpret_cast<int (*)[kMaxExperts]>(s_big);
    uint32_t* w_code = reinterpret_cast<uint32_t*>(s_big);
    int* w_loff = reinterpret_cast<int*>(s_big + 4 * kPadSlots);
    int (*w_hc)[kMaxRanks] = reinterpret_cast<int (*)[kMaxRanks]>(s_big + 8 * kPadSlots);
    int (*w_dc)[kMaxRanks] = reinterpret_cast<int (*)[kMaxRanks]>(s_big + 8 * kPadSlots + 4 * kW * kMaxRanks);
    uint64_t (*w_mask)[kMaxRanks] = reinterpret_cast<uint64_t (*)[kMaxRanks]>(s_big + 8 * kPadSlots + 8 * kW * kMaxRanks);

    const ScatterLds SL{s_cu, s_tot, s_base, s_loc, s_cnt, s_tmp, s_slot, s_pos};
    scatter_tile<NBE>(ids, src.pg.E, A, src, hdr, lout, SL, s_slot, s_pos);
    __syncthreads();
    const WriteLds WL{s_owner, s_cu_r, s_excl, s_ctp, s_doff, w_code, w_loff, w_hc, w_dc, w_mask, s_wtmp};
    plan_write_tile<KMAX, NB, kScatBlock>(WriteSrcLds{s_slot, s_pos, s_cu}, src.pg, src.pw, hdr, o, WL);
}

static PlanGeom plan_geom(int64_t N, int E, int K, int R, int S, int C, int64_t NvS) {
    PlanGeom g;
    g.N = (int)N;
    g.E = E;
    g.K = K;
    g.R = R;
    g.epn = E / R;
    g.S = S;
    g.n = (int)(N / S);
    g.TT = plan_tile_tokens(K);
    if (g.TT >= 2 && (int64_t)S * ceil_div64(g.n, g.TT / 2) <= kTileUnits) g.TT /= 2;
    g.tps = (int)ceil_div64(g.n, g.TT);
    g.ntiles = S * g.tps;
    g.ncols = 3 * R + E;
    g.C = C;
    g.NvS = NvS;
    int sub = (int)ceil_div64(g.ntiles, kCountTilesP);
    if (sub < 1) sub = 1;
    g.sub = sub;
    g.ctps = (int)ceil_div64(g.tps, sub);
    g.nct = S * g.ctps;
    g.ticketed = g.nct > kUnticketedCountTiles;
    g.direct = g.nct <= kDirectCountTiles;
    return g;
}

}  // namespace mep

namespace mep {

// Byte offsets of the parts of the plan workspace (each 256-byte aligned), and its size.
struct PlanWsLayout {
    size_t arrive, status3, statusE, tilehist, bytes;
};



static PlanWsLayout plan_ws_layout(const PlanGeom& g) {
    PlanWsLayout L;
    const size_t n3 = 3 * (size_t)g.R;
    // after the fused path's group sums, which only its kernels ever write
    L.arrive = sizeof(WsHeader) + kPathGsumBytes;
    L.status3 = L.arrive + kMaxCountTiles * sizeof(uint32_t);
    L.statusE = L.status3 + align256((size_t)g.nct * n3 * sizeof(uint64_t));
    L.tilehist = L.statusE + align256((size_t)g.nct * g.E * sizeof(uint64_t));
    L.bytes = L.tilehist + align256((size_t)g.ntiles * g.ncols * sizeof(uint64_t));
    return L;
}

}  // namespace mep

extern "C" size_t mep_plan_workspace_size(int64_t N, int E, int K, int R, int num_src) {
    using namespace mep;
    if (N < 0 || E < 1 || K < 1 || R < 1 || num_src < 1 || R > kMaxRanks || E > kMaxE)
        return sizeof(WsHeader);
    // large enough for both the count-tile kernels of mep_plan and the fused path's plan tiles
    const size_t a = plan_ws_layout(plan_geom(N, E, K, R, num_src, 1, 0)).bytes;
    const size_t b = path_workspace_bytes(N, E, K, R, num_src);
    return a > b ? a : b;
}

namespace mep {

// Checks of mep_plan and the launch arguments; MEP_OK or the error code.
int plan_prepare(const int32_t* topk_ids, const int32_t* cu_seqlens, const int32_t* expanded_to_permuted,
                 int64_t N, int E, int K, int alignment, int R, int num_src, int num_channels, int64_t NvS,
                 const mep_plan_outputs* out, void* ws, size_t ws_bytes, PlanCall& c) {
    if (!cu_seqlens || !out || !ws) return MEP_ERR_INVALID_ARG;
    if (N > 0 && (!topk_ids || !expanded_to_permuted)) return MEP_ERR_INVALID_ARG;  // N == 0 reads nothing
    if (N < 0 || E < 1 || K < 1 || R < 1 || num_src < 1 || num_channels < 1 || alignment < 1)
        return MEP_ERR_INVALID_ARG;
    const void* p4[] = {topk_ids, cu_seqlens, expanded_to_permuted, out->is_token_in_rank,
                        out->num_tokens_per_rank, out->num_tokens_per_expert, out->rank_prefix_matrix,
                        out->channel_prefix_matrix, out->recv_tokens, out->recv_cu_seqlens,
                        out->recv_zero_fill, out->dst, out->dup_counts, out->dup_offsets,
                        out->dup_groups, out->dup_loffs};
    for (const void* q : p4)
        if (q && !aligned(q, 4)) return MEP_ERR_INVALID_ARG;
    if (!aligned(ws, 256)) return MEP_ERR_INVALID_ARG;
    if (E > kMaxE || K > 32 || K > E || R > kMaxRanks) return MEP_ERR_UNSUPPORTED;
    if (E % R != 0) return MEP_ERR_UNSUPPORTED;
    if (num_src > kMaxSources) return MEP_ERR_UNSUPPORTED;
    if (N % num_src != 0) return MEP_ERR_INVALID_ARG;
    const int64_t NK = N * (int64_t)K;
    const int64_t bound = NK + (NK < E ? NK : (int64_t)E) * (int64_t)(alignment - 1);
    if (bound > INT32_MAX - (1 << 16)) return MEP_ERR_UNSUPPORTED;
    if ((int64_t)num_src * R * num_channels > INT32_MAX) return MEP_ERR_UNSUPPORTED;
    const int epn = E / R;
    const int64_t nvs_min = N * (int64_t)(K < epn ? K : epn) + (int64_t)epn * (alignment - 1);
    if (NvS < nvs_min || NvS < 1 || (int64_t)R * NvS > INT32_MAX) return MEP_ERR_CAPACITY;
    const int64_t g_max = epn >= 2 ? N * (int64_t)((K / 2) < R ? (K / 2) : R) : 0;
    const int64_t d_max = N * (int64_t)(K - (K + epn - 1) / epn);
    if (out->dup_groups && out->cap_groups < g_max) return MEP_ERR_CAPACITY;
    if (out->dup_loffs && out->cap_dups < d_max) return MEP_ERR_CAPACITY;
    if (ws_bytes < mep_plan_workspace_size(N, E, K, R, num_src)) return MEP_ERR_CAPACITY;

    c.g = plan_geom(N, E, K, R, num_src, num_channels, NvS);
    c.ids = topk_ids;
    c.cu = cu_seqlens;
    c.e2p = expanded_to_permuted;
    c.hdr = reinterpret_cast<WsHeader*>(ws);
    const PlanWsLayout L = plan_ws_layout(c.g);
    char* wsb = reinterpret_cast<char*>(ws);
    c.pw = PlanWs{reinterpret_cast<uint32_t*>(wsb + L.arrive), reinterpret_cast<uint64_t*>(wsb + L.status3),
                  reinterpret_cast<uint64_t*>(wsb + L.statusE), reinterpret_cast<uint64_t*>(wsb + L.tilehist)};
    c.o = PlanOutDev{out->is_token_in_rank, out->num_tokens_per_rank, out->num_tokens_per_expert,
                     out->rank_prefix_matrix, out->channel_prefix_matrix, out->recv_tokens,
                     out->recv_cu_seqlens, out->recv_zero_fill, out->dst, out->dup_counts,
                     out->dup_offsets, out->dup_groups, out->cap_groups, out->dup_loffs, out->cap_dups};
    return MEP_OK;
}

// The counting pass (reads the ids only) and the writing pass (also the layout's cu_seqlens and
// expanded_to_permuted), launched separately so that the counting pass can run alongside the
// layout kernels.
void plan_launch_count(const PlanCall& c, hipStream_t st) {
    const PlanGeom& g = c.g;
    if (g.ntiles == 0) return;
    auto launch = [&](auto kernel) {
        launch_ggl(kernel, dim3(g.ntiles), dim3(kPlanBlock), 0, st, c.ids, g, c.pw, c.hdr, c.o.itr);
    };
    if (g.K <= 8) {
        if (g.R <= 32) launch(plan_count_kernel<8, 1>);
        else launch(plan_count_kernel<8, 4>);
    } else {
        if (g.R <= 32) launch(plan_count_kernel<32, 1>);
        else launch(plan_count_kernel<32, 4>);
    }
}

void plan_launch_scatter_write(const LayoutCall& lc, const PlanCall& c, hipStream_t st) {
    const PlanGeom& g = c.g;
    if (g.K > 8) {  // the per-token arrays of K up to 32 need the registers of 512-thread groups
        layout_launch_scatter_from_plan(lc, c, st);
        plan_launch_write(c, st);
        return;
    }
    ScatterSrc src{};
    src.plan = 1;
    src.pg = g;
    src.pw = c.pw;
    const int grid = g.ntiles > 0 ? g.ntiles : 1;
    auto launch = [&](auto kernel) {
        launch_ggl(kernel, dim3(grid), dim3(kScatBlock), 0, st, c.ids, lc.A, src, c.hdr, lc.out, c.o);
    };
    const bool wideE = g.E > 256;  // expert ids need 10 bits for the scatter's wave matching
    if (g.R <= 8) wideE ? launch(plan_scatter_write_kernel<10, 8, 3>) : launch(plan_scatter_write_kernel<8, 8, 3>);
    else if (g.R <= 32) wideE ? launch(plan_scatter_write_kernel<10, 8, 5>) : launch(plan_scatter_write_kernel<8, 8, 5>);
    else wideE ? launch(plan_scatter_write_kernel<10, 8, 7>) : launch(plan_scatter_write_kernel<8, 8, 7>);
}

void plan_launch_write(const PlanCall& c, hipStream_t st) {
    const PlanGeom& g = c.g;
    const int grid = g.ntiles > 0 ? g.ntiles : 1;
    auto launch = [&](auto kernel) {
        launch_ggl(kernel, dim3(grid), dim3(kPlanBlock), 0, st, c.ids, c.cu, c.e2p, g, c.pw, c.hdr, c.o);
    };
    if (g.K <= 8) {
        if (g.R <= 8) launch(plan_write_kernel<8, 3>);
        else if (g.R <= 32) launch(plan_write_kernel<8, 5>);
        else launch(plan_write_kernel<8, 7>);
    } else {
        if (g.R <= 8) launch(plan_write_kernel<32, 3>);
        else if (g.R <= 32) launch(plan_write_kernel<32, 5>);
        else launch(plan_write_kernel<32, 7>);
    }
}

}  // namespace mep

extern "C" int mep_plan(const int32_t* topk_ids, const int32_t* cu_seqlens,
                        const int32_t* expanded_to_permuted, int64_t N, int E, int K, int alignment,
                        int R, int num_src, int num_channels, int64_t NvS, const mep_plan_outputs* out,
                        void* ws, size_t ws_bytes, void* stream) {
    mep::launch_begin();
    using namespace mep;
    PlanCall c;
    const int rc = plan_prepare(topk_ids, cu_seqlens, expanded_to_permuted, N, E, K, alignment, R, num_src,
                                num_channels, NvS, out, ws, ws_bytes, c);
    if (rc != MEP_OK) return rc;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (path_supported(N, E, K, R)) {
        // the plan-tile path: the counting kernel over the ids, then the plan-tile kernel, which
        // takes every slot's row and the group offsets from the given layout
        const PathCall pc = path_call_plan(c, cu_seqlens, expanded_to_permuted, alignment, ws);
        path_launch_count(pc, st);
        path_launch_plan(pc, st, nullptr, nullptr);
        return launch_status();
    }
    plan_launch_count(c, st);
    plan_launch_write(c, st);
    return launch_status();
}
