// The fused layout + plan path over plan tiles (path.h): the counting kernel (for ids given by
// the caller; the routing kernel does the same counting in its epilogue when it runs in the
// fused call), and the plan-tile kernel, which writes every per-slot and per-token output of the
// layout and the plan for one tile from the prefixes the counting epilogue left.  mep_plan runs
// the same two kernels with its layout as an input: the plan-tile kernel then takes each slot's
// row and the expert offsets from it and writes only the plan.
//
// Plan-tile kernel, one workgroup per tile (at most 4096 slots) of 1024 threads when every tile
// has a compute unit, else of 512 (two tiles per unit):
//   prologue   the tile's ids into LDS; the exclusive prefix of every column before the tile
//              (a sum of the rows the counting epilogue left, 16-byte loads spread over every
//              thread), cu_seqlens, the dedup segment starts;
//   tokens     a thread per token: owner ranks of its K slots, first slot per rank, slots per
//              rank -> a code per slot (expert, rank, head / duplicate / plain, slots on the rank);
//              is_token_in_rank; per-wave ballots of each rank's tokens (channel prefixes);
//   ranks      slots in slot order, 64 per wave step: a slot's rank among the same expert's
//              slots of its wave from one ballot per id bit (a wave64 stand-in for a warp match),
//              per-(wave, expert) counters in LDS; the same for dedup heads and duplicates per
//              rank.  The order is MoonEP planning.py run_c1's stable order, so the result is
//              deterministic;
//   write      expanded_to_permuted = cu[e] + prefix before the tile + earlier waves + rank;
//              permuted_to_expanded at that row; dst with the duplicate encoding (MoonEP
//              planning.py dst computation and duplicate canonicalisation); dedup groups and
//              duplicate offsets at their rank-major, token-ordered places;
//   per tile   channel prefixes ending in the tile (DeepEP intranode.cu notify_dispatch channel
//              part), the per-shard matrices from the shard's last tile, padding rows (-1) of
//              a share of the experts.
#include <limits.h>
#include <math.h>

#include "path.h"

namespace mep {

namespace {

constexpr int kCountNT = 512;
// Plan-tile workgroups: 1024 threads when every tile has a compute unit of its own, else 512
// (two tiles per compute unit at once, whose dependent chains then overlap).
constexpr int kPlanNTBig = 1024;
constexpr int kPlanNTSmall = 512;
constexpr int kPlanRowNT = 512;  // threads that load the prefix rows
static_assert(kPlanRowNT >= (kPathMaxNC + 3) / 4, "every column quad has a loader thread");
enum : uint32_t { kSlotPlain = 0, kSlotHead = 1, kSlotDup = 2 };

__device__ __forceinline__ uint32_t slot_code(int e, uint32_t type, int r, int h) {
    return (uint32_t)e | (type << 10) | ((uint32_t)r << 12) | ((uint32_t)h << 17);
}

// Exclusive scan over the 64 lanes of a wave; `total` gets the sum.  DPP row shifts by 1, 2, 4
// and 8 give the inclusive scan within each row of 16 lanes; the row broadcasts of lane 15 (into
// rows 1 and 3) and of lane 31 (into rows 2 and 3) carry it across rows.
__device__ __forceinline__ int wave_excl_scan(int v, int& total) {
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

}  // namespace

// ---- counting kernel (ids given) ---------------------------------------------------------------

// One counting workgroup per `sub` consecutive plan tiles: histogram rows in LDS, then the
// epilogue of path.h.
__global__ __launch_bounds__(kCountNT) void path_count_kernel(const int32_t* __restrict__ ids, PathGeom g,
                                                              PathWs w, WsHeader* hdr) {
    __shared__ int s_row[kPathMaxSub * kPathMaxNC];
    __shared__ int64_t s_tb[kPathMaxSub + 1];
    const int tid = threadIdx.x;
    const int j0 = blockIdx.x * g.sub;
    const int nsub = min(g.sub, g.ntiles - j0);
    for (int i = tid; i < nsub * g.NC; i += kCountNT) s_row[i] = 0;
    if (tid <= nsub) {
        int64_t a, b;
        path_tile_tokens(g, j0 + min(tid, nsub - 1), a, b);
        s_tb[tid] = tid < nsub ? a : b;
    }
    const uint32_t pcall = path_count_begin(hdr);
    __syncthreads();
    const int64_t tb0 = s_tb[0], tb1 = s_tb[nsub];
    const int K = g.K;
    const bool vec8 = K == 8 && (((uintptr_t)ids) & 15u) == 0;
    for (int64_t t = tb0 + tid; t < tb1; t += kCountNT) {
        int i = 0;
        while (i + 1 < nsub && t >= s_tb[i + 1]) ++i;
        int* row = s_row + i * g.NC;
        int id[kPathMaxK];
        if (vec8) {
            const MEP_GLOBAL u32x4* q = reinterpret_cast<const MEP_GLOBAL u32x4*>(gptr(ids) + t * 8);
            const u32x4 a = q[0], b = q[1];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                id[k] = (int)a[k];
                id[4 + k] = (int)b[k];
            }
        } else {
#pragma unroll
            for (int k = 0; k < kPathMaxK; ++k) id[k] = k < K ? gptr(ids)[t * K + k] : -1;
        }
        uint32_t m1 = 0u, m2 = 0u;
#pragma unroll
        for (int k = 0; k < kPathMaxK; ++k) {
            if (k < K) {
                atomicAdd(&row[id[k]], 1);
                const uint32_t bit = 1u << (id[k] / g.epn);
                m2 |= m1 & bit;
                m1 |= bit;
            }
        }
        path_count_ranks(g, row, m1, m2, 0, 1);
    }
    path_epilogue<kCountNT>(g, w, pcall, s_row);
}

// ---- totals -> cu_seqlens, dedup segment starts, small outputs --------------------------------

// By wave 0: the padded exclusive scan of the expert totals (cu_seqlens, [MOON] Phase B2 padded
// group scan) and the exclusive scans over the ranks of the dedup group and duplicate totals.
__device__ __forceinline__ void path_scan_totals(const PathGeom& g, const int* s_tot, int* s_cu,
                                                 int (*s_doff)[kPathMaxR + 1], const int32_t* cu_in) {
    const int lane = threadIdx.x & 63;
    const int E = g.E, R = g.R, A = g.A;
    constexpr int PER = kPathMaxE / 64;
    const int per = (E + 63) / 64;
    int pad[PER];
    int s = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane * per + i;
        int v = 0;
        if (i < per && e < E) {
            const int c = s_tot[e];
            v = c <= 0 ? 0 : g.ashift >= 0 ? ((c + A - 1) >> g.ashift) << g.ashift : ((c + A - 1) / A) * A;
        }
        pad[i] = v;
        s += v;
    }
    int total;
    int run = wave_excl_scan(s, total);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane * per + i;
        if (i < per && e < E) s_cu[e] = cu_in ? gptr(cu_in)[e] : run;  // the given layout's, else formed
        run += pad[i];
    }
    if (lane == 0) s_cu[E] = cu_in ? gptr(cu_in)[E] : total;
    const int ng_r = lane < R ? s_tot[path_col_c1(g, lane)] : 0;
    const int nd_r = lane < R ? s_tot[path_col_c2(g, lane)] : 0;
    int tg, td;
    const int eg = wave_excl_scan(ng_r, tg);
    const int ed = wave_excl_scan(nd_r, td);
    if (lane <= R) {
        s_doff[0][lane] = lane < R ? eg : tg;
        s_doff[1][lane] = lane < R ? ed : td;
    }
}

// By one workgroup: cu_seqlens, tokens_per_expert, zero_fill ([MOON] zero-fill ranges), the
// receive counts, offsets and zero-fill ranges ([DEEP] notify_dispatch), dedup counts and offsets.
template <int NT>
__device__ __forceinline__ void path_small_outputs(const PathGeom& g, const PathOut& o, const int* s_tot,
                                                   const int* s_cu, const int (*s_doff)[kPathMaxR + 1]) {
    const int tid = threadIdx.x;
    const int E = g.E, R = g.R;
    if (o.cu_seqlens)
        for (int e = tid; e <= E; e += NT) gptr(o.cu_seqlens)[e] = s_cu[e];
    for (int e = tid; e < E; e += NT) {
        const int c = s_tot[e];
        const int cu0 = s_cu[e];
        const int padded = s_cu[e + 1] - cu0;
        const bool z = c > 0 && padded > c;
        if (o.tokens_per_expert) gptr(o.tokens_per_expert)[e] = c;
        if (o.zero_fill) {
            gptr(o.zero_fill)[2 * e] = z ? cu0 + c : 0;
            gptr(o.zero_fill)[2 * e + 1] = z ? padded - c : 0;
        }
        if (o.p.recv_zf) {
            const int base = s_cu[(e / g.epn) * g.epn];
            gptr(o.p.recv_zf)[2 * e] = z ? cu0 + c - base : 0;
            gptr(o.p.recv_zf)[2 * e + 1] = z ? padded - c : 0;
        }
    }
    for (int r = tid; r <= R; r += NT) {
        if (o.p.dup_offsets) {
            gptr(o.p.dup_offsets)[2 * r] = s_doff[0][r];
            gptr(o.p.dup_offsets)[2 * r + 1] = s_doff[1][r];
        }
        if (r < R) {
            if (o.p.dup_counts) {
                gptr(o.p.dup_counts)[2 * r] = s_tot[path_col_c1(g, r)];
                gptr(o.p.dup_counts)[2 * r + 1] = s_tot[path_col_c2(g, r)];
            }
            if (o.p.recv_tokens) gptr(o.p.recv_tokens)[r] = s_tot[path_col_c0(g, r)];
        }
    }
    if (o.p.recv_cu)
        for (int p = tid; p < R * (g.epn + 1); p += NT) {
            const int r = p / (g.epn + 1);
            const int jj = p - r * (g.epn + 1);
            gptr(o.p.recv_cu)[p] = s_cu[r * g.epn + jj] - s_cu[r * g.epn];
        }
}

// ---- plan-tile kernel --------------------------------------------------------------------------

template <int NBE, int NBR, int kPlanNT>
__global__ __launch_bounds__(kPlanNT) void path_plan_kernel(const int32_t* __restrict__ ids, PathGeom g,
                                                            PathWs w, PathOut o, WsHeader* hdr) {
    constexpr int kPlanW = kPlanNT / 64;
    constexpr int kPlanRowBatch = 8;  // prefix rows a loader thread has in flight at once
    constexpr int kPlanIters = kPathSlots / kPlanNT;  // 64-slot steps per wave, at most
    __shared__ __align__(16) uint32_t s_code[kPathSlots];
    __shared__ int s_ecnt[kPlanW][kPathMaxE];
    __shared__ int s_rcnt[kPlanW][2][kPathMaxR];
    __shared__ int s_cu[kPathMaxE + 1];
    __shared__ int s_excl[kPathMaxNC];
    __shared__ int s_shx[kPathMaxNC];
    __shared__ int s_tot[kPathMaxNC];
    __shared__ int s_doff[2][kPathMaxR + 1];
    __shared__ int s_owner[kPathMaxE];
    __shared__ uint64_t s_mask[kPathTokens / 64][kPathMaxR];
    __shared__ u32x4 s_pq[3][kPlanRowNT];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int j = blockIdx.x;
    const int K = g.K, E = g.E, R = g.R, NC = g.NC;
    int64_t t0, t1;
    path_tile_tokens(g, j, t0, t1);
    const int nt = (int)(t1 - t0);
    const int ns = nt * K;
    const int64_t s0 = t0 * K;
    const int sh = j / g.tps;
    const int l = j - sh * g.tps;
    const bool shard_last = l == g.tps - 1;
    const int jf = sh * g.tps;
    const bool want_mask = o.p.chan || (shard_last && (o.p.rank_prefix || o.p.ntpr));
    const bool want_shx = o.p.chan || (shard_last && (o.p.ntpr || o.p.ntpe));

    // ---- prologue: every global load of the tile, issued together ----------------------------
    // The tile's ids: 16-byte loads into registers, stored into LDS only once the prefix rows'
    // loads below are in flight as well, so that the two round trips overlap (plain loads where
    // the slots are not 16-byte aligned).
    constexpr int kIdQ = kPathSlots / 4 / kPlanNT;  // id quads per thread, at most
    const MEP_GLOBAL int32_t* gid = gptr(ids) + s0;
    const int nq = ((s0 & 3) == 0) && ((((uintptr_t)ids) & 15u) == 0) ? ns >> 2 : 0;
    u32x4 idv[kIdQ];
#pragma unroll
    for (int i = 0; i < kIdQ; ++i)
        if (tid + i * kPlanNT < nq) idv[i] = reinterpret_cast<const MEP_GLOBAL u32x4*>(gid)[tid + i * kPlanNT];
    auto store_ids = [&]() {
#pragma unroll
        for (int i = 0; i < kIdQ; ++i) {
            const int q = tid + i * kPlanNT;
            if (q < nq) *reinterpret_cast<u32x4*>(&s_code[4 * q]) = idv[i];
        }
        for (int s = (nq << 2) + tid; s < ns; s += kPlanNT) s_code[s] = (uint32_t)gid[s];
    };
    // prefixes before this tile (and before the shard's first tile) and the totals: sums of rows
    // the counting epilogue left -- the group sum rows of both parities (one holds this call's
    // sums, the other is zero), the total rows of the earlier workgroups of the tile's group, the
    // tile's within-workgroup prefix row, and for the shard start the same two kinds of rows.
    // Each thread owns a column quad and a slice of the rows: 16-byte loads, all in flight at
    // once, summed in registers, then the slices summed through LDS.
    {
        const int NCs = g.NCs;
        const int NQ = NCs >> 2;
        const int ng = g.ng;
        const int wg = j / g.sub, grp = wg / g.GW, wg0 = grp * g.GW;
        const int wgf = jf / g.sub, grpf = wgf / g.GW, wgf0 = grpf * g.GW;
        // the shard start's prefix: every column for the shard's last tile (per-shard expert
        // counts), the rank token columns for the channel prefixes, none otherwise
        const bool shx_all = shard_last && o.p.ntpe;
        const bool shx_rank = o.p.chan || (shard_last && (o.p.ntpr || o.p.ntpe));
        const int r_w = 2 * ng;                 // first workgroup row of the tile's group
        const int r_t = r_w + (wg - wg0);       // the tile's prefix row
        const int r_f = r_t + 1;                // first workgroup row of the shard start's group
        const int nf = (shx_all || shx_rank) ? (wgf - wgf0) + 1 : 0;
        const int nrows = r_f + nf;
        const int r_l = nf > 0 ? nrows - 1 : nrows;  // the shard start's prefix row
        const int d_w = wg0 - r_w, d_f = wgf0 - r_f;  // row -> workgroup, in the two groups
        // row slices: as many as one batch of loads per thread needs (each slice is summed again
        // through LDS), within the loader threads
        const int nsl = min(kPlanRowNT / NQ, max(1, (nrows + kPlanRowBatch - 1) / kPlanRowBatch));
        const int q = tid % NQ, sl = tid / NQ;
        const bool need_f = shx_all || (shx_rank && 4 * q < E + R && 4 * q + 4 > E);
        // every row as a word offset from the first group sum row (rows past the list read group
        // row 0; they, and the shard start's rows in columns that do not need them, count nowhere)
        const MEP_GLOBAL uint32_t* base = gptr(w.gsum);
        const int64_t ow = w.wrow - w.gsum, ot = w.tpre - w.gsum;
        u32x4 tot = {0u, 0u, 0u, 0u}, ex = tot, sx = tot;
        u32x4 v[kPlanRowBatch];
        uint32_t use[kPlanRowBatch];  // bit 0: totals, bit 1: prefix of the tile, bit 2: of the shard start
        auto issue = [&](int r0) {
#pragma unroll
            for (int i = 0; i < kPlanRowBatch; ++i) {
                // the row's place from comparisons with the segment starts (group sum rows of
                // parity 0, of parity 1, total rows of the tile's group, the tile's prefix row,
                // total rows of the shard start's group, the shard start's prefix row, past the
                // list), one two-way select per statement: nested conditional expressions compile
                // to divergent branches
                const int r = r0 + i * nsl;
                const bool c1 = r >= ng, c2 = r >= r_w, c3 = r >= r_t, c4 = r >= r_f, c5 = r >= r_l,
                           c6 = r >= nrows;
                const int gi = c1 ? r - ng : r;
                const int i5 = c6 ? 0 : jf;
                const int i4 = c5 ? i5 : r + d_f;
                const int i3 = c4 ? i4 : j;
                const int i2 = c3 ? i3 : r + d_w;
                const int idx = c2 ? i2 : gi;
                const int64_t b_g = c1 ? (int64_t)kPathGsumWords : 0;
                const int64_t b_p = (c3 && !(c4 && !c5)) ? ot : ow;  // a prefix row, else a total row
                const int64_t b_w = c6 ? 0 : b_p;
                const int64_t rb = c2 ? b_w : b_g;
                const uint32_t u_g = 1u | (gi < grp ? 2u : 0u) | (gi < grpf ? 4u : 0u);
                const uint32_t u_f = (c6 || !need_f) ? 0u : 4u;
                const uint32_t u_w = c4 ? u_f : 2u;
                use[i] = c2 ? u_w : u_g;
                v[i] = reinterpret_cast<const MEP_GLOBAL u32x4*>(base + rb + (uint32_t)(idx * NCs))[q];
            }
        };
        auto accumulate = [&]() {
#pragma unroll
            for (int i = 0; i < kPlanRowBatch; ++i) {
                const u32x4 z = {0u, 0u, 0u, 0u};
                tot += (use[i] & 1u) ? v[i] : z;
                ex += (use[i] & 2u) ? v[i] : z;
                sx += (use[i] & 4u) ? v[i] : z;
            }
        };
        // the ids are stored on both sides of the branch, after the loads on the loaders' side (a
        // store after the join would wait for every load of the loaders)
        if (sl < nsl) {
            issue(sl);
            store_ids();
            accumulate();
            for (int r0 = sl + kPlanRowBatch * nsl; r0 < nrows; r0 += kPlanRowBatch * nsl) {
                issue(r0);
                accumulate();
            }
        } else {
            store_ids();
        }
        if (tid < kPlanRowNT) {
            s_pq[0][tid] = tot;
            s_pq[1][tid] = ex;
            s_pq[2][tid] = sx;
        }
        __syncthreads();
        for (int c = tid; c < NC; c += kPlanNT) {
            const int qc = c >> 2, ic = c & 3;
            uint32_t a = 0u, b = 0u, f = 0u;
            for (int s2 = 0; s2 < nsl; ++s2) {
                a += s_pq[0][s2 * NQ + qc][ic];
                b += s_pq[1][s2 * NQ + qc][ic];
                f += s_pq[2][s2 * NQ + qc][ic];
            }
            s_tot[c] = (int)a;
            s_excl[c] = (int)b;
            s_shx[c] = (int)f;
        }
    }
    for (int e = tid; e < E; e += kPlanNT) s_owner[e] = e / g.epn;
    for (int i = tid; i < kPlanW * E; i += kPlanNT) s_ecnt[i / E][i % E] = 0;
    for (int i = tid; i < kPlanW * 2 * R; i += kPlanNT) s_rcnt[i / (2 * R)][(i / R) & 1][i % R] = 0;
    __syncthreads();
    // ---- tokens (waves 0 .. kPlanW - 2): slot codes, is_token_in_rank, rank ballots; the last
    // wave meanwhile forms cu_seqlens and the dedup segment starts ---------------------------------
    if (wv == kPlanW - 1) path_scan_totals(g, s_tot, s_cu, s_doff, o.cu_in);
    for (int base = wv * 64; wv < kPlanW - 1 && base < nt; base += (kPlanW - 1) * 64) {
        const int tk = base + lane;
        const bool live = tk < nt;
        uint32_t m = 0u;
        if (live && K == 8 && R <= 8) {
            // eight slots, at most eight ranks: per-rank slot counts as 4-bit fields of one word
            const u32x4 a = *reinterpret_cast<const u32x4*>(&s_code[tk * 8]);
            const u32x4 b = *reinterpret_cast<const u32x4*>(&s_code[tk * 8 + 4]);
            const int e[8] = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
            int r[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) r[k] = g.eshift >= 0 ? e[k] >> g.eshift : s_owner[e[k]];
            uint32_t cnt = 0u;
#pragma unroll
            for (int k = 0; k < 8; ++k) cnt += 1u << (4 * r[k]);
            uint32_t cd[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t bit = 1u << r[k];
                const bool first = (m & bit) == 0u;
                m |= bit;
                const int h = (int)((cnt >> (4 * r[k])) & 15u);
                const uint32_t type = first ? (h >= 2 ? kSlotHead : kSlotPlain) : kSlotDup;
                cd[k] = slot_code(e[k], type, r[k], h);
            }
            *reinterpret_cast<u32x4*>(&s_code[tk * 8]) = u32x4{cd[0], cd[1], cd[2], cd[3]};
            *reinterpret_cast<u32x4*>(&s_code[tk * 8 + 4]) = u32x4{cd[4], cd[5], cd[6], cd[7]};
        } else if (live && R <= 8) {
            // fewer than eight slots, at most eight ranks: the same 4-bit per-rank counts
            int e[kPathMaxK], r[kPathMaxK];
            uint32_t cnt = 0u;
#pragma unroll
            for (int k = 0; k < kPathMaxK; ++k) {
                e[k] = k < K ? (int)s_code[tk * K + k] : 0;
                r[k] = g.eshift >= 0 ? e[k] >> g.eshift : s_owner[e[k]];
                cnt += k < K ? 1u << (4 * r[k]) : 0u;
            }
#pragma unroll
            for (int k = 0; k < kPathMaxK; ++k) {
                if (k < K) {
                    const uint32_t bit = 1u << r[k];
                    const bool first = (m & bit) == 0u;
                    m |= bit;
                    const int h = (int)((cnt >> (4 * r[k])) & 15u);
                    const uint32_t type = first ? (h >= 2 ? kSlotHead : kSlotPlain) : kSlotDup;
                    s_code[tk * K + k] = slot_code(e[k], type, r[k], h);
                }
            }
        } else if (live) {
            int e[kPathMaxK], r[kPathMaxK];
            uint32_t cd[kPathMaxK];
            if (K == 8) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(&s_code[tk * 8]);
                const u32x4 b = *reinterpret_cast<const u32x4*>(&s_code[tk * 8 + 4]);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    e[k] = (int)a[k];
                    e[4 + k] = (int)b[k];
                }
            } else if (K == 4) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(&s_code[tk * 4]);
#pragma unroll
                for (int k = 0; k < kPathMaxK; ++k) e[k] = k < 4 ? (int)a[k & 3] : 0;
            } else {
#pragma unroll
                for (int k = 0; k < kPathMaxK; ++k) e[k] = k < K ? (int)s_code[tk * K + k] : 0;
            }
            // up to 32 ranks: per-rank slot counts as 4-bit fields of four words (ranks 8q .. 8q + 7
            // in word q)
#pragma unroll
            for (int k = 0; k < kPathMaxK; ++k) r[k] = k < K ? (g.eshift >= 0 ? e[k] >> g.eshift : s_owner[e[k]]) : 0;
            uint32_t c4[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int k = 0; k < kPathMaxK; ++k) {
                const uint32_t inc = k < K ? 1u << (4 * (r[k] & 7)) : 0u;
#pragma unroll
                for (int q = 0; q < 4; ++q) c4[q] += (r[k] >> 3) == q ? inc : 0u;
            }
#pragma unroll
            for (int k = 0; k < kPathMaxK; ++k) {
                if (k >= K) continue;
                const int q = r[k] >> 3;
                const uint32_t wq = q == 0 ? c4[0] : q == 1 ? c4[1] : q == 2 ? c4[2] : c4[3];
                const int h = (int)((wq >> (4 * (r[k] & 7))) & 15u);
                const uint32_t bit = 1u << r[k];
                const bool first = (m & bit) == 0u;
                m |= bit;
                const uint32_t type = first ? (h >= 2 ? kSlotHead : kSlotPlain) : kSlotDup;
                cd[k] = slot_code(e[k], type, r[k], h);
            }
            if (K == 8) {
                *reinterpret_cast<u32x4*>(&s_code[tk * 8]) = u32x4{cd[0], cd[1], cd[2], cd[3]};
                *reinterpret_cast<u32x4*>(&s_code[tk * 8 + 4]) = u32x4{cd[4], cd[5], cd[6], cd[7]};
            } else if (K == 4) {
                *reinterpret_cast<u32x4*>(&s_code[tk * 4]) = u32x4{cd[0], cd[1], cd[2], cd[3]};
            } else {
#pragma unroll
                for (int k = 0; k < kPathMaxK; ++k)
                    if (k < K) s_code[tk * K + k] = cd[k];
            }
        }
        if (live) {
            if (o.p.itr) {
                MEP_GLOBAL uint8_t* row = gptr(o.p.itr) + (t0 + tk) * R;
                // four rank bits -> four bytes of 0 / 1 (the multiply places bit i at bit 8 i, with
                // no carries between the shifted copies)
                auto bytes4 = [](uint32_t b4) { return ((b4 & 15u) * 0x204081u) & 0x01010101u; };
                if ((R & 15) == 0 && (((uintptr_t)o.p.itr) & 15u) == 0) {
                    for (int bb = 0; bb < R; bb += 16) {
                        const u32x4 v = {bytes4(m >> bb), bytes4(m >> (bb + 4)), bytes4(m >> (bb + 8)),
                                         bytes4(m >> (bb + 12))};
                        *reinterpret_cast<MEP_GLOBAL u32x4*>(row + bb) = v;
                    }
                } else if ((R & 3) == 0) {
                    for (int bb = 0; bb < R; bb += 4)
                        *reinterpret_cast<MEP_GLOBAL uint32_t*>(row + bb) = bytes4(m >> bb);
                } else {
                    for (int bb = 0; bb < R; ++bb) row[bb] = (uint8_t)((m >> bb) & 1u);
                }
            }
        }
        if (want_mask) {
            // the wave's tokens on rank r as one 64-bit ballot, kept by lane r, then one store
            // per lane (no branch or LDS store inside the loop)
            const int tw = base >> 6;
            uint64_t mine = 0ull;
#pragma unroll 8
            for (int r = 0; r < R; ++r) {
                const uint64_t bm = __ballot((m >> r) & 1u);
                mine = lane == r ? bm : mine;
            }
            if (lane < R) s_mask[tw][lane] = mine;
        }
    }
    __syncthreads();
    if (j == 0) path_small_outputs<kPlanNT>(g, o, s_tot, s_cu, s_doff);

    // ---- stable ranks within the waves ------------------------------------------------------------
    const int spw = ((ns + kPlanNT - 1) / kPlanNT) * 64;  // slots per wave, a multiple of 64
    const int sbeg = wv * spw;
    int erank[kPlanIters], hrank[kPlanIters], drank[kPlanIters];
#pragma unroll
    for (int it = 0; it < kPlanIters; ++it) {
        erank[it] = hrank[it] = drank[it] = 0;
        if (it * 64 >= spw) continue;
        const int si = sbeg + it * 64 + lane;
        const bool valid = si < ns;
        const uint32_t code = valid ? s_code[si] : 0u;
        const int e = (int)(code & 1023u);
        const uint32_t type = (code >> 10) & 3u;
        const int r = (int)((code >> 12) & 31u);
        const uint64_t act = __ballot(valid);
        if (act == 0ull) continue;
        const uint64_t pe = match_peers<NBE>((uint32_t)e, act);
        const int eb = valid ? s_ecnt[wv][e] : 0;
        erank[it] = eb + popc64(pe & lanes_below());
        if (valid && (pe >> lane) == 1ull) s_ecnt[wv][e] = eb + popc64(pe);
        const uint64_t hm = __ballot(valid && type == kSlotHead);
        const uint64_t dm = __ballot(valid && type == kSlotDup);
        const uint64_t rel = hm | dm;
        if (rel != 0ull) {
            const bool inr = (rel >> lane) & 1ull;
            const uint64_t pr = match_peers<NBR>((uint32_t)r, rel);
            const uint64_t bl = pr & lanes_below();
            const int hb = inr ? s_rcnt[wv][0][r] : 0;
            const int db = inr ? s_rcnt[wv][1][r] : 0;
            hrank[it] = hb + popc64(bl & hm);
            drank[it] = db + popc64(bl & dm);
            if (inr && (pr >> lane) == 1ull) {
                s_rcnt[wv][0][r] = hb + popc64(pr & hm);
                s_rcnt[wv][1][r] = db + popc64(pr & dm);
            }
        }
    }
    __syncthreads();
    // per-(wave, column) counts -> exclusive prefixes over the waves; the tile's own expert counts
    for (int e = tid; e < E; e += kPlanNT) {
        int run = 0;
#pragma unroll
        for (int ww = 0; ww < kPlanW; ++ww) {
            const int x = s_ecnt[ww][e];
            s_ecnt[ww][e] = run;
            run += x;
        }
        if (shard_last && o.p.ntpe) gptr(o.p.ntpe)[(int64_t)sh * E + e] = s_excl[e] + run - s_shx[e];
    }
    for (int p = tid; p < 2 * R; p += kPlanNT) {
        const int q = p / R, r = p - (p / R) * R;
        int run = 0;
#pragma unroll
        for (int ww = 0; ww < kPlanW; ++ww) {
            const int x = s_rcnt[ww][q][r];
            s_rcnt[ww][q][r] = run;
            run += x;
        }
    }
    __syncthreads();

    // ---- per-slot outputs ----------------------------------------------------------------------
    const int epn = g.epn;
    const int NvS = (int)g.NvS;
#pragma unroll
    for (int it = 0; it < kPlanIters; ++it) {
        if (it * 64 >= spw) continue;
        const int si = sbeg + it * 64 + lane;
        if (si >= ns) continue;
        const uint32_t code = s_code[si];
        const int e = (int)(code & 1023u);
        const uint32_t type = (code >> 10) & 3u;
        const int r = (int)((code >> 12) & 31u);
        const int h = (int)(code >> 17);
        const int64_t gs = s0 + si;
        // the slot's permuted row: given (mep_plan), else its stable position
        const int P = o.p_in ? gptr(o.p_in)[gs] : s_cu[e] + s_excl[e] + s_ecnt[wv][e] + erank[it];
        if (o.e2p) gptr(o.e2p)[gs] = P;
        if (o.p2e) gptr(o.p2e)[P] = (int32_t)gs;
        const int loff = P - s_cu[r * epn];
        const int raw = r * NvS + loff;
        if (o.p.dst) gptr(o.p.dst)[gs] = type == kSlotDup ? -raw - 1 : raw;
        const int dloc = s_excl[path_col_c2(g, r)] + s_rcnt[wv][1][r] + drank[it];
        if (type == kSlotHead) {
            if (o.p.dup_groups) {
                const int64_t gpos = (int64_t)s_doff[0][r] + s_excl[path_col_c1(g, r)] + s_rcnt[wv][0][r] + hrank[it];
                if (gpos < o.p.cap_g) {
                    gptr(o.p.dup_groups)[3 * gpos + 0] = loff;
                    gptr(o.p.dup_groups)[3 * gpos + 1] = dloc;
                    gptr(o.p.dup_groups)[3 * gpos + 2] = h - 1;
                }
            }
        } else if (type == kSlotDup) {
            const int64_t dpos = (int64_t)s_doff[1][r] + dloc;
            if (o.p.dup_loffs && dpos < o.p.cap_d) gptr(o.p.dup_loffs)[dpos] = loff;
        }
    }

    // ---- channel prefixes ending in this tile --------------------------------------------------
    if (o.p.chan) {
        const int64_t q = ((int64_t)g.n + g.C - 1) / g.C;
        const int64_t tl0 = (int64_t)l * g.T, tl1 = tl0 + nt;
        const int c_lo = (int)(tl0 / q);
        int c_hi = c_lo;
        while (c_hi < g.C && ((int64_t)(c_hi + 1) * q < g.n ? (int64_t)(c_hi + 1) * q : (int64_t)g.n) <= tl1) ++c_hi;
        const int npairs = (c_hi - c_lo) * R;
        for (int p = tid; p < npairs; p += kPlanNT) {
            const int c = c_lo + p / R;
            const int r = p - (p / R) * R;
            const int64_t end = (int64_t)(c + 1) * q < g.n ? (int64_t)(c + 1) * q : (int64_t)g.n;
            const int L = (int)(end - tl0);  // tokens of the tile before the channel's end
            int cnt = 0;
            const int wf = L >> 6;
            for (int tw = 0; tw < wf; ++tw) cnt += popc64(s_mask[tw][r]);
            if (L & 63) cnt += popc64(s_mask[wf][r] & ((1ull << (L & 63)) - 1ull));
            const int c0 = path_col_c0(g, r);
            gptr(o.p.chan)[((int64_t)sh * R + r) * g.C + c] = s_excl[c0] - s_shx[c0] + cnt;
        }
    }

    // ---- per-shard matrices from the shard's last tile ----------------------------------------
    if (shard_last && (o.p.rank_prefix || o.p.ntpr)) {
        for (int r = tid; r < R; r += kPlanNT) {
            int own = 0;
            for (int tw = 0; tw * 64 < nt; ++tw) own += popc64(s_mask[tw][r]);
            const int c0 = path_col_c0(g, r);
            if (o.p.rank_prefix) gptr(o.p.rank_prefix)[(int64_t)sh * R + r] = s_excl[c0] + own;
            if (o.p.ntpr) gptr(o.p.ntpr)[(int64_t)sh * R + r] = s_excl[c0] + own - s_shx[c0];
        }
    }

    // ---- padding rows of a share of the experts -------------------------------------------------
    if (o.p2e) {
        for (int e = j; e < E; e += g.ntiles) {
            const int beg = s_cu[e] + s_tot[e];
            const int end = s_cu[e + 1];
            for (int row = beg + tid; row < end; row += kPlanNT) gptr(o.p2e)[row] = -1;
        }
    }
    if (j == 0 && tid == 0) __hip_atomic_fetch_add(&gptr(hdr)->pcall, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- host ----------------------------------------------------------------------------------------

PathGeom path_geom(int64_t N, int E, int K, int R, int S, int C, int A, int64_t NvS) {
    PathGeom g{};
    g.N = (int)N;
    g.E = E;
    g.K = K;
    g.R = R;
    g.epn = E / R;
    g.S = S;
    g.n = (int)(N / S);
    g.C = C;
    g.A = A;
    g.NvS = NvS;
    auto log2_exact = [](int v) {
        int k = 0;
        while (k < 30 && (1 << k) < v) ++k;
        return v > 0 && (1 << k) == v ? k : -1;
    };
    g.eshift = log2_exact(g.epn);
    g.ashift = log2_exact(A);
    int kp = 1;
    while (kp < K) kp <<= 1;
    g.T = kPathSlots / kp;
    if (g.T > kPathTokens) g.T = kPathTokens;
    // small batches: tiles of fewer tokens, so that the batch spreads over about kPathUnits
    // workgroups (each tile's latency-bound phases shrink with it), but not below 64 tokens
    const int64_t t_spread = ceil_div64(N, kPathUnits);
    const int t_fill = (int)(t_spread < kPathMinTileTokens ? kPathMinTileTokens : ceil_div64(t_spread, 64) * 64);
    if (g.T > t_fill) g.T = t_fill;
    if (g.T > g.n) g.T = g.n > 0 ? g.n : 1;
    g.tps = (int)ceil_div64(g.n, g.T);
    g.ntiles = S * g.tps;
    g.NC = E + 3 * R;
    g.NCs = (g.NC + 3) & ~3;
    int sub = (int)ceil_div64(g.ntiles, kPathUnits);
    if (sub < 1) sub = 1;
    if (sub > kPathMaxSub) sub = kPathMaxSub;
    g.sub = sub;
    g.nwg = (int)ceil_div64(g.ntiles, sub);
    int gw = (int)ceil(sqrt((double)g.nwg));
    const int gw_min = (int)ceil_div64(g.nwg, kPathMaxGroups);
    if (gw < gw_min) gw = gw_min;
    if (gw < 1) gw = 1;
    g.GW = gw;
    g.ng = (int)ceil_div64(g.nwg, gw);
    return g;
}

// The counters of mep_plan's count-tile kernels follow the group sums (8 KiB, always left at
// zero by those kernels); the rows of this path follow them, overlapping only parts of the
// workspace that every call of either kernel set rewrites before reading.
constexpr size_t kPlanArriveBytes = 8192;
// the plan-tile kernel reads the prefix rows as 16-byte quads: every row starts 16-byte aligned
// (the workspace is 256-byte aligned and rows are NCs words, a multiple of 4)
static_assert(sizeof(WsHeader) % 16 == 0 && kPathGsumWords * 4 % 16 == 0 && kPlanArriveBytes % 16 == 0,
              "prefix rows 16-byte aligned");

PathWsLayout path_ws_layout(const PathGeom& g) {
    PathWsLayout L;
    L.gsum = sizeof(WsHeader);
    size_t off = L.gsum + kPathGsumBytes + kPlanArriveBytes;
    L.wrow = off;
    off += align256((size_t)g.nwg * g.NCs * 4);
    L.tpre = off;
    off += align256((size_t)g.ntiles * g.NCs * 4);
    L.bytes = off;
    return L;
}

PathWs path_ws_views(void* ws, const PathGeom& g) {
    const PathWsLayout L = path_ws_layout(g);
    char* b = reinterpret_cast<char*>(ws);
    return PathWs{reinterpret_cast<uint32_t*>(b + L.gsum), reinterpret_cast<uint32_t*>(b + L.wrow),
                  reinterpret_cast<uint32_t*>(b + L.tpre)};
}

bool path_supported(int64_t N, int E, int K, int R) {
    return N > 0 && E <= kPathMaxE && K <= kPathMaxK && R <= kPathMaxR;
}

size_t path_workspace_bytes(int64_t N, int E, int K, int R, int S) {
    if (!path_supported(N, E, K, R) || S < 1 || N % S != 0) return 0;
    return path_ws_layout(path_geom(N, E, K, R, S, 1, 1, 0)).bytes;
}

PathCall path_call(const LayoutCall& lc, const PlanCall& pc, void* ws) {
    PathCall c;
    c.g = path_geom(pc.g.N, pc.g.E, pc.g.K, pc.g.R, pc.g.S, pc.g.C, lc.A, pc.g.NvS);
    c.w = path_ws_views(ws, c.g);
    c.hdr = reinterpret_cast<WsHeader*>(ws);
    c.o = PathOut{lc.out.tokens_per_expert, lc.out.cu_seqlens, lc.out.e2p, lc.out.p2e, lc.out.zero_fill, pc.o,
                  nullptr, nullptr};
    c.ids = pc.ids;
    return c;
}

PathCall path_call_plan(const PlanCall& pc, const int32_t* cu_seqlens, const int32_t* e2p, int A, void* ws) {
    PathCall c;
    c.g = path_geom(pc.g.N, pc.g.E, pc.g.K, pc.g.R, pc.g.S, pc.g.C, A, pc.g.NvS);
    c.w = path_ws_views(ws, c.g);
    c.hdr = reinterpret_cast<WsHeader*>(ws);
    c.o = PathOut{nullptr, nullptr, nullptr, nullptr, nullptr, pc.o, cu_seqlens, e2p};
    c.ids = pc.ids;
    return c;
}

void path_launch_count(const PathCall& c, hipStream_t st) {
    launch_ggl(path_count_kernel, dim3(c.g.nwg), dim3(kCountNT), 0, st, c.ids, c.g, c.w, c.hdr);
}

void path_launch_plan(const PathCall& c, hipStream_t st, hipEvent_t start, hipEvent_t stop) {
    auto launch = [&](auto kernel, int nt) {
        launch_ext(kernel, dim3(c.g.ntiles), dim3(nt), 0, st, start, stop, 0, c.ids, c.g, c.w, c.o, c.hdr);
    };
    const bool wideE = c.g.E > 256, wideR = c.g.R > 8;
    // 1024 threads when every tile has a compute unit and enough slots to share out; otherwise
    // 512 (two tiles per unit; fewer waves to clear and synchronise for a small tile)
    if (c.g.ntiles <= device_units() && (int64_t)c.g.T * c.g.K > 512) {
        constexpr int NT = kPlanNTBig;
        if (!wideR) wideE ? launch(path_plan_kernel<9, 3, NT>, NT) : launch(path_plan_kernel<8, 3, NT>, NT);
        else wideE ? launch(path_plan_kernel<9, 5, NT>, NT) : launch(path_plan_kernel<8, 5, NT>, NT);
    } else {
        constexpr int NT = kPlanNTSmall;
        if (!wideR) wideE ? launch(path_plan_kernel<9, 3, NT>, NT) : launch(path_plan_kernel<8, 3, NT>, NT);
        else wideE ? launch(path_plan_kernel<9, 5, NT>, NT) : launch(path_plan_kernel<8, 5, NT>, NT);
    }
}

}  // namespace mep
