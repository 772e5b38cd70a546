// mep_plan: expert-parallel dispatch plan over R virtual ranks, computed on one GPU's batch.
//
// Tokens are cut into tiles that never cross a source shard (TT tokens, TT*K <= 2048 slots).
// Per token, with owner(e) = e / epn:
//   c0[r]  1 if the token sends anything to r       (is_token_in_rank; DeepEP intranode.cu
//                                                     notify_dispatch counts and prefixes these)
//   c1[r]  1 if the token sends >= 2 slots to r     (one dedup group)
//   c2[r]  slots to r beyond the first              (duplicates: MoonEP planning.py duplicate
//                                                     canonicalisation encodes them as -dst-1)
//   cE[e]  1 if the token is routed to e            (per-shard expert counts)
//
//   count kernel  LDS histogram of the 3R+E columns per tile + decoupled look-back across tiles
//                 (exclusive/inclusive prefix of every column at every tile boundary); also
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

namespace mep {

constexpr int kPlanBlock = 256;
constexpr int kPlanWaves = kPlanBlock / kWave;
constexpr int kPlanSlots = 2048;  // slots per tile
constexpr int kMaxRanks = 128;
constexpr int kMaxE = 1024;
constexpr int kMaxCols = 3 * kMaxRanks + kMaxE;

static int plan_tile_tokens(int K) {
    int kp = 1;
    while (kp < K) kp <<= 1;
    int tt = kPlanSlots / kp;
    return tt > kPlanBlock ? kPlanBlock : tt;
}

struct PlanGeom {
    int N, E, K, R, epn, S, n, tps, ntiles, TT, ncols, C;
    int64_t NvS;
};

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
__device__ __forceinline__ void token_slots(TokenSlots<KMAX>& ts, const int32_t* ids, int64_t t,
                                            int K, int E, const int* s_owner) {
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        if (k < K) {
            const int id = ids[t * K + k];
            ts.ok[k] = (unsigned)id < (unsigned)E;
            ts.id[k] = ts.ok[k] ? id : 0;
            ts.r[k] = ts.ok[k] ? s_owner[ts.id[k]] : -1;
        } else {
            ts.ok[k] = false;
            ts.id[k] = 0;
            ts.r[k] = -1;
        }
    }
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

template <int KMAX>
__global__ __launch_bounds__(kPlanBlock) void plan_count_kernel(const int32_t* __restrict__ ids,
                                                                PlanGeom g, uint64_t* status,
                                                                WsHeader* hdr, uint8_t* itr) {
    __shared__ int s_cnt[kMaxCols];
    __shared__ int s_owner[kMaxE];
    __shared__ int s_tile;
    const int tid = threadIdx.x;
    for (int c = tid; c < g.ncols; c += kPlanBlock) s_cnt[c] = 0;
    for (int e = tid; e < g.E; e += kPlanBlock) s_owner[e] = e / g.epn;
    if (tid == 0) s_tile = take_ticket(hdr, (int)gridDim.x);
    __syncthreads();
    const int tile = s_tile;
    const uint32_t epoch = __hip_atomic_load(&hdr->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    const int sh = tile / g.tps;
    const int ct = tile - sh * g.tps;
    const int64_t t0 = (int64_t)sh * g.n + (int64_t)ct * g.TT;
    const int64_t t1 = min(t0 + g.TT, (int64_t)(sh + 1) * g.n);
    const int64_t t = t0 + tid;
    const int R = g.R;
    if (tid < g.TT && t < t1) {
        TokenSlots<KMAX> ts;
        token_slots<KMAX>(ts, ids, t, g.K, g.E, s_owner);
        uint32_t m[kMaxRanks / 32] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (!ts.ok[k]) continue;
            const int r = ts.r[k];
            atomicAdd(&s_cnt[3 * R + ts.id[k]], 1);
            if (ts.first[k]) {
                atomicAdd(&s_cnt[r], 1);
                if (ts.h[k] >= 2) atomicAdd(&s_cnt[R + r], 1);
#pragma unroll
                for (int q = 0; q < kMaxRanks / 32; ++q) m[q] |= ((r >> 5) == q) ? (1u << (r & 31)) : 0u;
            } else {
                atomicAdd(&s_cnt[2 * R + r], 1);
            }
        }
        if (itr) {
            uint8_t* row = itr + t * R;
            if ((R & 3) == 0) {
                for (int b = 0; b < R; b += 4) {
                    const uint32_t bits = m[b >> 5] >> (b & 31);
                    const uint32_t word = (bits & 1u) | (((bits >> 1) & 1u) << 8) |
                                          (((bits >> 2) & 1u) << 16) | (((bits >> 3) & 1u) << 24);
                    *reinterpret_cast<uint32_t*>(row + b) = word;
                }
            } else {
                for (int b = 0; b < R; ++b) row[b] = (uint8_t)((m[b >> 5] >> (b & 31)) & 1u);
            }
        }
    }
    __syncthreads();
    for (int c = tid; c < g.ncols; c += kPlanBlock)
        lookback_column(status, tile, g.ncols, c, epoch, (uint32_t)s_cnt[c]);
}

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

enum : uint32_t { kNone = 0, kHead = 1, kDup = 2 };

template <int KMAX>
__global__ __launch_bounds__(kPlanBlock) void plan_write_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ e2p, PlanGeom g, const uint64_t* status, WsHeader* hdr,
    PlanOutDev o) {
    __shared__ int s_owner[kMaxE];
    __shared__ int s_cu_r[kMaxRanks + 1];
    __shared__ int s_excl[3 * kMaxRanks];
    __shared__ int s_shard0[kMaxRanks];
    __shared__ int s_doff[2][kMaxRanks + 1];
    __shared__ uint32_t s_code[kPlanSlots];
    __shared__ int s_loff[kPlanSlots];
    __shared__ int s_hc[kPlanWaves][kMaxRanks];
    __shared__ int s_dc[kPlanWaves][kMaxRanks];
    __shared__ uint64_t s_mask[kPlanWaves][kMaxRanks];
    __shared__ int s_tmp[kPlanWaves];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int R = g.R;
    const int tile = g.ntiles > 0 ? (int)blockIdx.x : -1;
    const int sh = tile >= 0 ? tile / g.tps : 0;
    const int ct = tile >= 0 ? tile - sh * g.tps : 0;
    const int64_t t0 = (int64_t)sh * g.n + (int64_t)ct * g.TT;
    const int64_t t1 = tile >= 0 ? min(t0 + g.TT, (int64_t)(sh + 1) * g.n) : t0;
    const int first_tile_of_shard = sh * g.tps;

    auto total_of = [&](int col) -> int {
        return g.ntiles > 0 ? (int)status_value(status, g.ntiles - 1, g.ncols, col) : 0;
    };

    // ---- prologue --------------------------------------------------------------------------
    for (int e = tid; e < g.E; e += kPlanBlock) s_owner[e] = e / g.epn;
    for (int r = tid; r <= R; r += kPlanBlock) s_cu_r[r] = cu_seqlens[r * g.epn];
    for (int c = tid; c < 3 * R; c += kPlanBlock)
        s_excl[c] = tile > 0 ? (int)status_value(status, tile - 1, g.ncols, c) : 0;
    for (int r = tid; r < R; r += kPlanBlock)
        s_shard0[r] = first_tile_of_shard > 0
                          ? (int)status_value(status, first_tile_of_shard - 1, g.ncols, r)
                          : 0;
    for (int r = tid; r < R; r += kPlanBlock)
#pragma unroll
        for (int ww = 0; ww < kPlanWaves; ++ww) {
            s_hc[ww][r] = 0;
            s_dc[ww][r] = 0;
            s_mask[ww][r] = 0ull;
        }
    {
        // segment starts of every rank's groups and duplicates (exclusive prefix over ranks)
        const int ng = tid < R ? total_of(R + tid) : 0;
        const int nd = tid < R ? total_of(2 * R + tid) : 0;
        int tg, td;
        const int eg = block_exclusive_scan<kPlanBlock>(ng, s_tmp, tg);
        const int ed = block_exclusive_scan<kPlanBlock>(nd, s_tmp, td);
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
        const int64_t t = t0 + tid;
        const bool live = t < t1;
        uint32_t m[kMaxRanks / 32] = {0u, 0u, 0u, 0u};
        if (live) {
            TokenSlots<KMAX> ts;
            token_slots<KMAX>(ts, ids, t, g.K, g.E, s_owner);
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                if (k >= g.K) continue;
                const int si = tid * g.K + k;
                if (!ts.ok[k]) {
                    s_code[si] = kNone;
                    continue;
                }
                const int r = ts.r[k];
                const int loff = e2p[t * g.K + k] - s_cu_r[r];
                const int64_t raw = (int64_t)r * g.NvS + loff;
                if (o.dst) o.dst[t * g.K + k] = (int32_t)(ts.first[k] ? raw : -raw - 1);
                const uint32_t type = ts.first[k] ? (ts.h[k] >= 2 ? kHead : kNone) : kDup;
                s_code[si] = type | ((uint32_t)r << 2) | ((uint32_t)ts.h[k] << 10);
                s_loff[si] = loff;
                if (ts.first[k]) {
#pragma unroll
                    for (int q = 0; q < kMaxRanks / 32; ++q) m[q] |= ((r >> 5) == q) ? (1u << (r & 31)) : 0u;
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
    constexpr int kIters = kPlanSlots / kPlanWaves / kWave;  // 8
    const int per_wave = (nslots + kPlanWaves - 1) / kPlanWaves;
    const int wbeg = w * per_wave;
    const int wend = min(nslots, wbeg + per_wave);
    const int rbits = bits_for(R);
    int hrank[kIters];
    int drank[kIters];
    if (tile >= 0) {
#pragma unroll
        for (int it = 0; it < kIters; ++it) {
            const int si = wbeg + it * kWave + lane;
            const bool inb = si < wend;
            const uint32_t code = inb ? s_code[si] : kNone;
            const uint32_t type = code & 3u;
            const bool valid = type != kNone;
            const int r = valid ? (int)((code >> 2) & 0xFFu) : 0;
            const uint64_t act = __ballot(valid);
            const uint64_t hm = __ballot(valid && type == kHead);
            const uint64_t dm = __ballot(valid && type == kDup);
            const uint64_t peers = match_peers((uint32_t)r, rbits, act);
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
    for (int r = tid; r < R; r += kPlanBlock) {
        int hr = 0, dr = 0;
#pragma unroll
        for (int ww = 0; ww < kPlanWaves; ++ww) {
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
            const uint32_t code = s_code[si];
            const uint32_t type = code & 3u;
            if (type == kNone) continue;
            const int r = (int)((code >> 2) & 0xFFu);
            const int dup_local = s_excl[2 * R + r] + s_dc[w][r] + drank[it];  // within r's segment
            if (type == kHead) {
                const int64_t gpos = (int64_t)s_doff[0][r] + s_excl[R + r] + s_hc[w][r] + hrank[it];
                if (o.dup_groups && gpos < o.cap_g) {
                    const int h = (int)(code >> 10);
                    o.dup_groups[3 * gpos + 0] = s_loff[si];
                    o.dup_groups[3 * gpos + 1] = dup_local;
                    o.dup_groups[3 * gpos + 2] = h - 1;
                }
            } else {
                const int64_t dpos = (int64_t)s_doff[1][r] + dup_local;
                if (o.dup_loffs && dpos < o.cap_d) o.dup_loffs[dpos] = s_loff[si];
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
        for (int p = tid; p < npairs; p += kPlanBlock) {
            const int c = c_lo + p / R;
            const int r = p - (p / R) * R;
            const int L = (int)(min((int64_t)(c + 1) * q, (int64_t)g.n) - tl0);  // tokens before the end
            int cnt = 0;
            const int wf = L >> 6;
            for (int ww = 0; ww < wf; ++ww) cnt += popc64(s_mask[ww][r]);
            const int rem = L & 63;
            if (rem) cnt += popc64(s_mask[wf][r] & ((1ull << rem) - 1ull));
            o.chan[((int64_t)sh * R + r) * g.C + c] = s_excl[r] + cnt - s_shard0[r];
        }
    }

    // ---- per-shard matrices from the last tile of each shard -----------------------------
    if (tile >= 0 && ct == g.tps - 1) {
        for (int r = tid; r < R; r += kPlanBlock) {
            const int incl = (int)status_value(status, tile, g.ncols, r);
            if (o.rank_prefix) o.rank_prefix[(int64_t)sh * R + r] = incl;
            if (o.ntpr) o.ntpr[(int64_t)sh * R + r] = incl - s_shard0[r];
        }
        if (o.ntpe) {
            for (int e = tid; e < g.E; e += kPlanBlock) {
                const int col = 3 * R + e;
                const int prev = first_tile_of_shard > 0
                                     ? (int)status_value(status, first_tile_of_shard - 1, g.ncols, col)
                                     : 0;
                o.ntpe[(int64_t)sh * g.E + e] = (int)status_value(status, tile, g.ncols, col) - prev;
            }
        }
    }

    // ---- block 0: per-rank outputs, empty-shard case, workspace reset ---------------------
    if (blockIdx.x == 0) {
        for (int r = tid; r < R; r += kPlanBlock) {
            if (o.recv_tokens) o.recv_tokens[r] = total_of(r);
            if (o.dup_counts) {
                o.dup_counts[2 * r] = s_doff[0][r + 1] - s_doff[0][r];
                o.dup_counts[2 * r + 1] = s_doff[1][r + 1] - s_doff[1][r];
            }
        }
        if (o.dup_offsets)
            for (int r = tid; r <= R; r += kPlanBlock) {
                o.dup_offsets[2 * r] = s_doff[0][r];
                o.dup_offsets[2 * r + 1] = s_doff[1][r];
            }
        if (o.recv_cu)
            for (int p = tid; p < R * (g.epn + 1); p += kPlanBlock) {
                const int r = p / (g.epn + 1);
                const int j = p - r * (g.epn + 1);
                o.recv_cu[p] = cu_seqlens[r * g.epn + j] - s_cu_r[r];
            }
        if (o.recv_zf)
            for (int e = tid; e < g.E; e += kPlanBlock) {
                const int cnt = total_of(3 * R + e);
                const int padded = cu_seqlens[e + 1] - cu_seqlens[e];
                const bool z = cnt > 0 && padded > cnt;
                o.recv_zf[2 * e] = z ? cu_seqlens[e] + cnt - s_cu_r[s_owner[e]] : 0;
                o.recv_zf[2 * e + 1] = z ? padded - cnt : 0;
            }
        if (g.ntiles == 0) {  // no tokens: every per-shard matrix is zero
            for (int p = tid; p < g.S * R; p += kPlanBlock) {
                if (o.rank_prefix) o.rank_prefix[p] = 0;
                if (o.ntpr) o.ntpr[p] = 0;
            }
            if (o.ntpe)
                for (int p = tid; p < g.S * g.E; p += kPlanBlock) o.ntpe[p] = 0;
            if (o.chan)
                for (int64_t p = tid; p < (int64_t)g.S * R * g.C; p += kPlanBlock) o.chan[p] = 0;
        }
        if (tid == 0) {
            hdr->epoch = hdr->epoch + 1u;
            hdr->ticket = 0u;
        }
    }
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
    g.tps = (int)ceil_div64(g.n, g.TT);
    g.ntiles = S * g.tps;
    g.ncols = 3 * R + E;
    g.C = C;
    g.NvS = NvS;
    return g;
}

}  // namespace mep

extern "C" size_t mep_plan_workspace_size(int64_t N, int E, int K, int R, int num_src) {
    using namespace mep;
    if (N < 0 || E < 1 || K < 1 || R < 1 || num_src < 1) return sizeof(WsHeader);
    const int TT = plan_tile_tokens(K);
    const int64_t tps = ceil_div64(N / num_src, TT);
    return sizeof(WsHeader) + (size_t)(num_src * tps) * (size_t)(3 * R + E) * sizeof(uint64_t);
}

extern "C" int mep_plan(const int32_t* topk_ids, const int32_t* cu_seqlens,
                        const int32_t* expanded_to_permuted, int64_t N, int E, int K, int alignment,
                        int R, int num_src, int num_channels, int64_t NvS, const mep_plan_outputs* out,
                        void* ws, size_t ws_bytes, void* stream) {
    using namespace mep;
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

    PlanGeom g = plan_geom(N, E, K, R, num_src, num_channels, NvS);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    WsHeader* hdr = reinterpret_cast<WsHeader*>(ws);
    uint64_t* status = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(ws) + sizeof(WsHeader));
    PlanOutDev o{out->is_token_in_rank, out->num_tokens_per_rank, out->num_tokens_per_expert,
                 out->rank_prefix_matrix, out->channel_prefix_matrix, out->recv_tokens,
                 out->recv_cu_seqlens, out->recv_zero_fill, out->dst, out->dup_counts,
                 out->dup_offsets, out->dup_groups, out->cap_groups, out->dup_loffs, out->cap_dups};
    const int grid = g.ntiles > 0 ? g.ntiles : 1;
    if (K <= 8) {
        if (g.ntiles > 0)
            hipLaunchKernelGGL(plan_count_kernel<8>, dim3(g.ntiles), dim3(kPlanBlock), 0, st, topk_ids,
                               g, status, hdr, o.itr);
        hipLaunchKernelGGL(plan_write_kernel<8>, dim3(grid), dim3(kPlanBlock), 0, st, topk_ids,
                           cu_seqlens, expanded_to_permuted, g, status, hdr, o);
    } else {
        if (g.ntiles > 0)
            hipLaunchKernelGGL(plan_count_kernel<32>, dim3(g.ntiles), dim3(kPlanBlock), 0, st, topk_ids,
                               g, status, hdr, o.itr);
        hipLaunchKernelGGL(plan_write_kernel<32>, dim3(grid), dim3(kPlanBlock), 0, st, topk_ids,
                           cu_seqlens, expanded_to_permuted, g, status, hdr, o);
    }
    return launch_status();
}
