/*
 * mep.h -- C ABI of the MI355X (gfx950) MoE routing and dispatch-layout
 * library (libmep.so).
 *
 * Three calls form the data-parallel hot path of MoE expert dispatch on one
 * GPU's token batch:
 *
 *   mep_route_topk   router logits [N,E] -> top-K expert ids and weights
 *   mep_build_layout ids -> per-expert histogram, padded offsets, stable
 *                    expanded<->permuted maps
 *   mep_plan         ids + layout -> expert-parallel plan over R virtual
 *                    ranks (membership, counts, prefix matrices, rank-tagged
 *                    destinations with duplicate encoding, dedup lists)
 *   mep_layout_plan  the two calls above in one (two kernels instead of
 *                    four)
 *   mep_route_layout_plan
 *                    all three in one call; one kernel for small batches,
 *                    two for large ones (the routing kernel also counts)
 *   mep_tile_map     per-expert counts -> grouped-GEMM tile maps (the expert
 *                    and the row limit of every padded tile)
 *   mep_plan_balanced the plan with capacity rebalancing: token moves between
 *                    ranks, their split over experts, experts to copy, and
 *                    dst on the rank that computes each slot
 *   mep_permute_rows, mep_combine_rows
 *                    hidden-state rows into the permuted order (zero padding)
 *                    and back, summed over a token's K slots
 *
 * Sources, cited by page title and section:
 *   [TRT]  TensorRT-LLM RoutingKernel.cuh (blockScaleMoe routing helpers,
 *          histogram / offsets / permutation kernels)
 *   [MOON] MoonEP planning.py (PlanningKernel: histogram, stable scatter,
 *          padded group scan, dst computation, duplicate canonicalisation;
 *          caller-allocated outputs and host-side checks)
 *   [DEEP] DeepEP intranode.cu (notify_dispatch: rank prefix matrix,
 *          aligned receive counts, channel prefix matrix, host asserts)
 *
 * Conventions shared by every call
 *   - Pointers named as device buffers are device memory owned by the
 *     caller: inputs are read only, outputs are preallocated, all arrays are
 *     dense row-major.  `logits` must be 16-byte aligned, every other buffer
 *     4-byte aligned ([MOON] launch helper alignment rules).
 *   - Calls enqueue asynchronously on `stream` (a hipStream_t; NULL = the
 *     null stream) and never synchronise.  They allocate nothing.
 *   - Scratch lives in a caller-provided workspace of at least the size the
 *     matching *_workspace_size call reports.  A workspace must be zero-filled
 *     once before its first use; every call leaves it ready for the next one.
 *     Calls sharing a workspace must be ordered (same stream, or synchronised);
 *     overlapping calls on one workspace race.
 *   - All checks run on the host before anything is enqueued.  On error
 *     nothing is written and nothing is launched.  Capacities are checked
 *     against worst-case bounds, so kernels have no error path.
 *   - Optional outputs are marked "nullable"; NULL skips them.  With N == 0 the per-slot
 *     inputs and outputs (logits, ids, weights, permutation maps, dst) may be NULL.
 *   - No exceptions cross the ABI; mep_status_string names a return code.
 *   - Word 3 of every layout / plan workspace (uint32 at byte 12) holds sticky
 *     error bits: bit 0 is set when a bounded wait of a kernel ran out, which
 *     only overlapping calls on one workspace can cause (the results of such a
 *     call are wrong).  The library never clears it; zero-filling the
 *     workspace does.
 */
#ifndef MEP_H_
#define MEP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define MEP_OK 0
#define MEP_ERR_INVALID_ARG 1 /* NULL required pointer, bad enum, bad size, misalignment */
#define MEP_ERR_UNSUPPORTED 2 /* outside the supported envelope (see each call) */
#define MEP_ERR_CAPACITY 3    /* caller capacity or workspace below the bound */
#define MEP_ERR_DEVICE 4      /* a kernel launch of this call failed (its own return
                                 code; errors earlier calls left in the runtime are not
                                 reported) */

/* Logit element types. */
#define MEP_F32 0  /* IEEE binary32 */
#define MEP_BF16 1 /* bfloat16 (upper half of a binary32) */

/* Scoring functions. */
#define MEP_SOFTMAX 0
#define MEP_SIGMOID 1

typedef struct mep_route_params {
    int score_fn;    /* MEP_SOFTMAX or MEP_SIGMOID */
    int renormalize; /* 1: weights renormalised over the K selected experts */
    int n_group;     /* expert groups for group-limited selection; 1 = off */
    int topk_group;  /* groups kept when n_group > 1 */
    int group_topn;  /* keys summed into a group's score (1 or 2) */
    float scale;     /* factor applied to every weight */
} mep_route_params;

/*
 * mep_route_topk -- top-K expert selection and routing weights.
 *
 * Per token t (row of `logits`):
 *   key_e = logit_e                                 (MEP_SOFTMAX)
 *   s_e   = sigmoid(logit_e), correctly rounded to binary32,
 *   key_e = fl32(s_e + bias_e)                      (MEP_SIGMOID)
 *   The sigmoid is the real function of [TRT] sigmoid_accurate; the library
 *   returns its correctly rounded value so ids are reproducible bit for bit.
 *   With n_group > 1 the experts form n_group contiguous groups; a group's
 *   score is the binary32 sum of its group_topn largest keys (largest
 *   first); the topk_group best groups (score desc, group index asc) stay
 *   eligible.  The K best eligible experts (key desc, expert index asc) are
 *   written to topk_ids[t*K + k] in that order.
 *   Weights (computed in double, rounded once to binary32, then times scale):
 *     softmax, renormalize: softmax over the K selected logits
 *                           ([TRT] calcSoftmax over the top lanes)
 *     softmax, no renorm:   softmax probability over all E logits
 *                           ([TRT] calcSoftmax over the score vector)
 *     sigmoid, renormalize: s_k / sum of the K selected s (0 if that is 0)
 *     sigmoid, no renorm:   s_k
 *
 * Arguments
 *   logits       device, [N,E] of `dtype`, 16-byte aligned
 *   dtype        MEP_F32 or MEP_BF16
 *   N            tokens, >= 0
 *   E            experts, 1..1024
 *   K            experts per token, 1..min(E,32)
 *   bias         device, float[E]; required for MEP_SIGMOID, ignored otherwise
 *   p            host pointer to the parameters above
 *   topk_ids     device, int32[N,K] (output)
 *   topk_weights device, float[N,K] (output, nullable)
 * Returns MEP_ERR_UNSUPPORTED for E > 1024, K > min(E, 32), n_group > 32,
 * group_topn not in {1,2}, E % n_group != 0, or topk_group*(E/n_group) < K.
 * Non-finite logits give unspecified (but memory-safe) results.
 */
int mep_route_topk(const void* logits, int dtype, int64_t N, int E, int K,
                   const float* bias, const mep_route_params* p,
                   int32_t* topk_ids, float* topk_weights, void* stream);

/*
 * mep_route_topk_timed -- mep_route_topk with kernel timing.
 *
 * Computes exactly what mep_route_topk computes (same arguments, checks and
 * errors).  Every routing shape runs as one kernel; start_event and
 * stop_event (hipEvent_t created by the caller, either may be NULL) are
 * updated by that kernel's launch itself with its start and end times
 * (hipExtLaunchKernel), so hipEventElapsedTime(start, stop) is the kernel's
 * duration with no marker packet on the stream.  For measuring the kernel
 * in place inside a larger stream of work.  Events are left untouched when
 * the call returns an error or N == 0.
 */
int mep_route_topk_timed(const void* logits, int dtype, int64_t N, int E, int K,
                         const float* bias, const mep_route_params* p,
                         int32_t* topk_ids, float* topk_weights, void* stream,
                         void* start_event, void* stop_event);

/*
 * mep_build_layout -- padded per-expert layout of the N*K routed slots.
 *
 * Slot i = t*K + k holds expert e = topk_ids[i].
 *   tokens_per_expert[e] = #slots with expert e
 *                          ([TRT] routingIndicesHistogramKernel)
 *   padded_e = ceil(count_e / alignment) * alignment, 0 for an empty expert
 *   cu_seqlens[0] = 0, cu_seqlens[e+1] = cu_seqlens[e] + padded_e
 *                          ([MOON] Phase B2 padded group scan; [DEEP] aligned
 *                           per-expert receive counts)
 *   expanded_to_permuted[i] = cu_seqlens[e] + #{earlier slots with expert e}
 *                          (stable by slot index: [MOON] run_c1 passA)
 *   permuted_to_expanded[expanded_to_permuted[i]] = i; the padding rows of
 *     [0, cu_seqlens[E]) hold -1 ([MOON] empty-slot sentinel)
 *   zero_fill[e] = (cu_seqlens[e] + count_e, padded_e - count_e) if count_e > 0
 *     and padded_e > count_e, else (0, 0)  ([MOON] zero-fill ranges)
 *
 * Arguments
 *   topk_ids             device int32[N,K]; every id in [0,E) and the K ids of
 *                        a token distinct (true of mep_route_topk output);
 *                        other inputs give unspecified results
 *   alignment            >= 1
 *   tokens_per_expert    device int32[E] (nullable)
 *   cu_seqlens           device int32[E+1]
 *   expanded_to_permuted device int32[N*K]
 *   permuted_to_expanded device int32[permuted_cap] (nullable); only the
 *                        first cu_seqlens[E] entries are written
 *   permuted_cap         >= N*K + min(E, N*K)*(alignment-1) when
 *                        permuted_to_expanded is given, else ignored
 *   zero_fill            device int32[E,2] (nullable)
 *   ws, ws_bytes         workspace (see mep_layout_workspace_size)
 * Returns MEP_ERR_UNSUPPORTED for E > 1024, K > min(E, 32), or
 * N*K + min(E, N*K)*(alignment-1) > INT32_MAX - 65536.
 */
int mep_build_layout(const int32_t* topk_ids, int64_t N, int E, int K, int alignment,
                     int32_t* tokens_per_expert, int32_t* cu_seqlens,
                     int32_t* expanded_to_permuted, int32_t* permuted_to_expanded,
                     int64_t permuted_cap, int32_t* zero_fill,
                     void* ws, size_t ws_bytes, void* stream);

size_t mep_layout_workspace_size(int64_t N, int E, int K);

/* Outputs of mep_plan; every pointer is a device buffer and nullable. */
typedef struct mep_plan_outputs {
    uint8_t* is_token_in_rank;      /* [N,R]   1 iff some slot of t lands on r */
    int32_t* num_tokens_per_rank;   /* [S,R]   tokens of shard s sent to rank r */
    int32_t* num_tokens_per_expert; /* [S,E]   tokens of shard s routed to e */
    int32_t* rank_prefix_matrix;    /* [S,R]   sum over s' <= s of the above */
    int32_t* channel_prefix_matrix; /* [S,R,C] prefix over channels of shard s */
    int32_t* recv_tokens;           /* [R]     tokens rank r receives */
    int32_t* recv_cu_seqlens;       /* [R,epn+1] rank-local padded offsets */
    int32_t* recv_zero_fill;        /* [E,2]   rank-local zero-fill ranges */
    int32_t* dst;                   /* [N*K]   rank-tagged slot, dups as -raw-1 */
    int32_t* dup_counts;            /* [R,2]   (groups, dups) per rank */
    int32_t* dup_offsets;           /* [R+1,2] exclusive prefix of dup_counts */
    int32_t* dup_groups;            /* [cap_groups,3] (primary_loff, dup_begin, dup_count) */
    int64_t cap_groups;
    int32_t* dup_loffs;             /* [cap_dups] rank-local offsets of duplicates */
    int64_t cap_dups;
} mep_plan_outputs;

/*
 * mep_plan -- expert-parallel dispatch plan over R virtual ranks.
 *
 * Experts are split contiguously: owner(e) = e / epn, epn = E / R.  The
 * batch is the concatenation of num_src equal shards (virtual source ranks),
 * shard s = tokens [s*n, (s+1)*n), n = N / num_src.
 *   is_token_in_rank[t][r]      = 1 iff some k has owner(ids[t][k]) == r
 *   num_tokens_per_rank[s][r], num_tokens_per_expert[s][e]: per-shard counts
 *   rank_prefix_matrix[s][r]    = sum_{s' <= s} num_tokens_per_rank[s'][r]
 *                                 ([DEEP] notify_dispatch rank prefix)
 *   recv_tokens[r]              = rank_prefix_matrix[num_src-1][r]
 *   channel c of shard s covers tokens s*n + [min(c*q,n), min((c+1)*q,n)),
 *     q = ceil(n / num_channels); channel_prefix_matrix[s][r][c] counts the
 *     tokens of channels 0..c of shard s that go to r
 *                                 ([DEEP] notify_dispatch channel part)
 *   recv_cu_seqlens[r][j]       = cu_seqlens[r*epn+j] - cu_seqlens[r*epn]
 *   recv_zero_fill[e]           = zero-fill range of e relative to its rank's
 *                                 first row, (0,0) when e is empty or unpadded
 *   dst[i], slot i = t*K+k, expert e, owner r:
 *     raw = r*NvS + expanded_to_permuted[i] - cu_seqlens[r*epn]
 *     the first k of token t on rank r stores raw, later ones -raw-1
 *                                 ([MOON] dst computation without capacity
 *                                  moves; duplicate canonicalisation)
 *   dedup: for each rank r and each token t (ascending) with >= 2 slots on
 *     r, one group (primary_loff, dup_begin, dup_count): the rank-local slot
 *     of its first k, the index of its first duplicate within r's dup_loffs
 *     segment, and (slots on r) - 1.  The duplicates' rank-local slots follow
 *     in k order.  Groups of r start at dup_groups[dup_offsets[r][0]], its
 *     duplicates at dup_loffs[dup_offsets[r][1]]; dup_offsets[R] holds totals.
 *     (Shapes and counts from [MOON]'s plan record; the order is defined
 *     here and is deterministic.)
 *
 * Arguments
 *   topk_ids, cu_seqlens, expanded_to_permuted: device inputs as produced by
 *     mep_route_topk / mep_build_layout with the same N, E, K, alignment
 *   R          ranks, divides E, E/R <= 1024, R <= 128
 *   num_src    shards, divides N (N = 0 allowed)
 *   num_channels >= 1
 *   NvS        per-rank slot stride, >= N*min(K,epn) + epn*(alignment-1),
 *              R*NvS <= INT32_MAX
 *   out        host pointer to the output table; cap_groups must be >=
 *              N*min(K/2, R) and cap_dups >= N*(K - ceil(K/epn)) when their
 *              arrays are given (both bounds are 0 when epn == 1)
 *   ws, ws_bytes workspace (see mep_plan_workspace_size)
 */
int mep_plan(const int32_t* topk_ids, const int32_t* cu_seqlens,
             const int32_t* expanded_to_permuted, int64_t N, int E, int K,
             int alignment, int R, int num_src, int num_channels, int64_t NvS,
             const mep_plan_outputs* out, void* ws, size_t ws_bytes, void* stream);

size_t mep_plan_workspace_size(int64_t N, int E, int K, int R, int num_src);

/*
 * mep_layout_plan -- mep_build_layout followed by mep_plan in one call, with
 * the results of the two calls and the checks of both (the layout's
 * cu_seqlens and expanded_to_permuted are outputs of the first part and inputs
 * of the second, so both are required).
 *
 * Two kernels.  With K <= 8, R <= 32 and E <= 512 (and N > 0): a counting
 * kernel takes each plan tile's histogram of experts and rank columns
 * ([TRT] routingIndicesHistogramKernel; [DEEP] notify_dispatch counts) and
 * leaves per-tile, per-workgroup and per-group partial sums, without any
 * workgroup waiting for another; a plan-tile kernel then forms every prefix it
 * needs from those sums, writes the padded offsets ([MOON] Phase B2) and
 * scatters its tile stably ([MOON] run_c1 passA) while writing that tile's
 * part of the plan.  Other shapes: the plan's count-tile kernels, with one
 * kernel scattering the layout and writing the plan.
 *
 * Arguments as mep_build_layout (without its workspace) and mep_plan; `ws` is
 * a workspace of mep_plan_workspace_size(N, E, K, R, num_src) bytes, the only
 * scratch of the call, with the rules of every workspace (zero-filled before
 * first use, calls sharing it ordered).  It may be shared with mep_plan and
 * mep_route_layout_plan calls of any size, not with mep_build_layout calls.
 * Word 3 of the workspace holds the sticky error bits described above.
 */
int mep_layout_plan(const int32_t* topk_ids, int64_t N, int E, int K, int alignment,
                    int32_t* tokens_per_expert, int32_t* cu_seqlens,
                    int32_t* expanded_to_permuted, int32_t* permuted_to_expanded,
                    int64_t permuted_cap, int32_t* zero_fill, int R, int num_src,
                    int num_channels, int64_t NvS, const mep_plan_outputs* out, void* ws,
                    size_t ws_bytes, void* stream);

/*
 * mep_tile_map -- grouped-GEMM tile maps of a per-expert histogram
 * ([TRT] routingPermutation / routingIndicesOffsetsKernel: the per-expert
 * CTA bookkeeping after the histogram).
 *
 * With c_e = tokens_per_expert[e] and A = tile:
 *   tiles_e = ceil(c_e / A); off_e = sum_{e' < e} tiles_e'; T = sum of all
 *   for every j = off_e + i, 0 <= i < tiles_e:
 *     cta_to_expert[j] = e
 *     cta_mn_limit[j]  = min((j + 1) * A, off_e * A + c_e)
 *   permuted_idx_size[0] = T * A, num_ctas[0] = T
 * With the same A as mep_build_layout's alignment, tile j covers the permuted
 * rows [j*A, (j+1)*A) of that layout (off_e * A == cu_seqlens[e]): the rows
 * below its limit hold expert e's slots, the rest are padding.  Entries at and
 * beyond T are not written.  For the experts of one rank of mep_plan, pass
 * tokens_per_expert + r*epn with E = epn: the expert index is then rank-local
 * (the pages' local expert index with stride 1) and the tiles cover
 * recv_cu_seqlens[r].
 *
 * Arguments
 *   tokens_per_expert device int32[E], every count >= 0 (a negative count
 *                     counts as 0), summing to at most num_slots
 *   E                 1 .. 1024
 *   num_slots         >= sum of the counts (N*K for a whole layout)
 *   tile              A >= 1
 *   cta_to_expert, cta_mn_limit  device int32[cap_ctas] (nullable)
 *   cap_ctas          >= (num_slots + min(E, num_slots)*(A-1)) / A when
 *                     either array is given
 *   permuted_idx_size, num_ctas  device int32[1] (nullable)
 * Returns MEP_ERR_UNSUPPORTED for E > 1024 or
 * num_slots + min(E, num_slots)*(A-1) > INT32_MAX - 65536.  Counts that sum
 * above num_slots give unspecified values but no write beyond cap_ctas.
 */
int mep_tile_map(const int32_t* tokens_per_expert, int E, int64_t num_slots, int tile,
                 int32_t* cta_to_expert, int32_t* cta_mn_limit, int64_t cap_ctas,
                 int32_t* permuted_idx_size, int32_t* num_ctas, void* stream);

/* Outputs of mep_plan_balanced; device buffers, all required except
 * experts_to_copy when num_copies == 0 and dst when N == 0. */
typedef struct mep_balanced_outputs {
    int32_t* group_tokens;    /* [R]       slots owned by rank r before moves */
    int32_t* z;               /* [R,R]     slots moved from rank s to rank d */
    int32_t* alloc;           /* [R,E]     slots of expert e computed on rank r */
    int32_t* alloc_cumsum;    /* [E,R]     sum over r' <= r of alloc[r'][e] */
    int32_t* experts_to_copy; /* [R,B]     experts rank d receives a copy of, -1 = none */
    int32_t* remote_stats;    /* [R,2]     (remote experts with slots on r,
                                            copies of r's experts sent out) */
    int32_t* cu_seqlens;      /* [R,E+B]   end row of each group on rank r */
    int32_t* zero_fill;       /* [R,E+B,2] (start, length) padding of each group */
    int32_t* expert_offsets;  /* [R,E]     first row of expert e on rank r, -1 = none */
    int32_t* dst;             /* [N*K]     rank-tagged row, duplicates as -raw-1 */
} mep_balanced_outputs;

/*
 * mep_plan_balanced -- expert-parallel plan with capacity rebalancing and
 * redundant remote experts ([MOON] PlanningKernel: balancing loop, quota
 * allocation, experts to copy, group scan, dst search), for all R ranks.
 *
 * owner(e) = e / epn, epn = E / R; c_e = tokens_per_expert[e].
 *   group_tokens[r] = sum of c_e over r's experts; balance = that - capacity.
 *   Balancing: while the largest balance (lowest rank on ties) is > 0 and
 *     the smallest (lowest rank on ties) is < 0, the largest moves
 *     -smallest slots to the smallest (z), which ends at 0 -- in one move,
 *     even when that takes the giver below capacity.
 *   Quotas: each owner o hands z[o][r] out, largest quota first (lowest rank
 *     on ties), each time from its expert with the most slots left (lowest
 *     index on ties), min of the two at once; what is left stays at o.
 *     alloc[r][e] is the result, alloc_cumsum its prefix over r.
 *   Copies: for each rank d, the remote experts (owner != d) with slots on d
 *     are counted (remote_stats[d][0]); num_copies times the one with most
 *     slots (highest index on ties) is taken: experts_to_copy[d][b], or -1
 *     once none is left; each copy adds 1 to remote_stats[owner][1].
 *   Groups of rank d: E + B of them; group g < E is expert g with
 *     alloc[d][g] slots unless g was copied (then empty), group E + b the
 *     b-th copied expert.  Each holds round_up(slots, token_padding) rows;
 *     cu_seqlens[d][g] is the end of group g (inclusive prefix), zero_fill
 *     its padding (start, length) when it has slots and padding, else (0,0);
 *     expert_offsets[d][e] the start of e's group on d, -1 if e has no slots
 *     there.
 *   dst: slot i = t*K+k of expert e sits at q = expanded_to_permuted[i] -
 *     cu_seqlens_layout[e] among e's slots; its rank lo is the first with
 *     alloc_cumsum[e][lo] > q; dst = lo*NvS + expert_offsets[lo][e] + q -
 *     alloc_cumsum[e][lo-1] (0 for lo = 0).  A later k of token t whose rank
 *     repeats an earlier k's stores -dst-1.
 * The page runs the same steps on every rank from gathered per-rank counts;
 * on one GPU the layout's stable positions give q directly.
 *
 * Arguments
 *   topk_ids, cu_seqlens, expanded_to_permuted, tokens_per_expert: device
 *     inputs as produced by mep_build_layout (any alignment) for the same
 *     ids; tokens_per_expert is required even when N == 0
 *   R            divides E, R <= 128, E <= 1024, K <= min(E, 32)
 *   num_copies   B, 0 .. 64
 *   token_padding >= 1 (1 = no padding)
 *   capacity     slots per rank, 0 .. INT32_MAX
 *   NvS          per-rank row stride, >= max(N*min(K,epn), capacity) +
 *                (E+B)*(token_padding-1); R*NvS <= INT32_MAX
 * Two kernels; no workspace (the intermediate arrays are outputs).
 */
int mep_plan_balanced(const int32_t* topk_ids, const int32_t* tokens_per_expert,
                      const int32_t* cu_seqlens, const int32_t* expanded_to_permuted, int64_t N,
                      int E, int K, int R, int num_copies, int token_padding, int64_t capacity,
                      int64_t NvS, const mep_balanced_outputs* out, void* stream);

/*
 * mep_permute_rows -- one GPU's share of expert dispatch for hidden-state
 * rows ([DEEP] intranode dispatch: a token's row is copied to the slot of
 * every rank it is sent to; here the slots are the layout's permuted rows).
 *   x_permuted[expanded_to_permuted[t*K+k]] = x[t]   for every t, k
 *   x_permuted[start .. start+len) = 0 for every zero_fill[e] = (start, len)
 * Rows of [0, permuted_rows) covered by neither are not written (with the
 * layout's own zero_fill, every row of [0, cu_seqlens[E]) is covered).
 *
 * Arguments
 *   x                  device [N, H] rows of `dtype` (MEP_F32 or MEP_BF16; the
 *                      bytes are copied unchanged), 16-byte aligned
 *   H                  elements per row; H * sizeof(element) % 16 == 0
 *   K                  1 .. 32, N*K <= INT32_MAX
 *   expanded_to_permuted device int32[N*K] (from mep_build_layout); an entry
 *                      outside [0, permuted_rows) is skipped
 *   zero_fill, E       device int32[E,2] padding ranges (nullable; from
 *                      mep_build_layout), E >= 1 when given; a range that
 *                      leaves [0, permuted_rows) is skipped
 *   x_permuted         device [permuted_rows, H], 16-byte aligned
 *   permuted_rows      rows of x_permuted, <= INT32_MAX
 */
int mep_permute_rows(const void* x, int dtype, int64_t N, int64_t H, int K,
                     const int32_t* expanded_to_permuted, const int32_t* zero_fill, int E,
                     void* x_permuted, int64_t permuted_rows, void* stream);

/*
 * mep_combine_rows -- one GPU's share of expert combine ([DEEP] intranode
 * combine: a token's received rows are summed in fp32 and cast back to the
 * row type), with optional routing weights.
 *   acc = 0.0f; for k = 0 .. K-1 in order:
 *     acc = acc + w[t*K+k] * y[expanded_to_permuted[t*K+k]]   (with weights)
 *     acc = acc + y[expanded_to_permuted[t*K+k]]              (without)
 *   each step one binary32 multiply and one binary32 add, no fused
 *   multiply-add; out[t] = acc cast to the row type (bf16: round to nearest,
 *   ties to even, NaN kept quiet).
 *
 * Arguments
 *   y_permuted         device [permuted_rows, H] rows of `dtype`, 16-byte
 *                      aligned
 *   topk_weights       device float[N*K] (nullable: plain sum)
 *   out                device [N, H] rows of `dtype`, 16-byte aligned
 *   others             as mep_permute_rows; an index outside
 *                      [0, permuted_rows) drops its term
 */
int mep_combine_rows(const void* y_permuted, int dtype, int64_t N, int64_t H, int K,
                     const int32_t* expanded_to_permuted, const float* topk_weights,
                     int64_t permuted_rows, void* out, void* stream);

/*
 * mep_route_layout_plan -- mep_route_topk, then mep_layout_plan, in one call,
 * with the arguments, checks and results of the two (topk_ids is the
 * routing's output and the layout's input, so it is required).
 *
 * Small batches run as a single kernel of one workgroup ([TRT]
 * routingPermutation: a small batch's whole routing permutation without a
 * second launch): N*K <= 2048, E <= 256, K <= 8, R <= 8,
 * num_src*E <= 4096 and num_src*R*num_channels <= 4096.  That kernel routes
 * every token exactly (no fast-path certification to fail), keeps ids and
 * permuted positions in LDS, and uses no workspace.  Larger batches: where
 * mep_layout_plan takes two kernels (K <= 8, R <= 32, E <= 512) and the
 * sigmoid routing kernel covers the shape (E = 64, 128, 256 or 512, one
 * group of 32 experts per lane or no group limit), the routing kernel also
 * counts the plan tiles it routes, so the whole path is two kernels; else the
 * routing kernel is followed by mep_layout_plan's kernels.  Either way the
 * outputs equal those of mep_route_topk followed by mep_layout_plan; `ws` must
 * satisfy mep_layout_plan's rules in both cases.
 */
int mep_route_layout_plan(const void* logits, int dtype, int64_t N, int E, int K,
                          const float* bias, const mep_route_params* p, int32_t* topk_ids,
                          float* topk_weights, int alignment, int32_t* tokens_per_expert,
                          int32_t* cu_seqlens, int32_t* expanded_to_permuted,
                          int32_t* permuted_to_expanded, int64_t permuted_cap, int32_t* zero_fill,
                          int R, int num_src, int num_channels, int64_t NvS,
                          const mep_plan_outputs* out, void* ws, size_t ws_bytes, void* stream);

/*
 * mep_route_layout_plan_timed -- mep_route_layout_plan with kernel timing.
 *
 * Computes exactly what mep_route_layout_plan computes (same arguments, checks
 * and errors).  The four events (hipEvent_t created by the caller, each may be
 * NULL) are updated by kernel launches themselves (hipExtLaunchKernel), with no
 * marker packet on the stream: route_start / route_stop with the start and end
 * of the routing kernel (of the single kernel of a small batch), plan_start /
 * plan_stop with those of the plan-tile kernel of the fused path (left
 * untouched by small batches and by shapes outside the fused path).  For
 * measuring the kernels in place inside a stream of work.
 */
int mep_route_layout_plan_timed(const void* logits, int dtype, int64_t N, int E, int K,
                                const float* bias, const mep_route_params* p, int32_t* topk_ids,
                                float* topk_weights, int alignment, int32_t* tokens_per_expert,
                                int32_t* cu_seqlens, int32_t* expanded_to_permuted,
                                int32_t* permuted_to_expanded, int64_t permuted_cap, int32_t* zero_fill,
                                int R, int num_src, int num_channels, int64_t NvS,
                                const mep_plan_outputs* out, void* ws, size_t ws_bytes, void* stream,
                                void* route_start, void* route_stop, void* plan_start, void* plan_stop);

/*
 * mep_route_layout_plan_noalloc -- mep_route_layout_plan without a caller
 * workspace and without any allocation, for callers that cannot allocate:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.
 *
 * Same arguments (less ws / ws_bytes), checks, results and kernels as
 * mep_route_layout_plan.  The workspace is a device array of 8 MiB per GPU
 * inside the library (held by each GPU the library runs on until the process
 * ends); the first call on a device clears it with a small kernel on `stream`
 * and every call leaves it ready for the next.  Returns MEP_ERR_CAPACITY when
 * mep_plan_workspace_size(N, E, K, R, num_src) exceeds 8 MiB (nothing is
 * enqueued then), MEP_ERR_DEVICE when the array's address cannot be obtained.
 * Calls on one GPU share the array: calls that overlap on one GPU (two streams,
 * two host threads) race and must be ordered by the caller.
 */
int mep_route_layout_plan_noalloc(const void* logits, int dtype, int64_t N, int E, int K,
                                  const float* bias, const mep_route_params* p, int32_t* topk_ids,
                                  float* topk_weights, int alignment, int32_t* tokens_per_expert,
                                  int32_t* cu_seqlens, int32_t* expanded_to_permuted,
                                  int32_t* permuted_to_expanded, int64_t permuted_cap,
                                  int32_t* zero_fill, int R, int num_src, int num_channels,
                                  int64_t NvS, const mep_plan_outputs* out, void* stream);

/*
 * mep_sigmoid_eval -- the sigmoid evaluations the routing kernels use, applied
 * element-wise, for verifying them over every binary32 input (not a step of
 * the path).  The real function is the logistic sigmoid 1/(1+exp(-x)) of
 * [TRT] RoutingKernel.cuh (sigmoid_accurate), the scoring function of
 * sigmoid routing.
 *
 * x:          device, n binary32 inputs (4-byte aligned).
 * cr_out:     device, n binary32 (or NULL): sigma(x) correctly rounded to
 *             binary32 (round to nearest even, subnormals kept) -- the value
 *             every exact selection key is formed from.
 * filter_out: device, n binary32 (or NULL): the binary32 filter value
 *             rcp(1 + exp2(-x * log2 e)) of the certified fast selection.
 * weight_out: device, n binary64 (or NULL, 8-byte aligned): the binary64
 *             sigmoid the routing weights are computed from.
 * Returns MEP_ERR_INVALID_ARG for n < 0, a NULL x with n > 0, or a misaligned
 * pointer; MEP_OK with nothing enqueued for n == 0 or no output.
 */
int mep_sigmoid_eval(const float* x, int64_t n, float* cr_out, float* filter_out, double* weight_out,
                     void* stream);

/* Static, NUL-terminated name of a return code. */
const char* mep_status_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* MEP_H_ */
