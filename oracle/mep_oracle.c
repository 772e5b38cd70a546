/*
 * mep_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded CPU oracle for MoE routing, dispatch layout,
 * expert-parallel planning (plain, and with capacity rebalancing),
 * grouped-GEMM tile maps and the local permute / combine of hidden-state
 * rows.  Only tests, the smoke check and the CPU
 * baseline leg of the benchmark may load it; the product path never does.
 * It shares no code, header, table or constant with the HIP library.
 *
 * Every stage is written as the most direct reading of its definition:
 * nested loops, fp64 arithmetic for weights, repeated extraction for top-K,
 * a token-ordered walk for the stable permutation.  Nothing is blocked,
 * fused or reordered.
 *
 * Sources (web pages; cited by page title and section):
 *   [TRT]   TensorRT-LLM RoutingKernel.cuh (blockScaleMoe routing)
 *   [MOON]  MoonEP planning.py (PlanningKernel)
 *   [DEEP]  DeepEP intranode.cu (notify_dispatch)
 *
 * Readings taken where the pages are silent are listed next to the code
 * that takes them.  Parity status: every function here is pinned by the
 * CPU tests (brute force, exact-arithmetic sigmoid, closed forms,
 * stable-sort equivalence, plan invariants, row-by-row tile enumeration,
 * exact permute/combine round trips and sums, bf16 rounding against torch,
 * hand-worked rebalancing cases and the no-move reduction to the plain plan);
 * none is "parity unpinned".
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC
 *        mep_oracle.c -lquadmath -lm
 */
#include <math.h>
#include <quadmath.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_ERR_ARG 1
#define OR_ERR_CAP 3

/* ------------------------------------------------------------------ */
/* Scalar helpers                                                     */
/* ------------------------------------------------------------------ */

/* bfloat16 holds the upper 16 bits of a binary32 value, so widening is a
 * shift (exact). */
static float bf16_to_float(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static float logit_at(const void* logits, int dtype, int64_t i) {
    if (dtype == 0) return ((const float*)logits)[i];
    return bf16_to_float(((const uint16_t*)logits)[i]);
}

/* Which path decided the last sigmoid on this thread: 1 = double, 2 = quad.  For tests.
 * Thread-local, so routing calls on separate token ranges may run in parallel threads. */
static _Thread_local int g_sigmoid_path = 0;

/*
 * Logistic sigmoid 1/(1+exp(-x)), correctly rounded to binary32.
 * [TRT] sigmoid_accurate defines the same real function through tanh; the
 * page does not fix its rounding, so the oracle pins it as the correctly
 * rounded value (round to nearest, ties to even, subnormals kept).
 *
 * Ziv's strategy: evaluate in double, widen by an error bound far above
 * the true one, and accept if both ends of the interval round to the same
 * float.  Otherwise evaluate in binary128 (libquadmath) with a much
 * tighter interval.  If even that is ambiguous the oracle aborts loudly.
 */
float oracle_sigmoid(float x) {
    double xd = (double)x;
    double s = 1.0 / (1.0 + exp(-xd));
    /* glibc exp is within 1 ulp; the add and divide add 1 ulp: < 2^-51
     * relative.  2^-45 leaves a factor 64 of slack. */
    double err = s * 0x1p-45;
    float lo = (float)(s - err), hi = (float)(s + err);
    if (lo == hi) {
        g_sigmoid_path = 1;
        return lo;
    }
    __float128 xq = (__float128)x;
    __float128 sq = 1.0Q / (1.0Q + expq(-xq));
    __float128 errq = sq * 0x1p-100Q; /* expq is within ~1 ulp of 2^-112 */
    float loq = (float)(sq - errq), hiq = (float)(sq + errq);
    if (loq != hiq) {
        fprintf(stderr, "oracle_sigmoid: rounding undecided for x=%a\n", (double)x);
        abort();
    }
    g_sigmoid_path = 2;
    return loq;
}

int oracle_sigmoid_path(void) { return g_sigmoid_path; }

/* Batch form for tests. */
void oracle_sigmoid_batch(const float* x, int64_t n, float* out, int32_t* path) {
    for (int64_t i = 0; i < n; ++i) {
        out[i] = oracle_sigmoid(x[i]);
        if (path) path[i] = g_sigmoid_path;
    }
}

/* Order for top-K: a beats b iff key_a > key_b, or keys equal and
 * index_a < index_b.  Float comparison treats -0 and +0 as equal, so a
 * signed-zero pair is decided by index. */
static int beats(float ka, int ia, float kb, int ib) {
    if (ka > kb) return 1;
    if (ka < kb) return 0;
    return ia < ib;
}

/* ------------------------------------------------------------------ */
/* Routing                                                            */
/* ------------------------------------------------------------------ */

/*
 * Per token:
 *  1. keys.  Softmax scoring: key_e = logit_e (softmax is monotone, so the
 *     top-K of the probabilities is the top-K of the logits).  Sigmoid
 *     scoring: s_e = sigmoid(logit_e) correctly rounded, key_e = fl(s_e +
 *     bias_e) (bias steers selection only).
 *  2. group limit (n_group > 1): experts split into n_group contiguous
 *     groups; a group's score is the float sum, in descending order, of its
 *     group_topn largest keys; the topk_group best groups (score desc,
 *     group index asc) stay eligible.
 *  3. top-K among eligible experts by repeated extraction of the best
 *     remaining one (key desc, index asc); ids are written in that order.
 *  4. weights in fp64, rounded once to float:
 *       softmax, renormalize:  exp(x_k - x_1) / sum_{j in top-K} exp(x_j - x_1)
 *         -- [TRT] calcSoftmax over the NumTopExperts selected lanes;
 *            softmax-then-topK-then-renormalise is the same number.
 *       softmax, no renorm:   exp(x_k - M) / sum_{all e} exp(x_e - M), M = max
 *         -- [TRT] calcSoftmax over the full score vector.
 *       sigmoid, renormalize:  s_k / sum_{j in top-K} s_j  (0 if the sum is 0)
 *       sigmoid, no renorm:    s_k
 *     and every weight is then multiplied by `scale`.
 */
int oracle_route(const void* logits, int dtype, int64_t N, int E, int K,
                 const float* bias, int score_fn, int renormalize, int n_group,
                 int topk_group, int group_topn, float scale,
                 int32_t* topk_ids, float* topk_weights) {
    if (N < 0 || E <= 0 || K <= 0 || K > E) return OR_ERR_ARG;
    if (dtype != 0 && dtype != 1) return OR_ERR_ARG;
    if (score_fn != 0 && score_fn != 1) return OR_ERR_ARG;
    if (n_group < 1 || E % n_group != 0) return OR_ERR_ARG;
    int gsize = E / n_group;
    if (n_group > 1) {
        if (topk_group < 1 || topk_group > n_group) return OR_ERR_ARG;
        if (group_topn < 1 || group_topn > gsize) return OR_ERR_ARG;
        if ((int64_t)topk_group * gsize < K) return OR_ERR_ARG;
    }

    float* x = (float*)malloc(sizeof(float) * E);   /* logits as float */
    float* s = (float*)malloc(sizeof(float) * E);   /* sigmoid values */
    float* key = (float*)malloc(sizeof(float) * E);
    int* eligible = (int*)malloc(sizeof(int) * E);
    int* taken = (int*)malloc(sizeof(int) * E);
    float* gscore = (float*)malloc(sizeof(float) * n_group);
    int* gkept = (int*)malloc(sizeof(int) * n_group);
    int* sel = (int*)malloc(sizeof(int) * K);

    for (int64_t t = 0; t < N; ++t) {
        /* 1. keys */
        for (int e = 0; e < E; ++e) {
            x[e] = logit_at(logits, dtype, t * E + e);
            if (score_fn == 1) {
                s[e] = oracle_sigmoid(x[e]);
                float b = bias ? bias[e] : 0.0f;
                key[e] = s[e] + b; /* one binary32 addition */
            } else {
                key[e] = x[e];
            }
        }
        /* 2. group limit */
        for (int e = 0; e < E; ++e) eligible[e] = 1;
        if (n_group > 1) {
            for (int g = 0; g < n_group; ++g) {
                /* sum the group_topn largest keys, largest first */
                for (int e = g * gsize; e < (g + 1) * gsize; ++e) taken[e] = 0;
                float sum = 0.0f;
                for (int j = 0; j < group_topn; ++j) {
                    int best = -1;
                    for (int e = g * gsize; e < (g + 1) * gsize; ++e) {
                        if (taken[e]) continue;
                        if (best < 0 || beats(key[e], e, key[best], best)) best = e;
                    }
                    taken[best] = 1;
                    sum = (j == 0) ? key[best] : sum + key[best];
                }
                gscore[g] = sum;
                gkept[g] = 0;
            }
            for (int j = 0; j < topk_group; ++j) {
                int best = -1;
                for (int g = 0; g < n_group; ++g) {
                    if (gkept[g]) continue;
                    if (best < 0 || beats(gscore[g], g, gscore[best], best)) best = g;
                }
                gkept[best] = 1;
            }
            for (int e = 0; e < E; ++e) eligible[e] = gkept[e / gsize];
        }
        /* 3. top-K by repeated extraction */
        for (int e = 0; e < E; ++e) taken[e] = 0;
        for (int k = 0; k < K; ++k) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (!eligible[e] || taken[e]) continue;
                if (best < 0 || beats(key[e], e, key[best], best)) best = e;
            }
            taken[best] = 1;
            sel[k] = best;
            topk_ids[t * K + k] = best;
        }
        /* 4. weights */
        if (topk_weights) {
            double den = 0.0;
            if (score_fn == 0) {
                double m;
                if (renormalize) {
                    m = (double)x[sel[0]];
                    for (int k = 0; k < K; ++k) den += exp((double)x[sel[k]] - m);
                } else {
                    m = (double)x[0];
                    for (int e = 1; e < E; ++e)
                        if ((double)x[e] > m) m = (double)x[e];
                    for (int e = 0; e < E; ++e) den += exp((double)x[e] - m);
                }
                for (int k = 0; k < K; ++k) {
                    double w = exp((double)x[sel[k]] - m) / den;
                    topk_weights[t * K + k] = (float)(w * (double)scale);
                }
            } else {
                if (renormalize) {
                    for (int k = 0; k < K; ++k) den += (double)s[sel[k]];
                }
                for (int k = 0; k < K; ++k) {
                    double w;
                    if (renormalize)
                        w = den > 0.0 ? (double)s[sel[k]] / den : 0.0;
                    else
                        w = (double)s[sel[k]];
                    topk_weights[t * K + k] = (float)(w * (double)scale);
                }
            }
        }
    }
    free(x); free(s); free(key); free(eligible); free(taken);
    free(gscore); free(gkept); free(sel);
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* Dispatch layout                                                    */
/* ------------------------------------------------------------------ */

/*
 * Padded per-expert layout of the N*K routed slots.
 *   count[e]   = number of flat slots i = t*K+k with ids[i] == e
 *                ([TRT] routingIndicesHistogramKernel, [MOON] run_c1 1a)
 *   padded[e]  = ceil(count/A)*A, 0 for an empty expert
 *                ([MOON] Phase B2 padded group scan; [DEEP] notify_dispatch
 *                 aligns the per-expert receive count the same way)
 *   cu[0] = 0, cu[e+1] = cu[e] + padded[e]
 *   Walking slots in flat order, slot i of expert e gets position
 *     P[i] = cu[e] + (number of earlier slots of expert e)
 *   which is the stable counting sort of [MOON] run_c1 passA; Inv[P[i]] = i
 *   and Inv = -1 on padding rows ([MOON] src_info empty-slot sentinel).
 *   zero_fill[e] = (cu[e]+count, padded-count) when count > 0 and the
 *   expert was padded, else (0, 0) ([MOON] Phase B2 zero-fill ranges).
 * Reading: cu has E+1 entries with the total last; the inverse holds the
 * flat slot index t*K+k (the token is Inv/K).
 */
int oracle_layout(const int32_t* ids, int64_t N, int E, int K, int A,
                  int32_t* tokens_per_expert, int32_t* cu_seqlens,
                  int32_t* expanded_to_permuted, int32_t* permuted_to_expanded,
                  int64_t permuted_cap, int32_t* zero_fill) {
    if (N < 0 || E <= 0 || K <= 0 || A <= 0) return OR_ERR_ARG;
    int64_t NK = N * (int64_t)K;
    int64_t* count = (int64_t*)calloc((size_t)E, sizeof(int64_t));
    int64_t* cu = (int64_t*)calloc((size_t)E + 1, sizeof(int64_t));
    int64_t* fill = (int64_t*)calloc((size_t)E, sizeof(int64_t));
    for (int64_t i = 0; i < NK; ++i) {
        int e = ids[i];
        if (e < 0 || e >= E) { free(count); free(cu); free(fill); return OR_ERR_ARG; }
        count[e] += 1;
    }
    cu[0] = 0;
    for (int e = 0; e < E; ++e) {
        int64_t padded = count[e] > 0 ? ((count[e] + A - 1) / A) * A : 0;
        cu[e + 1] = cu[e] + padded;
    }
    int64_t T = cu[E];
    if (permuted_to_expanded && permuted_cap < T) {
        free(count); free(cu); free(fill);
        return OR_ERR_CAP;
    }
    if (permuted_to_expanded)
        for (int64_t p = 0; p < T; ++p) permuted_to_expanded[p] = -1;
    for (int64_t i = 0; i < NK; ++i) {
        int e = ids[i];
        int64_t p = cu[e] + fill[e];
        fill[e] += 1;
        expanded_to_permuted[i] = (int32_t)p;
        if (permuted_to_expanded) permuted_to_expanded[p] = (int32_t)i;
    }
    for (int e = 0; e < E; ++e) {
        if (tokens_per_expert) tokens_per_expert[e] = (int32_t)count[e];
        if (zero_fill) {
            int64_t padded = cu[e + 1] - cu[e];
            if (count[e] > 0 && padded > count[e]) {
                zero_fill[2 * e] = (int32_t)(cu[e] + count[e]);
                zero_fill[2 * e + 1] = (int32_t)(padded - count[e]);
            } else {
                zero_fill[2 * e] = 0;
                zero_fill[2 * e + 1] = 0;
            }
        }
    }
    for (int e = 0; e <= E; ++e) cu_seqlens[e] = (int32_t)cu[e];
    free(count); free(cu); free(fill);
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* Expert-parallel plan over R virtual ranks                          */
/* ------------------------------------------------------------------ */

/*
 * Experts are split contiguously over R ranks: owner(e) = e / epn,
 * epn = E / R.  The token batch is the concatenation of S equal shards
 * (virtual source ranks), shard s = tokens [s*n, (s+1)*n), n = N / S.
 *
 *   is_token_in_rank[t][r] = 1 iff some k has owner(ids[t][k]) == r
 *   num_tokens_per_rank[s][r]   = sum over t in shard s of itr[t][r]
 *   num_tokens_per_expert[s][e] = number of t in shard s routed to e
 *   rank_prefix_matrix[s][r]    = sum_{s' <= s} num_tokens_per_rank[s'][r]
 *        ([DEEP] notify_dispatch: column prefix over source ranks)
 *   recv_tokens[r] = rank_prefix_matrix[S-1][r]   ([DEEP] moe_recv_counter)
 *   channel c of shard s: tokens s*n + [min(c*q, n), min((c+1)*q, n)),
 *        q = ceil(n / C)  (reading: contiguous equal chunks, trailing ones
 *        may be empty -- the channel task range is not on the pages)
 *   channel_prefix_matrix[s][r][c] = sum_{c' <= c} (tokens of channel c'
 *        of shard s with itr[t][r])  ([DEEP] notify_dispatch channel part)
 *   recv_cu_seqlens[r][j] = cu[r*epn + j] - cu[r*epn], j = 0..epn
 *   recv_zero_fill[e] = zero-fill range of e made rank-local: (cu[e] +
 *        count[e] - cu[owner*epn], padded - count) when count > 0 and the
 *        expert was padded, else (0, 0)
 *   dst[i] for slot i = t*K+k with expert e, owner r:
 *        raw = r*NvS + (P[i] - cu[r*epn])   (rank-local slot, rank stride)
 *        the first k of token t that lands on rank r keeps raw; every later
 *        k of the same token on the same rank stores -raw-1
 *        ([MOON] dst computation without capacity moves, and its duplicate
 *         canonicalisation)
 *   dedup (the builder is not on the pages; this oracle defines it):
 *        for each rank r, for each token t ascending whose slots hit r at
 *        least twice: one group (primary_loff, dup_begin, dup_count) where
 *        primary_loff is the rank-local slot of the first such k,
 *        dup_count = (hits - 1), and the dup_count later slots' rank-local
 *        offsets are appended, in k order, to r's dup_loffs segment;
 *        dup_begin is the segment-relative index of the first of them.
 *        dup_counts[r] = (groups of r, dups of r); dup_offsets[r] is the
 *        exclusive prefix of dup_counts over r (row R holds the totals);
 *        groups of rank r sit at dup_groups[dup_offsets[r][0] + j], their
 *        dup offsets at dup_loffs[dup_offsets[r][1] + dup_begin + j].
 * All outputs may be NULL (skipped).
 */
int oracle_plan(const int32_t* ids, const int32_t* cu_seqlens,
                const int32_t* expanded_to_permuted, int64_t N, int E, int K,
                int R, int S, int C, int64_t NvS,
                uint8_t* is_token_in_rank, int32_t* num_tokens_per_rank,
                int32_t* num_tokens_per_expert, int32_t* rank_prefix_matrix,
                int32_t* channel_prefix_matrix, int32_t* recv_tokens,
                int32_t* recv_cu_seqlens, int32_t* recv_zero_fill, int32_t* dst,
                int32_t* dup_counts, int32_t* dup_offsets,
                int32_t* dup_groups, int64_t cap_g,
                int32_t* dup_loffs, int64_t cap_d) {
    if (N < 0 || E <= 0 || K <= 0 || R <= 0 || S <= 0 || C <= 0) return OR_ERR_ARG;
    if (E % R != 0 || N % S != 0) return OR_ERR_ARG;
    int epn = E / R;
    int64_t n = N / S;
    int64_t q = (n + C - 1) / C;

    /* itr and per-shard counts */
    uint8_t* itr = (uint8_t*)calloc((size_t)(N * R > 0 ? N * R : 1), 1);
    for (int64_t t = 0; t < N; ++t)
        for (int k = 0; k < K; ++k) itr[t * R + ids[t * K + k] / epn] = 1;
    if (is_token_in_rank) memcpy(is_token_in_rank, itr, (size_t)(N * R));

    int64_t* ntpr = (int64_t*)calloc((size_t)S * R, sizeof(int64_t));
    int64_t* ntpe = (int64_t*)calloc((size_t)S * E, sizeof(int64_t));
    for (int64_t t = 0; t < N; ++t) {
        int64_t s = t / n;
        for (int r = 0; r < R; ++r) ntpr[s * R + r] += itr[t * R + r];
        for (int k = 0; k < K; ++k) ntpe[s * E + ids[t * K + k]] += 1;
    }
    for (int64_t s = 0; s < S; ++s) {
        for (int r = 0; r < R; ++r) {
            if (num_tokens_per_rank) num_tokens_per_rank[s * R + r] = (int32_t)ntpr[s * R + r];
            int64_t pre = 0;
            for (int64_t s2 = 0; s2 <= s; ++s2) pre += ntpr[s2 * R + r];
            if (rank_prefix_matrix) rank_prefix_matrix[s * R + r] = (int32_t)pre;
            if (recv_tokens && s == S - 1) recv_tokens[r] = (int32_t)pre;
        }
        for (int e = 0; e < E; ++e)
            if (num_tokens_per_expert) num_tokens_per_expert[s * E + e] = (int32_t)ntpe[s * E + e];
    }
    /* channel prefix */
    if (channel_prefix_matrix) {
        for (int64_t s = 0; s < S; ++s)
            for (int r = 0; r < R; ++r) {
                int64_t run = 0;
                for (int c = 0; c < C; ++c) {
                    int64_t b = c * q < n ? c * q : n;
                    int64_t e_ = (c + 1) * q < n ? (c + 1) * q : n;
                    for (int64_t t = s * n + b; t < s * n + e_; ++t) run += itr[t * R + r];
                    channel_prefix_matrix[(s * R + r) * C + c] = (int32_t)run;
                }
            }
    }
    /* receive layout */
    if (recv_cu_seqlens)
        for (int r = 0; r < R; ++r)
            for (int j = 0; j <= epn; ++j)
                recv_cu_seqlens[r * (epn + 1) + j] = cu_seqlens[r * epn + j] - cu_seqlens[r * epn];
    if (recv_zero_fill) {
        for (int e = 0; e < E; ++e) {
            int64_t cnt = 0;
            for (int64_t s = 0; s < S; ++s) cnt += ntpe[s * E + e];
            int64_t padded = (int64_t)cu_seqlens[e + 1] - cu_seqlens[e];
            int r = e / epn;
            if (cnt > 0 && padded > cnt) {
                recv_zero_fill[2 * e] = (int32_t)(cu_seqlens[e] + cnt - cu_seqlens[r * epn]);
                recv_zero_fill[2 * e + 1] = (int32_t)(padded - cnt);
            } else {
                recv_zero_fill[2 * e] = 0;
                recv_zero_fill[2 * e + 1] = 0;
            }
        }
    }
    /* dst with duplicate encoding */
    if (dst) {
        for (int64_t t = 0; t < N; ++t)
            for (int k = 0; k < K; ++k) {
                int64_t i = t * K + k;
                int r = ids[i] / epn;
                int64_t raw = (int64_t)r * NvS + (expanded_to_permuted[i] - cu_seqlens[r * epn]);
                int earlier = 0;
                for (int k2 = 0; k2 < k; ++k2)
                    if (ids[t * K + k2] / epn == r) earlier = 1;
                dst[i] = (int32_t)(earlier ? -raw - 1 : raw);
            }
    }
    /* dedup */
    int64_t* ng = (int64_t*)calloc((size_t)R, sizeof(int64_t));
    int64_t* nd = (int64_t*)calloc((size_t)R, sizeof(int64_t));
    for (int64_t t = 0; t < N; ++t)
        for (int r = 0; r < R; ++r) {
            int hits = 0;
            for (int k = 0; k < K; ++k) hits += (ids[t * K + k] / epn == r);
            if (hits >= 2) { ng[r] += 1; nd[r] += hits - 1; }
        }
    int64_t gtot = 0, dtot = 0;
    for (int r = 0; r < R; ++r) {
        if (dup_counts) { dup_counts[2 * r] = (int32_t)ng[r]; dup_counts[2 * r + 1] = (int32_t)nd[r]; }
        if (dup_offsets) { dup_offsets[2 * r] = (int32_t)gtot; dup_offsets[2 * r + 1] = (int32_t)dtot; }
        gtot += ng[r];
        dtot += nd[r];
    }
    if (dup_offsets) { dup_offsets[2 * R] = (int32_t)gtot; dup_offsets[2 * R + 1] = (int32_t)dtot; }
    int rc = OR_OK;
    if ((dup_groups && cap_g < gtot) || (dup_loffs && cap_d < dtot)) rc = OR_ERR_CAP;
    if (rc == OR_OK && (dup_groups || dup_loffs)) {
        int64_t gpos = 0, dpos = 0;
        for (int r = 0; r < R; ++r) {
            int64_t dseg = dpos; /* start of r's dup_loffs segment */
            for (int64_t t = 0; t < N; ++t) {
                int hits = 0;
                for (int k = 0; k < K; ++k) hits += (ids[t * K + k] / epn == r);
                if (hits < 2) continue;
                int first = 1;
                int64_t begin = dpos - dseg;
                for (int k = 0; k < K; ++k) {
                    int64_t i = t * K + k;
                    if (ids[i] / epn != r) continue;
                    int32_t loff = expanded_to_permuted[i] - cu_seqlens[r * epn];
                    if (first) {
                        if (dup_groups) {
                            dup_groups[3 * gpos + 0] = loff;
                            dup_groups[3 * gpos + 1] = (int32_t)begin;
                            dup_groups[3 * gpos + 2] = hits - 1;
                        }
                        first = 0;
                    } else {
                        if (dup_loffs) dup_loffs[dpos] = loff;
                        dpos += 1;
                    }
                }
                gpos += 1;
            }
        }
    }
    free(itr); free(ntpr); free(ntpe); free(ng); free(nd);
    return rc;
}

/*
 * Grouped-GEMM tile maps, [TRT] routingPermutation / routingIndicesOffsetsKernel
 * (the per-expert CTA bookkeeping that follows the histogram).
 *   per expert e with count c_e: numCta_e = ceil(c_e / A) tiles of A rows;
 *   ctaOffset_e = exclusive prefix sum of numCta over experts, and the total
 *   (numNonExitingCtas) is the sum over all experts;
 *   for every tile index cta in [0, numCta_e), at position ctaOffset_e + cta:
 *     cta_to_expert = e   (the index of e within `counts`)
 *     mn_limit      = min((ctaOffset_e + cta + 1) * A, ctaOffset_e * A + c_e)
 *   permuted_idx_size = numNonExitingCtas * A.
 * Entries at and beyond the total are left untouched.  A negative count is
 * an argument error; a total above cap is OR_ERR_CAP with nothing written.
 * Pinned by the tile-map tests in test_oracle_pins.py.
 */
int oracle_tile_map(const int32_t* counts, int E, int A, int32_t* cta_to_expert,
                    int32_t* mn_limit, int64_t cap, int32_t* permuted_idx_size,
                    int32_t* num_ctas) {
    if (E <= 0 || A <= 0 || cap < 0) return OR_ERR_ARG;
    for (int e = 0; e < E; ++e)
        if (counts[e] < 0) return OR_ERR_ARG;
    int64_t* num_cta = (int64_t*)calloc((size_t)E, sizeof(int64_t));
    int64_t* cta_offset = (int64_t*)calloc((size_t)E, sizeof(int64_t));
    /* step 1: tiles per expert */
    for (int e = 0; e < E; ++e) num_cta[e] = ((int64_t)counts[e] + A - 1) / A;
    /* step 2: exclusive sum and its total */
    int64_t total = 0;
    for (int e = 0; e < E; ++e) {
        cta_offset[e] = total;
        total += num_cta[e];
    }
    if (total > cap) {
        free(num_cta);
        free(cta_offset);
        return OR_ERR_CAP;
    }
    /* step 3: each expert fills its own tiles */
    for (int e = 0; e < E; ++e)
        for (int64_t cta = 0; cta < num_cta[e]; ++cta) {
            int64_t lim1 = (cta_offset[e] + cta + 1) * (int64_t)A;
            int64_t lim2 = cta_offset[e] * (int64_t)A + counts[e];
            if (cta_to_expert) cta_to_expert[cta_offset[e] + cta] = e;
            if (mn_limit) mn_limit[cta_offset[e] + cta] = (int32_t)(lim1 < lim2 ? lim1 : lim2);
        }
    /* step 4: the two scalars */
    if (permuted_idx_size) *permuted_idx_size = (int32_t)(total * A);
    if (num_ctas) *num_ctas = (int32_t)total;
    free(num_cta);
    free(cta_offset);
    return OR_OK;
}

/*
 * Local permute and combine of hidden-state rows: one GPU's share of
 * [DEEP] intranode dispatch (each token's row copied to the slot of every
 * rank it goes to) and combine (a token's received rows summed in fp32 in
 * order, then cast back to the row type).  Here the destinations are the
 * permuted rows of the layout instead of per-rank channel buffers.
 *   permute:  out[expanded_to_permuted[t*K+k]] = x[t]  for every t, k;
 *             the zero-fill range (start, len) of every expert is set to 0.
 *   combine:  out[t] = cast(acc), acc = 0.0f then, for k = 0 .. K-1 in
 *             order, acc = acc + w[t*K+k] * y[expanded_to_permuted[t*K+k]]
 *             (or acc + y[...] when w is NULL), each step one binary32
 *             multiply and one binary32 add.
 * dtype 0 = fp32 rows, 1 = bf16 rows; H = elements per row.  The cast to
 * bf16 rounds to nearest, ties to even; a NaN stays a (quiet) NaN.
 */
static uint16_t bf16_round_nearest_even(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u); /* NaN: keep sign, force quiet */
    uint32_t upper = u >> 16;
    uint32_t lower = u & 0xffffu;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1; /* carries into exponent */
    return (uint16_t)upper;
}

static float row_value(const void* rows, int dtype, int64_t idx) {
    if (dtype == 0) return ((const float*)rows)[idx];
    uint32_t u = (uint32_t)((const uint16_t*)rows)[idx] << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

int oracle_permute_rows(const void* x, int dtype, int64_t N, int64_t H, int K,
                        const int32_t* expanded_to_permuted, const int32_t* zero_fill, int E,
                        void* out, int64_t T) {
    if (N < 0 || H <= 0 || K <= 0 || E <= 0 || T < 0) return OR_ERR_ARG;
    if (dtype != 0 && dtype != 1) return OR_ERR_ARG;
    size_t row = (size_t)H * (dtype == 0 ? 4 : 2);
    for (int64_t t = 0; t < N; ++t)
        for (int k = 0; k < K; ++k) {
            int64_t p = expanded_to_permuted[t * K + k];
            if (p < 0 || p >= T) return OR_ERR_ARG;
            memcpy((char*)out + (size_t)p * row, (const char*)x + (size_t)t * row, row);
        }
    if (zero_fill)
        for (int e = 0; e < E; ++e) {
            int64_t start = zero_fill[2 * e], len = zero_fill[2 * e + 1];
            if (len == 0) continue;
            if (start < 0 || start + len > T) return OR_ERR_ARG;
            memset((char*)out + (size_t)start * row, 0, (size_t)len * row);
        }
    return OR_OK;
}

int oracle_combine_rows(const void* y, int dtype, int64_t N, int64_t H, int K,
                        const int32_t* expanded_to_permuted, const float* topk_weights,
                        void* out, int64_t T) {
    if (N < 0 || H <= 0 || K <= 0 || T < 0) return OR_ERR_ARG;
    if (dtype != 0 && dtype != 1) return OR_ERR_ARG;
    for (int64_t t = 0; t < N; ++t)
        for (int k = 0; k < K; ++k) {
            int64_t p = expanded_to_permuted[t * K + k];
            if (p < 0 || p >= T) return OR_ERR_ARG;
        }
    for (int64_t t = 0; t < N; ++t)
        for (int64_t h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) {
                int64_t p = expanded_to_permuted[t * K + k];
                float v = row_value(y, dtype, p * H + h);
                if (topk_weights) {
                    float prod = topk_weights[t * K + k] * v;
                    acc = acc + prod;
                } else {
                    acc = acc + v;
                }
            }
            if (dtype == 0) ((float*)out)[t * H + h] = acc;
            else ((uint16_t*)out)[t * H + h] = bf16_round_nearest_even(acc);
        }
    return OR_OK;
}

/*
 * Capacity rebalancing with redundant remote experts: [MOON] PlanningKernel
 * phases after the gather of per-rank expert counts (the balancing loop,
 * the per-owner quota allocation, the per-destination choice of experts to
 * copy with its padded group scan, and the dst search), run for all R
 * ranks at once.  The N*K slots of the batch play every source rank in
 * turn: a slot's position among the slots of its expert (source-then-token
 * order, i.e. global slot order) is expanded_to_permuted - cu_seqlens[e].
 *
 *   total[e] = tokens_per_expert[e]; group_tokens[r] = sum of total over
 *     r's experts (owner(e) = e / epn).
 *   balance[r] = group_tokens[r] - CAP.  Repeat: the largest balance
 *     (lowest rank on ties) is the surplus, the smallest (lowest rank on
 *     ties) the deficit; stop when surplus <= 0 or deficit >= 0; otherwise
 *     move = -deficit (the deficit rank is refilled to CAP in one move even
 *     if that takes the surplus rank below CAP), z[surplus][deficit] = move,
 *     balance[surplus] -= move, balance[deficit] = 0.
 *   For every owner o: remaining[j] = total of o's j-th expert,
 *     quota[r] = z[o][r].  Repeat: the largest quota (lowest rank on ties);
 *     stop if <= 0; the largest remaining (lowest index on ties); stop if
 *     <= 0; take = min of the two; alloc[target][that expert] += take, both
 *     are reduced by take.  What is left stays at o.
 *   alloc_cumsum[e][r] = sum_{r' <= r} alloc[r'][e].
 *   For every destination d: counts[e] = alloc[d][e]; the remote ones
 *     (owner != d) with a count > 0 are counted in remote_stats[d][0]; B
 *     times the largest remote count is picked (highest index on ties) and
 *     cleared: experts_to_copy[d][slot] = that expert, or -1 when the
 *     largest is 0; each pick adds one to remote_stats[owner][1].
 *     E + B groups: group g < E holds expert g with counts[g] unless g was
 *     picked (then 0); group E + slot holds the picked expert's count.
 *     padded = round_up(count, tp) (tp <= 1: count).  An exclusive scan of
 *     padded gives each group's start; cu_seqlens[d][g] = its end;
 *     expert_offsets[d][expert] = its start when its count > 0 (else -1 here);
 *     zero_fill[d][g] = (start + count, padded - count) when count > 0 and
 *     padded > count, else (0, 0).
 *   dst of slot i with expert e and global position q: lo = the first rank
 *     with alloc_cumsum[e][lo] > q (binary search), pc = alloc_cumsum[e][lo-1]
 *     (0 for lo = 0); dst = lo*NvS + expert_offsets[lo][e] + (q - pc).  Then
 *     each token's later slots whose rank (dst / NvS) repeats an earlier
 *     slot's store -dst - 1.
 * Returns OR_ERR_ARG on bad sizes or a layout that does not match the
 * counts.  All outputs are required.
 */
static int beats_max_low(int64_t a, int ia, int64_t b, int ib) { return a > b || (a == b && ia < ib); }
static int beats_min_low(int64_t a, int ia, int64_t b, int ib) { return a < b || (a == b && ia < ib); }
static int beats_max_high(int64_t a, int ia, int64_t b, int ib) { return a > b || (a == b && ia > ib); }

int oracle_plan_balanced(const int32_t* ids, const int32_t* tokens_per_expert,
                         const int32_t* cu_seqlens, const int32_t* expanded_to_permuted,
                         int64_t N, int E, int K, int R, int B, int tp, int64_t CAP,
                         int64_t NvS, int32_t* group_tokens, int32_t* z, int32_t* alloc,
                         int32_t* alloc_cumsum, int32_t* experts_to_copy,
                         int32_t* remote_stats, int32_t* cu_out, int32_t* zero_fill,
                         int32_t* expert_offsets, int32_t* dst) {
    if (N < 0 || E <= 0 || K <= 0 || R <= 0 || B < 0 || CAP < 0 || NvS <= 0) return OR_ERR_ARG;
    if (E % R != 0) return OR_ERR_ARG;
    int epn = E / R;
    int G = E + B;
    int64_t* bal = (int64_t*)calloc((size_t)R, sizeof(int64_t));
    int64_t* counts = (int64_t*)calloc((size_t)E, sizeof(int64_t));
    int64_t* remote = (int64_t*)calloc((size_t)E, sizeof(int64_t));
    int* picked = (int*)calloc((size_t)E, sizeof(int));
    int* slot_expert = (int*)calloc((size_t)(B > 0 ? B : 1), sizeof(int));

    /* group totals */
    for (int r = 0; r < R; ++r) {
        int64_t s = 0;
        for (int j = 0; j < epn; ++j) s += tokens_per_expert[r * epn + j];
        group_tokens[r] = (int32_t)s;
    }
    /* balancing loop */
    for (int i = 0; i < R * R; ++i) z[i] = 0;
    for (int r = 0; r < R; ++r) bal[r] = (int64_t)group_tokens[r] - CAP;
    for (;;) {
        int sr = 0, dr = 0;
        for (int r = 1; r < R; ++r) {
            if (beats_max_low(bal[r], r, bal[sr], sr)) sr = r;
            if (beats_min_low(bal[r], r, bal[dr], dr)) dr = r;
        }
        if (bal[sr] <= 0 || bal[dr] >= 0) break;
        int64_t move = -bal[dr];
        bal[sr] -= move;
        bal[dr] = 0;
        z[sr * R + dr] = (int32_t)move;
    }
    /* quota allocation per owner */
    for (int i = 0; i < R * E; ++i) alloc[i] = 0;
    for (int o = 0; o < R; ++o) {
        int64_t* quota = (int64_t*)calloc((size_t)R, sizeof(int64_t));
        int64_t* rem = (int64_t*)calloc((size_t)epn, sizeof(int64_t));
        for (int r = 0; r < R; ++r) quota[r] = z[o * R + r];
        for (int j = 0; j < epn; ++j) rem[j] = tokens_per_expert[o * epn + j];
        for (;;) {
            int tr = 0;
            for (int r = 1; r < R; ++r)
                if (beats_max_low(quota[r], r, quota[tr], tr)) tr = r;
            if (quota[tr] <= 0) break;
            int sj = 0;
            for (int j = 1; j < epn; ++j)
                if (beats_max_low(rem[j], j, rem[sj], sj)) sj = j;
            if (rem[sj] <= 0) break;
            int64_t take = rem[sj] < quota[tr] ? rem[sj] : quota[tr];
            quota[tr] -= take;
            rem[sj] -= take;
            alloc[tr * E + o * epn + sj] += (int32_t)take;
        }
        for (int j = 0; j < epn; ++j) alloc[o * E + o * epn + j] += (int32_t)rem[j];
        free(quota);
        free(rem);
    }
    for (int e = 0; e < E; ++e) {
        int64_t run = 0;
        for (int r = 0; r < R; ++r) {
            run += alloc[r * E + e];
            alloc_cumsum[e * R + r] = (int32_t)run;
        }
    }
    /* per destination: experts to copy, groups, offsets */
    for (int i = 0; i < 2 * R; ++i) remote_stats[i] = 0;
    for (int d = 0; d < R; ++d) {
        int nremote = 0;
        for (int e = 0; e < E; ++e) {
            counts[e] = alloc[d * E + e];
            remote[e] = (e / epn == d) ? 0 : counts[e];
            picked[e] = 0;
            if (remote[e] > 0) nremote += 1;
        }
        remote_stats[2 * d] = nremote;
        for (int b = 0; b < B; ++b) {
            int best = 0;
            for (int e = 1; e < E; ++e)
                if (beats_max_high(remote[e], e, remote[best], best)) best = e;
            int chosen = remote[best] > 0 ? best : -1;
            remote[best] = 0;
            slot_expert[b] = chosen;
            experts_to_copy[d * B + b] = chosen;
            if (chosen >= 0) {
                remote_stats[2 * (chosen / epn) + 1] += 1;
                picked[chosen] = 1;
            }
        }
        for (int e = 0; e < E; ++e) expert_offsets[d * E + e] = -1;
        int64_t base = 0;
        for (int g = 0; g < G; ++g) {
            int64_t cnt = 0;
            int ex = -1;
            if (g < E) {
                if (!picked[g]) { cnt = counts[g]; ex = g; }
            } else if (slot_expert[g - E] >= 0) {
                ex = slot_expert[g - E];
                cnt = counts[ex];
            }
            int64_t padded = 0;
            if (cnt > 0) padded = tp > 1 ? ((cnt + tp - 1) / tp) * tp : cnt;
            if (cnt > 0) expert_offsets[d * E + ex] = (int32_t)base;
            cu_out[(int64_t)d * G + g] = (int32_t)(base + padded);
            if (cnt > 0 && padded > cnt) {
                zero_fill[2 * ((int64_t)d * G + g)] = (int32_t)(base + cnt);
                zero_fill[2 * ((int64_t)d * G + g) + 1] = (int32_t)(padded - cnt);
            } else {
                zero_fill[2 * ((int64_t)d * G + g)] = 0;
                zero_fill[2 * ((int64_t)d * G + g) + 1] = 0;
            }
            base += padded;
        }
    }
    /* dst: binary search over the expert's cumulative allocation */
    int rc = OR_OK;
    for (int64_t i = 0; i < N * K; ++i) {
        int e = ids[i];
        int64_t q = (int64_t)expanded_to_permuted[i] - cu_seqlens[e];
        if (e < 0 || e >= E || q < 0 || q >= alloc_cumsum[e * R + R - 1]) {
            rc = OR_ERR_ARG; /* the layout does not match the counts */
            goto done;
        }
        int lo = 0, hi = R;
        int64_t pc = 0;
        while (lo < hi) {
            int mid = (lo + hi) / 2;
            int64_t ac = alloc_cumsum[e * R + mid];
            if (ac > q) hi = mid;
            else { lo = mid + 1; pc = ac; }
        }
        dst[i] = (int32_t)((int64_t)lo * NvS + expert_offsets[lo * E + e] + (q - pc));
    }
    /* duplicate canonicalisation per token */
    for (int64_t t = 0; t < N; ++t)
        for (int k = 0; k < K; ++k) {
            int64_t rk = dst[t * K + k] / NvS;
            int seen = 0;
            for (int k2 = 0; k2 < k; ++k2) {
                int64_t v = dst[t * K + k2];
                int64_t raw = v < 0 ? -v - 1 : v;
                if (raw / NvS == rk) seen = 1;
            }
            if (seen) dst[t * K + k] = -dst[t * K + k] - 1;
        }
done:
    free(bal);
    free(counts);
    free(remote);
    free(picked);
    free(slot_expert);
    return rc;
}
