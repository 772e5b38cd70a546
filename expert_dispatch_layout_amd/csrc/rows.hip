// mep_permute_rows / mep_combine_rows: one GPU's share of expert dispatch and combine for the
// hidden-state rows, on the layout's permuted rows instead of per-rank channel buffers
// (DeepEP intranode.cu: dispatch copies each token's row to the slot of every rank it goes to;
// combine sums a token's received rows in fp32 and casts back to the row type).
//
// Both kernels give one wave to one token, so the token's K destination (or source) rows are
// read once as scalars and every memory instruction moves 1 KiB of one row (64 lanes x 16 B,
// fully coalesced).
//   permute  loads a chunk of the token's row once and stores it to its K permuted rows
//            (nontemporal stores: the permuted copy is written once and is far larger than the
//            caches).  Chunks of 2 KiB per wave measured fastest among 1, 2, 4 and 8 KiB at
//            N = 65536, H = 7168 bf16.  The first E workgroups zero the experts' padding
//            ranges instead.
//   combine  issues the K loads of a chunk before summing them, so a wave keeps K x 16 B per
//            lane in flight per chunk (nontemporal loads: each permuted row is read exactly
//            once); terms are added in slot order, one binary32 multiply and one binary32 add
//            each (no fused multiply-add), then cast once.
// Row indices come from device arrays; one outside [0, permuted_rows) is skipped rather than
// dereferenced.
#include <hip/hip_runtime.h>
#include <limits.h>

#include "host_common.h"

namespace mep {

namespace {

constexpr int kRowWaves = 4;
constexpr int kRowBlock = 64 * kRowWaves;
constexpr int kRowChunk = 2;  // 16-byte vectors per lane per step: 2 KiB of a row per wave
constexpr int kRowMaxK = 32;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Zero the padding range of expert `e`: 16-byte stores, rows striped over the workgroup's waves.
__device__ __forceinline__ void zero_range(const int32_t* __restrict__ zero_fill, int e, int64_t T,
                                           int64_t vec_per_row, u32x4* __restrict__ out) {
    const int64_t start = zero_fill[2 * e];
    const int64_t len = zero_fill[2 * e + 1];
    if (len <= 0 || start < 0 || start + len > T) return;
    const u32x4 z = {0u, 0u, 0u, 0u};
    u32x4* base = out + start * vec_per_row;
    const int64_t n = len * vec_per_row;
    for (int64_t i = threadIdx.x; i < n; i += kRowBlock) __builtin_nontemporal_store(z, base + i);
}

__global__ __launch_bounds__(kRowBlock) void permute_rows_kernel(const u32x4* __restrict__ x, int64_t N,
                                                                int64_t vec_per_row, int K,
                                                                const int32_t* __restrict__ e2p,
                                                                const int32_t* __restrict__ zero_fill,
                                                                int zero_blocks, int64_t T,
                                                                u32x4* __restrict__ out) {
    if ((int)blockIdx.x < zero_blocks) {
        zero_range(zero_fill, blockIdx.x, T, vec_per_row, out);
        return;
    }
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)(blockIdx.x - zero_blocks) * kRowWaves + (threadIdx.x >> 6);
    if (t >= N) return;
    const int my_p = lane < K ? e2p[t * K + lane] : -1;
    const u32x4* src = x + t * vec_per_row;
    for (int64_t c0 = 0; c0 < vec_per_row; c0 += 64 * kRowChunk) {
        u32x4 v[kRowChunk];
#pragma unroll
        for (int i = 0; i < kRowChunk; ++i) {
            const int64_t j = c0 + i * 64 + lane;
            if (j < vec_per_row) v[i] = src[j];
        }
        for (int k = 0; k < K; ++k) {
            const int p = wave_uniform(__shfl(my_p, k, 64));
            if (p < 0 || p >= T) continue;
            u32x4* dst = out + (int64_t)p * vec_per_row;
#pragma unroll
            for (int i = 0; i < kRowChunk; ++i) {
                const int64_t j = c0 + i * 64 + lane;
                if (j < vec_per_row) __builtin_nontemporal_store(v[i], dst + j);
            }
        }
    }
}

__device__ __forceinline__ float bf16_lo(unsigned int u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(unsigned int u) { return __uint_as_float(u & 0xffff0000u); }

// binary32 -> bf16 bits, round to nearest, ties to even; a NaN stays a quiet NaN
__device__ __forceinline__ unsigned int to_bf16(float f) {
    const unsigned int u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// acc += w * v, or acc += v without weights; kept as two separate binary32 operations
template <bool W>
__device__ __forceinline__ float add_term(float acc, float w, float v) {
    if (W) {
        const float prod = __fmul_rn(w, v);
        return __fadd_rn(acc, prod);
    }
    return __fadd_rn(acc, v);
}

template <bool BF16, bool W>
__global__ __launch_bounds__(kRowBlock) void combine_rows_kernel(const u32x4* __restrict__ y, int64_t N,
                                                                int64_t vec_per_row, int K,
                                                                const int32_t* __restrict__ e2p,
                                                                const float* __restrict__ weights,
                                                                int64_t T, u32x4* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * kRowWaves + (threadIdx.x >> 6);
    if (t >= N) return;
    const int my_p = lane < K ? e2p[t * K + lane] : -1;
    const float my_w = (W && lane < K) ? weights[t * K + lane] : 0.0f;
    for (int64_t c0 = 0; c0 < vec_per_row; c0 += 64 * 2) {
        constexpr int kE = BF16 ? 8 : 4;  // elements per 16-byte vector
        float acc[2][kE];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int q = 0; q < kE; ++q) acc[i][q] = 0.0f;
        for (int k0 = 0; k0 < K; k0 += 8) {
            u32x4 v[8][2];
            int ok[8];
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const int k = k0 + kk;
                const int p = wave_uniform(__shfl(my_p, k < K ? k : 0, 64));
                ok[kk] = k < K && p >= 0 && p < T;
                const u32x4* src = y + (int64_t)(ok[kk] ? p : 0) * vec_per_row;
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int64_t j = c0 + i * 64 + lane;
                    if (ok[kk] && j < vec_per_row) v[kk][i] = __builtin_nontemporal_load(src + j);
                }
            }
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                if (!ok[kk]) continue;
                const float w = W ? __shfl(my_w, k0 + kk, 64) : 1.0f;
#pragma unroll
                for (int i = 0; i < 2; ++i) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const unsigned int u = v[kk][i][q];
                        if (BF16) {
                            acc[i][2 * q] = add_term<W>(acc[i][2 * q], w, bf16_lo(u));
                            acc[i][2 * q + 1] = add_term<W>(acc[i][2 * q + 1], w, bf16_hi(u));
                        } else {
                            acc[i][q] = add_term<W>(acc[i][q], w, __uint_as_float(u));
                        }
                    }
                }
            }
        }
        u32x4* dst = out + t * vec_per_row;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int64_t j = c0 + i * 64 + lane;
            if (j >= vec_per_row) continue;
            u32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (BF16) o[q] = to_bf16(acc[i][2 * q]) | (to_bf16(acc[i][2 * q + 1]) << 16);
                else o[q] = __float_as_uint(acc[i][q]);
            }
            dst[j] = o;
        }
    }
}

// Shared checks; the row length in 16-byte vectors on success.
int rows_check(const void* a, int dtype, int64_t N, int64_t H, int K, const int32_t* e2p, int64_t T,
               const void* b, int64_t& vec_per_row) {
    if (N < 0 || H < 1 || K < 1 || T < 0) return MEP_ERR_INVALID_ARG;
    if (dtype != MEP_F32 && dtype != MEP_BF16) return MEP_ERR_INVALID_ARG;
    if (N > 0 && (!a || !b || !e2p)) return MEP_ERR_INVALID_ARG;
    if ((a && !aligned(a, 16)) || (b && !aligned(b, 16)) || (e2p && !aligned(e2p, 4)))
        return MEP_ERR_INVALID_ARG;
    const int64_t row_bytes = H * (dtype == MEP_BF16 ? 2 : 4);
    if (row_bytes % 16 != 0) return MEP_ERR_UNSUPPORTED;
    if (K > kRowMaxK || N > INT32_MAX / K || T > INT32_MAX) return MEP_ERR_UNSUPPORTED;
    vec_per_row = row_bytes / 16;
    return MEP_OK;
}

}  // namespace

}  // namespace mep

extern "C" int mep_permute_rows(const void* x, int dtype, int64_t N, int64_t H, int K,
                                const int32_t* expanded_to_permuted, const int32_t* zero_fill, int E,
                                void* x_permuted, int64_t permuted_rows, void* stream) {
    mep::launch_begin();
    using namespace mep;
    int64_t vpr = 0;
    int rc = rows_check(x, dtype, N, H, K, expanded_to_permuted, permuted_rows, x_permuted, vpr);
    if (rc != MEP_OK) return rc;
    if (zero_fill && (E < 1 || !aligned(zero_fill, 4))) return MEP_ERR_INVALID_ARG;
    if (zero_fill && !x_permuted) return MEP_ERR_INVALID_ARG;
    const int zb = zero_fill ? E : 0;
    const int64_t tok_blocks = ceil_div64(N, kRowWaves);
    const int64_t grid = tok_blocks + zb;
    if (grid == 0) return MEP_OK;
    if (grid > INT32_MAX) return MEP_ERR_UNSUPPORTED;
    launch_ggl(permute_rows_kernel, dim3((unsigned)grid), dim3(kRowBlock), 0,
                       reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const u32x4*>(x), N, vpr,
                       K, expanded_to_permuted, zero_fill, zb, permuted_rows,
                       reinterpret_cast<u32x4*>(x_permuted));
    return launch_status();
}

extern "C" int mep_combine_rows(const void* y_permuted, int dtype, int64_t N, int64_t H, int K,
                                const int32_t* expanded_to_permuted, const float* topk_weights,
                                int64_t permuted_rows, void* out, void* stream) {
    mep::launch_begin();
    using namespace mep;
    int64_t vpr = 0;
    int rc = rows_check(y_permuted, dtype, N, H, K, expanded_to_permuted, permuted_rows, out, vpr);
    if (rc != MEP_OK) return rc;
    if (topk_weights && !aligned(topk_weights, 4)) return MEP_ERR_INVALID_ARG;
    if (N == 0) return MEP_OK;
    const int64_t grid = ceil_div64(N, kRowWaves);
    const auto* yy = reinterpret_cast<const u32x4*>(y_permuted);
    auto* oo = reinterpret_cast<u32x4*>(out);
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const bool bf = dtype == MEP_BF16;
    if (bf && topk_weights)
        launch_ggl((combine_rows_kernel<true, true>), dim3((unsigned)grid), dim3(kRowBlock), 0, st, yy,
                           N, vpr, K, expanded_to_permuted, topk_weights, permuted_rows, oo);
    else if (bf)
        launch_ggl((combine_rows_kernel<true, false>), dim3((unsigned)grid), dim3(kRowBlock), 0, st, yy,
                           N, vpr, K, expanded_to_permuted, topk_weights, permuted_rows, oo);
    else if (topk_weights)
        launch_ggl((combine_rows_kernel<false, true>), dim3((unsigned)grid), dim3(kRowBlock), 0, st,
                           yy, N, vpr, K, expanded_to_permuted, topk_weights, permuted_rows, oo);
    else
        launch_ggl((combine_rows_kernel<false, false>), dim3((unsigned)grid), dim3(kRowBlock), 0, st,
                           yy, N, vpr, K, expanded_to_permuted, topk_weights, permuted_rows, oo);
    return launch_status();
}
