// mep_route_layout_plan_noalloc: mep_route_layout_plan for callers that cannot allocate (code
// under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
// workspace is a file-scope device array of kScratchBytes per GPU instead of a caller buffer.
//
// The array's name is only a host-side stand-in: its device address comes from
// hipGetSymbolAddress, taken once per device with that device current and kept per device; every
// kernel argument uses that address.  The workspace protocol of the fused path leaves the array
// ready for the next call after every call, so it only has to start at zero: the loader
// zero-fills the array, and the first call on each device also clears it with a fill kernel on
// the caller's stream (no hipMemset, so the call can be captured into a graph).  Calls on one GPU
// share the array: overlapping calls on one GPU race, as calls sharing any workspace do.
#include <mutex>

#include "calls.h"
#include "host_common.h"

namespace mep {

int route_layout_plan(const void* logits, int dtype, int64_t N, int E, int K, const float* bias,
                      const mep_route_params* p, int32_t* topk_ids, float* topk_weights, int alignment,
                      int32_t* tokens_per_expert, int32_t* cu_seqlens, int32_t* expanded_to_permuted,
                      int32_t* permuted_to_expanded, int64_t permuted_cap, int32_t* zero_fill, int R, int num_src,
                      int num_channels, int64_t NvS, const mep_plan_outputs* out, void* ws, size_t ws_bytes,
                      void* stream, const StepEvents& ev, bool validate_only);

namespace {

constexpr size_t kScratchBytes = 8u << 20;  // 8 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

__global__ __launch_bounds__(256) void scratch_clear_kernel(u32x4* p, size_t n16) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
        p[i] = u32x4{0u, 0u, 0u, 0u};
}

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {nullptr};

// The current device's array (its device address), cleared on the stream at first use.
int scratch_for_current_device(hipStream_t st, void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MEP_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MEP_ERR_DEVICE;
        launch_ggl(scratch_clear_kernel, dim3(256), dim3(256), 0, st, reinterpret_cast<u32x4*>(p),
                           kScratchBytes / 16);
        if (launch_status() != MEP_OK) return MEP_ERR_DEVICE;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return MEP_OK;
}

}  // namespace

}  // namespace mep

extern "C" int mep_route_layout_plan_noalloc(const void* logits, int dtype, int64_t N, int E, int K,
                                             const float* bias, const mep_route_params* p, int32_t* topk_ids,
                                             float* topk_weights, int alignment, int32_t* tokens_per_expert,
                                             int32_t* cu_seqlens, int32_t* expanded_to_permuted,
                                             int32_t* permuted_to_expanded, int64_t permuted_cap,
                                             int32_t* zero_fill, int R, int num_src, int num_channels, int64_t NvS,
                                             const mep_plan_outputs* out, void* stream) {
    mep::launch_begin();
    using namespace mep;
    // every check first (sizes beyond the array included); nothing is enqueued on an error
    if (N < 0 || E < 1 || K < 1 || R < 1 || num_src < 1) return MEP_ERR_INVALID_ARG;
    if (mep_plan_workspace_size(N, E, K, R, num_src) > kScratchBytes) return MEP_ERR_CAPACITY;
    void* const unchecked = reinterpret_cast<void*>(uintptr_t{256});  // aligned, never dereferenced
    int rc = route_layout_plan(logits, dtype, N, E, K, bias, p, topk_ids, topk_weights, alignment, tokens_per_expert,
                               cu_seqlens, expanded_to_permuted, permuted_to_expanded, permuted_cap, zero_fill, R,
                               num_src, num_channels, NvS, out, unchecked, kScratchBytes, stream, StepEvents{}, true);
    if (rc != MEP_OK) return rc;
    void* ws = nullptr;
    rc = scratch_for_current_device(reinterpret_cast<hipStream_t>(stream), &ws);
    if (rc != MEP_OK) return rc;
    return route_layout_plan(logits, dtype, N, E, K, bias, p, topk_ids, topk_weights, alignment, tokens_per_expert,
                             cu_seqlens, expanded_to_permuted, permuted_to_expanded, permuted_cap, zero_fill, R,
                             num_src, num_channels, NvS, out, ws, kScratchBytes, stream, StepEvents{}, false);
}
