// mep_sigmoid_eval: the three sigmoid evaluations of the routing kernels, element-wise over an
// array, so that each can be checked over every binary32 input:
//   - the correctly rounded binary32 sigmoid (sigmoid_cr: binary64 evaluation with an interval
//     test, double-double when the test cannot decide), from which every exact key is formed;
//   - the binary32 filter value s~ = rcp(1 + exp2(-x log2 e)) of the certified fast selection,
//     whose error bound |s~ - sigma| <= 3.23 * 2^-23 the certificates rest on;
//   - the binary64 sigmoid of the routing weights (relative error below 2^-30).
// The device functions are the ones the routing kernels inline.
#include "route_fast.h"

namespace mep {

namespace {

constexpr int kEvalBlock = 256;
constexpr int64_t kEvalMaxGrid = 8192;

__global__ __launch_bounds__(kEvalBlock) void sigmoid_eval_kernel(const float* __restrict__ x, int64_t n,
                                                                  float* __restrict__ cr,
                                                                  float* __restrict__ filter,
                                                                  double* __restrict__ weight) {
    const int64_t stride = (int64_t)gridDim.x * kEvalBlock;
    for (int64_t i = (int64_t)blockIdx.x * kEvalBlock + threadIdx.x; i < n; i += stride) {
        const float v = gptr(x)[i];
        if (cr) gptr(cr)[i] = sigmoid_cr(v);
        if (filter) gptr(filter)[i] = sigmoid_fast(v);
        if (weight) gptr(weight)[i] = sigmoid_f64_weight(v);
    }
}

}  // namespace

}  // namespace mep

extern "C" int mep_sigmoid_eval(const float* x, int64_t n, float* cr_out, float* filter_out, double* weight_out,
                                void* stream) {
    mep::launch_begin();
    using namespace mep;
    if (n < 0 || (n > 0 && !x)) return MEP_ERR_INVALID_ARG;
    if (!mep::aligned(x, 4) || !mep::aligned(cr_out, 4) || !mep::aligned(filter_out, 4) ||
        !mep::aligned(weight_out, 8))
        return MEP_ERR_INVALID_ARG;
    if (n == 0 || (!cr_out && !filter_out && !weight_out)) return MEP_OK;
    int64_t grid = ceil_div64(n, kEvalBlock);
    if (grid > kEvalMaxGrid) grid = kEvalMaxGrid;
    launch_ggl(sigmoid_eval_kernel, dim3((unsigned)grid), dim3(kEvalBlock), 0,
                       reinterpret_cast<hipStream_t>(stream), x, n, cr_out, filter_out, weight_out);
    return launch_status();
}
