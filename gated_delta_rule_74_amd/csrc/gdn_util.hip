// Small device utilities of the C ABI.
#include "gdn_common.hpp"
#include "gdn_launch.hpp"

namespace gdn {

// dst[i] = src ? src[i] : 0 for i < n (grid-stride); used for the results of
// an empty sequence, whose final state is the initial one and whose gradient
// with respect to the initial state is that of the final state
__global__ __launch_bounds__(NTHR) void copy_or_zero_kernel(float *__restrict__ dst,
                                                            const float *__restrict__ src, size_t n) {
    const size_t stride = (size_t)gridDim.x * NTHR;
    for (size_t i = (size_t)blockIdx.x * NTHR + threadIdx.x; i < n; i += stride) dst[i] = src ? src[i] : 0.f;
}

hipError_t launch_copy_or_zero(float *dst, const float *src, size_t n, hipStream_t st) {
    if (n == 0) return hipSuccess;
    const size_t blocks = (n + NTHR - 1) / NTHR;
    const int grid = (int)(blocks < 1024 ? blocks : 1024);
    hipLaunchKernelGGL(copy_or_zero_kernel, dim3(grid), dim3(NTHR), 0, st, dst, src, n);
    return hipGetLastError();
}

} // namespace gdn
