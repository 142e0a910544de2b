// The last step of the loss reductions: one block adds the per-block partial
// sums that a loss kernel left in the workspace, in a fixed order, so a loss
// is the same on every run with the same grid.
#include "ngv_internal.hpp"

namespace ngv {
namespace {

// Thread t sums the partials of blocks t, t + 256, ... in order, then a
// fixed-order tree.
__global__ __launch_bounds__(256) void partials_final_kernel(const double *__restrict__ partials, int nblocks,
                                                             double scale, double *__restrict__ loss,
                                                             int accumulate) {
    __shared__ double red[256];
    const int t = threadIdx.x;
    double s = 0.0;
    for (int b = t; b < nblocks; b += 256) s += partials[size_t(b) * kPartialStride];
    red[t] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (t < w) red[t] += red[t + w];
        __syncthreads();
    }
    if (t == 0) {
        const double v = scale * red[0];
        *loss = accumulate ? *loss + v : v;
    }
}

}  // namespace

hipError_t launch_partials_final(const double *partials, int nblocks, double scale, double *loss, int accumulate,
                                 hipStream_t s) {
    hipLaunchKernelGGL(partials_final_kernel, dim3(1), dim3(256), 0, s, partials, nblocks, scale, loss, accumulate);
    return hipGetLastError();
}

}  // namespace ngv
