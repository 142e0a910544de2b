// Mean squared error as the similarity term, with its gradient ("A Scalable
// Distributed Framework for Multimodal GigaVoxel Image Registration",
// Background and motivation: MSE among the similarity terms; Key design 5:
// a per-voxel loss whose shard sums add up to the whole):
//   loss = weight (1/N) sum (W - F)^2,   gW = 2 weight (W - F) / N.
//
// One streaming pass; per step a thread loads kU float4 chunks of F and W
// before it uses any (more bytes in flight per wave). The difference
// of two fp32 values is exact in fp64, so each thread's sum of squares is
// fp64 of exact terms; block sums go to the workspace partials and one block
// adds them in a fixed order (the loss is the same on every run).
#include "ngv_internal.hpp"

namespace ngv {
namespace {

constexpr int kThreads = 256;
// float4 chunks per thread and step, loaded before any is used (more bytes
// in flight per wave)
constexpr int kU = 2;
typedef float v4 __attribute__((ext_vector_type(4)));

__device__ inline void mse_chunk(const v4 &f, const v4 &w, float *gW, int64_t base, double gscale, int accumulate,
                                 double &acc) {
    v4 g;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const double d = double(w[k]) - double(f[k]);
        acc = fma(d, d, acc);
        g[k] = float(gscale * d);
    }
    if (gW) {
        if (accumulate) g += __builtin_nontemporal_load(reinterpret_cast<const v4 *>(gW + base));
        __builtin_nontemporal_store(g, reinterpret_cast<v4 *>(gW + base));
    }
}

__global__ __launch_bounds__(kThreads) void mse_kernel(const float *__restrict__ F, const float *__restrict__ W,
                                                       float *__restrict__ gW, int64_t n, double gscale,
                                                       int accumulate, double *__restrict__ partials) {
    __shared__ double red[kThreads / 64];
    constexpr int64_t kChunk = int64_t(kThreads) * 4, kPer = kChunk * kU;
    const ItemRange r = xcd_items((n + kPer - 1) / kPer);
    double acc = 0.0;
    for (int64_t it = r.begin; it < r.end; it += r.step) {
        const int64_t base = it * kPer + int64_t(threadIdx.x) * 4;
        if (base + (kU - 1) * kChunk + 3 < n) {
            // F and W stream through once: non-temporal
            v4 f[kU], w[kU];
#pragma unroll
            for (int c = 0; c < kU; ++c) {
                f[c] = __builtin_nontemporal_load(reinterpret_cast<const v4 *>(F + base + c * kChunk));
                w[c] = __builtin_nontemporal_load(reinterpret_cast<const v4 *>(W + base + c * kChunk));
            }
#pragma unroll
            for (int c = 0; c < kU; ++c) mse_chunk(f[c], w[c], gW, base + c * kChunk, gscale, accumulate, acc);
        } else {
            for (int c = 0; c < kU; ++c) {
                const int64_t b0 = base + c * kChunk;
                for (int64_t k = b0; k < n && k < b0 + 4; ++k) {
                    const double d = double(W[k]) - double(F[k]);
                    acc = fma(d, d, acc);
                    if (gW) {
                        const float g = float(gscale * d);
                        gW[k] = accumulate ? gW[k] + g : g;
                    }
                }
            }
        }
    }
    const double tot = block_sum(acc, red);
    if (threadIdx.x == 0) partials[size_t(blockIdx.x) * kPartialStride] = tot;
}

}  // namespace

hipError_t launch_mse(const float *F, const float *W, int64_t n, float weight, double *loss, float *gW,
                      int accumulate, void *ws, hipStream_t s) {
    double *partials = reinterpret_cast<double *>(static_cast<char *>(ws) + ws_layout(0).partials);
    const int64_t items = (n + kThreads * 4 * kU - 1) / (kThreads * 4 * kU);
    const int blocks = persistent_blocks(items, 8);
    const double N = double(n);
    hipLaunchKernelGGL(mse_kernel, dim3(blocks), dim3(kThreads), 0, s, F, W, gW, n, 2.0 * double(weight) / N,
                       accumulate, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_partials_final(partials, blocks, double(weight) / N, loss, accumulate, s);
}

}  // namespace ngv
