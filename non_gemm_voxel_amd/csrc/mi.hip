// Mattes mutual information with implicit Parzen windows ("A Scalable
// Distributed Framework for Multimodal GigaVoxel Image Registration", Key
// design 2; histogram merge, Key design 5).
//
// The B x N Parzen block is never formed. Three kernels:
//   hist     every block keeps a private joint histogram in LDS (32.32 fixed
//            point in u64, so the merges are exact and independent of order)
//            and adds each voxel's 4 x 4 cubic B-spline weights (a lane first
//            sums up to 64 of its samples' weights in fp32, see mi_device.hpp);
//            at the end the block adds its histogram into the global one (one
//            u64 atomic per non-empty bin) -- the block histograms are the
//            page's partial aggregates, merged by a plain sum.
//   finalize one block: p = H/N, marginals, MI, and the table
//            L_ab = ln(p_ab / (p_a p_b)) (0 where p_ab = 0).
//   grad     every voxel: gW = weight * (s_W / N) * sum_ab L_ab beta(a - cF) beta'(b - cW),
//            with L in LDS, 4 x 4 terms per voxel.
// The fixed image's kernel is a template parameter: the cubic B-spline (one
// kernel for both images), or the box (zero order) of Mattes et al.'s original
// pair, which puts each sample in one fixed bin (1 x 4 weights per voxel).
// Up to kMaxLdsBins bins the block histogram and the gradient's table live
// in LDS; beyond that (up to kMaxBins) the blocks add into the global
// histogram directly and the gradient reads the table from global memory.
// Extra device memory: bins^2 * 12 bytes, whatever the volume size.
#include "mi_device.hpp"

namespace ngv {
namespace {

using namespace mi;

constexpr int kThreads = 256;
__global__ __launch_bounds__(kThreads) void mi_zero_kernel(unsigned long long *__restrict__ hist, int nb2) {
    for (int i = threadIdx.x; i < nb2; i += blockDim.x) hist[i] = 0ull;
}

// Joint histogram. Work item = rz planes of a span of kSpan in-plane voxels;
// each thread owns 4 consecutive in-plane voxels and walks them up the rz
// planes, so its samples are spatial neighbours with nearby bins, and its
// register window (mi::hist_add) is flushed once per item. rz is 16, or less
// for volumes too small to give every CU two items. Dynamic LDS: the block's
// histogram, then the waves' rings of deferred samples.
constexpr int kRZ = 16;
constexpr int kSpan = kThreads * 4;

// kGlob: the histogram is too large for LDS (more than kMaxLdsBins bins), so
// the block adds straight into the global one (the same fixed-point values,
// so the same sums); LDS then holds only the rings.
template <int FO, bool kGlob>
__global__ __launch_bounds__(kThreads) void mi_hist_kernel(const float *__restrict__ F, const float *__restrict__ W,
                                                           int64_t plane, int64_t nz, int rz, int vec4, MiParams p,
                                                           unsigned long long *__restrict__ hist) {
    extern __shared__ unsigned long long lds[];
    const int nb = p.bins, nb2 = nb * nb;
    unsigned long long *h = kGlob ? hist : lds;
    if constexpr (!kGlob) {
        for (int i = threadIdx.x; i < nb2; i += blockDim.x) h[i] = 0ull;
        __syncthreads();
    }
    const int64_t spans = (plane + kSpan - 1) / kSpan, groups = (nz + rz - 1) / rz;
    const ItemRange r = xcd_items(spans * groups);
    HistCtx c;
    hist_init(c, reinterpret_cast<float2 *>(lds + (kGlob ? 0 : nb2)));
    for (int64_t it = r.begin; it < r.end; it += r.step) {
        const int64_t sp = it % spans, g = it / spans;
        const int64_t q0 = sp * kSpan + int64_t(threadIdx.x) * 4;  // in-plane index of the first voxel
        const int64_t z1 = (g + 1) * rz < nz ? (g + 1) * rz : nz;
        for (int64_t z = g * rz; z < z1; ++z) {
            const int64_t base = z * plane + q0;
            float fv[4] = {0.0f, 0.0f, 0.0f, 0.0f}, wv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            bool ok[4];
            if (vec4 && q0 + 3 < plane) {
                const float4 a = *reinterpret_cast<const float4 *>(F + base);
                const float4 b = *reinterpret_cast<const float4 *>(W + base);
                fv[0] = a.x; fv[1] = a.y; fv[2] = a.z; fv[3] = a.w;
                wv[0] = b.x; wv[1] = b.y; wv[2] = b.z; wv[3] = b.w;
                ok[0] = ok[1] = ok[2] = ok[3] = true;
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    ok[k] = q0 + k < plane;
                    if (ok[k]) {
                        fv[k] = F[base + k];
                        wv[k] = W[base + k];
                    }
                }
            }
            // every lane takes part in each hist_add (deferred samples are queued per wave)
#pragma unroll
            for (int k = 0; k < 4; ++k) hist_add<FO>(c, fv[k], wv[k], ok[k], p, h);
        }
        hist_flush<FO>(c, p, h);
    }
    if constexpr (!kGlob) {
        __syncthreads();
        for (int i = threadIdx.x; i < nb2; i += blockDim.x) {
            const unsigned long long v = h[i];
            if (v) atomicAdd(hist + i, v);
        }
    }
}

__global__ __launch_bounds__(1024) void mi_finalize_kernel(const unsigned long long *__restrict__ hist, MiParams p,
                                                           double inv_n, float *__restrict__ table,
                                                           double *__restrict__ loss, int accumulate) {
    __shared__ double pa[kMaxBins], pb[kMaxBins], red[16];
    const int nb = p.bins, nb2 = nb * nb;
    const double unit = inv_n / 4294967296.0;
    if (threadIdx.x < nb) {
        double s = 0.0;
        for (int b = 0; b < nb; ++b) s += double(hist[threadIdx.x * nb + b]) * unit;
        pa[threadIdx.x] = s;
    } else if (threadIdx.x >= 512 && threadIdx.x < 512 + nb) {
        const int b = threadIdx.x - 512;
        double s = 0.0;
        for (int a = 0; a < nb; ++a) s += double(hist[a * nb + b]) * unit;
        pb[b] = s;
    }
    __syncthreads();
    double mi = 0.0;
    for (int e = threadIdx.x; e < nb2; e += blockDim.x) {
        const double pab = double(hist[e]) * unit;
        double l = 0.0;
        if (pab > 0.0) {
            l = log(pab / (pa[e / nb] * pb[e % nb]));
            mi += pab * l;
        }
        table[e] = float(l);
    }
    mi = block_sum(mi, red);
    if (threadIdx.x == 0) {
        const double v = -double(p.weight) * mi;
        *loss = accumulate ? *loss + v : v;
    }
}

// kGlob: the table is too large for LDS (more than kMaxLdsBins bins) and is
// read from global memory (it stays in L2).
template <int FO, bool kGlob>
__global__ __launch_bounds__(kThreads) void mi_grad_kernel(const float *__restrict__ F, const float *__restrict__ W,
                                                           int64_t n, MiParams p, const float *__restrict__ table,
                                                           float gscale, float *__restrict__ gW, int accumulate) {
    extern __shared__ float lds_l[];
    const float *L = table;
    if constexpr (!kGlob) {
        const int nb2 = p.bins * p.bins;
        for (int i = threadIdx.x; i < nb2; i += blockDim.x) lds_l[i] = table[i];
        __syncthreads();
        L = lds_l;
    }
    const int64_t per = int64_t(kThreads) * 4;
    const int64_t total = (n + per - 1) / per;
    const ItemRange r = xcd_items(total);
    for (int64_t it = r.begin; it < r.end; it += r.step) {
        const int64_t base = it * per + int64_t(threadIdx.x) * 4;
        const int cnt = base + 3 < n ? 4 : int(n - base > 0 ? n - base : 0);
        float fv[4] = {0, 0, 0, 0}, wv[4] = {0, 0, 0, 0}, go[4] = {0, 0, 0, 0};
        if (cnt == 4) {
            const float4 a = *reinterpret_cast<const float4 *>(F + base);
            const float4 b = *reinterpret_cast<const float4 *>(W + base);
            fv[0] = a.x; fv[1] = a.y; fv[2] = a.z; fv[3] = a.w;
            wv[0] = b.x; wv[1] = b.y; wv[2] = b.z; wv[3] = b.w;
            if (accumulate) {
                const float4 c = *reinterpret_cast<const float4 *>(gW + base);
                go[0] = c.x; go[1] = c.y; go[2] = c.z; go[3] = c.w;
            }
        } else {
            for (int k = 0; k < cnt; ++k) {
                fv[k] = F[base + k];
                wv[k] = W[base + k];
                if (accumulate) go[k] = gW[base + k];
            }
        }
        float out[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) out[k] = go[k] + grad_value<FO>(fv[k], wv[k], p, L, gscale);
        if (cnt == 4) {
            *reinterpret_cast<float4 *>(gW + base) = make_float4(out[0], out[1], out[2], out[3]);
        } else {
            for (int k = 0; k < cnt; ++k) gW[base + k] = out[k];
        }
    }
}

}  // namespace

hipError_t launch_mi_zero(unsigned long long *hist, int bins, hipStream_t s) {
    hipLaunchKernelGGL(mi_zero_kernel, dim3(1), dim3(kThreads), 0, s, hist, bins * bins);
    return hipGetLastError();
}

hipError_t launch_mi_finalize(const unsigned long long *hist, const MiParams &p, int64_t n, float *table,
                              double *loss, int accumulate, hipStream_t s) {
    hipLaunchKernelGGL(mi_finalize_kernel, dim3(1), dim3(1024), 0, s, hist, p, 1.0 / double(n), table, loss,
                       accumulate);
    return hipGetLastError();
}

hipError_t launch_mi_grad(const float *F, const float *W, int64_t n, const MiParams &p, const float *table,
                          float *gW, int accumulate, hipStream_t s) {
    const float gscale = mi_grad_scale(p, n);
    const bool glob = p.bins > kMaxLdsBins;
    const size_t lds_l = glob ? 0 : size_t(p.bins) * p.bins * sizeof(float);
    const int64_t items = (n + kThreads * 4 - 1) / (kThreads * 4);
    const dim3 grid(persistent_blocks(items, 4));
    if (p.f_order == 0) {
        if (glob)
            hipLaunchKernelGGL((mi_grad_kernel<0, true>), grid, dim3(kThreads), 0, s, F, W, n, p, table, gscale, gW,
                               accumulate);
        else
            hipLaunchKernelGGL((mi_grad_kernel<0, false>), grid, dim3(kThreads), lds_l, s, F, W, n, p, table, gscale,
                               gW, accumulate);
    } else {
        if (glob)
            hipLaunchKernelGGL((mi_grad_kernel<3, true>), grid, dim3(kThreads), 0, s, F, W, n, p, table, gscale, gW,
                               accumulate);
        else
            hipLaunchKernelGGL((mi_grad_kernel<3, false>), grid, dim3(kThreads), lds_l, s, F, W, n, p, table, gscale,
                               gW, accumulate);
    }
    return hipGetLastError();
}

hipError_t launch_mi(const float *F, const float *W, int64_t plane, int64_t nz, const MiParams &p, double *loss,
                     float *gW, int accumulate, unsigned long long *hist, float *table, hipStream_t s) {
    const int64_t n = plane * nz;
    const int nb2 = p.bins * p.bins;
    hipError_t e = launch_mi_zero(hist, p.bins, s);
    if (e != hipSuccess) return e;
    const bool glob = p.bins > kMaxLdsBins;
    const size_t lds_h = (glob ? 0 : size_t(nb2) * sizeof(unsigned long long)) + ring_bytes(kThreads);
    const int64_t spans = (plane + kSpan - 1) / kSpan;
    int rz = kRZ;
    while (rz > 1 && spans * ((nz + rz - 1) / rz) < 2 * int64_t(device_info().cus)) rz /= 2;
    const int64_t hist_items = spans * ((nz + rz - 1) / rz);
    // eight blocks per CU (the 2048-block cap): on the 1280 x 1536 x 1280 pair
    // 9.85 ms against 10.3 with six and 10.6 with four; 640 x 768 x 640 the
    // same as with four (1.35 ms; six: 1.30). The histogram does not depend
    // on the grid: windows flush per item, and the rest is fixed point.
    const int blocks = persistent_blocks(hist_items, lds_h > 32768 ? 1 : 8);
    const void *kern = p.f_order == 0 ? reinterpret_cast<const void *>(mi_hist_kernel<0, false>)
                                      : reinterpret_cast<const void *>(mi_hist_kernel<3, false>);
    if (lds_h > 65536) {
        e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds_h));
        if (e != hipSuccess) return e;
    }
    const int vec4 = (plane % 4 == 0) ? 1 : 0;
    const dim3 grid(blocks);
    if (p.f_order == 0) {
        if (glob)
            hipLaunchKernelGGL((mi_hist_kernel<0, true>), grid, dim3(kThreads), lds_h, s, F, W, plane, nz, rz, vec4,
                               p, hist);
        else
            hipLaunchKernelGGL((mi_hist_kernel<0, false>), grid, dim3(kThreads), lds_h, s, F, W, plane, nz, rz, vec4,
                               p, hist);
    } else {
        if (glob)
            hipLaunchKernelGGL((mi_hist_kernel<3, true>), grid, dim3(kThreads), lds_h, s, F, W, plane, nz, rz, vec4,
                               p, hist);
        else
            hipLaunchKernelGGL((mi_hist_kernel<3, false>), grid, dim3(kThreads), lds_h, s, F, W, plane, nz, rz, vec4,
                               p, hist);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_mi_finalize(hist, p, n, table, loss, accumulate, s);
    if (e != hipSuccess || gW == nullptr) return e;
    return launch_mi_grad(F, W, n, p, table, gW, accumulate, s);
}

}  // namespace ngv
