// Mattes mutual information with implicit Parzen windows ("A Scalable
// Distributed Framework for Multimodal GigaVoxel Image Registration", Key
// design 2; histogram merge, Key design 5).
//
// The B x N Parzen block is never formed. Three kernels:
//   hist     every block keeps a private joint histogram in LDS (32.32 fixed
//            point in u64, so sums are exact and independent of order) and
//            adds each voxel's 4 x 4 cubic B-spline weights; at the end the
//            block adds its histogram into the global one (one u64 atomic per
//            non-empty bin) -- the block histograms are the page's partial
//            aggregates, merged by a plain sum.
//   finalize one block: p = H/N, marginals, MI, and the table
//            L_ab = ln(p_ab / (p_a p_b)) (0 where p_ab = 0).
//   grad     every voxel: gW = weight * (s_W / N) * sum_ab L_ab beta(a - cF) beta'(b - cW),
//            with L in LDS, 4 x 4 terms per voxel.
// Extra device memory: bins^2 * 12 bytes, whatever the volume size.
#include "ngv_internal.hpp"

namespace ngv {
namespace {

constexpr int kThreads = 256;
constexpr float kFix = 4294967296.0f;  // 2^32: fixed-point scale of the histogram

// Cubic B-spline weights of the four bins ia..ia+3 around bin coordinate c
// (ia = floor(c) - 1, t = c - floor(c)), the uniform cubic B-spline basis.
__device__ inline void bspline4(float c, int &ia, float w[4]) {
    const float fl = floorf(c);
    const float t = c - fl, t2 = t * t, t3 = t2 * t, s = 1.0f - t;
    ia = int(fl) - 1;
    w[0] = s * s * s * (1.0f / 6.0f);
    w[1] = fmaf(3.0f, t3, fmaf(-6.0f, t2, 4.0f)) * (1.0f / 6.0f);
    w[2] = fmaf(-3.0f, t3, fmaf(3.0f, t2, fmaf(3.0f, t, 1.0f))) * (1.0f / 6.0f);
    w[3] = t3 * (1.0f / 6.0f);
}

// Derivatives beta'(b - c) of the same four weights with respect to their
// argument b - c (so d/dc of weight b is minus this).
__device__ inline void bspline4_deriv(float c, int &ia, float d[4]) {
    const float fl = floorf(c);
    const float t = c - fl, t2 = t * t, s = 1.0f - t;
    ia = int(fl) - 1;
    d[0] = 0.5f * s * s;
    d[1] = fmaf(-1.5f, t2, 2.0f * t);
    d[2] = fmaf(1.5f, t2, -0.5f - t);
    d[3] = -0.5f * t2;
}

__device__ inline float bin_coord(float v, float lo, float hi, float scale) {
    return fmaf(fminf(fmaxf(v, lo), hi) - lo, scale, 2.0f);
}

__global__ __launch_bounds__(kThreads) void mi_zero_kernel(unsigned long long *__restrict__ hist, int nb2) {
    for (int i = threadIdx.x; i < nb2; i += blockDim.x) hist[i] = 0ull;
}

// Joint histogram. Work item = RZ planes of a span of kSpan in-plane voxels;
// each thread owns 4 consecutive in-plane voxels and walks them up the RZ
// planes, so its samples are spatial neighbours with nearby bins. A thread
// adds its voxels' 4 x 4 weight blocks into a private 6 x 6 window of the
// histogram held in registers (fp32), anchored one bin below its first
// sample's block; samples whose block falls outside the window go straight
// to the block's LDS histogram (u64 atomics). At the end of the item the
// windows are flushed to LDS in 32.32 fixed point -- summed across the wave
// first when every lane shares one anchor (the background, where thousands of
// samples hit the same bins and per-sample atomics would serialise).
constexpr int kRZ = 16;
constexpr int kSpan = kThreads * 4;
constexpr int kWin = 6;

struct HistCtx {
    float acc[kWin][kWin];
    int ha, hb;
    bool anchored;
};

__device__ inline void shift6(const float w[4], int d, float e[kWin]) {
    // e[j] = w[j - d] for 0 <= j - d < 4, else 0; d in {0, 1, 2}
    e[0] = d == 0 ? w[0] : 0.0f;
    e[1] = d == 0 ? w[1] : (d == 1 ? w[0] : 0.0f);
    e[2] = d == 0 ? w[2] : (d == 1 ? w[1] : w[0]);
    e[3] = d == 0 ? w[3] : (d == 1 ? w[2] : w[1]);
    e[4] = d == 0 ? 0.0f : (d == 1 ? w[3] : w[2]);
    e[5] = d == 2 ? w[3] : 0.0f;
}

__device__ inline void hist_add(HistCtx &c, float fv, float wv, const MiParams &p, unsigned long long *h) {
    const int nb = p.bins;
    int ia, ib;
    float wa[4], wb[4];
    bspline4(bin_coord(fv, p.f_lo, p.f_hi, p.f_scale), ia, wa);
    bspline4(bin_coord(wv, p.w_lo, p.w_hi, p.w_scale), ib, wb);
    if (!c.anchored) {
        c.ha = min(max(ia - 1, 0), nb - kWin);
        c.hb = min(max(ib - 1, 0), nb - kWin);
        c.anchored = true;
    }
    const int da = ia - c.ha, db = ib - c.hb;
    if (da >= 0 && da <= kWin - 4 && db >= 0 && db <= kWin - 4) {
        float ea[kWin], eb[kWin];
        shift6(wa, da, ea);
        shift6(wb, db, eb);
#pragma unroll
        for (int i = 0; i < kWin; ++i)
#pragma unroll
            for (int j = 0; j < kWin; ++j) c.acc[i][j] = fmaf(ea[i], eb[j], c.acc[i][j]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float wi = wa[i] * kFix;
            unsigned long long *row = h + (ia + i) * nb + ib;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const unsigned long long q = __float2ull_rn(wi * wb[j]);
                if (q) atomicAdd(row + j, q);
            }
        }
    }
}

__device__ inline void hist_flush(HistCtx &c, int nb, unsigned long long *h) {
    // lanes without samples carry zeros: give them the first anchored lane's anchor
    const unsigned long long have = __ballot(c.anchored);
    if (have == 0ull) return;
    const int src = __ffsll((long long)have) - 1;
    const int ha0 = __shfl(c.ha, src, 64), hb0 = __shfl(c.hb, src, 64);
    if (!c.anchored) {
        c.ha = ha0;
        c.hb = hb0;
    }
    const bool same = __all(c.ha == ha0 && c.hb == hb0);
    const int lane = threadIdx.x & 63;
    if (same) {
#pragma unroll
        for (int i = 0; i < kWin; ++i)
#pragma unroll
            for (int j = 0; j < kWin; ++j) {
                const float v = wave_sum(c.acc[i][j]);
                if (lane == i * kWin + j) {
                    const unsigned long long q = __float2ull_rn(v * kFix);
                    if (q) atomicAdd(h + (ha0 + i) * nb + hb0 + j, q);
                }
            }
    } else {
#pragma unroll
        for (int i = 0; i < kWin; ++i)
#pragma unroll
            for (int j = 0; j < kWin; ++j) {
                const unsigned long long q = __float2ull_rn(c.acc[i][j] * kFix);
                if (q) atomicAdd(h + (c.ha + i) * nb + c.hb + j, q);
            }
    }
#pragma unroll
    for (int i = 0; i < kWin; ++i)
#pragma unroll
        for (int j = 0; j < kWin; ++j) c.acc[i][j] = 0.0f;
    c.anchored = false;
}

__global__ __launch_bounds__(kThreads) void mi_hist_kernel(const float *__restrict__ F, const float *__restrict__ W,
                                                           int64_t plane, int64_t nz, int vec4, MiParams p,
                                                           unsigned long long *__restrict__ hist) {
    extern __shared__ unsigned long long h[];
    const int nb = p.bins, nb2 = nb * nb;
    for (int i = threadIdx.x; i < nb2; i += blockDim.x) h[i] = 0ull;
    __syncthreads();
    const int64_t spans = (plane + kSpan - 1) / kSpan, groups = (nz + kRZ - 1) / kRZ;
    const ItemRange r = xcd_items(spans * groups);
    HistCtx c;
#pragma unroll
    for (int i = 0; i < kWin; ++i)
#pragma unroll
        for (int j = 0; j < kWin; ++j) c.acc[i][j] = 0.0f;
    c.anchored = false;
    c.ha = c.hb = 0;
    for (int64_t it = r.begin; it < r.end; it += r.step) {
        const int64_t sp = it % spans, g = it / spans;
        const int64_t q0 = sp * kSpan + int64_t(threadIdx.x) * 4;  // in-plane index of the first voxel
        const int64_t z1 = (g + 1) * kRZ < nz ? (g + 1) * kRZ : nz;
        for (int64_t z = g * kRZ; z < z1; ++z) {
            const int64_t base = z * plane + q0;
            if (vec4 && q0 + 3 < plane) {
                const float4 a = *reinterpret_cast<const float4 *>(F + base);
                const float4 b = *reinterpret_cast<const float4 *>(W + base);
                hist_add(c, a.x, b.x, p, h);
                hist_add(c, a.y, b.y, p, h);
                hist_add(c, a.z, b.z, p, h);
                hist_add(c, a.w, b.w, p, h);
            } else {
                for (int k = 0; k < 4; ++k)
                    if (q0 + k < plane) hist_add(c, F[base + k], W[base + k], p, h);
            }
        }
        hist_flush(c, nb, h);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nb2; i += blockDim.x) {
        const unsigned long long v = h[i];
        if (v) atomicAdd(hist + i, v);
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

__global__ __launch_bounds__(kThreads) void mi_grad_kernel(const float *__restrict__ F, const float *__restrict__ W,
                                                           int64_t n, MiParams p, const float *__restrict__ table,
                                                           float gscale, float *__restrict__ gW, int accumulate) {
    extern __shared__ float L[];
    const int nb = p.bins, nb2 = nb * nb;
    for (int i = threadIdx.x; i < nb2; i += blockDim.x) L[i] = table[i];
    __syncthreads();
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
        for (int k = 0; k < 4; ++k) {
            float g = 0.0f;
            if (wv[k] >= p.w_lo && wv[k] <= p.w_hi) {
                int ia, ib;
                float wa[4], db[4];
                bspline4(bin_coord(fv[k], p.f_lo, p.f_hi, p.f_scale), ia, wa);
                bspline4_deriv(bin_coord(wv[k], p.w_lo, p.w_hi, p.w_scale), ib, db);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float *row = L + (ia + i) * nb + ib;
                    const float s = fmaf(row[0], db[0], fmaf(row[1], db[1], fmaf(row[2], db[2], row[3] * db[3])));
                    g = fmaf(wa[i], s, g);
                }
                g *= gscale;
            }
            out[k] = go[k] + g;
        }
        if (cnt == 4) {
            *reinterpret_cast<float4 *>(gW + base) = make_float4(out[0], out[1], out[2], out[3]);
        } else {
            for (int k = 0; k < cnt; ++k) gW[base + k] = out[k];
        }
    }
}

}  // namespace

hipError_t launch_mi(const float *F, const float *W, int64_t plane, int64_t nz, const MiParams &p, double *loss,
                     float *gW, int accumulate, void *ws, hipStream_t s) {
    const int64_t n = plane * nz;
    const WsLayout l = ws_layout(p.bins);
    char *base = static_cast<char *>(ws);
    auto *hist = reinterpret_cast<unsigned long long *>(base + l.hist);
    auto *table = reinterpret_cast<float *>(base + l.table);
    const int nb2 = p.bins * p.bins;
    hipLaunchKernelGGL(mi_zero_kernel, dim3(1), dim3(kThreads), 0, s, hist, nb2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t items = (n + kThreads * 4 - 1) / (kThreads * 4);
    const size_t lds_h = size_t(nb2) * sizeof(unsigned long long);
    const int64_t hist_items = ((plane + kSpan - 1) / kSpan) * ((nz + kRZ - 1) / kRZ);
    const int blocks = persistent_blocks(hist_items, lds_h > 32768 ? 1 : 4);
    if (lds_h > 65536) {
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(mi_hist_kernel),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(lds_h));
        if (e != hipSuccess) return e;
    }
    const int vec4 = (plane % 4 == 0) ? 1 : 0;
    hipLaunchKernelGGL(mi_hist_kernel, dim3(blocks), dim3(kThreads), lds_h, s, F, W, plane, nz, vec4, p, hist);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(mi_finalize_kernel, dim3(1), dim3(1024), 0, s, hist, p, 1.0 / double(n), table, loss,
                       accumulate);
    e = hipGetLastError();
    if (e != hipSuccess || gW == nullptr) return e;
    const float gscale = float(double(p.weight) * double(p.w_scale) / double(n));
    const size_t lds_l = size_t(nb2) * sizeof(float);
    hipLaunchKernelGGL(mi_grad_kernel, dim3(persistent_blocks(items, 4)), dim3(kThreads), lds_l, s, F, W, n, p,
                       table, gscale, gW, accumulate);
    return hipGetLastError();
}

}  // namespace ngv
