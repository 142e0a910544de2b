// Composite implicit grid sampler I(A x + t + S u(x)), forward and backward
// ("A Scalable Distributed Framework for Multimodal GigaVoxel Image
// Registration", Key design 1; slab partial sums, Key design 4).
//
// No coordinate grid exists in memory: every thread rebuilds its sample
// position from its own voxel index and its u(x), as
//   p = i + d,  d = (A_v - I) i + t_v + S_v u(i),
// where A_v, t_v, S_v are the map expressed in M's voxel units (prepared on
// the host in fp64). Splitting p into the integer i and the small offset d
// keeps the fractional part accurate at gigavoxel extents (floor(p) =
// i + floor(d) exactly) and makes the identity map land exactly on voxels.
//
// Work decomposition: items are spans of 1024 consecutive voxels of one
// z-plane, 4 per thread. A persistent grid walks the items in XCD-contiguous
// ranges (so the M rows a span gathers from are shared with its neighbours in
// one L2).
#include "ngv_internal.hpp"

namespace ngv {
namespace {

constexpr int kThreads = 256;

struct Sample {
    float c[8];  // corners, index (dz*2 + dy)*2 + dx
    float fx, fy, fz;
};

// Sample position and the 8 corner values of output voxel (ix, iy, iz);
// corners outside the moving grid or outside the held slab read as zero.
// The offset d is formed in fp64 (full rate on CDNA): fp32 positions carry
// ~1e-6 voxel of rounding at these extents, which is a 1e-3 relative error
// in W wherever the sample sits a hair inside a zero-padded face.
__device__ inline void gather(const WarpGeom &g, int64_t ix, int64_t iy, int64_t iz, float u0, float u1, float u2,
                              Sample &s) {
    const double di[3] = {double(ix), double(iy), double(iz)};
    const double du[3] = {double(u0), double(u1), double(u2)};
    int64_t i0[3];
    float f[3];
    const int64_t ii[3] = {ix, iy, iz};
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        double d = fma(g.a[j * 3 + 0], di[0], fma(g.a[j * 3 + 1], di[1], fma(g.a[j * 3 + 2], di[2], g.tv[j])));
        d += fma(g.sv[j * 3 + 0], du[0], fma(g.sv[j * 3 + 1], du[1], g.sv[j * 3 + 2] * du[2]));
        // clamp far-away offsets before the integer conversion (they sample zero)
        d = fmin(fmax(d, -1.0e9), 1.0e9);
        const double fl = floor(d);
        f[j] = float(d - fl);
        i0[j] = ii[j] + int64_t(fl);
    }
    s.fx = f[0];
    s.fy = f[1];
    s.fz = f[2];
    const int64_t x0 = i0[0], y0 = i0[1], z0 = i0[2];
    const bool inside = x0 >= 0 && x0 + 1 < g.mnx && y0 >= 0 && y0 + 1 < g.mny && z0 >= g.sz0 &&
                        z0 + 1 < g.sz0 + g.snz;
    if (inside) {
        const float *b = g.M + ((z0 - g.sz0) * g.mny + y0) * g.mnx + x0;
        const int64_t py = g.mnx, pz = g.mny * g.mnx;
        s.c[0] = b[0];
        s.c[1] = b[1];
        s.c[2] = b[py];
        s.c[3] = b[py + 1];
        s.c[4] = b[pz];
        s.c[5] = b[pz + 1];
        s.c[6] = b[pz + py];
        s.c[7] = b[pz + py + 1];
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int64_t x = x0 + (k & 1), y = y0 + ((k >> 1) & 1), z = z0 + (k >> 2);
            const bool ok = x >= 0 && x < g.mnx && y >= 0 && y < g.mny && z >= g.sz0 && z < g.sz0 + g.snz;
            s.c[k] = ok ? g.M[((z - g.sz0) * g.mny + y) * g.mnx + x] : 0.0f;
        }
    }
}

// Work item = one z-plane's span of kSpan consecutive in-plane voxels. Wave w
// of the block takes the 256 voxels [w*256, w*256 + 256) of the span and lane
// l the voxels l, l+64, l+128, l+192 of those, so every load, gather and
// store instruction is unit-stride across the wave and a thread has 4
// voxels' loads (32 corner gathers) in flight.
#ifndef NGV_WARP_VEC
#define NGV_WARP_VEC 4
#endif
constexpr int kVec = NGV_WARP_VEC;
constexpr int kSpan = kThreads * kVec;

struct Item {
    int64_t z, q[kVec];  // plane and in-plane index of each voxel
    int64_t x[kVec], y[kVec];
    bool ok[kVec];
};

__device__ inline bool item_at(const WarpGeom &g, int64_t it, int64_t spans, Item &m) {
    const int64_t plane = g.onx * g.ony;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t sp = it % spans;
    m.z = it / spans;
    const int64_t q0 = sp * kSpan + wave * (64 * kVec) + lane;
    int64_t y = q0 / g.onx, x = q0 - y * g.onx;
    bool any = false;
#pragma unroll
    for (int k = 0; k < kVec; ++k) {
        m.q[k] = q0 + 64 * k;
        m.ok[k] = m.q[k] < plane;
        any |= m.ok[k];
        m.x[k] = x;
        m.y[k] = y;
        x += 64;
        while (x >= g.onx) {
            x -= g.onx;
            ++y;
        }
    }
    return any;
}

__device__ inline void load4(const float *p, int64_t base, const Item &m, float v[kVec]) {
#pragma unroll
    for (int k = 0; k < kVec; ++k) v[k] = m.ok[k] ? p[base + m.q[k]] : 0.0f;
}

__device__ inline void store4(float *p, int64_t base, const Item &m, const float v[kVec]) {
#pragma unroll
    for (int k = 0; k < kVec; ++k)
        if (m.ok[k]) p[base + m.q[k]] = v[k];
}

__global__ __launch_bounds__(kThreads) void warp_fwd_kernel(WarpGeom g, float *__restrict__ W, int accumulate) {
    const int64_t plane = g.onx * g.ony, ostride = plane * g.onz;
    const int64_t spans = (plane + kSpan - 1) / kSpan;
    const ItemRange r = xcd_items(spans * g.onz);
    for (int64_t it = r.begin; it < r.end; it += r.step) {
        Item m;
        if (!item_at(g, it, spans, m)) continue;
        const int64_t o = m.z * plane;
        float u0[kVec], u1[kVec], u2[kVec], w[kVec];
        load4(g.u, o, m, u0);
        load4(g.u + ostride, o, m, u1);
        load4(g.u + 2 * ostride, o, m, u2);
        Sample s[kVec];
#pragma unroll
        for (int k = 0; k < kVec; ++k) gather(g, m.x[k], m.y[k], m.z, u0[k], u1[k], u2[k], s[k]);
#pragma unroll
        for (int k = 0; k < kVec; ++k) {
            const float e00 = fmaf(s[k].fx, s[k].c[1] - s[k].c[0], s[k].c[0]);
            const float e10 = fmaf(s[k].fx, s[k].c[3] - s[k].c[2], s[k].c[2]);
            const float e01 = fmaf(s[k].fx, s[k].c[5] - s[k].c[4], s[k].c[4]);
            const float e11 = fmaf(s[k].fx, s[k].c[7] - s[k].c[6], s[k].c[6]);
            const float f0 = fmaf(s[k].fy, e10 - e00, e00);
            const float f1 = fmaf(s[k].fy, e11 - e01, e01);
            w[k] = fmaf(s[k].fz, f1 - f0, f0);
        }
        if (accumulate) {
            float old[kVec];
            load4(W, o, m, old);
#pragma unroll
            for (int k = 0; k < kVec; ++k) w[k] += old[k];
        }
        store4(W, o, m, w);
    }
}

// Backward: g_pvox = dW/dp_vox * gW; gu = S_v^T g_pvox; the affine sums are
// accumulated as G_j = sum g_pvox,j and Gi_jk = sum g_pvox,j * i_k (12 sums per
// thread, fp32 within an item, fp64 across items), reduced per block into the
// workspace; warp_bwd_final turns them into dA, dt in a fixed order.
__global__ __launch_bounds__(kThreads) void warp_bwd_kernel(WarpGeom g, const float *__restrict__ gW,
                                                            float *__restrict__ gu, int accumulate,
                                                            double *__restrict__ partials) {
    const int64_t plane = g.onx * g.ony, ostride = plane * g.onz;
    const int64_t spans = (plane + kSpan - 1) / kSpan;
    const ItemRange r = xcd_items(spans * g.onz);
    float sv[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) sv[k] = float(g.sv[k]);
    double acc[12];
#pragma unroll
    for (int k = 0; k < 12; ++k) acc[k] = 0.0;
    for (int64_t it = r.begin; it < r.end; it += r.step) {
        Item m;
        if (!item_at(g, it, spans, m)) continue;
        const int64_t o = m.z * plane;
        float u0[kVec], u1[kVec], u2[kVec], gw[kVec];
        load4(g.u, o, m, u0);
        load4(g.u + ostride, o, m, u1);
        load4(g.u + 2 * ostride, o, m, u2);
        load4(gW, o, m, gw);
        Sample s[kVec];
#pragma unroll
        for (int k = 0; k < kVec; ++k) gather(g, m.x[k], m.y[k], m.z, u0[k], u1[k], u2[k], s[k]);
        float gout[3][kVec];
        float part[12];
#pragma unroll
        for (int k = 0; k < 12; ++k) part[k] = 0.0f;
#pragma unroll
        for (int k = 0; k < kVec; ++k) {
            const Sample &q = s[k];
            const float e00 = fmaf(q.fx, q.c[1] - q.c[0], q.c[0]);
            const float e10 = fmaf(q.fx, q.c[3] - q.c[2], q.c[2]);
            const float e01 = fmaf(q.fx, q.c[5] - q.c[4], q.c[4]);
            const float e11 = fmaf(q.fx, q.c[7] - q.c[6], q.c[6]);
            const float f0 = fmaf(q.fy, e10 - e00, e00);
            const float f1 = fmaf(q.fy, e11 - e01, e01);
            const float dx0 = fmaf(q.fy, (q.c[3] - q.c[2]) - (q.c[1] - q.c[0]), q.c[1] - q.c[0]);
            const float dx1 = fmaf(q.fy, (q.c[7] - q.c[6]) - (q.c[5] - q.c[4]), q.c[5] - q.c[4]);
            const float gvx = fmaf(q.fz, dx1 - dx0, dx0) * gw[k];
            const float gvy = fmaf(q.fz, (e11 - e01) - (e10 - e00), e10 - e00) * gw[k];
            const float gvz = (f1 - f0) * gw[k];
#pragma unroll
            for (int c = 0; c < 3; ++c)
                gout[c][k] = fmaf(sv[0 * 3 + c], gvx, fmaf(sv[1 * 3 + c], gvy, sv[2 * 3 + c] * gvz));
            if (m.ok[k]) {
                const float ii[3] = {float(m.x[k]), float(m.y[k]), float(m.z)};
                const float gp[3] = {gvx, gvy, gvz};
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    part[j] += gp[j];
#pragma unroll
                    for (int c = 0; c < 3; ++c) part[3 + j * 3 + c] = fmaf(gp[j], ii[c], part[3 + j * 3 + c]);
                }
            }
        }
#pragma unroll
        for (int k = 0; k < 12; ++k) acc[k] += double(part[k]);
#pragma unroll
        for (int c = 0; c < 3; ++c) {
            if (accumulate) {
                float old[kVec];
                load4(gu + c * ostride, o, m, old);
#pragma unroll
                for (int k = 0; k < kVec; ++k) gout[c][k] += old[k];
            }
            store4(gu + c * ostride, o, m, gout[c]);
        }
    }
    __shared__ double red[16];
#pragma unroll
    for (int k = 0; k < 12; ++k) {
        const double v = block_sum(acc[k], red);
        if (threadIdx.x == 0) partials[size_t(blockIdx.x) * kPartialStride + k] = v;
    }
}

// One block of 256 threads: thread t sums the partials of blocks t, t+256, ...
// in order, then a fixed-order tree over the threads; finally
//   dt_j = D_j G_j,  dA_jk = D_j (xmin_k G_j + delta_k Gi_jk).
__global__ __launch_bounds__(256) void warp_bwd_final(const double *__restrict__ partials, int nblocks,
                                                      WarpBwdFinal fin, double *__restrict__ gA9,
                                                      double *__restrict__ gt3, int accumulate) {
    __shared__ double red[12][256];
    const int t = threadIdx.x;
    double s[12];
#pragma unroll
    for (int k = 0; k < 12; ++k) s[k] = 0.0;
    for (int b = t; b < nblocks; b += 256)
#pragma unroll
        for (int k = 0; k < 12; ++k) s[k] += partials[size_t(b) * kPartialStride + k];
#pragma unroll
    for (int k = 0; k < 12; ++k) red[k][t] = s[k];
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (t < w)
#pragma unroll
            for (int k = 0; k < 12; ++k) red[k][t] += red[k][t + w];
        __syncthreads();
    }
    if (t < 3) {
        const double dt = fin.dm[t] * red[t][0];
        gt3[t] = accumulate ? gt3[t] + dt : dt;
    } else if (t < 12) {
        const int j = (t - 3) / 3, c = (t - 3) % 3;
        const double da = fin.dm[j] * (fin.xmin[c] * red[j][0] + fin.delta[c] * red[t][0]);
        gA9[j * 3 + c] = accumulate ? gA9[j * 3 + c] + da : da;
    }
}

}  // namespace

hipError_t launch_warp_fwd(const WarpGeom &g, float *W, int accumulate, hipStream_t s) {
    const int64_t plane = g.onx * g.ony;
    const int64_t items = ((plane + kSpan - 1) / kSpan) * g.onz;
    const int blocks = persistent_blocks(items, 8);
    hipLaunchKernelGGL(warp_fwd_kernel, dim3(blocks), dim3(kThreads), 0, s, g, W, accumulate);
    return hipGetLastError();
}

hipError_t launch_warp_bwd(const WarpGeom &g, const float *gW, float *gu, double *gA9, double *gt3,
                           const WarpBwdFinal &fin, int accumulate, void *ws, hipStream_t s) {
    const int64_t plane = g.onx * g.ony;
    const int64_t items = ((plane + kSpan - 1) / kSpan) * g.onz;
    const int blocks = persistent_blocks(items, 8);
    double *partials = reinterpret_cast<double *>(static_cast<char *>(ws) + ws_layout(0).partials);
    hipLaunchKernelGGL(warp_bwd_kernel, dim3(blocks), dim3(kThreads), 0, s, g, gW, gu, accumulate, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(warp_bwd_final, dim3(1), dim3(256), 0, s, partials, blocks, fin, gA9, gt3, accumulate);
    return hipGetLastError();
}

}  // namespace ngv
