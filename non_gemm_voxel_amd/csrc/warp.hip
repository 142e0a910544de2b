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
// Work decomposition: items are 64 (x) by 4 (y) output tiles of one z-plane,
// one wave per x-row, so loads of u and stores of W / gu are whole 256-byte
// rows. A persistent grid walks the items in XCD-contiguous ranges (so the
// M rows a tile gathers from are shared with its neighbours in one L2).
#include "ngv_internal.hpp"

namespace ngv {
namespace {

constexpr int kTX = 64, kTY = 4, kThreads = kTX * kTY;

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

__device__ inline int64_t tiles_total(const WarpGeom &g, int64_t &tiles_x, int64_t &tiles_y) {
    tiles_x = (g.onx + kTX - 1) / kTX;
    tiles_y = (g.ony + kTY - 1) / kTY;
    return tiles_x * tiles_y * g.onz;
}

__global__ __launch_bounds__(kThreads) void warp_fwd_kernel(WarpGeom g, float *__restrict__ W, int accumulate) {
    int64_t tiles_x, tiles_y;
    const int64_t total = tiles_total(g, tiles_x, tiles_y);
    const ItemRange r = xcd_items(total);
    const int lx = threadIdx.x % kTX, ly = threadIdx.x / kTX;
    const int64_t ostride = g.onx * g.ony * g.onz;
    for (int64_t it = r.begin; it < r.end; it += r.step) {
        const int64_t tx = it % tiles_x, rest = it / tiles_x;
        const int64_t ty = rest % tiles_y, iz = rest / tiles_y;
        const int64_t ix = tx * kTX + lx, iy = ty * kTY + ly;
        if (ix >= g.onx || iy >= g.ony) continue;
        const int64_t lin = (iz * g.ony + iy) * g.onx + ix;
        Sample s;
        gather(g, ix, iy, iz, g.u[lin], g.u[lin + ostride], g.u[lin + 2 * ostride], s);
        const float e00 = fmaf(s.fx, s.c[1] - s.c[0], s.c[0]);
        const float e10 = fmaf(s.fx, s.c[3] - s.c[2], s.c[2]);
        const float e01 = fmaf(s.fx, s.c[5] - s.c[4], s.c[4]);
        const float e11 = fmaf(s.fx, s.c[7] - s.c[6], s.c[6]);
        const float f0 = fmaf(s.fy, e10 - e00, e00);
        const float f1 = fmaf(s.fy, e11 - e01, e01);
        float w = fmaf(s.fz, f1 - f0, f0);
        if (accumulate) w += W[lin];
        W[lin] = w;
    }
}

// Backward: g_pvox = dW/dp_vox * gW; gu = S_v^T g_pvox; the affine sums are
// accumulated as G_j = sum g_pvox,j and Gi_jk = sum g_pvox,j * i_k (12 sums per
// thread, fp32 over batches of items, fp64 beyond), reduced per block into
// the workspace; warp_bwd_final turns them into dA, dt in a fixed order.
constexpr int kFlushEvery = 16;

__global__ __launch_bounds__(kThreads) void warp_bwd_kernel(WarpGeom g, const float *__restrict__ gW,
                                                            float *__restrict__ gu, int accumulate,
                                                            double *__restrict__ partials) {
    int64_t tiles_x, tiles_y;
    const int64_t total = tiles_total(g, tiles_x, tiles_y);
    const ItemRange r = xcd_items(total);
    const int lx = threadIdx.x % kTX, ly = threadIdx.x / kTX;
    const int64_t ostride = g.onx * g.ony * g.onz;
    double acc[12];
    float part[12];
#pragma unroll
    for (int k = 0; k < 12; ++k) {
        acc[k] = 0.0;
        part[k] = 0.0f;
    }
    int batch = 0;
    for (int64_t it = r.begin; it < r.end; it += r.step) {
        const int64_t tx = it % tiles_x, rest = it / tiles_x;
        const int64_t ty = rest % tiles_y, iz = rest / tiles_y;
        const int64_t ix = tx * kTX + lx, iy = ty * kTY + ly;
        if (ix < g.onx && iy < g.ony) {
            const int64_t lin = (iz * g.ony + iy) * g.onx + ix;
            Sample s;
            gather(g, ix, iy, iz, g.u[lin], g.u[lin + ostride], g.u[lin + 2 * ostride], s);
            const float e00 = fmaf(s.fx, s.c[1] - s.c[0], s.c[0]);
            const float e10 = fmaf(s.fx, s.c[3] - s.c[2], s.c[2]);
            const float e01 = fmaf(s.fx, s.c[5] - s.c[4], s.c[4]);
            const float e11 = fmaf(s.fx, s.c[7] - s.c[6], s.c[6]);
            const float f0 = fmaf(s.fy, e10 - e00, e00);
            const float f1 = fmaf(s.fy, e11 - e01, e01);
            const float dx0 = fmaf(s.fy, (s.c[3] - s.c[2]) - (s.c[1] - s.c[0]), s.c[1] - s.c[0]);
            const float dx1 = fmaf(s.fy, (s.c[7] - s.c[6]) - (s.c[5] - s.c[4]), s.c[5] - s.c[4]);
            const float dwx = fmaf(s.fz, dx1 - dx0, dx0);
            const float dwy = fmaf(s.fz, (e11 - e01) - (e10 - e00), e10 - e00);
            const float dwz = f1 - f0;
            const float gw = gW[lin];
            const float gp[3] = {dwx * gw, dwy * gw, dwz * gw};
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                float v = fmaf(float(g.sv[0 * 3 + k]), gp[0], fmaf(float(g.sv[1 * 3 + k]), gp[1], float(g.sv[2 * 3 + k]) * gp[2]));
                float *dst = gu + lin + k * ostride;
                if (accumulate) v += *dst;
                *dst = v;
            }
            const float ii[3] = {float(ix), float(iy), float(iz)};
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                part[j] += gp[j];
#pragma unroll
                for (int k = 0; k < 3; ++k) part[3 + j * 3 + k] = fmaf(gp[j], ii[k], part[3 + j * 3 + k]);
            }
        }
        if (++batch == kFlushEvery) {
            batch = 0;
#pragma unroll
            for (int k = 0; k < 12; ++k) {
                acc[k] += double(part[k]);
                part[k] = 0.0f;
            }
        }
    }
    __shared__ double red[16];
#pragma unroll
    for (int k = 0; k < 12; ++k) {
        const double v = block_sum(acc[k] + double(part[k]), red);
        if (threadIdx.x == 0) partials[size_t(blockIdx.x) * kPartialStride + k] = v;
    }
}

// One block: sums the per-block partials in block order and writes
//   dt_j = D_j G_j,  dA_jk = D_j (xmin_k G_j + delta_k Gi_jk).
__global__ __launch_bounds__(64) void warp_bwd_final(const double *__restrict__ partials, int nblocks,
                                                     WarpBwdFinal fin, double *__restrict__ gA9,
                                                     double *__restrict__ gt3, int accumulate) {
    __shared__ double sum[12];
    const int k = threadIdx.x;
    if (k < 12) {
        double s = 0.0;
        for (int b = 0; b < nblocks; ++b) s += partials[size_t(b) * kPartialStride + k];
        sum[k] = s;
    }
    __syncthreads();
    if (k < 3) {
        const double dt = fin.dm[k] * sum[k];
        gt3[k] = accumulate ? gt3[k] + dt : dt;
    } else if (k < 12) {
        const int j = (k - 3) / 3, c = (k - 3) % 3;
        const double da = fin.dm[j] * (fin.xmin[c] * sum[j] + fin.delta[c] * sum[k]);
        gA9[j * 3 + c] = accumulate ? gA9[j * 3 + c] + da : da;
    }
}

}  // namespace

hipError_t launch_warp_fwd(const WarpGeom &g, float *W, int accumulate, hipStream_t s) {
    const int64_t items = ((g.onx + kTX - 1) / kTX) * ((g.ony + kTY - 1) / kTY) * g.onz;
    const int blocks = persistent_blocks(items, 8);
    hipLaunchKernelGGL(warp_fwd_kernel, dim3(blocks), dim3(kThreads), 0, s, g, W, accumulate);
    return hipGetLastError();
}

hipError_t launch_warp_bwd(const WarpGeom &g, const float *gW, float *gu, double *gA9, double *gt3,
                           const WarpBwdFinal &fin, int accumulate, void *ws, hipStream_t s) {
    const int64_t items = ((g.onx + kTX - 1) / kTX) * ((g.ony + kTY - 1) / kTY) * g.onz;
    const int blocks = persistent_blocks(items, 8);
    double *partials = reinterpret_cast<double *>(static_cast<char *>(ws) + ws_layout(0).partials);
    hipLaunchKernelGGL(warp_bwd_kernel, dim3(blocks), dim3(kThreads), 0, s, g, gW, gu, accumulate, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(warp_bwd_final, dim3(1), dim3(64), 0, s, partials, blocks, fin, gA9, gt3, accumulate);
    return hipGetLastError();
}

}  // namespace ngv
