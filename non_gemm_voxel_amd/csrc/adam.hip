// Optimiser step on the displacement field ("A Scalable Distributed Framework
// for Multimodal GigaVoxel Image Registration", method overview: optimiser
// states m1, m2 and a gradient step after Sobolev smoothing), as Adam with
// bias correction.
//
// Without smoothing: one streaming pass, float4 over the 3 components.
// With smoothing (normalised Gaussian, taps -R..R, zero padding): one fused
// z-streaming pass, O(1) extra memory. A work item is (component, 32 x 16
// column tile, chunk of planes); per input plane the block convolves the
// tile + R halo along x and y in LDS, each thread keeps the last 2R+1
// xy-smoothed values of its column in registers, and the z tap sum at plane
// zi - R feeds the Adam update of u, m1, m2 there.
#include "ngv_internal.hpp"

namespace ngv {
namespace {

constexpr int kPlain = 256;

__global__ __launch_bounds__(kPlain) void adam_plain_kernel(float *__restrict__ u, const float *__restrict__ g,
                                                            float *__restrict__ m1, float *__restrict__ m2, int64_t n,
                                                            AdamParams p) {
    adam_resolve(p);
    const int64_t per = int64_t(kPlain) * 4;
    const int64_t total = (n + per - 1) / per;
    const ItemRange r = xcd_items(total);
    for (int64_t it = r.begin; it < r.end; it += r.step) {
        const int64_t base = it * per + int64_t(threadIdx.x) * 4;
        if (base + 3 < n) {
            // every array streams through once: non-temporal
            typedef float v4 __attribute__((ext_vector_type(4)));
            v4 uu = __builtin_nontemporal_load(reinterpret_cast<v4 *>(u + base));
            const v4 gg = __builtin_nontemporal_load(reinterpret_cast<const v4 *>(g + base));
            v4 a = __builtin_nontemporal_load(reinterpret_cast<v4 *>(m1 + base));
            v4 b = __builtin_nontemporal_load(reinterpret_cast<v4 *>(m2 + base));
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float x = uu[k], y = a[k], z = b[k];
                adam_one(x, y, z, gg[k], p);
                uu[k] = x;
                a[k] = y;
                b[k] = z;
            }
            __builtin_nontemporal_store(uu, reinterpret_cast<v4 *>(u + base));
            __builtin_nontemporal_store(a, reinterpret_cast<v4 *>(m1 + base));
            __builtin_nontemporal_store(b, reinterpret_cast<v4 *>(m2 + base));
        } else {
            for (int64_t k = base; k < n; ++k) adam_one(u[k], m1[k], m2[k], g[k], p);
        }
    }
}

constexpr int kTX = 32, kTY = 16, kThreads = kTX * kTY;

struct SmoothArgs {
    float *u;
    const float *g;
    float *m1, *m2;
    int64_t nx, ny, nz;
    int64_t tiles_x, tiles_y, chunk, nchunks;
    AdamParams p;
};

template <int R>
__global__ __launch_bounds__(kThreads) void adam_smooth_kernel(SmoothArgs a) {
    adam_resolve(a.p);
    constexpr int W = 2 * R + 1, HX = kTX + 2 * R, HY = kTY + 2 * R;
    __shared__ float raw[HY * HX];
    __shared__ float xs[HY * kTX];
    const int tid = threadIdx.x, tx = tid % kTX, ty = tid / kTX;
    const int64_t plane = a.nx * a.ny, vol = plane * a.nz;
    const int64_t total = 3 * a.tiles_x * a.tiles_y * a.nchunks;
    const ItemRange rng = xcd_items(total);
    for (int64_t it = rng.begin; it < rng.end; it += rng.step) {
        const int64_t bx = it % a.tiles_x, r1 = it / a.tiles_x;
        const int64_t by = r1 % a.tiles_y, r2 = r1 / a.tiles_y;
        const int64_t ch = r2 % a.nchunks, comp = r2 / a.nchunks;
        const int64_t x0 = bx * kTX, y0 = by * kTY;
        const int64_t zs = ch * a.chunk, ze = zs + a.chunk < a.nz ? zs + a.chunk : a.nz;
        const float *gc = a.g + comp * vol;
        const int64_t gxo = x0 + tx, gyo = y0 + ty;
        const bool col_in = gxo < a.nx && gyo < a.ny;
        float ring[W];
#pragma unroll
        for (int k = 0; k < W; ++k) ring[k] = 0.0f;
        const int64_t zbeg = zs - R, zend = ze + R;
        for (int64_t zb = zbeg; zb < zend; zb += W) {
#pragma unroll
            for (int slot = 0; slot < W; ++slot) {
                const int64_t zi = zb + slot;
                if (zi >= zend) break;
                const bool zin = zi >= 0 && zi < a.nz;
                for (int q = tid; q < HX * HY; q += kThreads) {
                    const int hx = q % HX, hy = q / HX;
                    const int64_t gx = x0 - R + hx, gy = y0 - R + hy;
                    float v = 0.0f;
                    if (zin && gx >= 0 && gx < a.nx && gy >= 0 && gy < a.ny) v = gc[zi * plane + gy * a.nx + gx];
                    raw[q] = v;
                }
                __syncthreads();
                for (int q = tid; q < HY * kTX; q += kThreads) {
                    const int ox = q % kTX, hy = q / kTX;
                    float s = 0.0f;
#pragma unroll
                    for (int k = 0; k < W; ++k) s = fmaf(a.p.taps[k], raw[hy * HX + ox + k], s);
                    xs[q] = s;
                }
                __syncthreads();
                float s = 0.0f;
#pragma unroll
                for (int k = 0; k < W; ++k) s = fmaf(a.p.taps[k], xs[(ty + k) * kTX + tx], s);
                ring[slot] = s;
                // z taps for plane zo = zi - R: planes zi-2R .. zi sit in slots
                // slot+1, ..., slot+2R+1 (mod W), oldest first
                const int64_t zo = zi - R;
                if (col_in && zo >= zs && zo < ze) {
                    float g = 0.0f;
#pragma unroll
                    for (int k = 0; k < W; ++k) g = fmaf(a.p.taps[k], ring[(slot + 1 + k) % W], g);
                    const int64_t o = comp * vol + zo * plane + gyo * a.nx + gxo;
                    float uu = a.u[o], mm1 = __builtin_nontemporal_load(a.m1 + o),
                          mm2 = __builtin_nontemporal_load(a.m2 + o);
                    adam_one(uu, mm1, mm2, g, a.p);
                    __builtin_nontemporal_store(uu, a.u + o);
                    __builtin_nontemporal_store(mm1, a.m1 + o);
                    __builtin_nontemporal_store(mm2, a.m2 + o);
                }
                // no trailing barrier: the next plane writes raw (read only
                // before this plane's second barrier) and then xs only after
                // its own first barrier, which follows every read of xs here
            }
        }
    }
}

__global__ __launch_bounds__(64) void adam_bc_kernel(const int32_t *__restrict__ step_dev, float beta1, float beta2,
                                                     float *__restrict__ bc) {
    if (threadIdx.x != 0) return;
    const int t = *step_dev < 1 ? 1 : *step_dev;
    bc[0] = float(1.0 / (1.0 - pow(double(beta1), double(t))));
    bc[1] = float(1.0 / (1.0 - pow(double(beta2), double(t))));
}

}  // namespace

hipError_t launch_adam_bc(const int32_t *step_dev, float beta1, float beta2, float *bc, hipStream_t s) {
    hipLaunchKernelGGL(adam_bc_kernel, dim3(1), dim3(64), 0, s, step_dev, beta1, beta2, bc);
    return hipGetLastError();
}

hipError_t launch_adam(float *u, const float *gu, float *m1, float *m2, int64_t nx, int64_t ny, int64_t nz,
                       const AdamParams &p, hipStream_t s) {
    if (p.radius == 0) {
        const int64_t n = 3 * nx * ny * nz;
        const int64_t items = (n + kPlain * 4 - 1) / (kPlain * 4);
        hipLaunchKernelGGL(adam_plain_kernel, dim3(persistent_blocks(items, 8)), dim3(kPlain), 0, s, u, gu, m1, m2,
                           n, p);
        return hipGetLastError();
    }
    SmoothArgs a;
    a.u = u;
    a.g = gu;
    a.m1 = m1;
    a.m2 = m2;
    a.nx = nx;
    a.ny = ny;
    a.nz = nz;
    a.tiles_x = (nx + kTX - 1) / kTX;
    a.tiles_y = (ny + kTY - 1) / kTY;
    const int64_t tiles = 3 * a.tiles_x * a.tiles_y;
    int64_t chunk = (nz * tiles + 4 * device_info().cus - 1) / (4 * device_info().cus);
    if (chunk < 8) chunk = 8;
    if (chunk > 64) chunk = 64;
    a.chunk = chunk;
    a.nchunks = (nz + chunk - 1) / chunk;
    a.p = p;
    const int64_t items = tiles * a.nchunks;
    const int blocks = persistent_blocks(items, 2);
    switch (p.radius) {
        case 1: hipLaunchKernelGGL(adam_smooth_kernel<1>, dim3(blocks), dim3(kThreads), 0, s, a); break;
        case 2: hipLaunchKernelGGL(adam_smooth_kernel<2>, dim3(blocks), dim3(kThreads), 0, s, a); break;
        case 3: hipLaunchKernelGGL(adam_smooth_kernel<3>, dim3(blocks), dim3(kThreads), 0, s, a); break;
        case 4: hipLaunchKernelGGL(adam_smooth_kernel<4>, dim3(blocks), dim3(kThreads), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ngv
