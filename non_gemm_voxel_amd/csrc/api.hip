// The C ABI of libngv.so: argument checks, the fp64 preparation of the
// sampler's voxel-space parameters, and the kernel launches. See ngv.h for
// the contract of every call.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "ngv_internal.hpp"

namespace ngv {

namespace {
thread_local std::string g_last_hip;
thread_local std::string g_status;

int hip_fail(hipError_t e) {
    g_last_hip = hipGetErrorString(e);
    return NGV_EHIP;
}

// Number of voxels of a grid, computed without overflow (0 for a null grid).
unsigned __int128 voxels(const ngv_dims *d) {
    return d ? (unsigned __int128)d->nx * (unsigned __int128)d->ny * (unsigned __int128)d->nz : 0;
}

// Every extent in [1, 2^31] and the volume at most 2^62 voxels, so that
// 64-bit index arithmetic cannot overflow.
bool dims_ok(const ngv_dims *d) {
    return d && d->nx >= 1 && d->ny >= 1 && d->nz >= 1 && d->nx <= (int64_t(1) << 31) &&
           d->ny <= (int64_t(1) << 31) && d->nz <= (int64_t(1) << 31) && voxels(d) <= ((unsigned __int128)1 << 62);
}

// The MI histogram holds each bin in 32.32 fixed point in 64 bits, and its
// entries sum to N * 2^32: N must stay below 2^32 voxels.
bool mi_size_ok(const ngv_dims *d) { return voxels(d) < ((unsigned __int128)1 << 32); }

bool finite(float v) { return std::isfinite(v); }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_ws(void *ws, size_t ws_bytes, size_t need) {
    if (!ws || !aligned(ws, 256) || ws_bytes < need) return NGV_EWORKSPACE;
    return NGV_OK;
}
}  // namespace

const DeviceInfo &device_info() {
    static std::mutex mu;
    static std::vector<DeviceInfo> cache;
    static std::vector<bool> have;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    std::lock_guard<std::mutex> lock(mu);
    if (int(cache.size()) <= dev) {
        cache.resize(dev + 1);
        have.resize(dev + 1, false);
    }
    if (!have[dev]) {
        DeviceInfo info;
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) info.cus = v;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess && v > 0)
            info.max_lds = size_t(v);
        cache[dev] = info;
        have[dev] = true;
    }
    return cache[dev];
}

// Voxel-space form of the composite map, in fp64 from the fp32 inputs:
//   p_vox = i + (A_v - I) i + t_v + S_v u
// with D = diag((n_M - 1)/2), delta = (xmax - xmin)/(n_O - 1):
//   A_v - I = (diag(D delta) - I) + D (A - I) diag(delta)
//   t_v     = D ((xmin + 1) + (A - I) xmin + t)
//   S_v     = D S
// The identity map on equal grids with bounds (-1, 1) gives exactly zero.
// The sampler's index arithmetic is 32-bit: every extent of both grids at
// most 2^30 and a moving-image plane below 2^31 voxels.
static bool sampler_size_ok(const ngv_dims *md, const ngv_dims *od) {
    const int64_t lim = int64_t(1) << 30;
    return md->nx <= lim && md->ny <= lim && md->nz <= lim && od->nx <= lim && od->ny <= lim && od->nz <= lim &&
           md->nx * md->ny < (int64_t(1) << 31);
}

// NGV_OK, NGV_EINVAL (non-finite map) or NGV_EUNSUPPORTED (sizes).
static int prepare_warp(const float *M, const ngv_dims *md, const ngv_slab *slab, const float *u,
                        const ngv_dims *od, const ngv_xform *xf, WarpGeom &g, WarpBwdFinal *fin) {
    for (int k = 0; k < 9; ++k)
        if (!finite(xf->A[k]) || !finite(xf->S[k])) return NGV_EINVAL;
    for (int k = 0; k < 3; ++k)
        if (!finite(xf->t[k]) || !finite(xf->xmin[k]) || !finite(xf->xmax[k])) return NGV_EINVAL;
    if (!sampler_size_ok(md, od)) return NGV_EUNSUPPORTED;
    const double mn[3] = {double(md->nx), double(md->ny), double(md->nz)};
    const double on[3] = {double(od->nx), double(od->ny), double(od->nz)};
    double D[3], delta[3], sigma[3], xmin[3];
    for (int k = 0; k < 3; ++k) {
        xmin[k] = xf->xmin[k];
        D[k] = (mn[k] - 1.0) / 2.0;
        const double span = double(xf->xmax[k]) - double(xf->xmin[k]);
        delta[k] = on[k] > 1.0 ? span / (on[k] - 1.0) : 0.0;
        sigma[k] = on[k] > 1.0 ? (mn[k] - 1.0) * span / (2.0 * (on[k] - 1.0)) : 0.0;
    }
    for (int j = 0; j < 3; ++j) {
        double tv = (xmin[j] + 1.0) + double(xf->t[j]);
        for (int k = 0; k < 3; ++k) {
            const double am = double(xf->A[j * 3 + k]) - (j == k ? 1.0 : 0.0);
            double v = (j == k ? sigma[j] - 1.0 : 0.0) + D[j] * am * delta[k];
            g.a[j * 3 + k] = v;
            tv += am * xmin[k];
            g.sv[j * 3 + k] = D[j] * double(xf->S[j * 3 + k]);
        }
        g.tv[j] = D[j] * tv;
    }
    g.M = M;
    g.mnx = md->nx;
    g.mny = md->ny;
    g.mnz = md->nz;
    g.sz0 = slab ? slab->z0 : 0;
    g.snz = slab ? slab->nz : md->nz;
    g.zrange = slab ? slab->zrange : nullptr;
    g.u = u;
    g.onx = od->nx;
    g.ony = od->ny;
    g.onz = od->nz;
    if (fin) {
        for (int k = 0; k < 3; ++k) {
            fin->dm[k] = D[k];
            fin->xmin[k] = xmin[k];
            fin->delta[k] = delta[k];
        }
    }
    return NGV_OK;
}

static int mi_params(int bins, float fmin, float fmax, float wmin, float wmax, float weight, MiParams &p,
                     int fixed_order = 3) {
    if (bins < 8 || bins > kMaxBins) return NGV_EINVAL;
    if (fixed_order != 0 && fixed_order != 3) return NGV_EINVAL;
    p.f_order = fixed_order;
    if (!finite(fmin) || !finite(fmax) || !finite(wmin) || !finite(wmax) || !finite(weight)) return NGV_EINVAL;
    if (!(fmax > fmin) || !(wmax > wmin)) return NGV_EINVAL;
    p.bins = bins;
    p.f_lo = fmin;
    p.f_hi = fmax;
    p.f_scale = float(double(bins - 5) / (double(fmax) - double(fmin)));
    p.w_lo = wmin;
    p.w_hi = wmax;
    p.w_scale = float(double(bins - 5) / (double(wmax) - double(wmin)));
    p.weight = weight;
    return NGV_OK;
}

static bool slab_ok(const ngv_slab *slab, const ngv_dims *md) {
    return !slab || (slab->z0 >= 0 && slab->nz >= 1 && slab->z0 + slab->nz <= md->nz &&
                     (!slab->zrange || aligned(slab->zrange, 8)));
}

}  // namespace ngv

// Scratch of ngv_mi_loss_fwd_bwd_noalloc: the MI joint histogram (bins^2
// u64) and log-ratio table (bins^2 f32) for up to kNoAllocBins bins, one copy
// per GPU in the library's device memory, held until the process ends. In
// host code `scratch` names a host-side stand-in: its device address comes
// from hipGetSymbolAddress (noalloc_scratch), once per device.
namespace ngv {
constexpr int kNoAllocBins = 128;
constexpr size_t kNoAllocHistBytes = size_t(kNoAllocBins) * kNoAllocBins * sizeof(unsigned long long);  // 128 KiB
constexpr size_t kNoAllocScratchBytes = kNoAllocHistBytes + size_t(kNoAllocBins) * kNoAllocBins * sizeof(float);
static_assert(kNoAllocHistBytes % 256 == 0, "table 256-byte aligned");
}  // namespace ngv

static __device__ __align__(256) unsigned char scratch[ngv::kNoAllocScratchBytes];

namespace ngv {
// The device address of `scratch` on the current device, looked up on the
// first call on each device and kept.
static int noalloc_scratch(char **out) {
    static std::mutex mu;
    static std::vector<char *> ptrs;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    std::lock_guard<std::mutex> lock(mu);
    if (int(ptrs.size()) <= dev) ptrs.resize(dev + 1, nullptr);
    if (!ptrs[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e);
        if (!ptr) return NGV_EHIP;
        ptrs[dev] = static_cast<char *>(ptr);
    }
    *out = ptrs[dev];
    return NGV_OK;
}
}  // namespace ngv

using namespace ngv;

extern "C" {

size_t ngv_workspace_bytes(int bins, int win) {
    const int b = bins > 0 ? (bins < kMaxBins ? bins : kMaxBins) : 0;
    const int bmax = b > 32 ? b : 32;
    size_t total = ws_layout(bmax).total;
    if (win >= 13 && win <= 31 && win % 2 == 1) {
        const size_t big = lncc_big_offset() + lncc_big_bytes(win);
        if (big > total) total = big;
    }
    return total;
}

const char *ngv_status_str(int status) {
    switch (status) {
        case NGV_OK: g_status = "ok"; break;
        case NGV_EINVAL: g_status = "invalid argument"; break;
        case NGV_EWORKSPACE: g_status = "workspace missing, too small or not 256-byte aligned"; break;
        case NGV_EHIP: g_status = "HIP error: " + g_last_hip; break;
        case NGV_EUNSUPPORTED: g_status = "unsupported parameters"; break;
        default: g_status = "unknown status " + std::to_string(status); break;
    }
    return g_status.c_str();
}

int ngv_warp_fwd(const float *M, const ngv_dims *md, const ngv_slab *slab, const float *u, const ngv_dims *od,
                 const ngv_xform *xf, float *W, int accumulate, void *stream) {
    if (!M || !u || !W || !xf || !dims_ok(md) || !dims_ok(od) || !slab_ok(slab, md)) return NGV_EINVAL;
    if (accumulate != 0 && accumulate != 1) return NGV_EINVAL;
    WarpGeom g;
    if (int e = prepare_warp(M, md, slab, u, od, xf, g, nullptr)) return e;
    hipError_t e = launch_warp_fwd(g, W, accumulate, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NGV_OK : hip_fail(e);
}

int ngv_warp_fwd_slab(const float *M, const ngv_dims *md, const ngv_slab *slab, const float *u,
                      const ngv_dims *od, const ngv_xform *xf, float *W, void *stream) {
    if (!M || !u || !W || !xf || !dims_ok(md) || !dims_ok(od) || !slab_ok(slab, md) || !slab || !slab->zrange)
        return NGV_EINVAL;
    WarpGeom g;
    if (int e = prepare_warp(M, md, slab, u, od, xf, g, nullptr)) return e;
    hipError_t e = launch_warp_fwd_seq(g, W, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NGV_OK : hip_fail(e);
}

int ngv_warp_bwd(const float *M, const ngv_dims *md, const ngv_slab *slab, const float *u, const ngv_dims *od,
                 const ngv_xform *xf, const float *gW, float *gu, double *gA9, double *gt3, int accumulate, void *ws,
                 size_t ws_bytes, void *stream) {
    if (!M || !u || !gW || !gu || !gA9 || !gt3 || !xf || !dims_ok(md) || !dims_ok(od) || !slab_ok(slab, md))
        return NGV_EINVAL;
    if (accumulate != 0 && accumulate != 1) return NGV_EINVAL;
    int st = check_ws(ws, ws_bytes, ngv_workspace_bytes(0, 0));
    if (st != NGV_OK) return st;
    WarpGeom g;
    WarpBwdFinal fin;
    if (int e = prepare_warp(M, md, slab, u, od, xf, g, &fin)) return e;
    hipError_t e = launch_warp_bwd(g, gW, gu, gA9, gt3, fin, accumulate, ws, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NGV_OK : hip_fail(e);
}

int ngv_mi_loss_fwd_bwd(const float *F, const float *W, const ngv_dims *d, int bins, float fmin, float fmax,
                        float wmin, float wmax, float weight, double *loss, float *gW, int accumulate, void *ws,
                        size_t ws_bytes, void *stream) {
    if (!F || !W || !loss || !dims_ok(d)) return NGV_EINVAL;
    if (accumulate != 0 && accumulate != 1) return NGV_EINVAL;
    if (!aligned(F, 16) || !aligned(W, 16) || (gW && !aligned(gW, 16))) return NGV_EINVAL;
    MiParams p;
    int st = mi_params(bins, fmin, fmax, wmin, wmax, weight, p);
    if (st != NGV_OK) return st;
    st = check_ws(ws, ws_bytes, ngv_workspace_bytes(bins, 0));
    if (st != NGV_OK) return st;
    if (!mi_size_ok(d)) return NGV_EUNSUPPORTED;
    const WsLayout l = ws_layout(bins);
    char *base = static_cast<char *>(ws);
    hipError_t e = launch_mi(F, W, d->nx * d->ny, d->nz, p, loss, gW, accumulate,
                             reinterpret_cast<unsigned long long *>(base + l.hist),
                             reinterpret_cast<float *>(base + l.table), static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NGV_OK : hip_fail(e);
}

int ngv_mi_loss_fwd_bwd_order(const float *F, const float *W, const ngv_dims *d, int bins, int fixed_order,
                              float fmin, float fmax, float wmin, float wmax, float weight, double *loss, float *gW,
                              int accumulate, void *ws, size_t ws_bytes, void *stream) {
    if (!F || !W || !loss || !dims_ok(d)) return NGV_EINVAL;
    if (accumulate != 0 && accumulate != 1) return NGV_EINVAL;
    if (!aligned(F, 16) || !aligned(W, 16) || (gW && !aligned(gW, 16))) return NGV_EINVAL;
    MiParams p;
    int st = mi_params(bins, fmin, fmax, wmin, wmax, weight, p, fixed_order);
    if (st != NGV_OK) return st;
    st = check_ws(ws, ws_bytes, ngv_workspace_bytes(bins, 0));
    if (st != NGV_OK) return st;
    if (!mi_size_ok(d)) return NGV_EUNSUPPORTED;
    const WsLayout l = ws_layout(bins);
    char *base = static_cast<char *>(ws);
    hipError_t e = launch_mi(F, W, d->nx * d->ny, d->nz, p, loss, gW, accumulate,
                             reinterpret_cast<unsigned long long *>(base + l.hist),
                             reinterpret_cast<float *>(base + l.table), static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NGV_OK : hip_fail(e);
}

int ngv_mi_loss_fwd_bwd_noalloc(const float *F, const float *W, const ngv_dims *d, int bins, float fmin, float fmax,
                                float wmin, float wmax, float weight, double *loss, float *gW, int accumulate,
                                void *stream) {
    if (!F || !W || !loss || !dims_ok(d)) return NGV_EINVAL;
    if (accumulate != 0 && accumulate != 1) return NGV_EINVAL;
    if (!aligned(F, 16) || !aligned(W, 16) || (gW && !aligned(gW, 16))) return NGV_EINVAL;
    MiParams p;
    int st = mi_params(bins, fmin, fmax, wmin, wmax, weight, p);
    if (st != NGV_OK) return st;
    if (bins > kNoAllocBins || !mi_size_ok(d)) return NGV_EUNSUPPORTED;
    char *sc = nullptr;
    st = noalloc_scratch(&sc);
    if (st != NGV_OK) return st;
    // the histogram is zeroed by a kernel at the start of the call; the table
    // is written whole before it is read
    hipError_t e = launch_mi(F, W, d->nx * d->ny, d->nz, p, loss, gW, accumulate,
                             reinterpret_cast<unsigned long long *>(sc),
                             reinterpret_cast<float *>(sc + kNoAllocHistBytes), static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NGV_OK : hip_fail(e);
}

int ngv_lncc_loss_fwd_bwd(const float *F, const float *W, const ngv_dims *d, int win, float eps, float weight,
                          double *loss, float *gW, int accumulate, void *ws, size_t ws_bytes, void *stream) {
    if (!F || !W || !loss || !dims_ok(d)) return NGV_EINVAL;
    if (win < 3 || win % 2 == 0 || win > 31) return NGV_EINVAL;
    if (!finite(eps) || eps < 0.0f || !finite(weight)) return NGV_EINVAL;
    if (accumulate != 0 && accumulate != 1) return NGV_EINVAL;
    int st = check_ws(ws, ws_bytes, ngv_workspace_bytes(0, win));
    if (st != NGV_OK) return st;
    hipError_t e = launch_lncc(F, W, d->nx, d->ny, d->nz, win, eps, weight, loss, gW, accumulate, ws,
                               static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NGV_OK : hip_fail(e);
}

// With a device step number the bias corrections are formed on the device,
// into the workspace, by a one-thread kernel enqueued before the update
// (adam_enqueue_bc); the update kernels read them from there.
static int adam_params(int step, const int32_t *step_dev, float lr, float beta1, float beta2, float eps,
                       float smooth_sigma, void *ws, AdamParams &p) {
    if (step_dev ? !aligned(step_dev, 4) : step < 1) return NGV_EINVAL;
    if (step_dev) step = 1;  // placeholder: the kernels read the device values
    if (!finite(lr) || !finite(beta1) || !finite(beta2) || !finite(eps) || !finite(smooth_sigma)) return NGV_EINVAL;
    if (beta1 < 0.0f || beta1 >= 1.0f || beta2 < 0.0f || beta2 >= 1.0f || eps < 0.0f || smooth_sigma < 0.0f)
        return NGV_EINVAL;
    p.lr = lr;
    p.beta1 = beta1;
    p.beta2 = beta2;
    p.eps = eps;
    p.inv_bc1 = float(1.0 / (1.0 - std::pow(double(beta1), double(step))));
    p.inv_bc2 = float(1.0 / (1.0 - std::pow(double(beta2), double(step))));
    p.bc = step_dev ? reinterpret_cast<const float *>(static_cast<const char *>(ws) + ws_layout(0).adam) : nullptr;
    p.radius = 0;
    for (int k = 0; k < 9; ++k) p.taps[k] = 0.0f;
    if (smooth_sigma > 0.0f) {
        const int R = int(std::ceil(3.0 * double(smooth_sigma)));
        if (R > 4) return NGV_EUNSUPPORTED;
        double t[9], tot = 0.0;
        for (int k = -R; k <= R; ++k) {
            t[k + R] = std::exp(-double(k * k) / (2.0 * double(smooth_sigma) * double(smooth_sigma)));
            tot += t[k + R];
        }
        for (int k = 0; k <= 2 * R; ++k) p.taps[k] = float(t[k] / tot);
        p.radius = R;
    }
    return NGV_OK;
}

static hipError_t adam_enqueue_bc(const int32_t *step_dev, const AdamParams &p, hipStream_t s) {
    return step_dev ? launch_adam_bc(step_dev, p.beta1, p.beta2, const_cast<float *>(p.bc), s) : hipSuccess;
}

int ngv_adam_step(float *u, const float *gu, float *m1, float *m2, const ngv_dims *d, int step,
                  const int32_t *step_dev, float lr, float beta1, float beta2, float eps, float smooth_sigma, void *ws,
                  size_t ws_bytes, void *stream) {
    if (!u || !gu || !m1 || !m2 || !dims_ok(d)) return NGV_EINVAL;
    if (!aligned(u, 16) || !aligned(gu, 16) || !aligned(m1, 16) || !aligned(m2, 16)) return NGV_EINVAL;
    AdamParams p;
    int st = adam_params(step, step_dev, lr, beta1, beta2, eps, smooth_sigma, ws, p);
    if (st != NGV_OK) return st;
    if (step_dev) {  // the workspace holds the device-side bias corrections
        st = check_ws(ws, ws_bytes, ngv_workspace_bytes(0, 0));
        if (st != NGV_OK) return st;
    }
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = adam_enqueue_bc(step_dev, p, s);
    if (e == hipSuccess) e = launch_adam(u, gu, m1, m2, d->nx, d->ny, d->nz, p, s);
    return e == hipSuccess ? NGV_OK : hip_fail(e);
}

int ngv_warp_bwd_adam(const float *M, const ngv_dims *md, const ngv_slab *slab, float *u, const ngv_dims *od,
                      const ngv_xform *xf, const float *gW, const float *gu_partial, float *m1, float *m2, int step,
                      const int32_t *step_dev, float lr, float beta1, float beta2, float eps, double *gA9, double *gt3,
                      int accumulate_affine, void *ws, size_t ws_bytes, void *stream) {
    if (!M || !u || !gW || !m1 || !m2 || !gA9 || !gt3 || !xf || !dims_ok(md) || !dims_ok(od) || !slab_ok(slab, md))
        return NGV_EINVAL;
    if (accumulate_affine != 0 && accumulate_affine != 1) return NGV_EINVAL;
    int st = check_ws(ws, ws_bytes, ngv_workspace_bytes(0, 0));
    if (st != NGV_OK) return st;
    AdamFuse f;
    st = adam_params(step, step_dev, lr, beta1, beta2, eps, 0.0f, ws, f.p);
    if (st != NGV_OK) return st;
    WarpGeom g;
    WarpBwdFinal fin;
    if (int e = prepare_warp(M, md, slab, u, od, xf, g, &fin)) return e;
    f.u = u;
    f.m1 = m1;
    f.m2 = m2;
    f.accumulate_affine = accumulate_affine;
    f.slab_mode = 0;
    hipError_t e = adam_enqueue_bc(step_dev, f.p, static_cast<hipStream_t>(stream));
    if (e == hipSuccess)
        e = launch_warp_bwd(g, gW, const_cast<float *>(gu_partial), gA9, gt3, fin, gu_partial ? 1 : 0, ws,
                            static_cast<hipStream_t>(stream), &f);
    return e == hipSuccess ? NGV_OK : hip_fail(e);
}

int ngv_warp_bwd_adam_mi(const float *M, const ngv_dims *md, float *u, const ngv_dims *od, const ngv_xform *xf,
                         const float *F, const float *gW, int bins, float fmin, float fmax, float wmin, float wmax,
                         float weight, float *m1, float *m2, int step, const int32_t *step_dev, float lr, float beta1,
                         float beta2, float eps, double *gA9, double *gt3, int accumulate_affine, void *ws,
                         size_t ws_bytes, void *stream) {
    if (!M || !u || !F || !m1 || !m2 || !gA9 || !gt3 || !xf || !dims_ok(md) || !dims_ok(od)) return NGV_EINVAL;
    if (accumulate_affine != 0 && accumulate_affine != 1) return NGV_EINVAL;
    MiFuse mf;
    int st = mi_params(bins, fmin, fmax, wmin, wmax, weight, mf.p);
    if (st != NGV_OK) return st;
    st = check_ws(ws, ws_bytes, ngv_workspace_bytes(bins, 0));
    if (st != NGV_OK) return st;
    if (!mi_size_ok(od) || bins > kMaxLdsBins) return NGV_EUNSUPPORTED;
    AdamFuse f;
    st = adam_params(step, step_dev, lr, beta1, beta2, eps, 0.0f, ws, f.p);
    if (st != NGV_OK) return st;
    WarpGeom g;
    WarpBwdFinal fin;
    if (int e = prepare_warp(M, md, nullptr, u, od, xf, g, &fin)) return e;
    mf.F = F;
    mf.table = reinterpret_cast<const float *>(static_cast<const char *>(ws) + ws_layout(bins).table);
    mf.gscale = mi_grad_scale(mf.p, od->nx * od->ny * od->nz);
    f.u = u;
    f.m1 = m1;
    f.m2 = m2;
    f.accumulate_affine = accumulate_affine;
    f.slab_mode = 0;
    hipError_t e = adam_enqueue_bc(step_dev, f.p, static_cast<hipStream_t>(stream));
    if (e == hipSuccess)
        e = launch_warp_bwd(g, gW, nullptr, gA9, gt3, fin, 0, ws, static_cast<hipStream_t>(stream), &f, &mf);
    return e == hipSuccess ? NGV_OK : hip_fail(e);
}

int ngv_warp_bwd_adam_slab(const float *M, const ngv_dims *md, const ngv_slab *slab, float *u, const ngv_dims *od,
                           const ngv_xform *xf, const float *gW, float *gu, float *m1, float *m2, int step,
                           const int32_t *step_dev, float lr, float beta1, float beta2, float eps, double *gA9,
                           double *gt3, int accumulate_affine, void *ws, size_t ws_bytes, void *stream) {
    if (!M || !u || !gW || !gu || !m1 || !m2 || !gA9 || !gt3 || !xf || !dims_ok(md) || !dims_ok(od) ||
        !slab_ok(slab, md) || !slab || !slab->zrange)
        return NGV_EINVAL;
    if (accumulate_affine != 0 && accumulate_affine != 1) return NGV_EINVAL;
    int st = check_ws(ws, ws_bytes, ngv_workspace_bytes(0, 0));
    if (st != NGV_OK) return st;
    AdamFuse f;
    st = adam_params(step, step_dev, lr, beta1, beta2, eps, 0.0f, ws, f.p);
    if (st != NGV_OK) return st;
    WarpGeom g;
    WarpBwdFinal fin;
    if (int e = prepare_warp(M, md, slab, u, od, xf, g, &fin)) return e;
    f.u = u;
    f.m1 = m1;
    f.m2 = m2;
    f.accumulate_affine = accumulate_affine;
    f.slab_mode = 1;
    hipError_t e = adam_enqueue_bc(step_dev, f.p, static_cast<hipStream_t>(stream));
    if (e == hipSuccess) e = launch_warp_bwd(g, gW, gu, gA9, gt3, fin, 0, ws, static_cast<hipStream_t>(stream), &f);
    return e == hipSuccess ? NGV_OK : hip_fail(e);
}

int ngv_warp_bwd_adam_slab_mi(const float *M, const ngv_dims *md, const ngv_slab *slab, float *u,
                              const ngv_dims *od, const ngv_xform *xf, const float *gW, const float *F,
                              const float *W, int bins, float fmin, float fmax, float wmin, float wmax,
                              float weight_mi, float *gu, float *m1, float *m2, int step, const int32_t *step_dev,
                              float lr, float beta1, float beta2, float eps, double *gA9, double *gt3,
                              int accumulate_affine, void *ws, size_t ws_bytes, void *stream) {
    if (!M || !u || !F || !W || !gu || !m1 || !m2 || !gA9 || !gt3 || !xf || !dims_ok(md) || !dims_ok(od) ||
        !slab_ok(slab, md) || !slab || !slab->zrange)
        return NGV_EINVAL;
    if (accumulate_affine != 0 && accumulate_affine != 1) return NGV_EINVAL;
    MiFuse mf;
    int st = mi_params(bins, fmin, fmax, wmin, wmax, weight_mi, mf.p);
    if (st != NGV_OK) return st;
    st = check_ws(ws, ws_bytes, ngv_workspace_bytes(bins, 0));
    if (st != NGV_OK) return st;
    if (!mi_size_ok(od) || bins > kMaxLdsBins) return NGV_EUNSUPPORTED;
    AdamFuse f;
    st = adam_params(step, step_dev, lr, beta1, beta2, eps, 0.0f, ws, f.p);
    if (st != NGV_OK) return st;
    WarpGeom g;
    WarpBwdFinal fin;
    if (int e = prepare_warp(M, md, slab, u, od, xf, g, &fin)) return e;
    mf.F = F;
    mf.W = W;
    mf.table = reinterpret_cast<const float *>(static_cast<const char *>(ws) + ws_layout(bins).table);
    mf.gscale = mi_grad_scale(mf.p, od->nx * od->ny * od->nz);
    f.u = u;
    f.m1 = m1;
    f.m2 = m2;
    f.accumulate_affine = accumulate_affine;
    f.slab_mode = 1;
    hipError_t e = adam_enqueue_bc(step_dev, f.p, static_cast<hipStream_t>(stream));
    if (e == hipSuccess)
        e = launch_warp_bwd(g, gW, gu, gA9, gt3, fin, 0, ws, static_cast<hipStream_t>(stream), &f, &mf);
    return e == hipSuccess ? NGV_OK : hip_fail(e);
}

int ngv_warp_fwd_mi(const float *M, const ngv_dims *md, const ngv_slab *slab, const float *u, const ngv_dims *od,
                    const ngv_xform *xf, float *W, int accumulate, const float *F, int bins, float fmin, float fmax,
                    float wmin, float wmax, float weight, double *loss, int accumulate_loss, void *ws,
                    size_t ws_bytes, void *stream) {
    if (!M || !u || !xf || !F || !loss || !dims_ok(md) || !dims_ok(od) || !slab_ok(slab, md)) return NGV_EINVAL;
    if (accumulate != 0 && accumulate != 1) return NGV_EINVAL;
    if (accumulate_loss != 0 && accumulate_loss != 1) return NGV_EINVAL;
    // without W the sample is not stored: one call over the whole moving image
    if (!W && (accumulate || (slab && (slab->z0 != 0 || slab->nz != md->nz)))) return NGV_EINVAL;
    MiParams p;
    int st = mi_params(bins, fmin, fmax, wmin, wmax, weight, p);
    if (st != NGV_OK) return st;
    st = check_ws(ws, ws_bytes, ngv_workspace_bytes(bins, 0));
    if (st != NGV_OK) return st;
    WarpGeom g;
    if (int e = prepare_warp(M, md, slab, u, od, xf, g, nullptr)) return e;
    if (!mi_size_ok(od) || bins > kMaxLdsBins) return NGV_EUNSUPPORTED;
    const WsLayout l = ws_layout(bins);
    char *base = static_cast<char *>(ws);
    auto *hist = reinterpret_cast<unsigned long long *>(base + l.hist);
    auto *table = reinterpret_cast<float *>(base + l.table);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_mi_zero(hist, bins, s);
    if (e == hipSuccess) e = launch_warp_fwd_hist(g, W, accumulate, F, p, hist, s);
    if (e == hipSuccess) e = launch_mi_finalize(hist, p, od->nx * od->ny * od->nz, table, loss, accumulate_loss, s);
    return e == hipSuccess ? NGV_OK : hip_fail(e);
}

int ngv_warp_lncc_mi_bwd(const float *M, const ngv_dims *md, const float *u, const ngv_dims *od, const ngv_xform *xf,
                         const float *F, int win, float eps, float weight_lncc, double *loss_lncc, int bins, float fmin,
                         float fmax, float wmin, float wmax, float weight_mi, float *gu, double *gA9, double *gt3,
                         int accumulate_affine, void *ws, size_t ws_bytes, void *stream) {
    if (!M || !u || !xf || !F || !loss_lncc || !gu || !gA9 || !gt3 || !dims_ok(md) || !dims_ok(od)) return NGV_EINVAL;
    if (accumulate_affine != 0 && accumulate_affine != 1) return NGV_EINVAL;
    if (win < 3 || win % 2 == 0 || win > 31) return NGV_EINVAL;
    if (!finite(eps) || eps < 0.0f || !finite(weight_lncc)) return NGV_EINVAL;
    // gu is written while u is read at other voxels: they must not overlap
    const uintptr_t ub = reinterpret_cast<uintptr_t>(u), gb = reinterpret_cast<uintptr_t>(gu);
    const size_t vb = 3 * sizeof(float) * size_t(od->nx * od->ny * od->nz);
    if (ub < gb + vb && gb < ub + vb) return NGV_EINVAL;
    MiFuse mf;
    if (bins != 0) {
        int st = mi_params(bins, fmin, fmax, wmin, wmax, weight_mi, mf.p);
        if (st != NGV_OK) return st;
    }
    // the fused sweep is the small-window kernel: windows 13..31 are valid
    // LNCC windows that it does not take
    if (win > 11) return NGV_EUNSUPPORTED;
    int st = check_ws(ws, ws_bytes, ngv_workspace_bytes(bins, 0));
    if (st != NGV_OK) return st;
    if (bins != 0 && !mi_size_ok(od)) return NGV_EUNSUPPORTED;
    WarpGeom g;
    WarpBwdFinal fin;
    if (int e = prepare_warp(M, md, nullptr, u, od, xf, g, &fin)) return e;
    if (bins != 0) {
        mf.F = F;
        mf.table = reinterpret_cast<const float *>(static_cast<const char *>(ws) + ws_layout(bins).table);
        mf.gscale = mi_grad_scale(mf.p, od->nx * od->ny * od->nz);
    }
    hipError_t e = launch_lncc_fused(g, fin, F, win, eps, weight_lncc, loss_lncc, bins != 0 ? &mf : nullptr, gu, gA9,
                                     gt3, accumulate_affine, ws, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NGV_OK : hip_fail(e);
}

int ngv_mi_grad(const float *F, const float *W, const ngv_dims *d, int bins, float fmin, float fmax, float wmin,
                float wmax, float weight, float *gW, int accumulate, void *ws, size_t ws_bytes, void *stream) {
    if (!F || !W || !gW || !dims_ok(d)) return NGV_EINVAL;
    if (accumulate != 0 && accumulate != 1) return NGV_EINVAL;
    if (!aligned(F, 16) || !aligned(W, 16) || !aligned(gW, 16)) return NGV_EINVAL;
    MiParams p;
    int st = mi_params(bins, fmin, fmax, wmin, wmax, weight, p);
    if (st != NGV_OK) return st;
    st = check_ws(ws, ws_bytes, ngv_workspace_bytes(bins, 0));
    if (st != NGV_OK) return st;
    if (!mi_size_ok(d)) return NGV_EUNSUPPORTED;
    const float *table = reinterpret_cast<const float *>(static_cast<const char *>(ws) + ws_layout(bins).table);
    hipError_t e = launch_mi_grad(F, W, d->nx * d->ny * d->nz, p, table, gW, accumulate,
                                  static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NGV_OK : hip_fail(e);
}

int ngv_warp_zrange(const float *u, const ngv_dims *od, const ngv_dims *md, const ngv_xform *xf, double *zrange,
                    void *ws, size_t ws_bytes, void *stream) {
    if (!u || !zrange || !xf || !dims_ok(od) || !dims_ok(md) || !aligned(zrange, 8)) return NGV_EINVAL;
    int st = check_ws(ws, ws_bytes, ngv_workspace_bytes(0, 0));
    if (st != NGV_OK) return st;
    WarpGeom g;
    if (int e = prepare_warp(nullptr, md, nullptr, u, od, xf, g, nullptr)) return e;
    hipError_t e = launch_warp_zrange(g, zrange, ws, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NGV_OK : hip_fail(e);
}

int ngv_mse_loss_fwd_bwd(const float *F, const float *W, const ngv_dims *d, float weight, double *loss, float *gW,
                         int accumulate, void *ws, size_t ws_bytes, void *stream) {
    if (!F || !W || !loss || !dims_ok(d)) return NGV_EINVAL;
    if (accumulate != 0 && accumulate != 1) return NGV_EINVAL;
    if (!finite(weight)) return NGV_EINVAL;
    if (!aligned(F, 16) || !aligned(W, 16) || (gW && !aligned(gW, 16))) return NGV_EINVAL;
    int st = check_ws(ws, ws_bytes, ngv_workspace_bytes(0, 0));
    if (st != NGV_OK) return st;
    hipError_t e = launch_mse(F, W, d->nx * d->ny * d->nz, weight, loss, gW, accumulate, ws,
                              static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NGV_OK : hip_fail(e);
}

int ngv_warp_compose(const float *uf, const ngv_dims *ud, const float *v, const ngv_dims *vd, const ngv_xform *xf,
                     float *w, void *stream) {
    if (!uf || !v || !w || !xf || !dims_ok(ud) || !dims_ok(vd)) return NGV_EINVAL;
    // w may be v itself, but must not overlap the sampled field
    const uintptr_t ub = reinterpret_cast<uintptr_t>(uf), wb = reinterpret_cast<uintptr_t>(w);
    const uintptr_t ue = ub + 3 * sizeof(float) * size_t(ud->nx * ud->ny * ud->nz);
    const uintptr_t we = wb + 3 * sizeof(float) * size_t(vd->nx * vd->ny * vd->nz);
    if (ub < we && wb < ue) return NGV_EINVAL;
    WarpGeom g;
    if (int e = prepare_warp(uf, ud, nullptr, v, vd, xf, g, nullptr)) return e;
    hipError_t e = launch_warp_compose(g, w, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NGV_OK : hip_fail(e);
}

}  // extern "C"
