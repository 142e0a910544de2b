// Internal declarations of libngv.so (HIP, gfx950). Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "ngv.h"

namespace ngv {

// MI355X: 256 compute units in 8 XCDs; work-groups are dealt to the XCDs
// round robin by block index.
constexpr int kXcds = 8;

// Persistent grids are capped at this many blocks; it fixes the number of
// per-block partial-sum slots in the workspace (O(1) in the volume size).
constexpr int kMaxBlocks = 2048;
constexpr int kPartialStride = 16;  // doubles per block slot
constexpr size_t kPartialBytes = size_t(kMaxBlocks) * kPartialStride * sizeof(double);
constexpr int kMaxBins = 256;
// MI bin counts whose u64 block histogram (and fp32 log-ratio table) fit in
// LDS; larger ones use the global histogram and table directly.
constexpr int kMaxLdsBins = 128;

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace layout (bytes from the base): [partials | optimiser bias
// corrections (2 f32) | MI histogram (u64) | MI log-ratio table (f32) |
// scalars].
struct WsLayout {
    size_t partials, adam, hist, table, scalars, total;
};
inline WsLayout ws_layout(int bins) {
    WsLayout l;
    size_t b2 = size_t(bins > 0 ? bins : 0) * size_t(bins > 0 ? bins : 0);
    l.partials = 0;
    l.adam = align_up(kPartialBytes, 256);
    l.hist = l.adam + 256;
    l.table = align_up(l.hist + b2 * sizeof(unsigned long long), 256);
    l.scalars = align_up(l.table + b2 * sizeof(float), 256);
    l.total = align_up(l.scalars + 256, 256);
    return l;
}

// The LNCC kernel for windows 13..31 keeps each block's state in a slice of
// the workspace (its size depends on the window only); the slices follow
// the largest MI layout, so that they never overlap the MI table that a
// later call of the same step reads.
constexpr int kLnccBigBlocks = 256;
inline size_t lncc_big_offset() { return align_up(ws_layout(kMaxBins).total, 256); }
size_t lncc_big_bytes(int win);  // 0 below 13

// Per-device launch facts, cached.
struct DeviceInfo {
    int cus = 256;
    size_t max_lds = 65536;
};
const DeviceInfo &device_info();

// Persistent-grid size: a multiple of kXcds, at most kMaxBlocks.
inline int persistent_blocks(int64_t items, int blocks_per_cu) {
    int64_t g = int64_t(device_info().cus) * blocks_per_cu;
    if (g > kMaxBlocks) g = kMaxBlocks;
    if (items < g) g = items;
    g = (g + kXcds - 1) / kXcds * kXcds;
    if (g < kXcds) g = kXcds;
    return int(g);
}

// ---------------------------------------------------------------- device side

// XCD-aware walk of a persistent grid over `total` work items: the blocks
// resident on one XCD take a contiguous eighth of the items, so neighbouring
// items (which share halo and gather data) meet in the same L2.
struct ItemRange {
    int64_t begin, end, step;
};
__device__ inline ItemRange xcd_items(int64_t total) {
    const int b = blockIdx.x, g = gridDim.x;
    const int x = b % kXcds, j = b / kXcds, per = g / kXcds;
    ItemRange r;
    r.begin = total * x / kXcds + j;
    r.end = total * (x + 1) / kXcds;
    r.step = per;
    return r;
}

__device__ inline double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Sum of `v` over the block (blockDim.x a multiple of 64, <= 1024), in a
// fixed order; the result is valid in thread 0. `red` is __shared__ scratch of
// at least 16 doubles.
__device__ inline double block_sum(double v, double *red) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    if (lane == 0) red[wid] = v;
    __syncthreads();
    double s = 0.0;
    if (threadIdx.x == 0) {
        const int nw = blockDim.x >> 6;
        for (int i = 0; i < nw; ++i) s += red[i];
    }
    __syncthreads();
    return s;
}

// ------------------------------------------------------------------ launchers
// Each returns a hipError_t from the launch; arguments are already checked.

struct WarpGeom {
    const float *M;
    int64_t mnx, mny, mnz;  // full moving grid
    int64_t sz0, snz;       // planes held by the buffer
    const float *u;
    int64_t onx, ony, onz;  // output grid
    double a[9];            // A_v - I in voxel units (row-major, on (ix, iy, iz))
    double tv[3];           // translation in M voxel units
    double sv[9];           // S_v = D_M S
    const double *zrange;   // bound of (S_v u)_z over the output grid, or null
};

struct WarpBwdFinal {
    double dm[3];    // (n_M - 1) / 2 per axis
    double xmin[3];  // output grid bounds
    double delta[3]; // output grid spacing
};

struct AdamParams {
    float lr, beta1, beta2, eps;
    float inv_bc1, inv_bc2;    // 1/(1 - b1^t), 1/(1 - b2^t)
    int radius;                // smoothing taps -radius..radius, 0: none
    float taps[9];
    const float *bc;  // non-null: inv_bc1, inv_bc2 are read here (device memory)
};

// The bias corrections that launch_adam_bc left in device memory (a step
// number held on the device); two uniform loads at the start of a kernel.
__device__ inline void adam_resolve(AdamParams &p) {
    if (!p.bc) return;
    p.inv_bc1 = p.bc[0];
    p.inv_bc2 = p.bc[1];
}

// Adam with bias correction on one value (shared by every kernel that
// updates u, so fused and separate updates are the same arithmetic).
__device__ inline void adam_one(float &u, float &m1, float &m2, float g, const AdamParams &p) {
    m1 = fmaf(p.beta1, m1, (1.0f - p.beta1) * g);
    m2 = fmaf(p.beta2, m2, (1.0f - p.beta2) * (g * g));
    const float den = sqrtf(m2 * p.inv_bc2) + p.eps;
    u -= p.lr * (m1 * p.inv_bc1) / den;
}

// Optimiser state for a sampler backward fused with the optimiser step.
struct AdamFuse {
    float *u, *m1, *m2;
    AdamParams p;
    int accumulate_affine;
    int slab_mode;  // one of a sequence of slab calls, each stepping the voxels it completes
};

struct MiFuse;

hipError_t launch_warp_fwd(const WarpGeom &g, float *W, int accumulate, hipStream_t s);
// One call of a forward slab sequence: the first slab that reaches an item
// writes it, later ones add, the top slab's call zeroes the items no slab
// reaches (a z-range bound is required).
hipError_t launch_warp_fwd_seq(const WarpGeom &g, float *W, hipStream_t s);
// zrange[0..1] = min, max over the output grid of (S_v u)_z.
hipError_t launch_warp_zrange(const WarpGeom &g, double *zrange, void *ws, hipStream_t s);
// adam == nullptr: store gu (accumulate: add to it). Otherwise gu (may be
// null) holds earlier slabs' partial gradient; the sum feeds the optimiser
// step and is not stored; dA, dt use adam->accumulate_affine. mi (with adam):
// the MI term's gradient is formed from F and W and added to gW (which may
// then be null) -- over the whole grid (no z-range bound) from the W the
// backward recomputes, or in slab mode from the stored W in mi->W.
hipError_t launch_warp_bwd(const WarpGeom &g, const float *gW, float *gu, double *gA9, double *gt3,
                           const WarpBwdFinal &fin, int accumulate, void *ws, hipStream_t s,
                           const AdamFuse *adam = nullptr, const MiFuse *mi = nullptr);

struct MiParams {
    int bins;
    int f_order;                // Parzen kernel of F: 3 cubic B-spline, 0 box
    float f_lo, f_hi, f_scale;  // clamp range and bin scale of F
    float w_lo, w_hi, w_scale;  // same for W
    float weight;
};
// d loss_MI / d W per voxel is (F's weights x W's weight derivatives against
// the log-ratio table) times this scale: weight * (W's bin scale) / N.
inline float mi_grad_scale(const MiParams &p, int64_t n) {
    return float(double(p.weight) * double(p.w_scale) / double(n));
}

// The MI gradient formed inside the fused sampler backward (the second sweep
// of a fused step): F on the output grid, the MI parameters and the log-ratio
// table (device memory, bins x bins floats) of the latest MI forward.
struct MiFuse {
    const float *F;
    MiParams p;
    const float *table;
    float gscale;  // mi_grad_scale(p, N)
    // the stored W (the whole forward result), for the backward slab
    // sequence, which cannot recompute W from one slab; null elsewhere
    const float *W = nullptr;
};

// hist: bins^2 u64 (zeroed here), table: bins^2 f32, both device memory
hipError_t launch_mi(const float *F, const float *W, int64_t plane, int64_t nz, const MiParams &p, double *loss,
                     float *gW, int accumulate, unsigned long long *hist, float *table, hipStream_t s);
// The pieces of launch_mi, for the sampler that builds the histogram in its
// own sweep: zero the global histogram; turn it into the loss and the
// log-ratio table; the gradient sweep from the table.
hipError_t launch_mi_zero(unsigned long long *hist, int bins, hipStream_t s);
hipError_t launch_mi_finalize(const unsigned long long *hist, const MiParams &p, int64_t n, float *table,
                              double *loss, int accumulate, hipStream_t s);
hipError_t launch_mi_grad(const float *F, const float *W, int64_t n, const MiParams &p, const float *table,
                          float *gW, int accumulate, hipStream_t s);
// The sampler forward (as launch_warp_fwd, every output voxel visited) that
// also adds the joint histogram of (F, final W) into hist.
hipError_t launch_warp_fwd_hist(const WarpGeom &g, float *W, int accumulate, const float *F, const MiParams &p,
                                unsigned long long *hist, hipStream_t s);

// loss (+)= scale * (sum of the first nblocks workspace partials), fixed order
hipError_t launch_partials_final(const double *partials, int nblocks, double scale, double *loss, int accumulate,
                                 hipStream_t s);
hipError_t launch_mse(const float *F, const float *W, int64_t n, float weight, double *loss, float *gW,
                      int accumulate, void *ws, hipStream_t s);
// w = v + U~(p) per component: g.M is U's first component (3 volumes of the
// moving grid), g.u the displacement v; no slab
hipError_t launch_warp_compose(const WarpGeom &g, float *w, hipStream_t s);
hipError_t launch_lncc(const float *F, const float *W, int64_t nx, int64_t ny, int64_t nz, int win, float eps,
                       float weight, double *loss, float *gW, int accumulate, void *ws, hipStream_t s);
// The fused second sweep: the LNCC kernel sampling W from g (whole moving
// image) itself, the LNCC (+ MI, when mi) gradient feeding the sampler
// backward at each output voxel: gu written, dA, dt and the LNCC loss.
hipError_t launch_lncc_big(const float *F, const float *W, int64_t nx, int64_t ny, int64_t nz, int win, float eps,
                           float weight, double *loss, float *gW, int accumulate, void *ws, hipStream_t s);
hipError_t launch_lncc_fused(const WarpGeom &g, const WarpBwdFinal &fin, const float *F, int win, float eps,
                             float weight, double *loss, const MiFuse *mi, float *gu, double *gA9, double *gt3,
                             int accumulate_affine, void *ws, hipStream_t s);
// dA, dt from per-block affine partial sums (slots 0..11 of the workspace
// partials) of nblocks blocks.
hipError_t launch_warp_bwd_final(const double *partials, int nblocks, const WarpBwdFinal &fin, double *gA9,
                                 double *gt3, int accumulate, hipStream_t s);

hipError_t launch_adam(float *u, const float *gu, float *m1, float *m2, int64_t nx, int64_t ny, int64_t nz,
                       const AdamParams &p, hipStream_t s);
// bc[0], bc[1] = 1/(1 - b1^t), 1/(1 - b2^t) for t = *step_dev (t < 1 counts as
// 1), formed as the host forms them from a host step: fp64, rounded to fp32.
hipError_t launch_adam_bc(const int32_t *step_dev, float beta1, float beta2, float *bc, hipStream_t s);

}  // namespace ngv
