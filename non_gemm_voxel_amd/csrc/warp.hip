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
// Work decomposition: 64 x 4 column tiles of a few consecutive planes (see
// below). u, gW and the optimiser state are read once per call and nothing
// reuses them from L2, so they are loaded non-temporally. A persistent grid
// walks the items in z-blocks dealt round the XCDs (the slab backward: single
// groups dealt round them), so the M rows and planes a tile gathers from are
// shared with its neighbours in one L2.
//
// Kernels: the forward (overwriting and accumulating instantiations), the
// composition of a 3-component field, the forward that also builds the MI
// histogram, the backward (alone, fused with the optimiser step, and fused
// over a slab sequence), and the z-range bound of the displacement.
#include "mi_device.hpp"
#include "sampler_device.hpp"

namespace ngv {
namespace {

using namespace sampler;

constexpr int kThreads = 256;

// Work item = a 64 (x) by 4 (y) tile of KZ consecutive z-planes. Lane l of
// wave w takes column (x0 + l, y0 + w) of the tile in all KZ planes: every
// load, gather and store instruction is unit-stride across the wave, a thread
// has KZ voxels' loads in flight, and the corner rows gathered for plane z + 1
// are largely those of plane z (reused through L1).
// planes per thread, measured best on the 640x768x640 workload: 5 for the
// overwriting forward pass (129 VGPRs, three waves per SIMD; 4 planes, four
// waves: 1.66 against 1.89 ms with a smooth displacement, 3.49 against 3.36
// with a rough one; 6: slower with both), 4 for the accumulating one (5:
// 30.0 against 29.7-29.9 ms for the 8-slab sequence on the 1280 x 1536 x
// 1280 grid; 3: 32.5), 2 for the backward pass, 3 for its slab sequence
// (on the 1280 x 1536 x 1280 grid in 8 slabs 55.3-55.5 against 56.3-57.5
// ms; 205 VGPRs, two waves per SIMD; the fused backward on the 640 x 768 x
// 640 grid went from 6.7 to 8.1 ms with three planes, losing its fourth wave)
constexpr int kTX = 64, kTY = 4, kKZF = 5, kKZFA = 4, kKZB = 2, kKZBS = 3;
constexpr bool kSlabPrefetch = true;
static_assert(kTX * kTY == kThreads, "tile");

struct Item {
    int x, y, z0;  // this thread's column and first plane
    int nzk;       // planes in this item (1..KZ); 0: column outside
};

// Plane k of an item for a load that every lane of the item issues: planes
// past the item's last read its last plane (nzk >= 1), whose value is not
// used. A load under a per-lane condition is waited for inside its branch,
// one round trip per load, where unconditional loads are in flight together.
// That helps the overwriting forward; in the accumulating forward and the
// backward, whose loads per item are more (u, W or gW, F, the partial
// gradient, the optimiser state), issuing them all at once measured slower
// (the 8-slab forward sequence on the 1280 x 1536 x 1280 grid 32.0 against
// 29.7 ms, its backward 57.0 against 56.6), and they keep the conditions.
__device__ inline int64_t load_plane(const Item &m, int k) { return k < m.nzk ? k : m.nzk - 1; }

template <int kKZ>
__device__ inline void item_at(const WarpGeom &g, int64_t it, int64_t tiles_x, int64_t tiles_y, Item &m) {
    const int64_t tx = it % tiles_x, r1 = it / tiles_x;
    const int64_t ty = r1 % tiles_y, zg = r1 / tiles_y;
    m.x = int(tx * kTX) + int(threadIdx.x & 63);
    m.y = int(ty * kTY) + int(threadIdx.x >> 6);
    m.z0 = int(zg * kKZ);
    const int64_t left = g.onz - m.z0;
    m.nzk = (m.x < g.onx && m.y < g.ony) ? int(left < kKZ ? left : kKZ) : 0;
}

template <int kKZ>
__device__ __host__ inline int64_t items_of(const WarpGeom &g, int64_t &tiles_x, int64_t &tiles_y) {
    tiles_x = (g.onx + kTX - 1) / kTX;
    tiles_y = (g.ony + kTY - 1) / kTY;
    return tiles_x * tiles_y * ((g.onz + kKZ - 1) / kKZ);
}

// Work items in z-blocks. The visited z-groups (a virtual index 0 ..
// ngroups - 1, which may stand for two ranges of groups) are cut into blocks
// of B groups, about 40 planes, but small enough that there are at least 32
// blocks; XCD x takes blocks x, x + 8, ..., and within a block the items go
// group fastest, then the tiles in x, then y. The items an XCD runs at once
// then cover a patch several groups deep, and as the walk moves on in y the
// moving-image rows and planes their samples share are still in its L2: with
// a rough displacement a plane's samples scatter over the neighbouring
// planes, which a walk through whole planes fetches again for every group.
// Dealing the blocks round the XCDs keeps their shares even where only part
// of the groups holds work (the band of a slab call, whose items reach the
// slab at a z that varies across the tiles). Measured on the 1280 x 1536 x
// 1280 grid after 5 and 25 optimiser steps: the forward 25.6 -> 23.2 and
// 36.5 -> 30.9 ms, its 8-slab sequence 33.4 -> 27.2 and 48.0 -> 35.4 ms (24.8
// against 27.7 at u = 0), the backward with Adam 55.7 -> 51.4 and 65.6 ->
// 58.2 ms (0.6 ms slower at u = 0). The backward's slab calls keep a walk of
// their own.
struct ZWalk {
    int64_t tiles, ngroups, B, nblk;
};

template <int kKZ>
__device__ inline ZWalk zwalk(int64_t tiles, int64_t ngroups) {
    constexpr int64_t kMax = (40 + kKZ - 1) / kKZ;
    int64_t B = ngroups / (4 * kXcds);
    B = B < 1 ? 1 : B > kMax ? kMax : B;
    return ZWalk{tiles, ngroups, B, (ngroups + B - 1) / B};
}

// This block's positions in its XCD's share: blocks of one XCD take every
// per-th item of it.
__device__ inline ItemRange zwalk_range(const ZWalk &w) {
    const int xcd = int(blockIdx.x) % kXcds, per = int(gridDim.x) / kXcds;
    int64_t n = 0;
    if (w.nblk > xcd) {
        n = (w.nblk - xcd + kXcds - 1) / kXcds * w.B * w.tiles;
        if ((w.nblk - 1) % kXcds == xcd) n -= (w.nblk * w.B - w.ngroups) * w.tiles;  // the last block is short
    }
    return ItemRange{int64_t(blockIdx.x) / kXcds, n, per};
}

// The item at position i0 of this XCD's share, as a virtual index
// (group * tiles + tile).
__device__ inline int64_t zwalk_item(const ZWalk &w, int64_t i0) {
    const int xcd = int(blockIdx.x) % kXcds;
    const int64_t lb = i0 / (w.tiles * w.B), vb = xcd + kXcds * lb;
    const int64_t r = i0 - lb * w.tiles * w.B;
    const int64_t zb = w.ngroups - vb * w.B < w.B ? w.ngroups - vb * w.B : w.B;
    const int64_t t = r / zb, k = r - t * zb;
    return (vb * w.B + k) * w.tiles + t;
}

// With a bound [lo, hi] of (S_v u)_z over the output grid, whether any sample
// of a box of output voxels can have a corner in the held planes
// [sz0, sz0 + snz): the corner plane is floor(iz + d_z), and iz + d_z is the
// affine part (1 + a_zz) iz + a_zx ix + a_zy iy + tv_z, extreme at the box
// corners, plus (S_v u)_z in [lo, hi]; a relative margin covers fp64
// rounding. For a work item's tile the answer is the same for the block.
// The same test for any range [zA, zB) of moving planes (empty: false). For
// contiguous ranges it splits exactly: reaching [zA, zC) is reaching [zA, zB)
// or [zB, zC).
__device__ inline bool box_reaches(const WarpGeom &g, double xl, double xh, double yl, double yh, double zl,
                                   double zh, int64_t zA, int64_t zB) {
    if (zB <= zA) return false;
    if (!g.zrange) return true;
    const double cx = g.a[6], cy = g.a[7], cz = 1.0 + g.a[8];
    const double pmin = g.tv[2] + (cx >= 0 ? cx * xl : cx * xh) + (cy >= 0 ? cy * yl : cy * yh) +
                        (cz >= 0 ? cz * zl : cz * zh);
    const double pmax = g.tv[2] + (cx >= 0 ? cx * xh : cx * xl) + (cy >= 0 ? cy * yh : cy * yl) +
                        (cz >= 0 ? cz * zh : cz * zl);
    const double lo = g.zrange[0], hi = g.zrange[1];
    const double margin = 1e-6 * (1.0 + fabs(pmin) + fabs(pmax) + fabs(lo) + fabs(hi));
    return pmax + hi + margin >= double(zA - 1) && pmin + lo - margin < double(zB);
}

__device__ inline bool box_touches_slab(const WarpGeom &g, double xl, double xh, double yl, double yh, double zl,
                                        double zh) {
    if (!g.zrange) return true;
    return box_reaches(g, xl, xh, yl, yh, zl, zh, g.sz0, g.sz0 + g.snz);
}

template <int kKZ>
__device__ inline bool item_reaches(const WarpGeom &g, int64_t it, int64_t tiles_x, int64_t tiles_y, int64_t zA,
                                    int64_t zB) {
    const int64_t tx = it % tiles_x, r1 = it / tiles_x;
    const int64_t ty = r1 % tiles_y, zg = r1 / tiles_y;
    return box_reaches(g, double(tx * kTX), double(min(tx * kTX + kTX, g.onx) - 1), double(ty * kTY),
                       double(min(ty * kTY + kTY, g.ony) - 1), double(zg * kKZ),
                       double(min(zg * kKZ + kKZ, g.onz) - 1), zA, zB);
}

template <int kKZ>
__device__ inline bool item_touches_slab(const WarpGeom &g, int64_t it, int64_t tiles_x, int64_t tiles_y) {
    if (!g.zrange) return true;
    return item_reaches<kKZ>(g, it, tiles_x, tiles_y, g.sz0, g.sz0 + g.snz);
}

// The slab tests of a block's next 64 work items as wave-uniform bit masks,
// one item per lane (it: the lane's item; valid: the lane has one). The fp64
// box test is the same for every thread of an item, so evaluating it once per
// item in this way takes 1/64 of the fp64 work of every thread testing every
// item (measured on the 1280 x 1536 x 1280 grid in 8 slabs: each test done
// per thread cost about 0.2 ms per sampler call). Bit j of a mask is the
// j-th of the 64 items: touch, the item reaches this slab; prev, an earlier
// slab reaches it; later, a later slab does; none, no slab does (only set in
// the top slab's call, top = true). Every lane of the wave must call it.
struct SlabMasks {
    uint64_t touch, prev, later, none;
};

template <int kKZ>
__device__ inline SlabMasks slab_masks(const WarpGeom &g, bool valid, int64_t it, int64_t tiles_x, int64_t tiles_y,
                                       bool top) {
    bool t = false, p = false, l = false, n = false;
    if (valid) {
        t = item_touches_slab<kKZ>(g, it, tiles_x, tiles_y);
        p = item_reaches<kKZ>(g, it, tiles_x, tiles_y, 0, g.sz0);
        l = item_reaches<kKZ>(g, it, tiles_x, tiles_y, g.sz0 + g.snz, g.mnz);
        n = top && !item_reaches<kKZ>(g, it, tiles_x, tiles_y, 0, g.mnz);
    }
    return SlabMasks{__ballot(t), __ballot(p), __ballot(l), __ballot(n)};
}

// The z-groups a slab call has to visit: with a z-range bound, only the
// groups whose planes can map into the held planes (a conservative band over
// the whole x, y extent; each item is then tested on its own tile). Returns
// the first group; `count` groups from there. Without a bound: all groups.
template <int kKZ>
__device__ inline int64_t slab_band(const WarpGeom &g, int64_t &count) {
    const int64_t nzg = (g.onz + kKZ - 1) / kKZ;
    count = nzg;
    if (!g.zrange) return 0;
    const double cx = g.a[6], cy = g.a[7], cz = 1.0 + g.a[8];
    if (!(cz > 1e-3)) return 0;  // planes not mapped forwards: visit everything
    const double xh = double(g.onx - 1), yh = double(g.ony - 1);
    const double mnxy = fmin(0.0, cx * xh) + fmin(0.0, cy * yh), mxxy = fmax(0.0, cx * xh) + fmax(0.0, cy * yh);
    const double lo = g.zrange[0], hi = g.zrange[1];
    const double margin = 1e-6 * (1.0 + fabs(g.tv[2]) + fabs(mnxy) + fabs(mxxy) + fabs(lo) + fabs(hi) +
                                  cz * double(g.onz));
    // planes z with tv + mxxy + cz z + hi >= sz0 - 1 and tv + mnxy + cz z + lo < sz0 + snz
    const double z_lo = (double(g.sz0 - 1) - margin - g.tv[2] - mxxy - hi) / cz;
    const double z_hi = (double(g.sz0 + g.snz) + margin - g.tv[2] - mnxy - lo) / cz;
    const double glo = floor(z_lo / kKZ) - 1.0, ghi = floor(z_hi / kKZ) + 1.0;
    if (!(glo < double(nzg)) || !(ghi >= 0.0)) {
        count = 0;
        return 0;
    }
    const int64_t b = glo < 0.0 ? 0 : int64_t(glo);
    const int64_t e = ghi >= double(nzg - 1) ? nzg - 1 : int64_t(ghi);
    count = e - b + 1;
    return b;
}

// The z-groups the top slab's backward call has to visit: its own band, and
// the groups that can hold an item no slab reaches (every sample below the
// moving grid, or every sample above it), which only that call steps. An item
// lies wholly below when its highest corner plane is under -1, which needs
// its group's lowest one to be (pmin + hi < -1); wholly above when its lowest
// is at nz or beyond, which needs its group's highest one to be (pmax + lo >=
// nz). With an increasing z map these are a prefix and a suffix of the
// groups. Returns up to two ranges [b0, b0 + n0), [b1, b1 + n1), ascending
// and disjoint; without a bound (or a z map that does not increase) all
// groups.
template <int kKZ>
__device__ inline void top_slab_walk(const WarpGeom &g, int64_t &b0, int64_t &n0, int64_t &b1, int64_t &n1) {
    const int64_t nzg = (g.onz + kKZ - 1) / kKZ;
    b0 = 0;
    n0 = nzg;
    b1 = nzg;
    n1 = 0;
    if (!g.zrange) return;
    const double cx = g.a[6], cy = g.a[7], cz = 1.0 + g.a[8];
    if (!(cz > 1e-3)) return;
    int64_t nband;
    const int64_t gb = slab_band<kKZ>(g, nband);
    const double xh = double(g.onx - 1), yh = double(g.ony - 1);
    const double mnxy = fmin(0.0, cx * xh) + fmin(0.0, cy * yh), mxxy = fmax(0.0, cx * xh) + fmax(0.0, cy * yh);
    const double lo = g.zrange[0], hi = g.zrange[1];
    const double margin = 1e-6 * (1.0 + fabs(g.tv[2]) + fabs(mnxy) + fabs(mxxy) + fabs(lo) + fabs(hi) +
                                  cz * double(g.onz));
    // groups whose first plane z has tv + mnxy + cz z + hi - margin < -1
    const double zb = (-1.0 + margin - g.tv[2] - mnxy - hi) / cz;
    // groups whose last plane z has tv + mxxy + cz z + lo + margin >= nz
    const double zt = (double(g.mnz) - margin - g.tv[2] - mxxy - lo) / cz;
    int64_t nbot = 0, ntop = nzg;
    if (zb > 0.0) nbot = zb >= double(g.onz) ? nzg : min(nzg, int64_t(floor(zb / kKZ)) + 2);
    if (zt < double(g.onz)) ntop = zt <= 0.0 ? 0 : max(int64_t(0), int64_t(floor((zt - kKZ + 1) / kKZ)) - 1);
    const int64_t hb = nband > 0 ? min(gb, ntop) : ntop;  // the band, then every group to the top
    if (nbot >= hb) return;                               // the ranges meet: all groups
    b0 = 0;
    n0 = nbot;
    b1 = hb;
    n1 = nzg - hb;
}

// Zero an output before a banded slab call that must overwrite it.
__global__ __launch_bounds__(kThreads) void fill_zero_kernel(float *__restrict__ p, int64_t n) {
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < n; i += stride) p[i] = 0.0f;
}

// W (+)= the sampler at the planes of item m (first voxel o0): u loads, the
// corner gathers, the trilinear form (the same arithmetic as warp_fwd_kernel,
// so W is bitwise the same); the final values are also returned.
template <int kKZ>
__device__ inline void fwd_planes(const WarpGeom &g, const Item &m, int64_t o0, int64_t plane, int64_t ostride,
                                  float *__restrict__ W, int accumulate, float (&w)[kKZ]) {
    float u0[kKZ], u1[kKZ], u2[kKZ];
#pragma unroll
    for (int k = 0; k < kKZ; ++k) {
        const bool ok = k < m.nzk;
        const int64_t o = o0 + k * plane;
        u0[k] = ok ? __builtin_nontemporal_load(g.u + o) : 0.0f;
        u1[k] = ok ? __builtin_nontemporal_load(g.u + o + ostride) : 0.0f;
        u2[k] = ok ? __builtin_nontemporal_load(g.u + o + 2 * ostride) : 0.0f;
    }
    Sample s[kKZ];
#pragma unroll
    for (int k = 0; k < kKZ; ++k) gather(g, m.x, m.y, m.z0 + k, u0[k], u1[k], u2[k], s[k]);
#pragma unroll
    for (int k = 0; k < kKZ; ++k) {
        w[k] = 0.0f;
        if (k >= m.nzk) continue;
        float v = trilerp(s[k].c, s[k].fx, s[k].fy, s[k].fz);
        const int64_t o = o0 + k * plane;
        if (accumulate) v += W[o];
        W[o] = v;
        w[k] = v;
    }
}

// Wait for this wave's LDS copies (and its other vector memory operations)
// to land; the memory clobber keeps the LDS reads that follow behind it.
__device__ inline void wait_lds_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// The overwriting forward: u of the item's planes into registers (all loads
// in flight together), the gathers, the trilinear form. With the sampler's
// index arithmetic in 32 bits this plain walk is as fast as one that copied
// the next item's u into LDS during this item's gathers, or faster: on the
// 640 x 768 x 640 grid 1.89 against 2.07 ms with a smooth displacement (a
// 3-degree rotation held in u), 3.36 against 3.41 ms with the rough one of 25
// optimiser steps. W is stored non-temporally, as in the accumulating
// forward: it is larger than the caches and its readers fetch it from HBM
// anyway (2.96-2.97 against 3.00-3.01 ms per call in the step on that grid).
__global__ __launch_bounds__(kThreads) void warp_fwd_kernel(WarpGeom g, float *__restrict__ W) {
    constexpr int kKZ = kKZF;
    const int64_t plane = g.onx * g.ony, ostride = plane * g.onz;
    int64_t tiles_x, tiles_y, ngroups;
    items_of<kKZ>(g, tiles_x, tiles_y);
    // a slab call with a z-range bound visits only its band of z-groups
    // (spread over every XCD)
    const int64_t gbeg = slab_band<kKZ>(g, ngroups), tiles = tiles_x * tiles_y;
    const int64_t base = gbeg * tiles;
    const ZWalk zw = zwalk<kKZ>(tiles, ngroups);
    const ItemRange r = zwalk_range(zw);
    for (int64_t it0 = r.begin; it0 < r.end; it0 += r.step) {
        const int64_t it = base + zwalk_item(zw, it0);
        if (!item_touches_slab<kKZ>(g, it, tiles_x, tiles_y)) continue;
        Item m;
        item_at<kKZ>(g, it, tiles_x, tiles_y, m);
        if (m.nzk == 0) continue;
        const int64_t o0 = m.z0 * plane + m.y * g.onx + m.x;
        float u0[kKZ], u1[kKZ], u2[kKZ];
#pragma unroll
        for (int k = 0; k < kKZ; ++k) {
            const int64_t o = o0 + load_plane(m, k) * plane;
            u0[k] = __builtin_nontemporal_load(g.u + o);
            u1[k] = __builtin_nontemporal_load(g.u + o + ostride);
            u2[k] = __builtin_nontemporal_load(g.u + o + 2 * ostride);
        }
        Sample s[kKZ];
#pragma unroll
        for (int k = 0; k < kKZ; ++k) gather(g, m.x, m.y, m.z0 + k, u0[k], u1[k], u2[k], s[k]);
#pragma unroll
        for (int k = 0; k < kKZ; ++k) {
            if (k >= m.nzk) break;
            __builtin_nontemporal_store(trilerp(s[k].c, s[k].fx, s[k].fy, s[k].fz), W + o0 + k * plane);
        }
    }
}

// The accumulating forward: W holds the earlier slabs' sum, to which this
// call adds (slab calls of a banded sequence). Its earlier-slab values are
// loaded with u, before the gathers, so their latency overlaps the gathers'.
// (The pipelined walk of the overwriting kernel was slower here: measured on
// the 1280 x 1536 x 1280 grid in 8 slabs, 33.5 ms against 35-39 ms.)
// kSeq: one call of a slab sequence (slabs in increasing z, covering the
// moving grid, all with the same z-range bound). An item's first reaching
// slab writes its part plus +0 (so W holds the same bits as after zeroing
// and adding, whatever W held before); later slabs add. The top slab's call also
// writes zero to the items no slab reaches, walking the groups that can hold
// them as the backward's top call does.
template <bool kSeq>
__global__ __launch_bounds__(kThreads) void warp_fwd_acc_kernel(WarpGeom g, float *__restrict__ W) {
    constexpr int kKZ = kKZFA;
    const int64_t plane = g.onx * g.ony, ostride = plane * g.onz;
    int64_t tiles_x, tiles_y;
    items_of<kKZ>(g, tiles_x, tiles_y);
    // a slab call with a z-range bound visits only its band of z-groups
    // (spread over every XCD); the caller has zeroed W when overwriting. The
    // top call of a sequence visits [gb0, gb0 + gn0) and [gb1, gb1 + gn1).
    int64_t gb0 = 0, gn0 = 0, gb1 = 0, gn1 = 0;
    const bool top = kSeq && g.sz0 + g.snz >= g.mnz;
    if (top)
        top_slab_walk<kKZ>(g, gb0, gn0, gb1, gn1);
    else
        gb0 = slab_band<kKZ>(g, gn0);
    const int64_t tiles = tiles_x * tiles_y, split = gn0 * tiles;
    const ZWalk zw = zwalk<kKZ>(tiles, gn0 + gn1);
    const ItemRange r = zwalk_range(zw);
    auto item_index = [&](int64_t i0) {
        const int64_t v = zwalk_item(zw, i0);
        return v < split ? gb0 * tiles + v : gb1 * tiles + (v - split);
    };
    SlabMasks sm{};
    int j = 0;
    for (int64_t it0 = r.begin; it0 < r.end; it0 += r.step, ++j) {
        if ((j & 63) == 0) {
            const int64_t il = it0 + int64_t(threadIdx.x & 63) * r.step;
            sm = slab_masks<kKZ>(g, il < r.end, il < r.end ? item_index(il) : 0, tiles_x, tiles_y, top);
        }
        const uint64_t bit = 1ull << (j & 63);
        const int64_t it = item_index(it0);
        Item m;
        item_at<kKZ>(g, it, tiles_x, tiles_y, m);
        if (m.nzk == 0) continue;
        const int64_t o0 = m.z0 * plane + m.y * g.onx + m.x;
        if (!(sm.touch & bit)) {
            // adds zero; in a sequence nothing else writes the items no slab reaches
            if (sm.none & bit)
                for (int k = 0; k < m.nzk; ++k) W[o0 + k * plane] = 0.0f;
            continue;
        }
        // where an item's sum starts (kSeq, no earlier slab reaches it) W is
        // still loaded, and its bits masked to +0: on the 1280 x 1536 x 1280
        // grid in 8 slabs reading the lines before writing them measured
        // faster than writing them unread (3.66 against 3.90 ms per call)
        const int keep = !kSeq || (sm.prev & bit) ? -1 : 0;
        float u0[kKZ], u1[kKZ], u2[kKZ], prev[kKZ];
#pragma unroll
        for (int k = 0; k < kKZ; ++k) {
            const bool ok = k < m.nzk;
            const int64_t o = o0 + k * plane;
            u0[k] = ok ? __builtin_nontemporal_load(g.u + o) : 0.0f;
            u1[k] = ok ? __builtin_nontemporal_load(g.u + o + ostride) : 0.0f;
            u2[k] = ok ? __builtin_nontemporal_load(g.u + o + 2 * ostride) : 0.0f;
            prev[k] = __int_as_float(__float_as_int(ok ? W[o] : 0.0f) & keep);
        }
        Sample s[kKZ];
#pragma unroll
        for (int k = 0; k < kKZ; ++k) gather(g, m.x, m.y, m.z0 + k, u0[k], u1[k], u2[k], s[k]);
#pragma unroll
        for (int k = 0; k < kKZ; ++k) {
            if (k >= m.nzk) break;
            float w = trilerp(s[k].c, s[k].fx, s[k].fy, s[k].fz);
            const int64_t o = o0 + k * plane;
            __builtin_nontemporal_store(w + prev[k], W + o);
        }
    }
}

// Warp composition (Background and motivation: warp composition is one of
// the profiled memory bottlenecks; Key design 1: the composite sampler):
//   w_c(i) = v_c(i) + U~_c(A x_i + t + S v(i)),  c = x, y, z,
// the three components of U sampled at one position, which is located once.
// Here g.M is U's x component (y and z follow at one moving-grid volume each)
// and g.u is v. w may be v itself: each thread reads its own voxels of v
// before it writes them, and no other thread reads them (U must not overlap
// w). Same tiles and XCD walk as the sampler forward; eight planes per thread
// (measured on the 640x768x640 grid: 4.1 ms against 4.2 for four and 4.7 for
// two). The call is bound by gather latency, not bandwidth: a grid of only
// the resident blocks fetches less from L2's backing memory but runs slower.
constexpr int kKZC = 8;

__global__ __launch_bounds__(kThreads) void warp_compose_kernel(WarpGeom g, float *w) {
    constexpr int kKZ = kKZC;
    const int64_t plane = g.onx * g.ony, ostride = plane * g.onz;
    const int64_t mstride = g.mnx * g.mny * g.mnz;
    int64_t tiles_x, tiles_y;
    items_of<kKZ>(g, tiles_x, tiles_y);
    const ZWalk zw = zwalk<kKZ>(tiles_x * tiles_y, (g.onz + kKZ - 1) / kKZ);
    const ItemRange r = zwalk_range(zw);
    for (int64_t it = r.begin; it < r.end; it += r.step) {
        Item m;
        item_at<kKZ>(g, zwalk_item(zw, it), tiles_x, tiles_y, m);
        if (m.nzk == 0) continue;
        const int64_t o0 = m.z0 * plane + m.y * g.onx + m.x;
        float v[3][kKZ];
#pragma unroll
        for (int k = 0; k < kKZ; ++k) {
            const bool ok = k < m.nzk;
            const int64_t o = o0 + k * plane;
#pragma unroll
            for (int c = 0; c < 3; ++c) v[c][k] = ok ? __builtin_nontemporal_load(g.u + o + c * ostride) : 0.0f;
        }
        Cell cell[kKZ];
#pragma unroll
        for (int k = 0; k < kKZ; ++k) locate(g, m.x, m.y, m.z0 + k, v[0][k], v[1][k], v[2][k], cell[k]);
#pragma unroll
        for (int k = 0; k < kKZ; ++k) {
            if (k >= m.nzk) break;
            float cc[3][8];
#pragma unroll
            for (int c = 0; c < 3; ++c) corners(g, g.M + c * mstride, cell[k], cc[c]);
            const int64_t o = o0 + k * plane;
#pragma unroll
            for (int c = 0; c < 3; ++c)
                __builtin_nontemporal_store(v[c][k] + trilerp(cc[c], cell[k].fx, cell[k].fy, cell[k].fz),
                                            w + o + c * ostride);
        }
    }
}

// The sampler forward that also builds the MI joint histogram of (F, final W)
// in the same sweep (the first sweep of a fused step: W is read once less).
// Work item = a 64 x 4 tile of kKZH planes, sampled one plane at a time (the
// histogram window and more planes in flight do not fit four waves per SIMD);
// each thread's register window of the histogram is flushed once per item.
// Measured on the 640x768x640 workload it is slower (4.7 ms) than the two
// separate sweeps (2.7 + 1.75 ms): the histogram's VALU work and the
// sampler's latency-bound gathers do not overlap in one kernel.
// Every output voxel is visited (the histogram needs the final W of all of
// them); with a z-range bound, tiles this slab cannot reach skip the gather
// and only add the W of earlier slabs to the histogram.
constexpr int kKZH = 16;

__global__ __launch_bounds__(kThreads) void warp_fwd_hist_kernel(WarpGeom g, float *__restrict__ W, int accumulate,
                                                                 const float *__restrict__ F, MiParams p,
                                                                 unsigned long long *__restrict__ hist) {
    extern __shared__ unsigned long long h[];
    const int nb = p.bins, nb2 = nb * nb;
    for (int i = threadIdx.x; i < nb2; i += blockDim.x) h[i] = 0ull;
    __syncthreads();
    const int64_t plane = g.onx * g.ony, ostride = plane * g.onz;
    int64_t tiles_x, tiles_y;
    items_of<kKZH>(g, tiles_x, tiles_y);
    const ZWalk zw = zwalk<kKZH>(tiles_x * tiles_y, (g.onz + kKZH - 1) / kKZH);
    const ItemRange r = zwalk_range(zw);
    mi::HistCtx c;
    mi::hist_init(c, reinterpret_cast<float2 *>(h + nb2));
    for (int64_t i0 = r.begin; i0 < r.end; i0 += r.step) {
        const int64_t it = zwalk_item(zw, i0);
        Item m;
        item_at<kKZH>(g, it, tiles_x, tiles_y, m);
        const int64_t tx = it % tiles_x, ty = (it / tiles_x) % tiles_y;
#pragma unroll 1
        for (int k0 = 0; k0 < kKZH; ++k0) {
            if (m.z0 + k0 >= g.onz) break;  // uniform
            Item ms = m;
            ms.z0 = m.z0 + k0;
            ms.nzk = m.nzk > k0 ? 1 : 0;
            const int64_t o0 = ms.z0 * plane + m.y * g.onx + m.x;
            const bool touch = box_touches_slab(g, double(tx * kTX), double(min(tx * kTX + kTX, g.onx) - 1),
                                                double(ty * kTY), double(min(ty * kTY + kTY, g.ony) - 1),
                                                double(ms.z0), double(ms.z0));
            float w[1] = {0.0f};
            if (touch) {
                if (W) {
                    fwd_planes<1>(g, ms, o0, plane, ostride, W, accumulate, w);
                } else if (ms.nzk) {
                    // W not stored (the first sweep of a fused step): the sample alone
                    Sample q;
                    gather(g, m.x, m.y, ms.z0, __builtin_nontemporal_load(g.u + o0),
                           __builtin_nontemporal_load(g.u + o0 + ostride),
                           __builtin_nontemporal_load(g.u + o0 + 2 * ostride), q);
                    w[0] = trilerp(q.c, q.fx, q.fy, q.fz);
                }
            } else if (ms.nzk && W) {
                // nothing of this slab reaches here: W is the earlier slabs' sum
                w[0] = accumulate ? W[o0] : 0.0f;
                if (!accumulate) W[o0] = 0.0f;
            }
            // every lane takes part (deferred samples are queued per wave)
            mi::hist_add(c, ms.nzk ? F[o0] : 0.0f, w[0], ms.nzk != 0, p, h);
        }
        mi::hist_flush(c, p, h);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nb2; i += blockDim.x) {
        const unsigned long long v = h[i];
        if (v) atomicAdd(hist + i, v);
    }
}

// Backward: g_pvox = dW/dp_vox * gW; gu = S_v^T g_pvox; the affine sums are
// accumulated as G_j = sum g_pvox,j and Gi_jk = sum g_pvox,j * i_k (12 sums per
// thread, fp32 within an item, fp64 across items), reduced per block into the
// workspace; warp_bwd_final turns them into dA, dt in a fixed order.
// With kAdam the gradient of u is not stored: it is added to the partial
// gradient of earlier slabs (gu, may be null) and fed straight into the
// optimiser step of this voxel's u, m1, m2 (each thread reads and writes only
// its own voxel's state, so the update is done in place).
// kSlabs (with a z-range bound): this call is one of a sequence over
// contiguous slabs in increasing z. An item's first slab starts its gradient
// (earlier slabs reach none of its samples), the others add to the partial
// gradient in gu; in its last slab (no later slab reaches it) the optimiser
// step takes the gradient and gu is not written. The call of the top slab
// also steps the items that no slab reaches, with a zero gradient.
struct AdamArgs {
    float *u, *m1, *m2;
    AdamParams p;
};

// g_p = dW/dp_vox * gW at one sample.
__device__ inline void sample_grad(const Sample &q, float gw, float (&gp)[3]) {
    float w, dw[3];
    sample_terms(q, w, dw);
    gp[0] = dw[0] * gw;
    gp[1] = dw[1] * gw;
    gp[2] = dw[2] * gw;
}

// The item's affine sums: part[j] += g_p,j and part[3 + 3j + c] += g_p,j i_c
// at the voxel of plane k. No contraction of g_p's product into the plain
// sum: whether the compiler would fuse it differs between kernels, and they
// must form the same affine sums.
__device__ inline void affine_add(float (&part)[12], const float (&gp)[3], const Item &m, int k) {
#pragma clang fp contract(off)
    const float ii[3] = {float(m.x), float(m.y), float(m.z0 + k)};
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        part[j] = part[j] + gp[j];
#pragma unroll
        for (int c = 0; c < 3; ++c) part[3 + j * 3 + c] = fmaf(gp[j], ii[c], part[3 + j * 3 + c]);
    }
}

// kMi (slab mode): the MI term's gradient is formed here from F, the stored
// W (the whole forward result: no one slab call can recompute it) and the
// log-ratio table in LDS, and added to gW's value as ngv_mi_grad adds it.
struct SlabMi {
    const float *F, *W;
    MiParams p;
    const float *table;
    float gscale;
};

template <bool kAdam, bool kSlabs = false, bool kMi = false>
__global__ __launch_bounds__(kThreads) void warp_bwd_kernel(WarpGeom g, const float *__restrict__ gW,
                                                            float *__restrict__ gu, int accumulate,
                                                            double *__restrict__ partials, AdamArgs ad, SlabMi mi) {
    constexpr int kKZ = kSlabs ? kKZBS : kKZB;
    extern __shared__ float mi_table[];
    if constexpr (kMi) {
        const int nb2 = mi.p.bins * mi.p.bins;
        for (int i = threadIdx.x; i < nb2; i += kThreads) mi_table[i] = mi.table[i];
        __syncthreads();
    }
    if (kAdam) adam_resolve(ad.p);
    const int64_t plane = g.onx * g.ony, ostride = plane * g.onz;
    int64_t tiles_x, tiles_y, ngroups;
    items_of<kKZ>(g, tiles_x, tiles_y);
    // without the optimiser step, a slab call with a z-range bound visits only
    // its band (the caller has zeroed gu when overwriting); the optimiser step
    // needs every voxel, except in slab mode, where only the top slab's call
    // looks beyond its band (for the items no slab reaches)
    // the groups visited: one range [gb0, gb0 + gn0), or, for the top slab's
    // call in slab mode, that and a second range [gb1, gb1 + gn1)
    int64_t gb0 = 0, gn0 = 0, gb1 = 0, gn1 = 0;
    const bool top = g.sz0 + g.snz >= g.mnz;  // the slab holding the top planes
    if (kAdam && !kSlabs)
        gn0 = (g.onz + kKZ - 1) / kKZ;
    else if (kAdam && top)
        top_slab_walk<kKZ>(g, gb0, gn0, gb1, gn1);
    else
        gb0 = slab_band<kKZ>(g, gn0);
    ngroups = gn0 + gn1;
    const int64_t tiles = tiles_x * tiles_y;
    // XCD x takes the visited groups x, x + 8, ... (counting through both
    // ranges): a slab's band of groups is shared by all XCDs, x-neighbouring
    // tiles of a group still run together on one XCD, and with or without the
    // optimiser step the same block sums the same items in the same order.
    // (The z-block walk of the other sampler kernels made this kernel slower:
    // on the 1280 x 1536 x 1280 grid in 8 slabs 6.6 -> 7.4 ms per slab call
    // in blocks of 4 groups, 10.3 ms in blocks of 8.)
    const int xcd = int(blockIdx.x) % kXcds, per = int(gridDim.x) / kXcds;
    const int64_t xgroups = ngroups > xcd ? (ngroups - xcd + kXcds - 1) / kXcds : 0;
    const ItemRange r{int64_t(blockIdx.x) / kXcds, xgroups * tiles, per};
    float sv[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) sv[k] = float(g.sv[k]);
    double acc[12];
#pragma unroll
    for (int k = 0; k < 12; ++k) acc[k] = 0.0;
    auto item_index = [&](int64_t i0) {
        const int64_t vg = xcd + kXcds * (i0 / tiles);
        return (vg < gn0 ? gb0 + vg : gb1 + (vg - gn0)) * tiles + i0 % tiles;
    };
    SlabMasks sm{};
    int j = 0;
    for (int64_t it0 = r.begin; it0 < r.end; it0 += r.step, ++j) {
        if ((j & 63) == 0) {
            const int64_t il = it0 + int64_t(threadIdx.x & 63) * r.step;
            sm = slab_masks<kKZ>(g, il < r.end, il < r.end ? item_index(il) : 0, tiles_x, tiles_y, top);
        }
        const uint64_t bit = 1ull << (j & 63);
        const int64_t it = item_index(it0);
        Item m;
        item_at<kKZ>(g, it, tiles_x, tiles_y, m);
        if (m.nzk == 0) continue;
        const int64_t o0 = m.z0 * plane + m.y * g.onx + m.x;
        // slab mode: whether an earlier slab reaches the item (its partial
        // gradient is in gu) and whether a later one will (it keeps it there)
        bool first = false, last = true;
        if (kSlabs) {
            first = !(sm.prev & bit);
            last = !(sm.later & bit);
        }
        if (!(sm.touch & bit)) {
            // slab mode: only the top slab's call steps the items no slab reaches
            if (kSlabs && !(sm.none & bit)) continue;
            // this slab adds nothing to the item's gradient or affine sums; the
            // optimiser step still takes the earlier slabs' gradient
            if (kAdam)
                for (int k = 0; k < m.nzk; ++k)
                    for (int c = 0; c < 3; ++c) {
                        const int64_t oc = o0 + k * plane + c * ostride;
                        float uu = ad.u[oc], a1 = __builtin_nontemporal_load(ad.m1 + oc),
                              a2 = __builtin_nontemporal_load(ad.m2 + oc);
                        adam_one(uu, a1, a2, accumulate && !kSlabs ? gu[oc] : 0.0f, ad.p);
                        __builtin_nontemporal_store(uu, ad.u + oc);
                        __builtin_nontemporal_store(a1, ad.m1 + oc);
                        __builtin_nontemporal_store(a2, ad.m2 + oc);
                    }
            continue;
        }
        float u0[kKZ], u1[kKZ], u2[kKZ], gw[kKZ], fv[kKZ], wv[kKZ];
#pragma unroll
        for (int k = 0; k < kKZ; ++k) {
            const bool ok = k < m.nzk;
            const int64_t o = o0 + k * plane;
            u0[k] = ok ? __builtin_nontemporal_load(g.u + o) : 0.0f;
            u1[k] = ok ? __builtin_nontemporal_load(g.u + o + ostride) : 0.0f;
            u2[k] = ok ? __builtin_nontemporal_load(g.u + o + 2 * ostride) : 0.0f;
            gw[k] = ok && gW ? __builtin_nontemporal_load(gW + o) : 0.0f;
            if constexpr (kMi) {
                fv[k] = ok ? __builtin_nontemporal_load(mi.F + o) : 0.0f;
                wv[k] = ok ? __builtin_nontemporal_load(mi.W + o) : 0.0f;
            }
        }
        // the earlier slabs' gradient of the item is loaded with u, before the
        // gathers, so that its latency overlaps theirs instead of following it
        // once per voxel and component (loading the optimiser state early as
        // well costs a wave per SIMD and is slower)
        float prev[kKZ][3], st1[kKZ][3], st2[kKZ][3];
#pragma unroll
        for (int k = 0; k < kKZ; ++k)
#pragma unroll
            for (int c = 0; c < 3; ++c) {
                const bool ok = k < m.nzk;
                const bool has_prev = kSlabs ? !first : accumulate != 0;
                const int64_t oc = o0 + k * plane + c * ostride;
                prev[k][c] = has_prev && ok ? gu[oc] : 0.0f;
                // in slab mode the optimiser state of the items this call
                // completes is loaded here too (the kernel runs at three waves
                // per SIMD there anyway)
                st1[k][c] = kSlabs && kSlabPrefetch && last && ok ? __builtin_nontemporal_load(ad.m1 + oc) : 0.0f;
                st2[k][c] = kSlabs && kSlabPrefetch && last && ok ? __builtin_nontemporal_load(ad.m2 + oc) : 0.0f;
            }
        Sample s[kKZ];
#pragma unroll
        for (int k = 0; k < kKZ; ++k) gather(g, m.x, m.y, m.z0 + k, u0[k], u1[k], u2[k], s[k]);
        float part[12];
#pragma unroll
        for (int k = 0; k < 12; ++k) part[k] = 0.0f;
#pragma unroll
        for (int k = 0; k < kKZ; ++k) {
            if (k >= m.nzk) break;
            float gp[3];
            float gt = gw[k];
            if constexpr (kMi) gt = gt + mi::grad_value<3>(fv[k], wv[k], mi.p, mi_table, mi.gscale);
            sample_grad(s[k], gt, gp);
            const int64_t o = o0 + k * plane;
#pragma unroll
            for (int c = 0; c < 3; ++c) {
                float v = su_component(sv, gp, c);
                const int64_t oc = o + c * ostride;
                v += prev[k][c];
                if (kSlabs && !last) {
                    gu[oc] = v;  // a later slab adds to it and takes the step
                } else if (kAdam) {
                    // this voxel's u was read above and nothing else reads it
                    // the optimiser state streams through once: non-temporal
                    float uu = c == 0 ? u0[k] : (c == 1 ? u1[k] : u2[k]);
                    float a1 = kSlabs && kSlabPrefetch ? st1[k][c] : __builtin_nontemporal_load(ad.m1 + oc);
                    float a2 = kSlabs && kSlabPrefetch ? st2[k][c] : __builtin_nontemporal_load(ad.m2 + oc);
                    adam_one(uu, a1, a2, v, ad.p);
                    __builtin_nontemporal_store(uu, ad.u + oc);
                    __builtin_nontemporal_store(a1, ad.m1 + oc);
                    __builtin_nontemporal_store(a2, ad.m2 + oc);
                } else {
                    gu[oc] = v;
                }
            }
            affine_add(part, gp, m, k);
        }
#pragma unroll
        for (int k = 0; k < 12; ++k) acc[k] += double(part[k]);
    }
    __shared__ double red[16];
#pragma unroll
    for (int k = 0; k < 12; ++k) {
        const double v = block_sum(acc[k], red);
        if (threadIdx.x == 0) partials[size_t(blockIdx.x) * kPartialStride + k] = v;
    }
}

// The backward fused with the optimiser step over the whole output grid (no
// z-range bound, not a slab sequence), software-pipelined like the
// overwriting forward: everything a work item reads besides its gathers -- u,
// gW, the earlier slabs' gradient when accumulating, F when the MI gradient is
// formed here, and the optimiser state -- is copied into LDS
// (double-buffered) while the item before it gathers. Same walk, same items
// per block in the same order and same arithmetic as warp_bwd_kernel, so the
// results are bit for bit the same. Measured on the 640 x 768 x 640 grid:
// 5.81 ms against 5.91 ms (three waves per SIMD here, four there; the call
// moves 80 B/voxel and runs near the copy rate either way). Without the
// optimiser step the pipelined walk needs 129 VGPRs and gained nothing, so
// the plain backward keeps warp_bwd_kernel.
//
// kMi (the second sweep of a fused step): the MI term's gradient is formed
// here instead of being read from gW. The backward gathers the sample's
// corners anyway, so W at the voxel is the trilinear form on them (the
// forward's value, bit for bit); with F at the voxel and the log-ratio table
// (in LDS) it gives d loss_MI / d W, to which gW (the other terms' gradient,
// or none) is added, in the order the MI sweep and an accumulating loss call
// would have added them.

// LDS rows of one plane in the copy (one float per thread each); -1: absent.
struct BwdRows {
    int u, g, p, f, m1, m2, n;
};

__device__ inline void bwd_to_lds(const WarpGeom &g, const float *gW, const float *gu, const float *F,
                                  const AdamArgs &ad, const BwdRows &R, const Item &m, int64_t o0, int64_t plane,
                                  int64_t ostride, float (*buf)[kThreads]) {
    const int wb = threadIdx.x & ~63;
#pragma unroll
    for (int k = 0; k < kKZB; ++k) {
        if (k < m.nzk) {
            const int64_t o = o0 + k * plane;
            float(*row)[kThreads] = buf + k * R.n;
#pragma unroll
            for (int c = 0; c < 3; ++c)
                __builtin_amdgcn_global_load_lds(g.u + o + c * ostride, &row[R.u + c][wb], 4, 0, 0);
            if (R.g >= 0) __builtin_amdgcn_global_load_lds(gW + o, &row[R.g][wb], 4, 0, 0);
            if (R.p >= 0)
#pragma unroll
                for (int c = 0; c < 3; ++c)
                    __builtin_amdgcn_global_load_lds(gu + o + c * ostride, &row[R.p + c][wb], 4, 0, 0);
            if (R.f >= 0) __builtin_amdgcn_global_load_lds(F + o, &row[R.f][wb], 4, 0, 0);
#pragma unroll
            for (int c = 0; c < 3; ++c) {
                __builtin_amdgcn_global_load_lds(ad.m1 + o + c * ostride, &row[R.m1 + c][wb], 4, 0, 0);
                __builtin_amdgcn_global_load_lds(ad.m2 + o + c * ostride, &row[R.m2 + c][wb], 4, 0, 0);
            }
        }
    }
}

// Dynamic LDS: the two copy buffers (2 x kKZB x R.n rows of kThreads
// floats), then with kMi the bins x bins log-ratio table.
template <bool kMi>
__global__ __launch_bounds__(kThreads) void warp_bwd_adam_pipe_kernel(WarpGeom g, const float *__restrict__ gW,
                                                                      float *__restrict__ gu,
                                                                      double *__restrict__ partials, AdamArgs ad,
                                                                      BwdRows R, MiFuse mf) {
    constexpr int kKZ = kKZB;
    extern __shared__ float lds[];
    float(*bufs)[kThreads] = reinterpret_cast<float(*)[kThreads]>(lds);
    const int brows = kKZ * R.n;  // rows per buffer
    float *L = lds + size_t(2 * brows) * kThreads;
    if (kMi) {
        const int nb2 = mf.p.bins * mf.p.bins;
        for (int i = threadIdx.x; i < nb2; i += kThreads) L[i] = mf.table[i];
        __syncthreads();
    }
    adam_resolve(ad.p);
    const int64_t plane = g.onx * g.ony, ostride = plane * g.onz;
    int64_t tiles_x, tiles_y;
    items_of<kKZ>(g, tiles_x, tiles_y);
    const int64_t ngroups = (g.onz + kKZ - 1) / kKZ, tiles = tiles_x * tiles_y;
    // the walk of warp_bwd_kernel without a band
    const ZWalk zw = zwalk<kKZ>(tiles, ngroups);
    const ItemRange r = zwalk_range(zw);
    auto item_of = [&](int64_t it0) { return zwalk_item(zw, it0); };
    float sv[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) sv[k] = float(g.sv[k]);
    double acc[12];
#pragma unroll
    for (int k = 0; k < 12; ++k) acc[k] = 0.0;
    Item m;
    m.nzk = 0;
    int64_t o0 = 0;
    if (r.begin < r.end) {
        item_at<kKZ>(g, item_of(r.begin), tiles_x, tiles_y, m);
        o0 = m.z0 * plane + m.y * g.onx + m.x;
        bwd_to_lds(g, gW, gu, mf.F, ad, R, m, o0, plane, ostride, bufs);
        wait_lds_copies();
    }
    int b = 0;
    for (int64_t it0 = r.begin; it0 < r.end; it0 += r.step) {
        const int64_t nx0 = it0 + r.step;
        Item mn;
        mn.nzk = 0;
        int64_t on = 0;
        if (nx0 < r.end) {
            item_at<kKZ>(g, item_of(nx0), tiles_x, tiles_y, mn);
            on = mn.z0 * plane + mn.y * g.onx + mn.x;
            bwd_to_lds(g, gW, gu, mf.F, ad, R, mn, on, plane, ostride, bufs + (b ^ 1) * brows);
        }
        const float(*cur)[kThreads] = bufs + b * brows;
        float u0[kKZ], u1[kKZ], u2[kKZ], gw[kKZ];
#pragma unroll
        for (int k = 0; k < kKZ; ++k) {
            const bool ok = k < m.nzk;
            u0[k] = ok ? cur[k * R.n + R.u + 0][threadIdx.x] : 0.0f;
            u1[k] = ok ? cur[k * R.n + R.u + 1][threadIdx.x] : 0.0f;
            u2[k] = ok ? cur[k * R.n + R.u + 2][threadIdx.x] : 0.0f;
            gw[k] = ok && R.g >= 0 ? cur[k * R.n + R.g][threadIdx.x] : 0.0f;
        }
        float part[12], gv[kKZ][3];
#pragma unroll
        for (int k = 0; k < 12; ++k) part[k] = 0.0f;
        if (m.nzk > 0) {
            Sample s[kKZ];
#pragma unroll
            for (int k = 0; k < kKZ; ++k) gather(g, m.x, m.y, m.z0 + k, u0[k], u1[k], u2[k], s[k]);
#pragma unroll
            for (int k = 0; k < kKZ; ++k) {
                if (k >= m.nzk) break;
                float gp[3];
                if (kMi) {
                    float w, dw[3];
                    sample_terms(s[k], w, dw);
                    const float fv = cur[k * R.n + R.f][threadIdx.x];
                    const float gt = gw[k] + mi::grad_value<3>(fv, w, mf.p, L, mf.gscale);
                    gp[0] = dw[0] * gt;
                    gp[1] = dw[1] * gt;
                    gp[2] = dw[2] * gt;
                } else {
                    sample_grad(s[k], gw[k], gp);
                }
#pragma unroll
                for (int c = 0; c < 3; ++c) {
                    float v = su_component(sv, gp, c);
                    v += R.p >= 0 ? cur[k * R.n + R.p + c][threadIdx.x] : 0.0f;
                    gv[k][c] = v;
                }
                affine_add(part, gp, m, k);
            }
#pragma unroll
            for (int k = 0; k < 12; ++k) acc[k] += double(part[k]);
        }
        // the next item's copies (and this item's gathers) are in
        wait_lds_copies();
#pragma unroll
        for (int k = 0; k < kKZ; ++k) {
            if (k >= m.nzk) break;
            const int64_t o = o0 + k * plane;
#pragma unroll
            for (int c = 0; c < 3; ++c) {
                const int64_t oc = o + c * ostride;
                float uu = c == 0 ? u0[k] : (c == 1 ? u1[k] : u2[k]);
                float a1 = cur[k * R.n + R.m1 + c][threadIdx.x];
                float a2 = cur[k * R.n + R.m2 + c][threadIdx.x];
                adam_one(uu, a1, a2, gv[k][c], ad.p);
                __builtin_nontemporal_store(uu, ad.u + oc);
                __builtin_nontemporal_store(a1, ad.m1 + oc);
                __builtin_nontemporal_store(a2, ad.m2 + oc);
            }
        }
        m = mn;
        o0 = on;
        b ^= 1;
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

// Range of (S_v u)_z over the output grid: per-thread fp64 min and max (the
// same expression the sampler forms), per-block reduction into the partial
// slots, then one block folds the slots. Min and max do not depend on order.
__global__ __launch_bounds__(kThreads) void warp_zrange_kernel(WarpGeom g, double *__restrict__ partials) {
    const int64_t n = g.onx * g.ony * g.onz;
    const double s6 = g.sv[6], s7 = g.sv[7], s8 = g.sv[8];
    double lo = INFINITY, hi = -INFINITY;
    const ItemRange r = xcd_items((n + kThreads - 1) / kThreads);
    const float *uz = g.u + 2 * n;
    if (s6 == 0.0 && s7 == 0.0 && (reinterpret_cast<uintptr_t>(uz) & 15) == 0) {
        // S's z row holds only u_z (a diagonal S, as for the usual
        // normalisation): one field is read instead of three, with the same
        // values for finite u (the zero terms add exact zeros); 16-byte loads,
        // the last n mod 4 values in block 0
        const int64_t n4 = n / 4;
        const float4 *q = reinterpret_cast<const float4 *>(uz);
        const ItemRange r4 = xcd_items((n4 + kThreads - 1) / kThreads);
        for (int64_t it = r4.begin; it < r4.end; it += r4.step) {
            const int64_t o = it * kThreads + threadIdx.x;
            if (o < n4) {
                const float4 t = q[o];
                const double a = s8 * double(t.x), b = s8 * double(t.y), c = s8 * double(t.z),
                             d = s8 * double(t.w);
                lo = fmin(lo, fmin(fmin(a, b), fmin(c, d)));
                hi = fmax(hi, fmax(fmax(a, b), fmax(c, d)));
            }
        }
        if (blockIdx.x == 0 && threadIdx.x < n - 4 * n4) {
            const double v = s8 * double(uz[4 * n4 + threadIdx.x]);
            lo = fmin(lo, v);
            hi = fmax(hi, v);
        }
    } else if (s6 == 0.0 && s7 == 0.0) {
        for (int64_t it = r.begin; it < r.end; it += r.step) {
            const int64_t o = it * kThreads + threadIdx.x;
            if (o < n) {
                const double v = s8 * double(g.u[o + 2 * n]);
                lo = fmin(lo, v);
                hi = fmax(hi, v);
            }
        }
    } else {
        for (int64_t it = r.begin; it < r.end; it += r.step) {
            const int64_t o = it * kThreads + threadIdx.x;
            if (o < n) {
                const double v = fma(s6, double(g.u[o]), fma(s7, double(g.u[o + n]), s8 * double(g.u[o + 2 * n])));
                lo = fmin(lo, v);
                hi = fmax(hi, v);
            }
        }
    }
    __shared__ double rl[kThreads], rh[kThreads];
    rl[threadIdx.x] = lo;
    rh[threadIdx.x] = hi;
    __syncthreads();
    for (int w = kThreads / 2; w > 0; w >>= 1) {
        if (threadIdx.x < w) {
            rl[threadIdx.x] = fmin(rl[threadIdx.x], rl[threadIdx.x + w]);
            rh[threadIdx.x] = fmax(rh[threadIdx.x], rh[threadIdx.x + w]);
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        partials[size_t(blockIdx.x) * kPartialStride] = rl[0];
        partials[size_t(blockIdx.x) * kPartialStride + 1] = rh[0];
    }
}

__global__ __launch_bounds__(256) void warp_zrange_final(const double *__restrict__ partials, int nblocks,
                                                         double *__restrict__ zrange) {
    __shared__ double rl[256], rh[256];
    const int t = threadIdx.x;
    double lo = INFINITY, hi = -INFINITY;
    for (int b = t; b < nblocks; b += 256) {
        lo = fmin(lo, partials[size_t(b) * kPartialStride]);
        hi = fmax(hi, partials[size_t(b) * kPartialStride + 1]);
    }
    rl[t] = lo;
    rh[t] = hi;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (t < w) {
            rl[t] = fmin(rl[t], rl[t + w]);
            rh[t] = fmax(rh[t], rh[t + w]);
        }
        __syncthreads();
    }
    if (t == 0) {
        // all-NaN or empty input: a range that skips nothing
        zrange[0] = rl[0] <= rh[0] ? rl[0] : -INFINITY;
        zrange[1] = rl[0] <= rh[0] ? rh[0] : INFINITY;
    }
}

}  // namespace

hipError_t launch_warp_zrange(const WarpGeom &g, double *zrange, void *ws, hipStream_t s) {
    const int64_t n = g.onx * g.ony * g.onz;
    const int blocks = persistent_blocks((n + kThreads - 1) / kThreads, 8);
    double *partials = reinterpret_cast<double *>(static_cast<char *>(ws) + ws_layout(0).partials);
    hipLaunchKernelGGL(warp_zrange_kernel, dim3(blocks), dim3(kThreads), 0, s, g, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(warp_zrange_final, dim3(1), dim3(256), 0, s, partials, blocks, zrange);
    return hipGetLastError();
}

// A banded slab call (z-range bound) skips whole z-groups, so when it has to
// overwrite its output the output is zeroed first and the call adds.
static hipError_t zero_fill(float *p, int64_t n, hipStream_t s) {
    const int blocks = persistent_blocks((n + kThreads - 1) / kThreads, 8);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(kThreads), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_warp_fwd(const WarpGeom &g, float *W, int accumulate, hipStream_t s) {
    int64_t tx, ty;
    if (g.zrange && !accumulate) {
        hipError_t e = zero_fill(W, g.onx * g.ony * g.onz, s);
        if (e != hipSuccess) return e;
        accumulate = 1;
    }
    if (accumulate)
        hipLaunchKernelGGL(warp_fwd_acc_kernel<false>, dim3(persistent_blocks(items_of<kKZFA>(g, tx, ty), 8)),
                           dim3(kThreads), 0, s, g, W);
    else
        hipLaunchKernelGGL(warp_fwd_kernel, dim3(persistent_blocks(items_of<kKZF>(g, tx, ty), 8)),
                           dim3(kThreads), 0, s, g, W);
    return hipGetLastError();
}

hipError_t launch_warp_bwd_final(const double *partials, int nblocks, const WarpBwdFinal &fin, double *gA9,
                                 double *gt3, int accumulate, hipStream_t s) {
    hipLaunchKernelGGL(warp_bwd_final, dim3(1), dim3(256), 0, s, partials, nblocks, fin, gA9, gt3, accumulate);
    return hipGetLastError();
}

hipError_t launch_warp_fwd_seq(const WarpGeom &g, float *W, hipStream_t s) {
    int64_t tx, ty;
    hipLaunchKernelGGL(warp_fwd_acc_kernel<true>, dim3(persistent_blocks(items_of<kKZFA>(g, tx, ty), 8)),
                       dim3(kThreads), 0, s, g, W);
    return hipGetLastError();
}

hipError_t launch_warp_compose(const WarpGeom &g, float *w, hipStream_t s) {
    int64_t tx, ty;
    const int blocks = persistent_blocks(items_of<kKZC>(g, tx, ty), 8);
    hipLaunchKernelGGL(warp_compose_kernel, dim3(blocks), dim3(kThreads), 0, s, g, w);
    return hipGetLastError();
}

hipError_t launch_warp_fwd_hist(const WarpGeom &g, float *W, int accumulate, const float *F, const MiParams &p,
                                unsigned long long *hist, hipStream_t s) {
    int64_t tx, ty;
    const size_t lds_h = size_t(p.bins) * p.bins * sizeof(unsigned long long) + mi::ring_bytes(kThreads);
    if (lds_h > 65536) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(warp_fwd_hist_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, int(lds_h));
        if (e != hipSuccess) return e;
    }
    const int blocks = persistent_blocks(items_of<kKZH>(g, tx, ty), lds_h > 32768 ? 1 : 4);
    hipLaunchKernelGGL(warp_fwd_hist_kernel, dim3(blocks), dim3(kThreads), lds_h, s, g, W, accumulate, F, p, hist);
    return hipGetLastError();
}

hipError_t launch_warp_bwd(const WarpGeom &g, const float *gW, float *gu, double *gA9, double *gt3,
                           const WarpBwdFinal &fin, int accumulate, void *ws, hipStream_t s,
                           const AdamFuse *adam, const MiFuse *mi) {
    int64_t tx, ty;
    const bool seq = adam && adam->slab_mode;  // the slab sequence's instantiations take kKZBS planes
    const int blocks = persistent_blocks(seq ? items_of<kKZBS>(g, tx, ty) : items_of<kKZB>(g, tx, ty), 8);
    double *partials = reinterpret_cast<double *>(static_cast<char *>(ws) + ws_layout(0).partials);
    AdamArgs ad{};
    if (adam) {
        ad.u = adam->u;
        ad.m1 = adam->m1;
        ad.m2 = adam->m2;
        ad.p = adam->p;
        if (adam->slab_mode && mi) {
            const SlabMi smi{mi->F, mi->W, mi->p, mi->table, mi->gscale};
            const size_t lds = size_t(mi->p.bins) * mi->p.bins * sizeof(float);
            if (lds > 65536) {
                hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(warp_bwd_kernel<true, true, true>),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
                if (e != hipSuccess) return e;
            }
            hipLaunchKernelGGL((warp_bwd_kernel<true, true, true>), dim3(blocks), dim3(kThreads), lds, s, g, gW, gu,
                               accumulate, partials, ad, smi);
        } else if (adam->slab_mode)
            hipLaunchKernelGGL((warp_bwd_kernel<true, true>), dim3(blocks), dim3(kThreads), 0, s, g, gW, gu, accumulate,
                               partials, ad, SlabMi{});
        else if (!g.zrange) {
            // LDS rows of one plane: u, gW (when given), the earlier gradient
            // (when accumulating), F (with the MI gradient), m1, m2
            BwdRows R;
            int n = 3;
            R.u = 0;
            R.g = gW ? n++ : -1;
            R.p = accumulate ? n : -1;
            n += accumulate ? 3 : 0;
            R.f = mi ? n++ : -1;
            R.m1 = n;
            R.m2 = n + 3;
            R.n = n + 6;
            const size_t lds = size_t(2 * kKZB * R.n) * kThreads * sizeof(float) +
                               (mi ? size_t(mi->p.bins) * mi->p.bins * sizeof(float) : 0);
            const void *kern = mi ? reinterpret_cast<const void *>(warp_bwd_adam_pipe_kernel<true>)
                                  : reinterpret_cast<const void *>(warp_bwd_adam_pipe_kernel<false>);
            if (lds > 65536) {
                hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
                if (e != hipSuccess) return e;
            }
            const MiFuse mf = mi ? *mi : MiFuse{};
            if (mi)
                hipLaunchKernelGGL(warp_bwd_adam_pipe_kernel<true>, dim3(blocks), dim3(kThreads), lds, s, g, gW, gu,
                                   partials, ad, R, mf);
            else
                hipLaunchKernelGGL(warp_bwd_adam_pipe_kernel<false>, dim3(blocks), dim3(kThreads), lds, s, g, gW, gu,
                                   partials, ad, R, mf);
        } else
            hipLaunchKernelGGL(warp_bwd_kernel<true>, dim3(blocks), dim3(kThreads), 0, s, g, gW, gu, accumulate,
                               partials, ad, SlabMi{});
    } else {
        const int affine_acc = accumulate;
        if (g.zrange && !accumulate) {
            hipError_t e = zero_fill(gu, 3 * g.onx * g.ony * g.onz, s);
            if (e != hipSuccess) return e;
            accumulate = 1;
        }
        hipLaunchKernelGGL(warp_bwd_kernel<false>, dim3(blocks), dim3(kThreads), 0, s, g, gW, gu, accumulate,
                           partials, ad, SlabMi{});
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(warp_bwd_final, dim3(1), dim3(256), 0, s, partials, blocks, fin, gA9, gt3, affine_acc);
        return hipGetLastError();
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(warp_bwd_final, dim3(1), dim3(256), 0, s, partials, blocks, fin, gA9, gt3,
                       adam ? adam->accumulate_affine : accumulate);
    return hipGetLastError();
}

}  // namespace ngv
