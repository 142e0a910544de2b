// Device helpers of the composite implicit grid sampler ("A Scalable
// Distributed Framework for Multimodal GigaVoxel Image Registration", Key
// design 1), shared by the sampler kernels and the LNCC kernel that samples
// W itself in the fused second sweep: the sample position p = i + d of an
// output voxel, the 8 corners of its cell, the trilinear form and its
// derivative. The same functions give the same values in every kernel.
#pragma once

#include "ngv_internal.hpp"

namespace ngv {
namespace sampler {

struct Sample {
    float c[8];  // corners, index (dz*2 + dy)*2 + dx
    float fx, fy, fz;
};

// Two x-adjacent corners in one 8-byte load; only 4-byte alignment is known.
struct __attribute__((aligned(4))) Pair {
    float a, b;
};

// The cell of a sample: its floor corner in M's voxel grid and the
// fractional offsets. Index arithmetic is 32-bit: the sampling calls take
// extents of at most 2^30 voxels and moving-image planes of fewer than 2^31
// voxels, and offsets are clamped to +-1e9 voxels, so a corner index
// i + floor(d) and a plane offset y * nx + x inside M both fit an int. (With
// 64-bit indices the int64 conversions, compares and products made up about
// a quarter of the vector instructions in the forward kernel's code.)
struct Cell {
    int x0, y0, z0;
    float fx, fy, fz;
};

// Sample position of output voxel (ix, iy, iz) with displacement (u0, u1, u2).
// The offset d is formed in fp64 (full rate on CDNA): fp32 positions carry
// ~1e-6 voxel of rounding at these extents, which is a 1e-3 relative error
// in W wherever the sample sits a hair inside a zero-padded face.
__device__ inline void locate(const WarpGeom &g, int ix, int iy, int iz, float u0, float u1, float u2, Cell &c) {
    const double di[3] = {double(ix), double(iy), double(iz)};
    const double du[3] = {double(u0), double(u1), double(u2)};
    const int ii[3] = {ix, iy, iz};
    int i0[3];
    float f[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        double d = fma(g.a[j * 3 + 0], di[0], fma(g.a[j * 3 + 1], di[1], fma(g.a[j * 3 + 2], di[2], g.tv[j])));
        d += fma(g.sv[j * 3 + 0], du[0], fma(g.sv[j * 3 + 1], du[1], g.sv[j * 3 + 2] * du[2]));
        // clamp far-away offsets before the integer conversion (they sample zero)
        d = fmin(fmax(d, -1.0e9), 1.0e9);
        const double fl = floor(d);
        f[j] = float(d - fl);
        i0[j] = ii[j] + int(fl);
    }
    c.fx = f[0];
    c.fy = f[1];
    c.fz = f[2];
    c.x0 = i0[0];
    c.y0 = i0[1];
    c.z0 = i0[2];
}

// The 8 corner values of cell c in volume V (M's grid and held planes);
// corners outside the moving grid or outside the held slab read as zero.
__device__ inline void corners(const WarpGeom &g, const float *V, const Cell &c, float (&v)[8]) {
    const int nx = int(g.mnx), ny = int(g.mny), nz = int(g.snz), pz = int(g.mnx * g.mny);
    const int x0 = c.x0, y0 = c.y0, zr = c.z0 - int(g.sz0);  // zr: plane within the held slab
    // 0 <= x0 < nx - 1 and so on, as unsigned compares
    const bool inside = unsigned(x0) < unsigned(nx - 1) && unsigned(y0) < unsigned(ny - 1) &&
                        unsigned(zr) < unsigned(nz - 1);
    if (inside) {
        const float *b = V + (int64_t(zr) * pz + (y0 * nx + x0));
        const Pair p0 = *reinterpret_cast<const Pair *>(b);
        const Pair p1 = *reinterpret_cast<const Pair *>(b + nx);
        const Pair p2 = *reinterpret_cast<const Pair *>(b + pz);
        const Pair p3 = *reinterpret_cast<const Pair *>(b + pz + nx);
        v[0] = p0.a;
        v[1] = p0.b;
        v[2] = p1.a;
        v[3] = p1.b;
        v[4] = p2.a;
        v[5] = p2.b;
        v[6] = p3.a;
        v[7] = p3.b;
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int x = x0 + (k & 1), y = y0 + ((k >> 1) & 1), z = zr + (k >> 2);
            const bool ok = unsigned(x) < unsigned(nx) && unsigned(y) < unsigned(ny) && unsigned(z) < unsigned(nz);
            v[k] = ok ? V[int64_t(z) * pz + (y * nx + x)] : 0.0f;
        }
    }
}

// Sample position and the 8 corner values of M for output voxel (ix, iy, iz).
__device__ inline void gather(const WarpGeom &g, int ix, int iy, int iz, float u0, float u1, float u2, Sample &s) {
    Cell c;
    locate(g, ix, iy, iz, u0, u1, u2, c);
    s.fx = c.fx;
    s.fy = c.fy;
    s.fz = c.fz;
    corners(g, g.M, c, s.c);
}

// The trilinear form on the corners of a cell (x first, then y, then z).
__device__ inline float trilerp(const float (&c)[8], float fx, float fy, float fz) {
    const float e00 = fmaf(fx, c[1] - c[0], c[0]);
    const float e10 = fmaf(fx, c[3] - c[2], c[2]);
    const float e01 = fmaf(fx, c[5] - c[4], c[4]);
    const float e11 = fmaf(fx, c[7] - c[6], c[6]);
    const float f0 = fmaf(fy, e10 - e00, e00);
    const float f1 = fmaf(fy, e11 - e01, e01);
    return fmaf(fz, f1 - f0, f0);
}

// The per-sample terms of the backward: W at the sample (the trilinear form,
// the same arithmetic as trilerp, so the same value as the forward's) and
// dW/dp_vox, the form's derivative in each axis at the sample's fractional
// position.
__device__ inline void sample_terms(const Sample &q, float &w, float (&dw)[3]) {
    const float e00 = fmaf(q.fx, q.c[1] - q.c[0], q.c[0]);
    const float e10 = fmaf(q.fx, q.c[3] - q.c[2], q.c[2]);
    const float e01 = fmaf(q.fx, q.c[5] - q.c[4], q.c[4]);
    const float e11 = fmaf(q.fx, q.c[7] - q.c[6], q.c[6]);
    const float f0 = fmaf(q.fy, e10 - e00, e00);
    const float f1 = fmaf(q.fy, e11 - e01, e01);
    const float dx0 = fmaf(q.fy, (q.c[3] - q.c[2]) - (q.c[1] - q.c[0]), q.c[1] - q.c[0]);
    const float dx1 = fmaf(q.fy, (q.c[7] - q.c[6]) - (q.c[5] - q.c[4]), q.c[5] - q.c[4]);
    w = fmaf(q.fz, f1 - f0, f0);
    dw[0] = fmaf(q.fz, dx1 - dx0, dx0);
    dw[1] = fmaf(q.fz, (e11 - e01) - (e10 - e00), e10 - e00);
    dw[2] = f1 - f0;
}

// Component c of S_v^T g_p (sv holds S_v row-major in fp32).
__device__ inline float su_component(const float (&sv)[9], const float (&gp)[3], int c) {
    return fmaf(sv[0 * 3 + c], gp[0], fmaf(sv[1 * 3 + c], gp[1], sv[2 * 3 + c] * gp[2]));
}

}  // namespace sampler
}  // namespace ngv
