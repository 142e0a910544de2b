/*
 * ngv_oracle.c -- the oracle: a plain, slow, fp64 CPU implementation of one
 * optimisation step of affine + deformable image registration.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library. It shares no source,
 * header, table or helper with the HIP library and includes nothing from it.
 *
 * Source of every definition below: the papernotes.org summary page
 * "A Scalable Distributed Framework for Multimodal GigaVoxel Image
 * Registration" (ICLR 2026), cited by its section names:
 *   Background      objective L(phi) = C(F, M o phi) + R(phi) with the
 *                   composite map phi(x) = A x + t + u(x)
 *   Key design 1    the composite implicit grid sampler I(A x + t + S u(x)),
 *                   identity grid given only by its bounds x_bounds
 *   Key design 2    Mattes MI as the KL divergence between the joint and the
 *                   product of marginals, with Parzen (kernel density)
 *                   estimates P_I(v) = (1/N) sum_k kappa(v - I_k) on B bins;
 *                   LNCC from I, J, I^2, J^2, IJ and their w-box sums
 *   Key design 4    interpolation splits into partial sums over image shards
 *   Key design 5    the global histogram is the N_h/N weighted sum of the
 *                   shard histograms
 *   Method overview optimiser states m1, m2 and a gradient step after
 *                   Sobolev smoothing
 * Points the page leaves open are settled by the readings listed at each
 * function (frame, padding, kernel, bin mapping, LNCC form, optimiser).
 *
 * Every function computes the plain definition, voxel by voxel. The only
 * liberties: a w^3 window sum is evaluated as nested axis sums (a
 * re-bracketing of the same finite sum), and OpenMP splits loops over z,
 * with partial sums combined in a fixed order.
 *
 * Layout: volumes are fp32, x fastest: index (z*ny + y)*nx + x. Vector fields
 * (u, gu) are three such volumes back to back, components (x, y, z).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_API __attribute__((visibility("default")))

ORC_API int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the parallel loops that follow (n >= 1). */
ORC_API void orc_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------ */
/* Grid sampler (Key design 1)                                              */
/* ------------------------------------------------------------------------ */

/* Parameters of one sampler call. Coordinates are the normalised frame
 * [-1, 1] per axis with the end voxels' centres at -1 and +1 (reading:
 * align_corners=True, the plainest PyTorch-like frame). The output grid is
 * the implicit identity grid spanning [xmin, xmax]; M is the moving image on
 * the full grid of size mn, of which the buffer holds planes [sz0, sz0+snz). */
typedef struct {
    const float *M;
    int64_t mn[3];          /* moving grid size (x, y, z) */
    int64_t sz0, snz;       /* planes of M present in the buffer */
    const float *u;         /* displacement, [3][on_z][on_y][on_x] */
    int64_t on[3];          /* output grid size (x, y, z) */
    double A[9], t[3], S[9], xmin[3], xmax[3];
} warp_prm;

static void unpack_prm(warp_prm *w, const float *M, const int64_t *mn, int64_t sz0, int64_t snz,
                       const float *u, const int64_t *on, const double *prm) {
    int k;
    w->M = M;
    w->u = u;
    for (k = 0; k < 3; ++k) {
        w->mn[k] = mn[k];
        w->on[k] = on[k];
    }
    w->sz0 = sz0;
    w->snz = snz;
    memcpy(w->A, prm + 0, 9 * sizeof(double));
    memcpy(w->t, prm + 9, 3 * sizeof(double));
    memcpy(w->S, prm + 12, 9 * sizeof(double));
    memcpy(w->xmin, prm + 21, 3 * sizeof(double));
    memcpy(w->xmax, prm + 24, 3 * sizeof(double));
}

/* Moving image value at an integer voxel, zero outside the volume (reading:
 * zero padding) and zero for planes not held by this slab (Key design 4:
 * each shard contributes only the corners it owns). */
static double m_at(const warp_prm *w, int64_t x, int64_t y, int64_t z) {
    if (x < 0 || y < 0 || z < 0 || x >= w->mn[0] || y >= w->mn[1] || z >= w->mn[2]) return 0.0;
    if (z < w->sz0 || z >= w->sz0 + w->snz) return 0.0;
    return (double)w->M[((z - w->sz0) * w->mn[1] + y) * w->mn[0] + x];
}

/* Normalised coordinate of output voxel index i along axis k. */
static double grid_coord(const warp_prm *w, int k, int64_t i) {
    double delta = w->on[k] > 1 ? (w->xmax[k] - w->xmin[k]) / (double)(w->on[k] - 1) : 0.0;
    return w->xmin[k] + delta * (double)i;
}

/* Sample position in M's voxel units for output voxel (ix, iy, iz), and the
 * normalised grid point x. p = A x + t + S u(x), then p_vox = (p + 1)(n - 1)/2.
 * Positions within 1e-10 (relative) of a lattice point are taken as that
 * lattice point: this undoes the fp64 rounding of the normalised round trip,
 * so that the identity map lands exactly on voxels as in exact arithmetic. */
static void sample_pos(const warp_prm *w, int64_t ix, int64_t iy, int64_t iz, double pv[3], double x[3]) {
    int64_t N = w->on[0] * w->on[1] * w->on[2];
    int64_t lin = (iz * w->on[1] + iy) * w->on[0] + ix;
    double uu[3], p[3];
    int j, k;
    x[0] = grid_coord(w, 0, ix);
    x[1] = grid_coord(w, 1, iy);
    x[2] = grid_coord(w, 2, iz);
    for (k = 0; k < 3; ++k) uu[k] = (double)w->u[k * N + lin];
    for (j = 0; j < 3; ++j) {
        p[j] = w->t[j];
        for (k = 0; k < 3; ++k) p[j] += w->A[j * 3 + k] * x[k] + w->S[j * 3 + k] * uu[k];
        pv[j] = (p[j] + 1.0) * (double)(w->mn[j] - 1) / 2.0;
        {
            double q = nearbyint(pv[j]);
            if (fabs(pv[j] - q) <= 1e-10 * fmax(1.0, fabs(q))) pv[j] = q;
        }
    }
}

/* Trilinear interpolation of M at pv (floor cell), its derivative with
 * respect to pv (the derivative of the floor cell's trilinear form, so a
 * forward difference at exact lattice positions), and the distance of the
 * fractional parts to the nearest cell face. */
static double trilinear(const warp_prm *w, const double pv[3], double dW[3], double *kink) {
    int64_t i0[3];
    double f[3], val = 0.0;
    int cx, cy, cz, k;
    for (k = 0; k < 3; ++k) {
        double fl = floor(pv[k]);
        i0[k] = (int64_t)fl;
        f[k] = pv[k] - fl;
    }
    dW[0] = dW[1] = dW[2] = 0.0;
    for (cz = 0; cz < 2; ++cz)
        for (cy = 0; cy < 2; ++cy)
            for (cx = 0; cx < 2; ++cx) {
                double v = m_at(w, i0[0] + cx, i0[1] + cy, i0[2] + cz);
                double wx = cx ? f[0] : 1.0 - f[0];
                double wy = cy ? f[1] : 1.0 - f[1];
                double wz = cz ? f[2] : 1.0 - f[2];
                val += wx * wy * wz * v;
                dW[0] += (cx ? 1.0 : -1.0) * wy * wz * v;
                dW[1] += wx * (cy ? 1.0 : -1.0) * wz * v;
                dW[2] += wx * wy * (cz ? 1.0 : -1.0) * v;
            }
    if (kink) {
        double kd = 1.0;
        for (k = 0; k < 3; ++k) {
            double d = fmin(f[k], 1.0 - f[k]);
            if (d < kd) kd = d;
        }
        *kink = kd;
    }
    return val;
}

/* W(i) = M~(p_vox(i)) for output planes [z_lo, z_hi). W and kink (optional)
 * are full output volumes; only the requested planes are written. */
ORC_API void orc_warp_fwd(const float *M, const int64_t *mn, int64_t sz0, int64_t snz, const float *u,
                          const int64_t *on, const double *prm, int64_t z_lo, int64_t z_hi, double *W,
                          double *kink) {
    warp_prm w;
    int64_t iz;
    unpack_prm(&w, M, mn, sz0, snz, u, on, prm);
#pragma omp parallel for schedule(dynamic, 1)
    for (iz = z_lo; iz < z_hi; ++iz) {
        int64_t iy, ix;
        for (iy = 0; iy < w.on[1]; ++iy)
            for (ix = 0; ix < w.on[0]; ++ix) {
                double pv[3], x[3], dW[3], kd;
                int64_t lin = (iz * w.on[1] + iy) * w.on[0] + ix;
                sample_pos(&w, ix, iy, iz, pv, x);
                W[lin] = trilinear(&w, pv, dW, &kd);
                if (kink) kink[lin] = kd;
            }
    }
}

/* The same at a list of output voxels (linear indices), for sampled checks of
 * volumes too large to warp whole on the host. dWdp (optional) gets the 3
 * derivatives per point. */
ORC_API void orc_warp_points(const float *M, const int64_t *mn, int64_t sz0, int64_t snz, const float *u,
                             const int64_t *on, const double *prm, const int64_t *idx, int64_t npts,
                             double *W, double *dWdp, double *kink) {
    warp_prm w;
    int64_t q;
    unpack_prm(&w, M, mn, sz0, snz, u, on, prm);
#pragma omp parallel for schedule(static)
    for (q = 0; q < npts; ++q) {
        int64_t lin = idx[q];
        int64_t ix = lin % w.on[0], iy = (lin / w.on[0]) % w.on[1], iz = lin / (w.on[0] * w.on[1]);
        double pv[3], x[3], dW[3], kd;
        sample_pos(&w, ix, iy, iz, pv, x);
        W[q] = trilinear(&w, pv, dW, &kd);
        if (dWdp) {
            dWdp[3 * q + 0] = dW[0];
            dWdp[3 * q + 1] = dW[1];
            dWdp[3 * q + 2] = dW[2];
        }
        if (kink) kink[q] = kd;
    }
}

/* Backward of the sampler for output planes [z_lo, z_hi) (Key design 1: the
 * gradients reach u and the affine part). With g_p = dL/dp the chain rule
 * through p_vox = (p + 1)(n - 1)/2 gives
 *   g_p[j] = (n_j - 1)/2 * dW/dpv_j * gW,   gu = S^T g_p,
 *   dA[j][k] += g_p[j] * x[k],              dt[j] += g_p[j].
 * No gradient to M (it is data). gu is a full [3][volume] array (planes in
 * range written); dA, dt and mag are accumulated in fixed plane order.
 * mag accumulates sum |g_p| |x|, a conditioning scale for tests. */
ORC_API void orc_warp_bwd(const float *M, const int64_t *mn, int64_t sz0, int64_t snz, const float *u,
                          const int64_t *on, const double *prm, const double *gW, int64_t z_lo, int64_t z_hi,
                          double *gu, double *dA, double *dt, double *mag) {
    warp_prm w;
    int64_t iz, nzr = z_hi - z_lo, N;
    double *part;
    unpack_prm(&w, M, mn, sz0, snz, u, on, prm);
    N = w.on[0] * w.on[1] * w.on[2];
    if (nzr <= 0) return;
    part = (double *)calloc((size_t)nzr * 13, sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
    for (iz = z_lo; iz < z_hi; ++iz) {
        double *pp = part + (iz - z_lo) * 13;
        int64_t iy, ix;
        for (iy = 0; iy < w.on[1]; ++iy)
            for (ix = 0; ix < w.on[0]; ++ix) {
                double pv[3], x[3], dW[3], gp[3];
                int64_t lin = (iz * w.on[1] + iy) * w.on[0] + ix;
                int j, k;
                double gn = 0.0, xn = 0.0;
                sample_pos(&w, ix, iy, iz, pv, x);
                trilinear(&w, pv, dW, NULL);
                for (j = 0; j < 3; ++j) gp[j] = (double)(w.mn[j] - 1) / 2.0 * dW[j] * gW[lin];
                for (k = 0; k < 3; ++k) {
                    double s = 0.0;
                    for (j = 0; j < 3; ++j) s += w.S[j * 3 + k] * gp[j];
                    if (gu) gu[k * N + lin] = s;
                }
                for (j = 0; j < 3; ++j) {
                    for (k = 0; k < 3; ++k) pp[j * 3 + k] += gp[j] * x[k];
                    pp[9 + j] += gp[j];
                    gn += gp[j] * gp[j];
                    xn += x[j] * x[j];
                }
                pp[12] += sqrt(gn) * sqrt(xn);
            }
    }
    for (iz = 0; iz < nzr; ++iz) {
        int j;
        for (j = 0; j < 9; ++j) dA[j] += part[iz * 13 + j];
        for (j = 0; j < 3; ++j) dt[j] += part[iz * 13 + 9 + j];
        if (mag) *mag += part[iz * 13 + 12];
    }
    free(part);
}

/* orc_warp_fwd for planes [z_lo, z_hi), written chunk-relative:
 * W[(iz - z_lo) * plane + iy * nx + ix]. For volumes too large to hold in fp64. */
ORC_API void orc_warp_fwd_chunk(const float *M, const int64_t *mn, int64_t sz0, int64_t snz, const float *u,
                                const int64_t *on, const double *prm, int64_t z_lo, int64_t z_hi, double *W) {
    warp_prm w;
    int64_t iz;
    unpack_prm(&w, M, mn, sz0, snz, u, on, prm);
#pragma omp parallel for schedule(dynamic, 1)
    for (iz = z_lo; iz < z_hi; ++iz) {
        int64_t iy, ix;
        for (iy = 0; iy < w.on[1]; ++iy)
            for (ix = 0; ix < w.on[0]; ++ix) {
                double pv[3], x[3], dW[3];
                sample_pos(&w, ix, iy, iz, pv, x);
                W[((iz - z_lo) * w.on[1] + iy) * w.on[0] + ix] = trilinear(&w, pv, dW, NULL);
            }
    }
}

/* Sampler backward at a list of output voxels: gu (3 per point) = S^T g_p with
 * g_p[j] = (n_j - 1)/2 * dW/dpv_j * gW, given gW at those points. */
ORC_API void orc_warp_bwd_points(const float *M, const int64_t *mn, int64_t sz0, int64_t snz, const float *u,
                                 const int64_t *on, const double *prm, const int64_t *idx, int64_t npts,
                                 const double *gW, double *gu) {
    warp_prm w;
    int64_t q;
    unpack_prm(&w, M, mn, sz0, snz, u, on, prm);
#pragma omp parallel for schedule(static)
    for (q = 0; q < npts; ++q) {
        int64_t lin = idx[q];
        int64_t ix = lin % w.on[0], iy = (lin / w.on[0]) % w.on[1], iz = lin / (w.on[0] * w.on[1]);
        double pv[3], x[3], dW[3], gp[3];
        int j, k;
        sample_pos(&w, ix, iy, iz, pv, x);
        trilinear(&w, pv, dW, NULL);
        for (j = 0; j < 3; ++j) gp[j] = (double)(w.mn[j] - 1) / 2.0 * dW[j] * gW[q];
        for (k = 0; k < 3; ++k) {
            double s = 0.0;
            for (j = 0; j < 3; ++j) s += w.S[j * 3 + k] * gp[j];
            gu[3 * q + k] = s;
        }
    }
}

/* Derivative with respect to pv of the trilinear form of the cell with lower
 * corner i0, at fractional position f inside (or just outside) that cell. */
static void cell_deriv(const warp_prm *w, const int64_t i0[3], const double f[3], double dW[3]) {
    int cx, cy, cz;
    dW[0] = dW[1] = dW[2] = 0.0;
    for (cz = 0; cz < 2; ++cz)
        for (cy = 0; cy < 2; ++cy)
            for (cx = 0; cx < 2; ++cx) {
                double v = m_at(w, i0[0] + cx, i0[1] + cy, i0[2] + cz);
                double wx = cx ? f[0] : 1.0 - f[0];
                double wy = cy ? f[1] : 1.0 - f[1];
                double wz = cz ? f[2] : 1.0 - f[2];
                dW[0] += (cx ? 1.0 : -1.0) * wy * wz * v;
                dW[1] += wx * (cy ? 1.0 : -1.0) * wz * v;
                dW[2] += wx * wy * (cz ? 1.0 : -1.0) * v;
            }
}

/* Where the sample of an output voxel lies within `band` of a cell face, the
 * derivative of the sampler there is one-sided and both sides are valid
 * (reading: the floor cell is taken, but an evaluation in other precision
 * may fall on the other side of the face). For each voxel and component k
 * this writes the largest |gu_k(alt) - gu_k(floor cell)| over the cells that
 * share the faces within the band (each combination of those axes shifted to
 * the neighbouring cell), for the gradient gW: zero away from faces. A test
 * scale, like the kink distance: the spread of the valid answers. */
ORC_API void orc_warp_kink_spread(const float *M, const int64_t *mn, int64_t sz0, int64_t snz, const float *u,
                                  const int64_t *on, const double *prm, double band, const double *gW,
                                  double *spread) {
    warp_prm w;
    int64_t iz, N;
    unpack_prm(&w, M, mn, sz0, snz, u, on, prm);
    N = w.on[0] * w.on[1] * w.on[2];
#pragma omp parallel for schedule(dynamic, 1)
    for (iz = 0; iz < w.on[2]; ++iz) {
        int64_t iy, ix;
        for (iy = 0; iy < w.on[1]; ++iy)
            for (ix = 0; ix < w.on[0]; ++ix) {
                double pv[3], x[3], f[3], d0[3], best[3] = {0.0, 0.0, 0.0};
                int64_t i0[3], lin = (iz * w.on[1] + iy) * w.on[0] + ix;
                int side[3], k, j, m;
                sample_pos(&w, ix, iy, iz, pv, x);
                for (k = 0; k < 3; ++k) {
                    double fl = floor(pv[k]);
                    i0[k] = (int64_t)fl;
                    f[k] = pv[k] - fl;
                    side[k] = f[k] < band ? -1 : (f[k] > 1.0 - band ? 1 : 0);
                }
                if (side[0] || side[1] || side[2]) {
                    cell_deriv(&w, i0, f, d0);
                    for (m = 1; m < 8; ++m) {
                        int64_t i1[3];
                        double f1[3], d1[3], gp[3];
                        int ok = 1;
                        for (k = 0; k < 3; ++k) {
                            i1[k] = i0[k];
                            f1[k] = f[k];
                            if (m & (1 << k)) {
                                if (!side[k]) ok = 0;
                                i1[k] += side[k];
                                f1[k] -= side[k];
                            }
                        }
                        if (!ok) continue;
                        cell_deriv(&w, i1, f1, d1);
                        for (j = 0; j < 3; ++j) gp[j] = (double)(w.mn[j] - 1) / 2.0 * (d1[j] - d0[j]) * gW[lin];
                        for (k = 0; k < 3; ++k) {
                            double sdiff = 0.0;
                            for (j = 0; j < 3; ++j) sdiff += w.S[j * 3 + k] * gp[j];
                            if (fabs(sdiff) > best[k]) best[k] = fabs(sdiff);
                        }
                    }
                }
                for (k = 0; k < 3; ++k) spread[k * N + lin] = best[k];
            }
    }
}

/* ------------------------------------------------------------------------ */
/* Mattes mutual information (Key design 2, Key design 5)                   */
/* ------------------------------------------------------------------------ */

/* Parzen kernels. order 3: the cubic B-spline (reading: one cubic B-spline
 * kernel for both images, as the config's "cubic B-spline Parzen" says);
 * order 0: the unit box on (-1/2, 1/2], which turns the estimate into the
 * hard histogram: a sample with bin coordinate c falls in the one bin a with
 * a - c in (-1/2, 1/2], i.e. a = floor(c + 1/2), and a sample exactly half
 * way between two bin centres goes to the upper bin (reading: the page
 * defines the estimate P(v) = (1/N) sum_k kappa(v - I_k) and fixes no side
 * for the box's edges). Evaluated in fp64 on a - c, which is exact here. */
static double parzen(int order, double x) {
    double ax = fabs(x);
    if (order == 0) return (x > -0.5 && x <= 0.5) ? 1.0 : 0.0;
    if (ax < 1.0) return (4.0 - 6.0 * x * x + 3.0 * ax * ax * ax) / 6.0;
    if (ax < 2.0) return (2.0 - ax) * (2.0 - ax) * (2.0 - ax) / 6.0;
    return 0.0;
}

static double parzen_deriv(int order, double x) {
    double ax = fabs(x);
    if (order == 0) return 0.0;
    if (ax < 1.0) return -2.0 * x + 1.5 * x * ax;
    if (ax < 2.0) return (x > 0 ? -1.0 : 1.0) * (2.0 - ax) * (2.0 - ax) / 2.0;
    return 0.0;
}

/* Second derivative (used only for a conditioning scale, see orc_mi_grad). */
static double parzen_deriv2(int order, double x) {
    double ax = fabs(x);
    if (order == 0) return 0.0;
    if (ax < 1.0) return 3.0 * ax - 2.0;
    if (ax < 2.0) return 2.0 - ax;
    return 0.0;
}

/* Continuous bin coordinate of intensity v (reading: fixed range
 * [vmin, vmax] per image, values clamped into it, two bins of padding each
 * side so that the whole kernel mass of every sample lies inside the B bins). */
#define MI_PAD 2
static double bin_scale(int bins, double vmin, double vmax) {
    return (double)(bins - 1 - 2 * MI_PAD) / (vmax - vmin);
}
static double bin_coord(double v, int bins, double vmin, double vmax) {
    double c = v < vmin ? vmin : (v > vmax ? vmax : v);
    return (double)MI_PAD + (c - vmin) * bin_scale(bins, vmin, vmax);
}

/* Weight of F bin a for the fixed sample with bin coordinate cf: the
 * kernel of order forder at a - cf (forder 0 with a cubic W kernel is the
 * zero-order fixed kernel of Mattes et al.'s original pair: 1 at the box bin
 * floor(cf + 1/2), 0 elsewhere). */
static double fixed_weight(int forder, int a, double cf) {
    return parzen(forder, (double)a - cf);
}

#define MI_CHUNK 65536

/* Joint Parzen histogram, accumulated into H[a*bins + b] (a: F bin, b: W bin):
 *   H_ab += sum_k kappa_F(a - cF(F_k)) kappa(b - cW(W_k)),
 * kappa the kernel of the given order for W, kappa_F that of forder for F
 * (equal orders: one kernel for both images; forder 0 with order 3: the
 * zero-order fixed and cubic moving kernels of Mattes et al.'s original MI).
 * Summed in fixed chunks in fixed order, so the result does not depend on the
 * thread count. Accumulating calls over disjoint parts of a volume give the
 * whole-volume histogram (Key design 5). */
ORC_API void orc_mi_hist(const float *F, const double *W, int64_t n, int bins, double fmin, double fmax,
                         double wmin, double wmax, int forder, int order, double *H) {
    int64_t nch = (n + MI_CHUNK - 1) / MI_CHUNK, ch;
    int64_t B2 = (int64_t)bins * bins;
    int64_t group = 256; /* chunks per partial buffer, bounds memory */
    int64_t g0;
    double *part = (double *)malloc((size_t)(group * B2) * sizeof(double));
    for (g0 = 0; g0 < nch; g0 += group) {
        int64_t g1 = g0 + group < nch ? g0 + group : nch;
        memset(part, 0, (size_t)(group * B2) * sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
        for (ch = g0; ch < g1; ++ch) {
            double *h = part + (ch - g0) * B2;
            int64_t k0 = ch * MI_CHUNK, k1 = k0 + MI_CHUNK < n ? k0 + MI_CHUNK : n, k;
            for (k = k0; k < k1; ++k) {
                double cf = bin_coord((double)F[k], bins, fmin, fmax);
                double cw = bin_coord(W[k], bins, wmin, wmax);
                int a0 = (int)floor(cf) - 2, b0 = (int)floor(cw) - 2, a, b;
                for (a = a0; a <= a0 + 4; ++a) {
                    double wa;
                    if (a < 0 || a >= bins) continue;
                    wa = fixed_weight(forder, a, cf);
                    if (wa == 0.0) continue;
                    for (b = b0; b <= b0 + 4; ++b) {
                        if (b < 0 || b >= bins) continue;
                        h[(int64_t)a * bins + b] += wa * parzen(order, (double)b - cw);
                    }
                }
            }
        }
        for (ch = 0; ch < g1 - g0; ++ch) {
            int64_t q;
            for (q = 0; q < B2; ++q) H[q] += part[ch * B2 + q];
        }
    }
    free(part);
}

/* MI from the joint histogram of N samples: p = H/N, marginals as row and
 * column sums, MI = sum_{p_ab > 0} p_ab ln(p_ab / (p_a p_b)) (natural log,
 * 0 ln 0 = 0). L (optional, bins^2) gets ln(p_ab / (p_a p_b)) where p_ab > 0
 * and 0 elsewhere: the per-bin factor of the gradient. Returns MI. */
ORC_API double orc_mi_finalize(const double *H, int bins, double N, double *L) {
    double *pa = (double *)calloc((size_t)bins, sizeof(double));
    double *pb = (double *)calloc((size_t)bins, sizeof(double));
    double mi = 0.0;
    int a, b;
    for (a = 0; a < bins; ++a)
        for (b = 0; b < bins; ++b) {
            double p = H[a * bins + b] / N;
            pa[a] += p;
            pb[b] += p;
        }
    for (a = 0; a < bins; ++a)
        for (b = 0; b < bins; ++b) {
            double p = H[a * bins + b] / N, l = 0.0;
            if (p > 0.0) {
                l = log(p / (pa[a] * pb[b]));
                mi += p * l;
            }
            if (L) L[a * bins + b] = l;
        }
    free(pa);
    free(pb);
    return mi;
}

/* Gradient of loss = -weight * MI with respect to W_k. Differentiating
 * MI = sum p ln p - sum p_a ln p_a - sum p_b ln p_b gives
 *   dMI = sum_ab dp_ab (L_ab - 1) and sum_ab dp_ab = 0 (the kernel sums to 1),
 * and dp_ab/dW_k = -(s/N) kappa_F(a - cF_k) kappa'(b - cW_k) inside the clamp
 * range (s: bin scale). Hence
 *   gW_k = weight (s/N) sum_ab L_ab kappa_F(a - cF_k) kappa'(b - cW_k)
 * for wmin <= W_k <= wmax (clamp passes the gradient at its end points), else 0.
 * accumulate != 0 adds into gW. mode != 0 writes instead a conditioning scale
 * for comparing a lower-precision evaluation of the same sum (|weight| s/N
 * times): mode 1, sum_ab |L_ab kappa_F kappa'|, the magnitude of its terms;
 * mode 2, sum_ab |L_ab| (|kappa_F'| |kappa'| + |kappa_F| |kappa''|), the
 * magnitude of its derivative with respect to the two bin coordinates. */
ORC_API void orc_mi_grad(const float *F, const double *W, int64_t n, int bins, double fmin, double fmax,
                         double wmin, double wmax, int forder, int order, const double *L, double weight, double N,
                         double *gW, int accumulate, int mode) {
    double s = bin_scale(bins, wmin, wmax);
    int64_t k;
#pragma omp parallel for schedule(static)
    for (k = 0; k < n; ++k) {
        double g = 0.0;
        if (W[k] >= wmin && W[k] <= wmax) {
            double cf = bin_coord((double)F[k], bins, fmin, fmax);
            double cw = bin_coord(W[k], bins, wmin, wmax);
            int a0 = (int)floor(cf) - 2, b0 = (int)floor(cw) - 2, a, b;
            for (a = a0; a <= a0 + 4; ++a) {
                double wa;
                if (a < 0 || a >= bins) continue;
                wa = fixed_weight(forder, a, cf);
                if (wa == 0.0) continue;
                for (b = b0; b <= b0 + 4; ++b) {
                    if (b < 0 || b >= bins) continue;
                    double xb = (double)b - cw;
                    if (mode == 0)
                        g += L[a * bins + b] * wa * parzen_deriv(order, xb);
                    else if (mode == 1)
                        g += fabs(L[a * bins + b] * wa * parzen_deriv(order, xb));
                    else
                        g += fabs(L[a * bins + b]) *
                             (fabs(parzen_deriv(forder, (double)a - cf) * parzen_deriv(order, xb)) +
                              fabs(wa * parzen_deriv2(order, xb)));
                }
            }
            g *= (mode ? fabs(weight) : weight) * s / N;
        }
        gW[k] = accumulate ? gW[k] + g : g;
    }
}

/* ------------------------------------------------------------------------ */
/* LNCC (Key design 2)                                                      */
/* ------------------------------------------------------------------------ */

/* Readings: w odd, r = w/2, window = the w^3 cube centred on the voxel, zero
 * padding outside the volume, n = w^3 for every voxel, and the squared local
 * correlation cc = cross^2 / (v_F v_W + eps) with
 *   cross = s_FW - s_F s_W / n,  v_F = s_FF - s_F^2 / n,  v_W = s_WW - s_W^2 / n
 * where s_* are window sums of the moment images F, W, F^2, W^2, FW.
 * Loss = -weight * (1/N) sum_x cc(x). */

/* Window sums of the five moment images for centre planes [za, zb). out holds
 * 5 consecutive blocks of (zb - za) planes: s_F, s_W, s_FF, s_WW, s_FW. The
 * cube sum is evaluated as a sum over z of sums over y of sums over x. */
static void lncc_window_sums(const float *F, const double *W, int64_t nx, int64_t ny, int64_t nz, int r,
                             int64_t za, int64_t zb, double *out) {
    int64_t pl = nx * ny;
    int64_t ia = za - r < 0 ? 0 : za - r, ib = zb + r > nz ? nz : zb + r; /* input planes used */
    int64_t nin = ib - ia, nout = zb - za, z;
    double *sx = (double *)calloc((size_t)(5 * nin * pl), sizeof(double)); /* sums over x */
    double *sxy = (double *)calloc((size_t)(5 * nin * pl), sizeof(double)); /* then over y */
#pragma omp parallel for schedule(dynamic, 1)
    for (z = ia; z < ib; ++z) {
        int64_t y, x, d, m;
        for (y = 0; y < ny; ++y)
            for (x = 0; x < nx; ++x) {
                double acc[5] = {0, 0, 0, 0, 0};
                for (d = -r; d <= r; ++d) {
                    int64_t xx = x + d, q;
                    double f, g;
                    if (xx < 0 || xx >= nx) continue;
                    q = z * pl + y * nx + xx;
                    f = (double)F[q];
                    g = W[q];
                    acc[0] += f;
                    acc[1] += g;
                    acc[2] += f * f;
                    acc[3] += g * g;
                    acc[4] += f * g;
                }
                for (m = 0; m < 5; ++m) sx[(m * nin + (z - ia)) * pl + y * nx + x] = acc[m];
            }
        for (y = 0; y < ny; ++y)
            for (x = 0; x < nx; ++x)
                for (m = 0; m < 5; ++m) {
                    double acc = 0.0;
                    for (d = -r; d <= r; ++d) {
                        int64_t yy = y + d;
                        if (yy < 0 || yy >= ny) continue;
                        acc += sx[(m * nin + (z - ia)) * pl + yy * nx + x];
                    }
                    sxy[(m * nin + (z - ia)) * pl + y * nx + x] = acc;
                }
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (z = za; z < zb; ++z) {
        int64_t q, m, d;
        for (m = 0; m < 5; ++m)
            for (q = 0; q < pl; ++q) {
                double acc = 0.0;
                for (d = -r; d <= r; ++d) {
                    int64_t zz = z + d;
                    if (zz < 0 || zz >= nz) continue;
                    acc += sxy[(m * nin + (zz - ia)) * pl + q];
                }
                out[(m * nout + (z - za)) * pl + q] = acc;
            }
    }
    free(sx);
    free(sxy);
}

/* cc and its partial derivatives with respect to the window sums:
 *   d[0] = dcc/ds_FW = 2 cross / D
 *   d[1] = dcc/ds_WW = -cross^2 v_F / D^2
 *   d[2] = dcc/ds_W  = -2 cross s_F / (n D) + 2 cross^2 v_F s_W / (n D^2)
 * with D = v_F v_W + eps. */
static double lncc_cc(const double s[5], double n, double eps, double d[3]) {
    double cross = s[4] - s[0] * s[1] / n;
    double vf = s[2] - s[0] * s[0] / n;
    double vw = s[3] - s[1] * s[1] / n;
    double D = vf * vw + eps;
    if (d) {
        d[0] = 2.0 * cross / D;
        d[1] = -cross * cross * vf / (D * D);
        d[2] = -2.0 * cross * s[0] / (n * D) + 2.0 * cross * cross * vf * s[1] / (n * D * D);
    }
    return cross * cross / D;
}

/* cc(x) for centres in planes [z_lo, z_hi), written into the full volume cc. */
ORC_API void orc_lncc_cc(const float *F, const double *W, const int64_t *dims, int win, double eps,
                         int64_t z_lo, int64_t z_hi, double *cc) {
    int64_t nx = dims[0], ny = dims[1], nz = dims[2], pl = nx * ny, nr = z_hi - z_lo, z;
    int r = win / 2;
    double n = (double)win * win * win;
    double *s;
    if (nr <= 0) return;
    s = (double *)malloc((size_t)(5 * nr * pl) * sizeof(double));
    lncc_window_sums(F, W, nx, ny, nz, r, z_lo, z_hi, s);
#pragma omp parallel for schedule(static)
    for (z = 0; z < nr; ++z) {
        int64_t q, m;
        for (q = 0; q < pl; ++q) {
            double v[5];
            for (m = 0; m < 5; ++m) v[m] = s[(m * nr + z) * pl + q];
            cc[(z_lo + z) * pl + q] = lncc_cc(v, n, eps, NULL);
        }
    }
    free(s);
}

/* Sum of cc over centres in planes [z_lo, z_hi), summed in plane order. */
ORC_API double orc_lncc_sum(const float *F, const double *W, const int64_t *dims, int win, double eps,
                            int64_t z_lo, int64_t z_hi) {
    int64_t nx = dims[0], ny = dims[1], nz = dims[2], pl = nx * ny, nr = z_hi - z_lo, z;
    int r = win / 2;
    double n = (double)win * win * win, total = 0.0;
    double *s, *part;
    if (nr <= 0) return 0.0;
    s = (double *)malloc((size_t)(5 * nr * pl) * sizeof(double));
    part = (double *)calloc((size_t)nr, sizeof(double));
    lncc_window_sums(F, W, nx, ny, nz, r, z_lo, z_hi, s);
#pragma omp parallel for schedule(static)
    for (z = 0; z < nr; ++z) {
        int64_t q, m;
        for (q = 0; q < pl; ++q) {
            double v[5];
            for (m = 0; m < 5; ++m) v[m] = s[(m * nr + z) * pl + q];
            part[z] += lncc_cc(v, n, eps, NULL);
        }
    }
    for (z = 0; z < nr; ++z) total += part[z];
    free(s);
    free(part);
    return total;
}

/* Gradient of loss = -weight * (1/N) sum_x cc(x) with respect to W(y), for
 * y in planes [z_lo, z_hi). W(y) enters s_W, s_WW and s_FW of every window
 * containing y, so with the same zero-padded box (symmetric, hence its own
 * adjoint) over centres x inside the volume:
 *   gW(y) = -(weight/N) [ box(dcc/ds_W) + 2 W(y) box(dcc/ds_WW) + F(y) box(dcc/ds_FW) ](y).
 * gW is a full volume; accumulate != 0 adds. */
ORC_API void orc_lncc_grad(const float *F, const double *W, const int64_t *dims, int win, double eps,
                           double weight, double N, int64_t z_lo, int64_t z_hi, double *gW, int accumulate) {
    int64_t nx = dims[0], ny = dims[1], nz = dims[2], pl = nx * ny;
    int r = win / 2;
    double n = (double)win * win * win;
    int64_t ca = z_lo - r < 0 ? 0 : z_lo - r, cb = z_hi + r > nz ? nz : z_hi + r; /* centre planes */
    int64_t nc = cb - ca, z;
    double *s, *coef, *bx, *bxy;
    if (z_hi <= z_lo) return;
    s = (double *)malloc((size_t)(5 * nc * pl) * sizeof(double));
    coef = (double *)malloc((size_t)(3 * nc * pl) * sizeof(double));
    lncc_window_sums(F, W, nx, ny, nz, r, ca, cb, s);
#pragma omp parallel for schedule(static)
    for (z = 0; z < nc; ++z) {
        int64_t q, m;
        for (q = 0; q < pl; ++q) {
            double v[5], d[3];
            for (m = 0; m < 5; ++m) v[m] = s[(m * nc + z) * pl + q];
            lncc_cc(v, n, eps, d);
            for (m = 0; m < 3; ++m) coef[(m * nc + z) * pl + q] = d[m];
        }
    }
    /* box of the three coefficient fields over centres inside the volume, as
     * nested axis sums (x, then y, then z), at the output planes */
    bx = (double *)malloc((size_t)(3 * nc * pl) * sizeof(double));
    bxy = (double *)malloc((size_t)(3 * nc * pl) * sizeof(double));
#pragma omp parallel for schedule(static)
    for (z = 0; z < nc; ++z) {
        int64_t y, x, d;
        int m;
        for (m = 0; m < 3; ++m)
            for (y = 0; y < ny; ++y)
                for (x = 0; x < nx; ++x) {
                    double acc = 0.0;
                    for (d = -r; d <= r; ++d)
                        if (x + d >= 0 && x + d < nx) acc += coef[(m * nc + z) * pl + y * nx + x + d];
                    bx[(m * nc + z) * pl + y * nx + x] = acc;
                }
        for (m = 0; m < 3; ++m)
            for (y = 0; y < ny; ++y)
                for (x = 0; x < nx; ++x) {
                    double acc = 0.0;
                    for (d = -r; d <= r; ++d)
                        if (y + d >= 0 && y + d < ny) acc += bx[(m * nc + z) * pl + (y + d) * nx + x];
                    bxy[(m * nc + z) * pl + y * nx + x] = acc;
                }
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (z = z_lo; z < z_hi; ++z) {
        int64_t q, d;
        for (q = 0; q < pl; ++q) {
            double b[3] = {0, 0, 0}, g;
            int64_t lin = z * pl + q;
            int m;
            for (d = -r; d <= r; ++d) {
                int64_t zz = z + d;
                if (zz < 0 || zz >= nz) continue;
                for (m = 0; m < 3; ++m) b[m] += bxy[(m * nc + (zz - ca)) * pl + q];
            }
            g = -(weight / N) * (b[2] + 2.0 * W[lin] * b[1] + (double)F[lin] * b[0]);
            gW[lin] = accumulate ? gW[lin] + g : g;
        }
    }
    free(bx);
    free(bxy);
    free(s);
    free(coef);
}

/* The LNCC gradient at single voxels, by direct sums over the w^3 windows (no
 * separable sums, no shared intermediates). F and W are a sub-volume of the
 * full volume (origin org, size sd, both (x, y, z)); it must contain every
 * in-volume voxel within 2r of each point. pts are full-volume coordinates
 * (x, y, z, 3 per point). Positions outside the full volume count as zero. */
static double sub_val_f(const float *F, const int64_t *org, const int64_t *sd, const int64_t *fd, int64_t x,
                        int64_t y, int64_t z) {
    if (x < 0 || y < 0 || z < 0 || x >= fd[0] || y >= fd[1] || z >= fd[2]) return 0.0;
    return (double)F[((z - org[2]) * sd[1] + (y - org[1])) * sd[0] + (x - org[0])];
}
static double sub_val_d(const double *W, const int64_t *org, const int64_t *sd, const int64_t *fd, int64_t x,
                        int64_t y, int64_t z) {
    if (x < 0 || y < 0 || z < 0 || x >= fd[0] || y >= fd[1] || z >= fd[2]) return 0.0;
    return W[((z - org[2]) * sd[1] + (y - org[1])) * sd[0] + (x - org[0])];
}

ORC_API void orc_lncc_grad_at(const float *F, const double *W, const int64_t *org, const int64_t *sd,
                              const int64_t *fd, int win, double eps, double weight, double N, const int64_t *pts,
                              int64_t npts, double *out) {
    int r = win / 2;
    double n = (double)win * win * win;
    int64_t q;
#pragma omp parallel for schedule(dynamic, 1)
    for (q = 0; q < npts; ++q) {
        int64_t py = pts[3 * q + 1], px = pts[3 * q + 0], pz = pts[3 * q + 2];
        double b[3] = {0, 0, 0};
        int64_t cz, cy, cx;
        for (cz = pz - r; cz <= pz + r; ++cz)
            for (cy = py - r; cy <= py + r; ++cy)
                for (cx = px - r; cx <= px + r; ++cx) {
                    double sm[5] = {0, 0, 0, 0, 0}, d[3];
                    int64_t wz, wy, wx;
                    int m;
                    if (cx < 0 || cy < 0 || cz < 0 || cx >= fd[0] || cy >= fd[1] || cz >= fd[2]) continue;
                    for (wz = cz - r; wz <= cz + r; ++wz)
                        for (wy = cy - r; wy <= cy + r; ++wy)
                            for (wx = cx - r; wx <= cx + r; ++wx) {
                                double f = sub_val_f(F, org, sd, fd, wx, wy, wz);
                                double g = sub_val_d(W, org, sd, fd, wx, wy, wz);
                                sm[0] += f;
                                sm[1] += g;
                                sm[2] += f * f;
                                sm[3] += g * g;
                                sm[4] += f * g;
                            }
                    lncc_cc(sm, n, eps, d);
                    for (m = 0; m < 3; ++m) b[m] += d[m];
                }
        out[q] = -(weight / N) *
                 (b[2] + 2.0 * sub_val_d(W, org, sd, fd, px, py, pz) * b[1] + sub_val_f(F, org, sd, fd, px, py, pz) * b[0]);
    }
}

/* ------------------------------------------------------------------------ */
/* Optimiser (Method overview: states m1, m2, a gradient step after Sobolev */
/* smoothing)                                                               */
/* ------------------------------------------------------------------------ */

/* Reading: Adam with bias correction (Kingma & Ba 2015), step t >= 1:
 *   m1 = b1 m1 + (1-b1) g,  m2 = b2 m2 + (1-b2) g^2,
 *   u -= lr * (m1 / (1 - b1^t)) / (sqrt(m2 / (1 - b2^t)) + eps). */
ORC_API void orc_adam(double *u, const double *g, double *m1, double *m2, int64_t n, int step, double lr,
                      double b1, double b2, double eps) {
    double c1 = 1.0 - pow(b1, (double)step), c2 = 1.0 - pow(b2, (double)step);
    int64_t k;
#pragma omp parallel for schedule(static)
    for (k = 0; k < n; ++k) {
        m1[k] = b1 * m1[k] + (1.0 - b1) * g[k];
        m2[k] = b2 * m2[k] + (1.0 - b2) * g[k] * g[k];
        u[k] -= lr * (m1[k] / c1) / (sqrt(m2[k] / c2) + eps);
    }
}

/* Reading of the Sobolev step: the gradient is smoothed with a normalised
 * Gaussian of standard deviation sigma (voxels), taps k = -R..R with
 * R = ceil(3 sigma), zero padding, applied along x, then y, then z (the 3D
 * Gaussian is the product of the three). One scalar volume. */
ORC_API void orc_gauss_smooth(const double *g, const int64_t *dims, double sigma, double *out) {
    int64_t nx = dims[0], ny = dims[1], nz = dims[2], pl = nx * ny, N = pl * nz, z;
    int R = (int)ceil(3.0 * sigma), k;
    double *tap = (double *)malloc((size_t)(2 * R + 1) * sizeof(double)), tot = 0.0;
    double *t1 = (double *)malloc((size_t)N * sizeof(double));
    double *t2 = (double *)malloc((size_t)N * sizeof(double));
    for (k = -R; k <= R; ++k) {
        tap[k + R] = exp(-(double)(k * k) / (2.0 * sigma * sigma));
        tot += tap[k + R];
    }
    for (k = 0; k <= 2 * R; ++k) tap[k] /= tot;
#pragma omp parallel for schedule(static)
    for (z = 0; z < nz; ++z) {
        int64_t y, x, d;
        for (y = 0; y < ny; ++y)
            for (x = 0; x < nx; ++x) {
                double a = 0.0;
                for (d = -R; d <= R; ++d)
                    if (x + d >= 0 && x + d < nx) a += tap[d + R] * g[z * pl + y * nx + x + d];
                t1[z * pl + y * nx + x] = a;
            }
    }
#pragma omp parallel for schedule(static)
    for (z = 0; z < nz; ++z) {
        int64_t y, x, d;
        for (y = 0; y < ny; ++y)
            for (x = 0; x < nx; ++x) {
                double a = 0.0;
                for (d = -R; d <= R; ++d)
                    if (y + d >= 0 && y + d < ny) a += tap[d + R] * t1[z * pl + (y + d) * nx + x];
                t2[z * pl + y * nx + x] = a;
            }
    }
#pragma omp parallel for schedule(static)
    for (z = 0; z < nz; ++z) {
        int64_t q, d;
        for (q = 0; q < pl; ++q) {
            double a = 0.0;
            for (d = -R; d <= R; ++d)
                if (z + d >= 0 && z + d < nz) a += tap[d + R] * t2[(z + d) * pl + q];
            out[z * pl + q] = a;
        }
    }
    free(tap);
    free(t1);
    free(t2);
}
