"""ctypes wrapper of the oracle library (test infrastructure only).

Arrays are numpy: the stored inputs (F, M, u) as float32, every quantity the
oracle computes itself (W, gW, gu, histograms) as float64. Sizes are (nx, ny,
nz) with x fastest, the same as the volumes' C order (nz, ny, nx).

Sampler parameters are the fp32 values a caller hands the HIP library,
widened to fp64: ``prm`` packs A (9, row-major, acting on (x, y, z)), t (3),
S (9), xmin (3), xmax (3).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

_f32 = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64 = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i64 = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_c_i64 = ctypes.c_int64
_c_d = ctypes.c_double
_c_i = ctypes.c_int
_vp = ctypes.c_void_p


def lib():
    """Load the oracle library, building it first only if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        _build.build_oracle()
    L = ctypes.CDLL(_build.LIB)
    L.orc_num_threads.restype = _c_i
    L.orc_set_num_threads.argtypes = [_c_i]
    L.orc_warp_fwd.argtypes = [_f32, _i64, _c_i64, _c_i64, _f32, _i64, _f64, _c_i64, _c_i64, _f64, _vp]
    L.orc_warp_points.argtypes = [_f32, _i64, _c_i64, _c_i64, _f32, _i64, _f64, _i64, _c_i64, _f64, _vp, _vp]
    L.orc_warp_bwd.argtypes = [_f32, _i64, _c_i64, _c_i64, _f32, _i64, _f64, _f64, _c_i64, _c_i64,
                               _vp, _f64, _f64, _vp]
    L.orc_warp_kink_spread.argtypes = [_f32, _i64, _c_i64, _c_i64, _f32, _i64, _f64, _c_d, _f64, _f64]
    L.orc_warp_fwd_chunk.argtypes = [_f32, _i64, _c_i64, _c_i64, _f32, _i64, _f64, _c_i64, _c_i64, _f64]
    L.orc_warp_bwd_points.argtypes = [_f32, _i64, _c_i64, _c_i64, _f32, _i64, _f64, _i64, _c_i64, _f64, _f64]
    L.orc_lncc_grad_at.argtypes = [_f32, _f64, _i64, _i64, _i64, _c_i, _c_d, _c_d, _c_d, _i64, _c_i64, _f64]
    L.orc_mi_hist.argtypes = [_f32, _f64, _c_i64, _c_i, _c_d, _c_d, _c_d, _c_d, _c_i, _c_i, _f64]
    L.orc_mi_finalize.argtypes = [_f64, _c_i, _c_d, _vp]
    L.orc_mi_finalize.restype = _c_d
    L.orc_mi_grad.argtypes = [_f32, _f64, _c_i64, _c_i, _c_d, _c_d, _c_d, _c_d, _c_i, _c_i, _f64, _c_d, _c_d,
                              _f64, _c_i, _c_i]
    L.orc_lncc_cc.argtypes = [_f32, _f64, _i64, _c_i, _c_d, _c_i64, _c_i64, _f64]
    L.orc_lncc_sum.argtypes = [_f32, _f64, _i64, _c_i, _c_d, _c_i64, _c_i64]
    L.orc_lncc_sum.restype = _c_d
    L.orc_lncc_grad.argtypes = [_f32, _f64, _i64, _c_i, _c_d, _c_d, _c_d, _c_i64, _c_i64, _f64, _c_i]
    L.orc_adam.argtypes = [_f64, _f64, _f64, _f64, _c_i64, _c_i, _c_d, _c_d, _c_d, _c_d]
    L.orc_gauss_smooth.argtypes = [_f64, _i64, _c_d, _f64]
    _lib = L
    return L


def num_threads():
    return lib().orc_num_threads()


def set_num_threads(n):
    """Threads of the oracle's parallel loops from now on."""
    lib().orc_set_num_threads(int(n))


def _sz(vol):
    """(nx, ny, nz) of a C-ordered (nz, ny, nx) volume."""
    nz, ny, nx = vol.shape[-3:]
    return np.array([nx, ny, nz], dtype=np.int64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def pack_prm(A, t, S=None, xmin=(-1.0, -1.0, -1.0), xmax=(1.0, 1.0, 1.0)):
    """Sampler parameters as the HIP library receives them (fp32), widened to fp64."""
    S = np.eye(3) if S is None else S
    parts = [np.asarray(A, np.float32).reshape(9), np.asarray(t, np.float32).reshape(3),
             np.asarray(S, np.float32).reshape(9), np.asarray(xmin, np.float32).reshape(3),
             np.asarray(xmax, np.float32).reshape(3)]
    return np.concatenate(parts).astype(np.float64)


def _mn_full(M, slab, mdims):
    if mdims is not None:
        return np.asarray(mdims, dtype=np.int64)
    mn = _sz(M)
    if slab is not None:
        raise ValueError("a slab needs the full moving grid size")
    return mn


def warp_fwd(M, u, prm, slab=None, mdims=None, z_range=None, want_kink=False):
    """W = M~(A x + t + S u(x)) on the output grid of u. slab = (z0, nz) when M
    holds only those planes of a moving image of size mdims (nx, ny, nz)."""
    M = np.ascontiguousarray(M, np.float32)
    u = np.ascontiguousarray(u, np.float32)
    mn = _mn_full(M, slab, mdims)
    on = _sz(u)
    z0, snz = slab if slab is not None else (0, int(mn[2]))
    zl, zh = z_range if z_range is not None else (0, int(on[2]))
    W = np.zeros(u.shape[1:], np.float64)
    kink = np.ones(u.shape[1:], np.float64) if want_kink else None
    lib().orc_warp_fwd(M, mn, z0, snz, u, on, np.ascontiguousarray(prm, np.float64), zl, zh, W, _ptr(kink))
    return (W, kink) if want_kink else W


def warp_points(M, u, prm, idx, slab=None, mdims=None):
    """W, dW/dp_vox (n, 3) and kink distance at linear output indices idx."""
    M = np.ascontiguousarray(M, np.float32)
    u = np.ascontiguousarray(u, np.float32)
    mn = _mn_full(M, slab, mdims)
    z0, snz = slab if slab is not None else (0, int(mn[2]))
    idx = np.ascontiguousarray(idx, np.int64)
    n = idx.size
    W = np.zeros(n, np.float64)
    d = np.zeros((n, 3), np.float64)
    k = np.zeros(n, np.float64)
    lib().orc_warp_points(M, mn, z0, snz, u, _sz(u), np.ascontiguousarray(prm, np.float64), idx, n, W,
                          _ptr(d), _ptr(k))
    return W, d, k


def warp_bwd(M, u, prm, gW, slab=None, mdims=None, z_range=None, want_gu=True):
    """Returns (gu (3, nz, ny, nx) or None, dA (3, 3), dt (3), mag) where mag is
    sum |g_p| |x| over the voxels, a conditioning scale for the affine sums."""
    M = np.ascontiguousarray(M, np.float32)
    u = np.ascontiguousarray(u, np.float32)
    mn = _mn_full(M, slab, mdims)
    on = _sz(u)
    z0, snz = slab if slab is not None else (0, int(mn[2]))
    zl, zh = z_range if z_range is not None else (0, int(on[2]))
    gu = np.zeros(u.shape, np.float64) if want_gu else None
    dA = np.zeros(9, np.float64)
    dt = np.zeros(3, np.float64)
    mag = np.zeros(1, np.float64)
    lib().orc_warp_bwd(M, mn, z0, snz, u, on, np.ascontiguousarray(prm, np.float64),
                       np.ascontiguousarray(gW, np.float64), zl, zh, _ptr(gu), dA, dt, _ptr(mag))
    return gu, dA.reshape(3, 3), dt, float(mag[0])


def warp_kink_spread(M, u, prm, gW, band=1e-4, mdims=None):
    """Per voxel and component, the largest difference between the sampler
    backward's gu in the floor cell and in a cell across a face within `band`
    of the sample (both one-sided derivatives are valid there); zero away from
    faces. Returns (3, nz, ny, nx) fp64."""
    M = np.ascontiguousarray(M, np.float32)
    u = np.ascontiguousarray(u, np.float32)
    mn = _mn_full(M, None, mdims)
    out = np.zeros(u.shape, np.float64)
    lib().orc_warp_kink_spread(M, mn, 0, int(mn[2]), u, _sz(u), np.ascontiguousarray(prm, np.float64), float(band),
                               np.ascontiguousarray(gW, np.float64), out)
    return out


def warp_fwd_chunk(M, u, prm, z_range, slab=None, mdims=None, out=None):
    """W for output planes z_range only, as a (z1-z0, ny, nx) fp64 array."""
    M = np.ascontiguousarray(M, np.float32)
    mn = _mn_full(M, slab, mdims)
    z0, snz = slab if slab is not None else (0, int(mn[2]))
    on = _sz(u)
    zl, zh = z_range
    if out is None:
        out = np.zeros((zh - zl,) + u.shape[2:], np.float64)
    lib().orc_warp_fwd_chunk(M, mn, z0, snz, u, on, np.ascontiguousarray(prm, np.float64), zl, zh, out)
    return out


def warp_bwd_points(M, u, prm, idx, gW_pts, slab=None, mdims=None):
    """gu (n, 3) at linear output indices idx, given gW there."""
    M = np.ascontiguousarray(M, np.float32)
    mn = _mn_full(M, slab, mdims)
    z0, snz = slab if slab is not None else (0, int(mn[2]))
    idx = np.ascontiguousarray(idx, np.int64)
    gu = np.zeros((idx.size, 3), np.float64)
    lib().orc_warp_bwd_points(M, mn, z0, snz, u, _sz(u), np.ascontiguousarray(prm, np.float64), idx, idx.size,
                              np.ascontiguousarray(gW_pts, np.float64), gu)
    return gu


def lncc_grad_at(F_sub, W_sub, origin_zyx, full_shape, pts_zyx, win, eps=1e-5, weight=1.0, N=None):
    """LNCC gradient at points (k, 3) given in (z, y, x) full-volume coordinates,
    from a sub-volume (F_sub float32, W_sub float64) whose first voxel is at
    origin_zyx and which contains every in-volume voxel within 2r of each point."""
    F_sub = np.ascontiguousarray(F_sub, np.float32)
    W_sub = np.ascontiguousarray(W_sub, np.float64)
    nz, ny, nx = full_shape
    N = float(nx * ny * nz) if N is None else float(N)
    org = np.array([origin_zyx[2], origin_zyx[1], origin_zyx[0]], np.int64)
    sd = _sz(F_sub)
    fd = np.array([nx, ny, nz], np.int64)
    p = np.ascontiguousarray(np.asarray(pts_zyx, np.int64)[:, ::-1])
    out = np.zeros(p.shape[0], np.float64)
    lib().orc_lncc_grad_at(F_sub, W_sub, org, sd, fd, win, eps, weight, N, p, p.shape[0], out)
    return out


def _fo(order, forder):
    return order if forder is None else forder


def mi_grad_values(F_vals, W_vals, L, bins=32, frange=(0.0, 1.0), wrange=(0.0, 1.0), weight=1.0, N=None, order=3,
                   forder=None, mode=0):
    """MI gradient at individual samples given the log-ratio table L of the
    whole volume's histogram (N samples). order: the Parzen kernel of W;
    forder: that of F (None: the same). mode 1 or 2: instead of the gradient,
    a conditioning scale for comparing a lower-precision evaluation of its
    sum, |weight| (s/N) times: 1, sum |L_ab kappa_F kappa'| (the magnitude of
    the terms); 2, sum |L_ab| (|kappa_F'| |kappa'| + |kappa_F| |kappa''|) (the
    magnitude of the sum's derivative with respect to the bin coordinates)."""
    F_vals = np.ascontiguousarray(F_vals, np.float32).reshape(-1)
    W_vals = np.ascontiguousarray(W_vals, np.float64).reshape(-1)
    g = np.zeros(F_vals.size, np.float64)
    lib().orc_mi_grad(F_vals, W_vals, F_vals.size, bins, frange[0], frange[1], wrange[0], wrange[1],
                      _fo(order, forder), order,
                      np.ascontiguousarray(L, np.float64), weight, float(N), g, 0, int(mode))
    return g


def mi_hist(F, W, bins=32, frange=(0.0, 1.0), wrange=(0.0, 1.0), order=3, H=None, forder=None):
    F = np.ascontiguousarray(F, np.float32).reshape(-1)
    W = np.ascontiguousarray(W, np.float64).reshape(-1)
    if H is None:
        H = np.zeros((bins, bins), np.float64)
    lib().orc_mi_hist(F, W, F.size, bins, frange[0], frange[1], wrange[0], wrange[1], _fo(order, forder), order, H)
    return H


def mi_finalize(H, N):
    bins = H.shape[0]
    L = np.zeros((bins, bins), np.float64)
    mi = lib().orc_mi_finalize(np.ascontiguousarray(H, np.float64), bins, float(N), _ptr(L))
    return mi, L


def mi_loss_grad(F, W, bins=32, frange=(0.0, 1.0), wrange=(0.0, 1.0), weight=1.0, order=3, want_grad=True,
                 forder=None):
    """loss = -weight * MI(F, W) and its gradient with respect to W. order is
    the Parzen kernel of W and forder that of F (None: the same); forder=0
    with order=3 is Mattes et al.'s original pair."""
    shape = np.shape(W)
    F = np.ascontiguousarray(F, np.float32).reshape(-1)
    W = np.ascontiguousarray(W, np.float64).reshape(-1)
    N = F.size
    H = mi_hist(F, W, bins, frange, wrange, order, forder=forder)
    mi, L = mi_finalize(H, N)
    g = None
    if want_grad:
        g = np.zeros(N, np.float64)
        lib().orc_mi_grad(F, W, N, bins, frange[0], frange[1], wrange[0], wrange[1], _fo(order, forder), order, L,
                          weight, float(N), g, 0, 0)
        g = g.reshape(shape)
    return -weight * mi, g, H


def lncc_sum(F, W, win, eps=1e-5, z_range=None):
    F = np.ascontiguousarray(F, np.float32)
    W = np.ascontiguousarray(W, np.float64)
    zl, zh = z_range if z_range is not None else (0, F.shape[0])
    return lib().orc_lncc_sum(F, W, _sz(F), win, eps, zl, zh)


def lncc_cc(F, W, win, eps=1e-5):
    """The local squared correlation cc at every voxel."""
    F = np.ascontiguousarray(F, np.float32)
    W = np.ascontiguousarray(W, np.float64)
    cc = np.zeros(F.shape, np.float64)
    lib().orc_lncc_cc(F, W, _sz(F), win, eps, 0, F.shape[0], cc)
    return cc


def lncc_loss_grad(F, W, win, eps=1e-5, weight=1.0, want_grad=True):
    """loss = -weight * mean(cc) and its gradient with respect to W."""
    F = np.ascontiguousarray(F, np.float32)
    W = np.ascontiguousarray(W, np.float64)
    N = F.size
    loss = -weight * lncc_sum(F, W, win, eps) / N
    g = None
    if want_grad:
        g = np.zeros(F.shape, np.float64)
        lib().orc_lncc_grad(F, W, _sz(F), win, eps, weight, float(N), 0, F.shape[0], g, 0)
    return loss, g


def lncc_grad_range(F, W, win, eps, weight, N, z_range, gW):
    """Writes the LNCC gradient for planes z_range into the full volume gW."""
    F = np.ascontiguousarray(F, np.float32)
    W = np.ascontiguousarray(W, np.float64)
    lib().orc_lncc_grad(F, W, _sz(F), win, eps, weight, float(N), z_range[0], z_range[1], gW, 0)


def adam(u, g, m1, m2, step, lr, b1=0.9, b2=0.999, eps=1e-8):
    """One Adam step in fp64 on copies; returns (u, m1, m2)."""
    u = np.array(u, np.float64).reshape(-1)
    m1 = np.array(m1, np.float64).reshape(-1)
    m2 = np.array(m2, np.float64).reshape(-1)
    g = np.ascontiguousarray(g, np.float64).reshape(-1)
    lib().orc_adam(u, g, m1, m2, u.size, step, lr, b1, b2, eps)
    return u, m1, m2


def gauss_smooth(g, sigma):
    """Zero-padded separable Gaussian smoothing of one scalar volume."""
    g = np.ascontiguousarray(g, np.float64)
    out = np.zeros_like(g)
    lib().orc_gauss_smooth(g, _sz(g), sigma, out)
    return out


def mse_loss_grad(F, W, weight=1.0, want_grad=True):
    """Mean squared error as a similarity term and its gradient.

    Page "A Scalable Distributed Framework for Multimodal GigaVoxel Image
    Registration", Background and motivation: MSE is one of the similarity
    terms C(F, M o phi); Key design 5: it is a per-voxel loss, so shard sums
    of the same expression add up to the whole. Reading taken: the mean over
    the N output voxels, C = weight * (1/N) sum (W - F)^2, and
    dC/dW = 2 weight (W - F) / N. Returns (loss, gW or None) in fp64."""
    d = np.asarray(W, np.float64) - np.asarray(F, np.float64)
    N = d.size
    loss = float(weight) * float(np.sum(d * d)) / N
    gW = (2.0 * float(weight) / N) * d if want_grad else None
    return loss, gW


def compose(uf, v, prm, mdims=None):
    """Warp composition by the composite sampler, per component c:
        w_c(x) = v_c(x) + uf_c~(A x + t + S v(x)),
    uf~ the trilinear, zero-padded interpolation of the field uf on its own
    grid (the moving grid of the sampler). With phi_v(x) = A x + t + S v(x)
    and phi_u(y) = y + S uf(y) this is phi_u(phi_v(x)) = A x + t + S w(x).

    Page "A Scalable Distributed Framework for Multimodal GigaVoxel Image
    Registration", Background and motivation (warp composition is one of the
    three profiled memory bottlenecks) and Key design 1 (the sampler that
    evaluates each component at the composite position). Each component is
    the oracle's own sampler applied to uf_c with v as the displacement.
    Returns w (3, nz, ny, nx) in fp64 on the grid of v."""
    uf = np.ascontiguousarray(uf, np.float32)
    v = np.ascontiguousarray(v, np.float32)
    if uf.shape[0] != 3 or v.shape[0] != 3:
        raise ValueError("uf and v are 3-component fields")
    w = np.empty(v.shape, np.float64)
    for c in range(3):
        w[c] = v[c].astype(np.float64) + warp_fwd(uf[c], v, prm, mdims=mdims)
    return w
