"""Degenerate and boundary sizes through the C ABI, against the oracle: axes
of one voxel (the implicit grid then sits at x_min on that axis), moving
grids of one voxel along an axis, volumes smaller than the LNCC window, a
single voxel, extents one past a tile (64 + 1 columns, 4 + 1 rows), and
samples far outside the moving grid.
"""
import numpy as np
import pytest
import torch

from non_gemm_voxel_amd import synth
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def ngv():
    from non_gemm_voxel_amd import ngv as lib
    lib.lib()
    return lib


def _say(*a):
    print("[case]", *a, flush=True)


def _dev(x):
    return torch.as_tensor(np.ascontiguousarray(x)).to(DEV)


def _affine(seed):
    r = synth.scalars(seed, 1, 12)
    R = synth.euler_rotation(*(0.1 * (2 * r[:3] - 1)))
    A = R @ np.diag(1.0 + 0.05 * (2 * r[3:6] - 1))
    t = 0.05 * (2 * r[6:9] - 1)
    return A.astype(np.float32), t.astype(np.float32)


SAMPLER_CASES = [
    # (output shape, moving shape), (nz, ny, nx)
    ((1, 1, 9), (1, 1, 9)),
    ((1, 13, 1), (3, 5, 7)),
    ((5, 1, 1), (1, 1, 1)),
    ((2, 3, 2), (4, 4, 4)),
    ((4, 5, 65), (6, 6, 60)),
    ((9, 9, 9), (1, 9, 9)),
]


@pytest.mark.parametrize("case", range(len(SAMPLER_CASES)))
def test_sampler_degenerate_shapes(orc, ngv, case):
    oshape, mshape = SAMPLER_CASES[case]
    _say("sampler", oshape, mshape)
    M = synth.random_volume(mshape, 30 + case, 0).numpy()
    A, t = _affine(30 + case)
    u = (0.05 * synth.random_field(oshape, 30 + case, 1, 1.0)).numpy()
    gW = synth.random_volume(oshape, 30 + case, 2, -1.0, 1.0).numpy()
    xf = ngv.make_xform(A, t)
    prm = orc.pack_prm(A, t)
    W = torch.empty(oshape, device=DEV)
    ngv.ngv_warp_fwd(_dev(M), _dev(u), xf, W)
    gu = torch.empty((3,) + oshape, device=DEV)
    gA = torch.zeros(9, dtype=torch.float64, device=DEV)
    gt = torch.zeros(3, dtype=torch.float64, device=DEV)
    ngv.ngv_warp_bwd(_dev(M), _dev(u), xf, _dev(gW), gu, gA, gt)
    torch.cuda.synchronize()
    W_ref, kink = orc.warp_fwd(M, u, prm, want_kink=True)
    P.elementwise(P.to_np(W), W_ref, P.RTOL_W, what="W")
    gu_ref, dA, dt, mag = orc.warp_bwd(M, u, prm, gW.astype(np.float64))
    mask = P.off_kink(kink)
    for k in range(3):
        P.elementwise(P.to_np(gu[k]), gu_ref[k], P.RTOL_GRAD, mask=mask, what=f"gu[{k}]")
    P.affine_sums(P.to_np(gA), dA.ravel(), mag, "dA")
    P.affine_sums(P.to_np(gt), dt, mag, "dt")


@pytest.mark.parametrize("shape", [(1, 1, 1), (1, 1, 5), (2, 1, 3), (3, 4, 5)])
def test_losses_on_tiny_volumes(orc, ngv, shape):
    """MI, LNCC (window larger than the volume) and MSE on a few voxels."""
    _say("losses", shape)
    F = synth.random_volume(shape, 40, 0).numpy()
    W = (0.5 * F + 0.5 * synth.random_volume(shape, 40, 1).numpy()).astype(np.float32)
    Fd, Wd = _dev(F), _dev(W)
    l_mi = torch.zeros(1, dtype=torch.float64, device=DEV)
    g_mi = torch.empty(shape, device=DEV)
    ngv.ngv_mi_loss_fwd_bwd(Fd, Wd, l_mi, g_mi, bins=16)
    l_cc = torch.zeros(1, dtype=torch.float64, device=DEV)
    g_cc = torch.empty(shape, device=DEV)
    ngv.ngv_lncc_loss_fwd_bwd(Fd, Wd, l_cc, g_cc, win=9)
    l_ms = torch.zeros(1, dtype=torch.float64, device=DEV)
    g_ms = torch.empty(shape, device=DEV)
    ngv.ngv_mse_loss_fwd_bwd(Fd, Wd, l_ms, g_ms)
    torch.cuda.synchronize()
    W64 = W.astype(np.float64)
    lo, go, _ = orc.mi_loss_grad(F, W64, bins=16)
    # one sample: the joint factorises and MI is zero; the kernel's fp32 spline
    # weights sum to 1 only within a few ulps, so its mass and hence its MI are
    # off by ~1e-7 (absolute; a loss of order 1 sees it as 1e-7 relative)
    assert abs(float(l_mi[0]) - lo) <= 1e-4 * abs(lo) + 1e-6
    if F.size == 1:
        # and its gradient is zero: the kernel's is its log-ratio table's
        # rounding (~1e-7) times the bin scale (bins - 5) / range and 1/N
        assert np.abs(P.to_np(g_mi)).max() <= 1e-6 * (16 - 5)
    else:
        P.elementwise(P.to_np(g_mi), go, P.RTOL_GRAD, what="MI gW")
    lo, go = orc.lncc_loss_grad(F, W64, 9)
    P.scalar(float(l_cc[0]), lo, what="LNCC loss")
    P.elementwise(P.to_np(g_cc), go, P.RTOL_GRAD, what="LNCC gW")
    lo, go = orc.mse_loss_grad(F, W64)
    P.scalar(float(l_ms[0]), lo, what="MSE loss")
    P.elementwise(P.to_np(g_ms), go, P.RTOL_GRAD, what="MSE gW")


@pytest.mark.parametrize("shape", [(1, 1, 1), (1, 2, 3)])
def test_adam_and_compose_on_tiny_fields(orc, ngv, shape):
    _say("adam/compose", shape)
    u = (0.1 * synth.random_volume((3,) + shape, 41, 0, -1.0, 1.0)).numpy()
    g = synth.random_volume((3,) + shape, 41, 1, -1.0, 1.0).numpy()
    z = np.zeros_like(u)
    ud, m1, m2 = _dev(u), _dev(z), _dev(z)
    ngv.ngv_adam_step(ud, _dev(g), m1, m2, step=1, lr=0.01)
    v = (0.2 * synth.random_volume((3,) + shape, 41, 2, -1.0, 1.0)).numpy()
    uf = synth.random_volume((3,) + shape, 41, 3, -1.0, 1.0).numpy()
    w = torch.empty((3,) + shape, device=DEV)
    A, t = _affine(41)
    ngv.ngv_warp_compose(_dev(uf), _dev(v), ngv.make_xform(A, t), w)
    torch.cuda.synchronize()
    ur, m1r, m2r = orc.adam(u, g, z, z, 1, 0.01)
    P.elementwise(P.to_np(ud).ravel(), ur, P.RTOL_GRAD, what="u")
    P.elementwise(P.to_np(m1).ravel(), m1r, P.RTOL_GRAD, what="m1")
    P.elementwise(P.to_np(m2).ravel(), m2r, P.RTOL_GRAD, what="m2")
    ref = orc.compose(uf, v, orc.pack_prm(A, t))
    for c in range(3):
        P.elementwise(P.to_np(w[c]), ref[c], P.RTOL_W, what=f"w[{c}]")


@pytest.mark.parametrize("case", range(len(SAMPLER_CASES)))
def test_fused_backward_adam_degenerate_shapes(ngv, case):
    """The sampler backward fused with the Adam step on the same degenerate
    shapes (blocks with one item or none, rows and columns past the grid's
    edge, one-plane items) equals the backward and the Adam step as two
    calls, bit for bit."""
    oshape, mshape = SAMPLER_CASES[case]
    _say("fused backward + adam", oshape, mshape)
    M = _dev(synth.random_volume(mshape, 50 + case, 0).numpy())
    A, t = _affine(50 + case)
    vol = (3,) + oshape
    u = (0.05 * synth.random_field(oshape, 50 + case, 1, 1.0)).numpy()
    gW = _dev(synth.random_volume(oshape, 50 + case, 2, -1.0, 1.0).numpy())
    m1 = synth.random_volume(vol, 50 + case, 3, -0.1, 0.1).numpy()
    m2 = synth.random_volume(vol, 50 + case, 4, 0.0, 0.1).numpy()
    xf = ngv.make_xform(A, t)
    out = []
    for fused in (False, True):
        ud, m1d, m2d = _dev(u), _dev(m1), _dev(m2)
        gA = torch.zeros(9, dtype=torch.float64, device=DEV)
        gt = torch.zeros(3, dtype=torch.float64, device=DEV)
        if fused:
            ngv.ngv_warp_bwd_adam(M, ud, xf, gW, m1d, m2d, 2, 0.01, gA, gt)
        else:
            gu = torch.empty(vol, device=DEV)
            ngv.ngv_warp_bwd(M, ud, xf, gW, gu, gA, gt)
            ngv.ngv_adam_step(ud, gu, m1d, m2d, 2, 0.01)
        out.append((ud, m1d, m2d, gA, gt))
    torch.cuda.synchronize()
    for a, b, what in zip(out[0], out[1], ("u", "m1", "m2", "dA", "dt")):
        assert torch.equal(a, b), what


def test_sampler_far_samples(orc, ngv):
    """Samples far outside the moving grid, against the oracle: displacements
    of 1e2 to 1e9 (normalised units, so offsets up to about 3e10 voxels) on a
    quarter of the components. Such samples read zero and get no gradient;
    the kernels clamp the offset before taking its 32-bit floor, so the
    corner index cannot wrap into the grid. The rest of the volume, and the
    slab sequence whose z-range bound the far samples stretch, are as
    usual."""
    oshape, mshape = (6, 9, 70), (7, 8, 66)
    _say("far samples", oshape, mshape)
    M = synth.random_volume(mshape, 77, 0).numpy()
    A, t = _affine(77)
    u = (0.05 * synth.random_field(oshape, 77, 1, 1.0)).numpy()
    pick = synth.random_volume((3,) + oshape, 77, 3).numpy()
    sign = np.where(synth.random_volume((3,) + oshape, 77, 4).numpy() < 0.5, -1.0, 1.0)
    scales = np.array([1e2, 1e5, 3e7, 1e9])
    for j, s in enumerate(scales):
        sel = (pick >= j / 16) & (pick < (j + 1) / 16)
        u[sel] = (sign[sel] * s).astype(np.float32)
    assert (np.abs(u) >= 1e2).mean() > 0.2
    gW = synth.random_volume(oshape, 77, 2, -1.0, 1.0).numpy()
    xf = ngv.make_xform(A, t)
    prm = orc.pack_prm(A, t)
    Md, ud = _dev(M), _dev(u)
    W = torch.full(oshape, float("nan"), device=DEV)
    ngv.ngv_warp_fwd(Md, ud, xf, W)
    gu = torch.empty((3,) + oshape, device=DEV)
    gA = torch.zeros(9, dtype=torch.float64, device=DEV)
    gt = torch.zeros(3, dtype=torch.float64, device=DEV)
    ngv.ngv_warp_bwd(Md, ud, xf, _dev(gW), gu, gA, gt)
    # the forward slab sequence over three slabs
    bounds = [(0, 2), (2, 5), (5, 7)]
    zr = torch.empty(2, dtype=torch.float64, device=DEV)
    ngv.ngv_warp_zrange(ud, xf, zr, mshape)
    Ws = torch.full(oshape, 7.0, device=DEV)
    for z0, z1 in bounds:
        ngv.ngv_warp_fwd_slab(Md[z0:z1].contiguous(), ud, xf, Ws, (z0, z1 - z0, zr), mdims=mshape)
    torch.cuda.synchronize()
    W_ref, kink = orc.warp_fwd(M, u, prm, want_kink=True)
    far = (np.abs(u) >= 1e2).any(axis=0)
    assert (W_ref[far] == 0).all()
    P.elementwise(P.to_np(W), W_ref, P.RTOL_W, what="W")
    P.elementwise(P.to_np(Ws), W_ref, P.RTOL_W, what="W by slabs")
    assert (P.to_np(W)[far] == 0).all() and (P.to_np(Ws)[far] == 0).all()
    gu_ref, dA, dt, mag = orc.warp_bwd(M, u, prm, gW.astype(np.float64))
    mask = P.off_kink(kink)
    for k in range(3):
        P.elementwise(P.to_np(gu[k]), gu_ref[k], P.RTOL_GRAD, mask=mask, what=f"gu[{k}]")
        assert (P.to_np(gu[k])[far] == 0).all()
    P.affine_sums(P.to_np(gA), dA.ravel(), mag, "dA")
    P.affine_sums(P.to_np(gt), dt, mag, "dt")
