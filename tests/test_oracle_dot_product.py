"""Dot-product pins of the oracle's whole gradient: for random smooth
directions, the central difference of the oracle's loss (sampler, then MI
and/or LNCC) equals the inner product with the oracle's gradient with
respect to u, A and t. This checks the sampler backward, both loss
gradients and their sum as one linear map on volumes well beyond the sizes
of the per-voxel finite-difference pins, with a non-identity S (the S^T in
gu) and a window larger than 11.

Everything is fp64 except u, which the oracle takes in fp32 like the
kernels: the u steps are taken on the fp32 values and the inner product
uses the step actually taken. The sampler's kinks make the loss piecewise
smooth: a sample that crosses a cell face within the step changes the
difference by the jump in slope times the overshoot (a 1e-3 relative error
at steps of 1e-5 voxel here), so the steps move samples by at most about
1e-6 voxel, where no sample of these volumes crosses a face.
"""
import numpy as np
import pytest

from non_gemm_voxel_amd import synth


def _prm(A, t, S):
    """fp64 sampler parameters (A, t, S, the output grid's x bounds)."""
    return np.concatenate([np.asarray(A, np.float64).ravel(), np.asarray(t, np.float64),
                           np.asarray(S, np.float64).ravel(), -np.ones(3), np.ones(3)])


def _loss_grad(orc, F, M, u, prm, bins, win):
    W = orc.warp_fwd(M, u, prm)
    loss, gW = 0.0, np.zeros_like(W)
    if bins:
        l, g, _ = orc.mi_loss_grad(F, W, bins=bins)
        loss += l
        gW += g
    if win:
        l, g = orc.lncc_loss_grad(F, W, win)
        loss += l
        gW += g
    return loss, gW


def _loss(orc, F, M, u, prm, bins, win):
    W = orc.warp_fwd(M, u, prm)
    loss = 0.0
    if bins:
        loss += orc.mi_loss_grad(F, W, bins=bins, want_grad=False)[0]
    if win:
        loss += orc.lncc_loss_grad(F, W, win, want_grad=False)[0]
    return loss


@pytest.mark.parametrize("shape,bins,win,S", [
    ((18, 20, 22), 32, 5, np.eye(3)),
    ((16, 18, 21), None, 13, np.diag([0.5, 1.0, 2.0])),
    ((20, 17, 19), 16, None, np.array([[1.0, 0.2, 0.0], [0.0, 0.8, 0.1], [0.1, 0.0, 1.2]])),
])
def test_directional_derivatives(orc, shape, bins, win, S):
    seed = shape[0]
    F = synth.random_volume(shape, seed, 0).numpy()
    # a smooth moving image (a blurred random volume) so the loss varies smoothly with u
    M = orc.gauss_smooth(synth.random_volume(shape, seed, 1).numpy().astype(np.float64), 1.5).astype(np.float32)
    r = synth.scalars(seed, 2, 12)
    A = synth.euler_rotation(*(0.1 * (2 * r[:3] - 1))) @ np.diag(1.0 + 0.04 * (2 * r[3:6] - 1))
    t = 0.03 * (2 * r[6:9] - 1)
    prm = _prm(A, t, S)
    unit = 2.0 / (max(shape) - 1)
    u0 = (0.4 * unit * synth.random_field(shape, seed, 3, 1.0)).numpy().astype(np.float32)
    du = (unit * synth.random_field(shape, seed, 4, 1.0)).numpy()
    _, gW = _loss_grad(orc, F, M, u0, prm, bins, win)
    gu, dA, dt, _ = orc.warp_bwd(M, u0, prm, gW)
    # u: the fp32 points actually sampled
    h = 1e-6
    up = (u0 + h * du).astype(np.float32)
    um = (u0 - h * du).astype(np.float32)
    step = up.astype(np.float64) - um.astype(np.float64)
    fd = _loss(orc, F, M, up, prm, bins, win) - _loss(orc, F, M, um, prm, bins, win)
    an = float(np.sum(gu * step))
    mag = float(np.sum(np.abs(gu * step)))
    assert abs(fd - an) <= 1e-5 * abs(an) + 1e-9 * mag, (fd, an, mag)
    # A and t (fp64 parameters)
    rng = np.random.default_rng(seed)
    hA = 1e-7
    for what, dA_dir, dt_dir, grad in (("A", rng.uniform(-1, 1, (3, 3)), np.zeros(3), dA),
                                       ("t", np.zeros((3, 3)), rng.uniform(-1, 1, 3), dt)):
        pp = _prm(A + hA * dA_dir, t + hA * dt_dir, S)
        pm = _prm(A - hA * dA_dir, t - hA * dt_dir, S)
        fd = _loss(orc, F, M, u0, pp, bins, win) - _loss(orc, F, M, u0, pm, bins, win)
        d = dA_dir if what == "A" else dt_dir
        an = float(np.sum(np.asarray(grad).reshape(d.shape) * 2 * hA * d))
        assert abs(fd - an) <= 1e-5 * abs(an) + 1e-14, (what, fd, an)
