"""Dot-product tests of the whole step's gradient at sizes where the oracle
cannot give every voxel: for a random smooth direction du, the central
difference of the kernels' own loss, (L(u + h du) - L(u - h du)) / 2h, must
equal <gu, du> from the kernels' backward; likewise for A and t against dA
and dt. This pins the sampler backward, the MI and LNCC gradients and their
sum as one linear map at the full 640x768x640 size, and the slab sequence's
gradient on the gigavoxel recipe (at a reduced size), through the C ABI.

The loss is piecewise smooth in u (trilinear interpolation has kinks at cell
faces), so the base point u0 is a random smooth field that keeps samples
off the lattice, and h moves samples by at most 2.5e-4 voxel: the samples that cross a
face within that distance perturb the difference by well under the bar
(relative 2e-3 of |<g, du>| plus 1e-6 of sum |g du|, the latter covering the
fp32 rounding of W in each loss evaluation).
"""
import numpy as np
import pytest
import torch

from non_gemm_voxel_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(*a):
    print("[case]", *a, flush=True)


def _loss(st):
    st.forward()
    return float(st.loss[0] if st.bins else 0.0) + float(st.loss[1] if st.win else 0.0)


def _check(fd, an, mag, what):
    _say(what, f"difference {fd:.9e} analytic {an:.9e} (sum |terms| {mag:.3e})")
    assert abs(fd - an) <= 2e-3 * abs(an) + 1e-6 * mag, (what, fd, an)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wl_name,shape,slabs", [
    ("c2", (40, 48, 56), 1),
    ("c3", (48, 48, 48), 1),
    ("c5", (96, 112, 96), 8),
    ("c4", None, 1),
])
def test_directional_derivatives(wl_name, shape, slabs):
    from non_gemm_voxel_amd import ngv
    from non_gemm_voxel_amd.step import RegistrationStep
    wl = synth.WORKLOADS[wl_name]
    c = synth.make_case(wl, shape=shape, device=DEV)
    shp = c.shape
    _say("dot product", wl_name, shp, "slabs", slabs)
    # the stored path: gu, dA, dt written by the sampler backward (slab by slab)
    st = RegistrationStep(c.F, c.M, c.A, c.t, bins=wl.bins, win=wl.win, lr=c.lr, slabs=slabs, fused=False,
                          mi_in_backward=False)
    unit = 2.0 / (max(shp) - 1)  # one voxel of the longest axis in normalised units
    u0 = synth.random_field(shp, wl.seed, 60, 0.4 * unit, device=DEV)
    du = synth.random_field(shp, wl.seed, 61, 1.0 * unit, device=DEV)
    h = 2.5e-4
    st.u.copy_(u0)
    _loss(st)
    st.backward()
    torch.cuda.synchronize()
    gu = st.gu.clone()
    gA = st.gA.cpu().numpy().reshape(3, 3)
    gt = st.gt.cpu().numpy()
    prod = gu.double() * du.double()
    an = float(prod.sum())
    mag = float(prod.abs().sum())
    st.u.copy_(u0 + h * du)
    lp = _loss(st)
    st.u.copy_(u0 - h * du)
    lm = _loss(st)
    _check((lp - lm) / (2 * h), an, mag, f"{wl_name} u")
    # the affine part at u0: a random direction in A and in t (the sampler
    # receives fp32 parameters, so the steps are taken on the fp32 values)
    st.u.copy_(u0)
    rng = np.random.default_rng(wl.seed)
    dA = rng.uniform(-1.0, 1.0, (3, 3))
    dt = rng.uniform(-1.0, 1.0, 3)
    hA = 5e-6
    A0, t0 = np.asarray(c.A, np.float64), np.asarray(c.t, np.float64)
    for what, dir_A, dir_t, grad in (("A", dA, np.zeros(3), gA), ("t", np.zeros((3, 3)), dt, gt)):
        Ap, Am = (A0 + hA * dir_A).astype(np.float32), (A0 - hA * dir_A).astype(np.float32)
        tp, tm = (t0 + hA * dir_t).astype(np.float32), (t0 - hA * dir_t).astype(np.float32)
        # the step actually taken in fp32
        step = (Ap.astype(np.float64) - Am.astype(np.float64)) if what == "A" else \
            (tp.astype(np.float64) - tm.astype(np.float64))
        st.xf = ngv.make_xform(Ap, tp)
        lp = _loss(st)
        st.xf = ngv.make_xform(Am, tm)
        lm = _loss(st)
        an = float(np.sum(grad * step))
        _check(lp - lm, an, float(np.sum(np.abs(grad * step))), f"{wl_name} {what}")
    del st
    torch.cuda.empty_cache()
